// Stage 1: candidate-index normalisation on gfx950.
//
// "5.1.1 · 从索引到 Kernel" §1.1 eq. (1) (S = unique(D ∪ W ∪ A), dedup is
// required), §1.2 eq. (2) (token -> logical block, block union and in-page
// mask), §7.3 (dedup by logical identity with a bitmap; eq. (16)-(17)),
// §7.4 eq. (19) (CSR row pointers); "HiSparse" walkthrough, token -> global
// slot id conversion (slot = table[block] * page + offset, -1 propagation).
//
// The work is small (a few thousand ids per token) and latency bound, so
// the kernels are built to keep the chain of dependent memory round trips
// short rather than to stream bytes.
//
// normalize_kernel: one 256-thread workgroup per query token holds a bitmap
// of the token's visible positions in LDS (plus the request's page-table row
// when it fits).  The token's D entries are loaded before anything else (they
// do not depend on the request), then D, W and A set bits with LDS atomicOr
// (duplicates collapse for free).  S is emitted in ascending order by each
// wave over its own run of 64-word batches: a wave scan of the words'
// popcounts gives every word its output offset; sparse words are walked by
// their own lane, dense ones (the window) by the whole wave, one lane per
// bit.  Block division uses a precomputed 2^32 / P multiplier.
//
// block_fill_kernel (block view only): one workgroup per token rebuilds the
// token's bitmap from its sorted S, derives the touched blocks and their
// in-page masks, and writes them at the token's CSR offset.  The offset is a
// prefix over the other tokens' block counts; the first kernel stores each
// count as -(count + 1) in blk_indptr[i + 1] and this kernel replaces it by
// the inclusive prefix, so a workgroup reading its predecessors sees, for
// each, either the raw count or an inclusive prefix that ends the look-back.
// Both are valid whatever the order of the workgroups, so nothing waits.

#include "stp_internal.h"

namespace {

constexpr int kMaxPositions = 1 << 20;     // bitmap of 128 KiB LDS
constexpr int kLdsBudget = 150 * 1024;     // dynamic LDS a workgroup may use
constexpr int kDenseWord = 8;              // words with more bits go wave-wide
#ifndef STP_NORM_THREADS
#define STP_NORM_THREADS 1024
#endif
constexpr int kNThreads = STP_NORM_THREADS;  // normalize_kernel's workgroup
constexpr int kNWaves = kNThreads / 64;
constexpr int kNDPer = kNThreads >= 1024 ? 2 : (kNThreads >= 512 ? 4 : 8);  // D entries per thread
constexpr int kFThreads = 1024;            // block_fill_kernel's workgroup
constexpr int kFWaves = kFThreads / 64;
constexpr int kFDPer = 2;                  // entries of S per thread in flight

struct NormArgs {
  const int32_t* topk;
  const int32_t* req_id;
  const int32_t* q_pos;
  const int32_t* block_table;
  int top_k, num_reqs, max_blocks, P, window, num_sinks, cap;
  int nwords_alloc;
  int vec_out;    // cap % 4 == 0 and 16-byte aligned output rows: vector stores
  uint64_t pdiv;  // ceil(2^32 / P): t / P == (t * pdiv) >> 32 for t < 2^20
  int32_t* tok_out;
  int32_t* slot_out;
  int32_t* count_out;
  int32_t* dropped_out;
  int32_t* blk_indptr;  // nullable; receives -(block count + 1) per token
};

__device__ __forceinline__ int div_p(int t, uint64_t pdiv) {
  return (int)(((uint64_t)(uint32_t)t * pdiv) >> 32);
}

// Bits of positions [lo, hi) (0 < hi - lo <= 64) taken from the bitmap.
__device__ __forceinline__ uint64_t bits_in_range(const uint64_t* bm, int lo, int hi) {
  const int w0 = lo >> 6, w1 = (hi - 1) >> 6;
  const int a = lo & 63;
  uint64_t acc = bm[w0] >> a;
  if (w1 != w0) acc |= bm[w1] << (64 - a);
  const int n = hi - lo;
  return n == 64 ? acc : (acc & ((1ull << n) - 1));
}

template <int kW>
__device__ __forceinline__ int block_sum(int v, int* scratch) {
  v = stp::wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) s += scratch[w];
  return s;
}

// LDS of normalize_kernel: the bitmap (nwords_alloc words), then the
// request's page-table row (kTableLds), then the emitted list S (kListLds).
template <bool kTableLds, bool kListLds>
__global__ __launch_bounds__(kNThreads) void normalize_kernel(NormArgs a) {
  extern __shared__ uint64_t bitmap[];
  __shared__ int s_wave_total[kNWaves];
  __shared__ int s_wave_blocks[kNWaves];
  __shared__ int s_wave_dropped[kNWaves];

  const int i = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // D first: independent of the request, so its loads overlap the rest.
  const int32_t* drow = a.topk + (int64_t)i * a.top_k;
  int dv[kNDPer];
#pragma unroll
  for (int u = 0; u < kNDPer; ++u) {
    const int j = tid + u * kNThreads;
    dv[u] = j < a.top_k ? drow[j] : -1;
  }
  const int r = a.req_id[i];
  const int q = a.q_pos[i];
  int32_t* tok_row = a.tok_out + (int64_t)i * a.cap;
  int32_t* slot_row = a.slot_out + (int64_t)i * a.cap;

  if (r < 0 || r >= a.num_reqs || q < 0) {  // padding row (uniform branch)
    for (int j = tid; j < a.cap; j += kNThreads) {
      tok_row[j] = -1;
      slot_row[j] = -1;
    }
    if (tid == 0) {
      a.count_out[i] = 0;
      if (a.dropped_out) a.dropped_out[i] = 0;
      if (a.blk_indptr) a.blk_indptr[i + 1] = -1;
    }
    return;
  }

  const int P = a.P;
  const int32_t* g_table = a.block_table + (int64_t)r * a.max_blocks;
  const int limit = min(q, a.max_blocks * P - 1);  // last position that can be visible
  const int nwords = (limit >> 6) + 1;
  const int used_blocks = div_p(limit, a.pdiv) + 1;
  int32_t* l_table = (int32_t*)(bitmap + a.nwords_alloc);
  int32_t* l_list = l_table + (kTableLds ? a.max_blocks : 0);
  if (kTableLds) {
    // all of a thread's table loads in flight before its stores
    for (int b0 = 0; b0 < used_blocks; b0 += 4 * kNThreads) {
      int tv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int b = b0 + tid + u * kNThreads;
        tv[u] = b < used_blocks ? g_table[b] : -1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int b = b0 + tid + u * kNThreads;
        if (b < used_blocks) l_table[b] = tv[u];
      }
    }
  }
  for (int w = tid; w < nwords; w += kNThreads) bitmap[w] = 0;
  __syncthreads();
  const int32_t* table = kTableLds ? l_table : g_table;

  auto set_bit = [&](int t) {
    atomicOr((unsigned long long*)&bitmap[t >> 6], 1ull << (t & 63));
  };
  // D entries: every table read first, then branch-free visibility.
  int my_dropped = 0;
  auto add_d = [&](const int (&tv)[kNDPer]) {
    int pg[kNDPer];
#pragma unroll
    for (int u = 0; u < kNDPer; ++u) {
      const int tc = min(max(tv[u], 0), limit);  // in-range stand-in for the read
      pg[u] = table[div_p(tc, a.pdiv)];
    }
#pragma unroll
    for (int u = 0; u < kNDPer; ++u) {
      const int t = tv[u];
      const int b = div_p(max(t, 0), a.pdiv);
      const bool ok = t >= 0 && t <= limit && pg[u] >= 0 &&
                      (int64_t)pg[u] * P + (t - b * P) <= INT32_MAX;
      my_dropped += (t >= 0 && !ok) ? 1 : 0;
      if (ok) set_bit(t);
    }
  };
  add_d(dv);
  for (int j0 = kNDPer * kNThreads; j0 < a.top_k; j0 += kNDPer * kNThreads) {
#pragma unroll
    for (int u = 0; u < kNDPer; ++u) {
      const int j = j0 + tid + u * kNThreads;
      dv[u] = j < a.top_k ? drow[j] : -1;
    }
    add_d(dv);
  }
  auto visible = [&](int t) -> bool {  // 0 <= t <= limit
    const int b = div_p(t, a.pdiv);
    const int page = table[b];
    return page >= 0 && (int64_t)page * P + (t - b * P) <= INT32_MAX;
  };
  // W: the local window ending at the query's own position.
  if (a.window > 0)
    for (int t = max(0, q - a.window + 1) + tid; t <= q; t += kNThreads)
      if (t <= limit && visible(t)) set_bit(t);
  // A: the sink positions.
  const int na = min(a.num_sinks, q + 1);
  for (int t = tid; t < na; t += kNThreads)
    if (t <= limit && visible(t)) set_bit(t);
  __syncthreads();  // bitmap complete

  // One pass over the bitmap for the three totals, published together: the
  // set's size (each wave owns a contiguous run of 64-word batches), the
  // touched logical blocks (one block per thread) and the dropped entries.
  const int nbatch = (nwords + 63) >> 6;
  const int bpw = (nbatch + kNWaves - 1) / kNWaves;
  const int b0 = min(nbatch, wave * bpw), b1 = min(nbatch, b0 + bpw);
  int cnt = 0;
  for (int bb = b0; bb < b1; ++bb) {
    const int w = bb * 64 + lane;
    cnt += w < nwords ? __popcll(bitmap[w]) : 0;
  }
  int my_blocks = 0;
  if (a.blk_indptr) {
    for (int b = tid; b < used_blocks; b += kNThreads) {
      const int lo = b * P, hi = min(lo + P, limit + 1);
      if (bits_in_range(bitmap, lo, hi)) ++my_blocks;
    }
  }
  cnt = stp::wave_sum(cnt);
  my_blocks = stp::wave_sum(my_blocks);
  my_dropped = stp::wave_sum(my_dropped);
  if (lane == 0) {
    s_wave_total[wave] = cnt;
    s_wave_blocks[wave] = my_blocks;
    s_wave_dropped[wave] = my_dropped;
  }
  __syncthreads();
  int base = 0, total = 0, nb = 0, dropped = 0;
#pragma unroll
  for (int w = 0; w < kNWaves; ++w) {
    const int sw = s_wave_total[w];
    base += w < wave ? sw : 0;
    total += sw;
    nb += s_wave_blocks[w];
    dropped += s_wave_dropped[w];
  }

  // Ascending emission: into the LDS list (then written out below in one
  // coalesced pass), or straight to global memory when the list does not
  // fit in LDS.
  auto emit = [&](int t, int pos) {
    if (kListLds) {
      l_list[pos] = t;
    } else {
      const int b = div_p(t, a.pdiv);
      tok_row[pos] = t;
      slot_row[pos] = table[b] * P + (t - b * P);
    }
  };
  for (int bb = b0; bb < b1; ++bb) {
    const int w = bb * 64 + lane;
    const uint64_t x = w < nwords ? bitmap[w] : 0ull;
    const int c = __popcll(x);
    const int incl = stp::wave_incl_sum(c);
    int off = base + incl - c;
    base += __builtin_amdgcn_readlane(incl, 63);
    // sparse words: the owning lane walks its bits
    uint64_t bits = c < kDenseWord ? x : 0ull;
    while (bits) {
      emit(w * 64 + __builtin_ctzll(bits), off++);
      bits &= bits - 1;
    }
    // dense words: one lane per bit
    uint64_t dense = __ballot(c >= kDenseWord);
    while (dense) {
      const int src = __builtin_ctzll(dense);
      dense &= dense - 1;
      const uint32_t xlo = __builtin_amdgcn_readlane((uint32_t)x, src);
      const uint32_t xhi = __builtin_amdgcn_readlane((uint32_t)(x >> 32), src);
      const int woff = __builtin_amdgcn_readlane(off, src);
      const uint32_t below = __builtin_amdgcn_mbcnt_hi(xhi, __builtin_amdgcn_mbcnt_lo(xlo, 0u));
      const bool mine = ((lane < 32 ? xlo >> lane : xhi >> (lane - 32)) & 1u) != 0;
      if (mine) emit((bb * 64 + src) * 64 + lane, woff + (int)below);
    }
  }
  if (kListLds && a.vec_out) {
    __syncthreads();  // list complete
    // one coalesced pass, four consecutive entries per thread written as
    // 16-byte vectors: tokens, slots and the -1 tail
    for (int j0 = 4 * tid; j0 < a.cap; j0 += 4 * kNThreads) {
      int tv[4], sl[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) tv[u] = j0 + u < total ? l_list[j0 + u] : -1;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = tv[u];
        const int b = div_p(max(t, 0), a.pdiv);
        sl[u] = t >= 0 ? table[b] * P + (t - b * P) : -1;
      }
      *(int4*)(tok_row + j0) = make_int4(tv[0], tv[1], tv[2], tv[3]);
      *(int4*)(slot_row + j0) = make_int4(sl[0], sl[1], sl[2], sl[3]);
    }
  } else if (kListLds) {
    __syncthreads();  // list complete
    // one coalesced pass: tokens, slots and the -1 tail
    for (int j0 = 0; j0 < a.cap; j0 += 4 * kNThreads) {
      int tv[4], sl[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + tid + u * kNThreads;
        tv[u] = j < total ? l_list[j] : -1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = tv[u];
        const int b = div_p(max(t, 0), a.pdiv);
        sl[u] = t >= 0 ? table[b] * P + (t - b * P) : -1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + tid + u * kNThreads;
        if (j < a.cap) {
          tok_row[j] = tv[u];
          slot_row[j] = sl[u];
        }
      }
    }
  } else {
    for (int j = total + tid; j < a.cap; j += kNThreads) {
      tok_row[j] = -1;
      slot_row[j] = -1;
    }
  }

  if (tid == 0) {
    a.count_out[i] = total;
    if (a.dropped_out) a.dropped_out[i] = dropped;
    if (a.blk_indptr) a.blk_indptr[i + 1] = -(nb + 1);
  }
}

struct FillArgs {
  const int32_t* tok_out;
  const int32_t* count_out;
  const int32_t* req_id;
  const int32_t* q_pos;
  const int32_t* block_table;
  int num_reqs, max_blocks, P, cap;
  uint64_t pdiv;
  int nwords_alloc;  // bitmap words; the staged table row follows them in LDS
  int32_t* blk_indptr;
  int32_t* blk_logical;
  int32_t* blk_page;
  uint64_t* blk_mask;
};

// Per token: CSR offset by look-back, then the touched blocks from a bitmap
// rebuilt out of the token's sorted S.  The request's page-table row is
// staged in LDS (after the bitmap) while the look-back runs, when it fits.
template <bool kTableLds>
__global__ __launch_bounds__(kFThreads) void block_fill_kernel(FillArgs a) {
  extern __shared__ uint64_t bitmap[];
  __shared__ int s_red[kFWaves];
  __shared__ int s_scan[kFWaves];
  const int i = blockIdx.x;
  const int tid = threadIdx.x;

  // written as -(count + 1) by the normalisation; only this workgroup turns it
  // into the inclusive prefix, so a value >= 0 means this token's view is
  // already complete (a repeated fill over the same arrays): nothing to do
  const int raw = a.blk_indptr[i + 1];
  if (raw >= 0) return;
  const int own = -raw - 1;
  const int n = a.count_out[i];
  const int r = a.req_id[i];
  const int q = a.q_pos[i];
  const bool pad = r < 0 || r >= a.num_reqs || q < 0;
  const int32_t* tok = a.tok_out + (int64_t)i * a.cap;
  // the token's first entries of S and its table row, loaded while the
  // look-back runs
  int tv[kFDPer];
#pragma unroll
  for (int u = 0; u < kFDPer; ++u) {
    const int j = tid + u * kFThreads;
    tv[u] = j < n ? tok[j] : -1;
  }
  const int P = a.P;
  const int limit = pad ? 0 : min(q, a.max_blocks * P - 1);
  const int nwords = (limit >> 6) + 1;
  const int used_blocks = div_p(limit, a.pdiv) + 1;
  const int32_t* g_table = a.block_table + (int64_t)(pad ? 0 : r) * a.max_blocks;
  int32_t* l_table = (int32_t*)(bitmap + a.nwords_alloc);
  // the first look-back window's entries (tokens i-1 .. i-kFThreads; never
  // this token's own entry), in flight with the loads above
  const int k_first = i - 1 - tid;
  const int v_first = k_first >= 0 ? a.blk_indptr[k_first + 1] : -1;
  if (kTableLds && !pad && own > 0) {
    for (int b0 = 0; b0 < used_blocks; b0 += 2 * kFThreads) {
      int pv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int b = b0 + tid + u * kFThreads;
        pv[u] = b < used_blocks ? g_table[b] : -1;
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int b = b0 + tid + u * kFThreads;
        if (b < used_blocks) l_table[b] = pv[u];
      }
    }
  }
  __syncthreads();  // every thread has its `own` before thread 0 rewrites the entry

  // Look-back over tokens i-1, i-2, ...: raw counts until an inclusive prefix.
  int prefix = 0;
  for (int hi = i; hi > 0; hi -= kFThreads) {
    const int k = hi - 1 - tid;  // token index this thread reads
    const int v = hi == i ? v_first : (k >= 0 ? a.blk_indptr[k + 1] : -1);
    // the newest (largest k) inclusive prefix in this window, if any
    const int kp = (k >= 0 && v >= 0) ? k : -1;
    // (an LDS atomic max over the workgroup)
    __syncthreads();
    if (tid == 0) s_red[0] = -1;
    __syncthreads();
    if (kp >= 0) atomicMax(&s_red[0], kp);
    __syncthreads();
    const int kstar = s_red[0];
    int contrib = 0;
    if (k >= 0 && k > kstar) contrib = -v - 1;  // raw count after the newest prefix
    if (k >= 0 && k == kstar) contrib = v;      // the prefix itself
    prefix += block_sum<kFWaves>(contrib, s_red);
    if (kstar >= 0) break;
  }

  if (tid == 0) {
    if (i == 0) a.blk_indptr[0] = 0;
    a.blk_indptr[i + 1] = prefix + own;
  }
  if (own == 0 || pad) return;

  const int32_t* table = kTableLds ? l_table : g_table;
  for (int w = tid; w < nwords; w += kFThreads) bitmap[w] = 0;
  __syncthreads();
  auto set_bits = [&](const int (&v)[kFDPer]) {
#pragma unroll
    for (int u = 0; u < kFDPer; ++u)
      if (v[u] >= 0) atomicOr((unsigned long long*)&bitmap[v[u] >> 6], 1ull << (v[u] & 63));
  };
  set_bits(tv);
  for (int j0 = kFDPer * kFThreads; j0 < n; j0 += kFDPer * kFThreads) {
#pragma unroll
    for (int u = 0; u < kFDPer; ++u) {
      const int j = j0 + tid + u * kFThreads;
      tv[u] = j < n ? tok[j] : -1;
    }
    set_bits(tv);
  }
  __syncthreads();

  // Blocks in chunks of kFThreads, one per thread: in-page mask, page,
  // position by a block-wide scan of the flags.
  int k0 = prefix;
  for (int c0 = 0; c0 < used_blocks; c0 += kFThreads) {
    const int b = c0 + tid;
    uint64_t m = 0;
    if (b < used_blocks) {
      const int lo = b * P, hi = min(lo + P, limit + 1);
      m = bits_in_range(bitmap, lo, hi);
    }
    const int page = m ? table[b] : 0;
    int tot;
    const int k = k0 + stp::block_exclusive_scan<kFWaves>(m ? 1 : 0, s_scan, &tot);
    if (m) {
      a.blk_logical[k] = b;
      a.blk_page[k] = page;
      a.blk_mask[k] = m;
    }
    k0 += tot;
  }
}

// Dynamic LDS above the default limit for every kernel of this file, once.
int set_lds_attrs() {
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)normalize_kernel<true, true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget) !=
            hipSuccess ||
        hipFuncSetAttribute((const void*)normalize_kernel<true, false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget) !=
            hipSuccess ||
        hipFuncSetAttribute((const void*)normalize_kernel<false, true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget) !=
            hipSuccess ||
        hipFuncSetAttribute((const void*)normalize_kernel<false, false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget) !=
            hipSuccess ||
        hipFuncSetAttribute((const void*)block_fill_kernel<true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget) != hipSuccess ||
        hipFuncSetAttribute((const void*)block_fill_kernel<false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget) != hipSuccess)
      return stp::fail(STP_ERR_HIP, "normalize_indices: hipFuncSetAttribute failed");
    attr_set = true;
  }
  return STP_OK;
}

// The block-view pass of a normalisation whose counts are in blk_indptr.
int launch_block_fill(const int32_t* tok_out, const int32_t* count_out, const int32_t* req_id,
                      const int32_t* q_pos, int32_t T, const int32_t* block_table,
                      int32_t num_reqs, int32_t max_blocks, int32_t page_size, int32_t cap,
                      int32_t* blk_indptr, int32_t* blk_logical, int32_t* blk_page,
                      uint64_t* blk_mask, hipStream_t stream) {
  if (num_reqs == 0 || max_blocks == 0) num_reqs = 0;  // every token is a padding row
  const int nwords = max(1, (int)(((int64_t)max_blocks * page_size + 63) / 64));
  const size_t bitmap_bytes = (size_t)nwords * sizeof(uint64_t);
  const bool table_in_lds = bitmap_bytes + (size_t)max_blocks * 4 <= (size_t)kLdsBudget;
  const uint64_t pdiv = ((1ull << 32) + (uint64_t)page_size - 1) / (uint64_t)page_size;
  FillArgs fa{tok_out, count_out, req_id, q_pos, block_table, num_reqs, max_blocks, page_size,
              cap, pdiv, nwords, blk_indptr, blk_logical, blk_page, blk_mask};
  if (table_in_lds)
    block_fill_kernel<true><<<T, kFThreads, bitmap_bytes + (size_t)max_blocks * 4, stream>>>(fa);
  else
    block_fill_kernel<false><<<T, kFThreads, bitmap_bytes, stream>>>(fa);
  return stp::check_launch("block_fill_kernel");
}

}  // namespace

static int normalize_impl(const int32_t* topk, int32_t top_k, const int32_t* req_id,
                          const int32_t* q_pos, int32_t T, const int32_t* block_table,
                          int32_t num_reqs, int32_t max_blocks, int32_t page_size,
                          int32_t window, int32_t num_sinks, int32_t cap, int32_t* tok_out,
                          int32_t* slot_out, int32_t* count_out, int32_t* dropped_out,
                          int32_t* blk_indptr, int32_t* blk_logical, int32_t* blk_page,
                          uint64_t* blk_mask, hipStream_t stream, bool defer_fill) {
  using stp::fail;
  if (T < 0 || top_k < 0 || num_reqs < 0 || max_blocks < 0 || window < 0 || num_sinks < 0 ||
      cap < 0)
    return fail(STP_ERR_INVALID_ARG, "normalize_indices: negative size");
  if (page_size < 1 || page_size > 64)
    return fail(STP_ERR_INVALID_ARG, "normalize_indices: page_size %d not in [1, 64]", page_size);
  if ((int64_t)cap < (int64_t)top_k + window + num_sinks)
    return fail(STP_ERR_INVALID_ARG, "normalize_indices: cap %d < top_k + window + num_sinks",
                cap);
  if ((int64_t)max_blocks * page_size > kMaxPositions)
    return fail(STP_ERR_INVALID_ARG,
                "normalize_indices: max_blocks * page_size exceeds %d positions", kMaxPositions);
  if (T == 0) return STP_OK;
  if (!req_id || !q_pos || !tok_out || !slot_out || !count_out || (top_k > 0 && !topk) ||
      (num_reqs > 0 && max_blocks > 0 && !block_table))
    return fail(STP_ERR_INVALID_ARG, "normalize_indices: null pointer");
  if (blk_indptr && (!blk_logical || !blk_page || !blk_mask))
    return fail(STP_ERR_INVALID_ARG, "normalize_indices: block view arrays missing");
  if (num_reqs == 0 || max_blocks == 0) {
    // No request has a mapped page: every token is a padding row.
    num_reqs = 0;
  }

  const int nwords = max(1, (int)(((int64_t)max_blocks * page_size + 63) / 64));
  const size_t bitmap_bytes = (size_t)nwords * sizeof(uint64_t);
  const bool table_in_lds = bitmap_bytes + (size_t)max_blocks * 4 <= (size_t)kLdsBudget;
  size_t lds = bitmap_bytes + (table_in_lds ? (size_t)max_blocks * 4 : 0);
  const bool list_in_lds = lds + (size_t)cap * 4 <= (size_t)kLdsBudget;
  if (list_in_lds) lds += (size_t)cap * 4;
  if (int rc = set_lds_attrs()) return rc;
  const uint64_t pdiv = ((1ull << 32) + (uint64_t)page_size - 1) / (uint64_t)page_size;
  const int vec_out = cap % 4 == 0 && (uintptr_t)tok_out % 16 == 0 &&
                      (uintptr_t)slot_out % 16 == 0;
  NormArgs na{topk, req_id, q_pos, block_table, top_k, num_reqs, max_blocks, page_size, window,
              num_sinks, cap, nwords, vec_out, pdiv, tok_out, slot_out, count_out,
              dropped_out, blk_indptr};
  if (table_in_lds && list_in_lds)
    normalize_kernel<true, true><<<T, kNThreads, lds, stream>>>(na);
  else if (table_in_lds)
    normalize_kernel<true, false><<<T, kNThreads, lds, stream>>>(na);
  else if (list_in_lds)
    normalize_kernel<false, true><<<T, kNThreads, lds, stream>>>(na);
  else
    normalize_kernel<false, false><<<T, kNThreads, lds, stream>>>(na);
  if (int rc = stp::check_launch("normalize_kernel")) return rc;
  if (blk_indptr && !defer_fill)
    return launch_block_fill(tok_out, count_out, req_id, q_pos, T, block_table, num_reqs,
                             max_blocks, page_size, cap, blk_indptr, blk_logical, blk_page,
                             blk_mask, stream);
  return STP_OK;
}

extern "C" int stp_normalize_indices(const int32_t* topk, int32_t top_k, const int32_t* req_id,
                                     const int32_t* q_pos, int32_t T,
                                     const int32_t* block_table, int32_t num_reqs,
                                     int32_t max_blocks, int32_t page_size, int32_t window,
                                     int32_t num_sinks, int32_t cap, int32_t* tok_out,
                                     int32_t* slot_out, int32_t* count_out, int32_t* dropped_out,
                                     int32_t* blk_indptr, int32_t* blk_logical,
                                     int32_t* blk_page, uint64_t* blk_mask, hipStream_t stream) {
  return normalize_impl(topk, top_k, req_id, q_pos, T, block_table, num_reqs, max_blocks,
                        page_size, window, num_sinks, cap, tok_out, slot_out, count_out,
                        dropped_out, blk_indptr, blk_logical, blk_page, blk_mask, stream, false);
}

extern "C" int stp_normalize_indices_deferred(
    const int32_t* topk, int32_t top_k, const int32_t* req_id, const int32_t* q_pos, int32_t T,
    const int32_t* block_table, int32_t num_reqs, int32_t max_blocks, int32_t page_size,
    int32_t window, int32_t num_sinks, int32_t cap, int32_t* tok_out, int32_t* slot_out,
    int32_t* count_out, int32_t* dropped_out, int32_t* blk_indptr, int32_t* blk_logical,
    int32_t* blk_page, uint64_t* blk_mask, hipStream_t stream) {
  return normalize_impl(topk, top_k, req_id, q_pos, T, block_table, num_reqs, max_blocks,
                        page_size, window, num_sinks, cap, tok_out, slot_out, count_out,
                        dropped_out, blk_indptr, blk_logical, blk_page, blk_mask, stream, true);
}

extern "C" int stp_block_view_fill(const int32_t* tok_out, const int32_t* count_out,
                                   const int32_t* req_id, const int32_t* q_pos, int32_t T,
                                   const int32_t* block_table, int32_t num_reqs,
                                   int32_t max_blocks, int32_t page_size, int32_t cap,
                                   int32_t* blk_indptr, int32_t* blk_logical, int32_t* blk_page,
                                   uint64_t* blk_mask, hipStream_t stream) {
  using stp::fail;
  if (T < 0 || num_reqs < 0 || max_blocks < 0 || cap < 0)
    return fail(STP_ERR_INVALID_ARG, "block_view_fill: negative size");
  if (page_size < 1 || page_size > 64)
    return fail(STP_ERR_INVALID_ARG, "block_view_fill: page_size %d not in [1, 64]", page_size);
  if ((int64_t)max_blocks * page_size > kMaxPositions)
    return fail(STP_ERR_INVALID_ARG, "block_view_fill: max_blocks * page_size too large");
  if (T == 0) return STP_OK;
  if (!tok_out || !count_out || !req_id || !q_pos || !blk_indptr || !blk_logical || !blk_page ||
      !blk_mask || (num_reqs > 0 && max_blocks > 0 && !block_table))
    return fail(STP_ERR_INVALID_ARG, "block_view_fill: null pointer");
  if (int rc = set_lds_attrs()) return rc;
  return launch_block_fill(tok_out, count_out, req_id, q_pos, T, block_table, num_reqs,
                           max_blocks, page_size, cap, blk_indptr, blk_logical, blk_page,
                           blk_mask, stream);
}
