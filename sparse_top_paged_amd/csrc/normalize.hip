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
// normalize_kernel: one 1024-thread workgroup per query token holds a bitmap
// of the token's visible positions in LDS (plus the request's page-table row
// when it fits).  The token's D entries are loaded before anything else (they
// do not depend on the request), then D, W and A set bits with LDS atomicOr
// (duplicates collapse for free).  S is emitted in ascending order by each
// wave over its own run of 64-word batches: a wave scan of the words'
// popcounts gives every word its output offset; sparse words are walked by
// their own lane, dense ones (the window) by the whole wave, one lane per
// bit.  Block division uses a precomputed 2^32 / P multiplier.
//
// block_fill_kernel (block view only): one workgroup per token runs the
// block-view pass (block_view.h): the token's CSR offset by a wait-free
// look-back over the counts the first kernel left in blk_indptr, then its
// touched blocks, their pages and in-page masks from a bitmap rebuilt out of
// the token's sorted S and slot ids.

#include "block_view.h"
#include "stp_internal.h"

namespace {

using namespace stp::bv;

constexpr int kMaxPositions = 1 << 20;     // bitmap of 128 KiB LDS
constexpr int kLdsBudget = 150 * 1024;     // dynamic LDS a workgroup may use
constexpr int kDenseWord = 8;              // words with more bits go wave-wide
#ifndef STP_NORM_THREADS
#define STP_NORM_THREADS 1024
#endif
constexpr int kNThreads = STP_NORM_THREADS;  // normalize_kernel's workgroup
constexpr int kNWaves = kNThreads / 64;
constexpr int kNDPer = kNThreads >= 1024 ? 2 : (kNThreads >= 512 ? 4 : 8);  // D entries per thread

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

template <bool kPageLds>
__global__ __launch_bounds__(kFThreads) void block_fill_kernel(FillArgs a) {
  extern __shared__ uint64_t bitmap[];
  __shared__ int s_red[kFWaves];
  __shared__ int s_scan[kFWaves];
  block_fill_token<kPageLds>(a, blockIdx.x, bitmap, s_red, s_scan);
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

}  // namespace

namespace stp {

int launch_block_fill(const BlockViewPass& p, int32_t T, hipStream_t stream) {
  if (int rc = set_lds_attrs()) return rc;
  // no request with a mapped page: every token is a padding row
  const int num_reqs = (p.num_reqs == 0 || p.max_blocks == 0) ? 0 : p.num_reqs;
  const int nwords = max(1, (int)(((int64_t)p.max_blocks * p.page_size + 63) / 64));
  const size_t bitmap_bytes = (size_t)nwords * sizeof(uint64_t);
  const bool pages_in_lds = bitmap_bytes + (size_t)p.max_blocks * 4 <= (size_t)kLdsBudget;
  const uint64_t pdiv = ((1ull << 32) + (uint64_t)p.page_size - 1) / (uint64_t)p.page_size;
  FillArgs fa{p.tok_out, p.slot_out, p.req_id, p.q_pos, p.block_table, num_reqs,
              p.max_blocks, p.page_size, p.cap, pdiv, nwords, p.blk_indptr, p.blk_logical,
              p.blk_page, p.blk_mask};
  if (pages_in_lds)
    block_fill_kernel<true><<<T, kFThreads, bitmap_bytes + (size_t)p.max_blocks * 4, stream>>>(fa);
  else
    block_fill_kernel<false><<<T, kFThreads, bitmap_bytes, stream>>>(fa);
  return check_launch("block_fill_kernel");
}

int check_block_view_args(const char* what, const int32_t* tok_out, const int32_t* slot_out,
                          const int32_t* req_id, const int32_t* q_pos, int32_t T,
                          const int32_t* block_table, int32_t num_reqs, int32_t max_blocks,
                          int32_t page_size, int32_t cap, int32_t* blk_indptr,
                          int32_t* blk_logical, int32_t* blk_page, uint64_t* blk_mask) {
  if (T < 0 || num_reqs < 0 || max_blocks < 0 || cap < 0)
    return fail(STP_ERR_INVALID_ARG, "%s: negative size", what);
  if (page_size < 1 || page_size > 64)
    return fail(STP_ERR_INVALID_ARG, "%s: page_size %d not in [1, 64]", what, page_size);
  if ((int64_t)max_blocks * page_size > kMaxPositions)
    return fail(STP_ERR_INVALID_ARG, "%s: max_blocks * page_size too large", what);
  if (T == 0) return STP_OK;
  if (!tok_out || !slot_out || !req_id || !q_pos || !blk_indptr || !blk_logical || !blk_page ||
      !blk_mask || (num_reqs > 0 && max_blocks > 0 && !block_table))
    return fail(STP_ERR_INVALID_ARG, "%s: null pointer", what);
  return STP_OK;
}

}  // namespace stp

namespace stp {

int check_normalize_args(const char* what, const int32_t* topk, int32_t top_k,
                         const int32_t* req_id, const int32_t* q_pos, int32_t T,
                         const int32_t* block_table, int32_t num_reqs, int32_t max_blocks,
                         int32_t page_size, int32_t window, int32_t num_sinks, int32_t cap,
                         const int32_t* tok_out, const int32_t* slot_out,
                         const int32_t* count_out) {
  if (T < 0 || top_k < 0 || num_reqs < 0 || max_blocks < 0 || window < 0 || num_sinks < 0 ||
      cap < 0)
    return fail(STP_ERR_INVALID_ARG, "%s: negative size", what);
  if (page_size < 1 || page_size > 64)
    return fail(STP_ERR_INVALID_ARG, "%s: page_size %d not in [1, 64]", what, page_size);
  if ((int64_t)cap < (int64_t)top_k + window + num_sinks)
    return fail(STP_ERR_INVALID_ARG, "%s: cap %d < top_k + window + num_sinks", what, cap);
  if ((int64_t)max_blocks * page_size > kMaxPositions)
    return fail(STP_ERR_INVALID_ARG, "%s: max_blocks * page_size exceeds %d positions", what,
                kMaxPositions);
  if (T == 0) return STP_OK;
  if (!req_id || !q_pos || !tok_out || !slot_out || !count_out || (top_k > 0 && !topk) ||
      (num_reqs > 0 && max_blocks > 0 && !block_table))
    return fail(STP_ERR_INVALID_ARG, "%s: null pointer", what);
  return STP_OK;
}

}  // namespace stp

static int normalize_impl(const int32_t* topk, int32_t top_k, const int32_t* req_id,
                          const int32_t* q_pos, int32_t T, const int32_t* block_table,
                          int32_t num_reqs, int32_t max_blocks, int32_t page_size,
                          int32_t window, int32_t num_sinks, int32_t cap, int32_t* tok_out,
                          int32_t* slot_out, int32_t* count_out, int32_t* dropped_out,
                          int32_t* blk_indptr, int32_t* blk_logical, int32_t* blk_page,
                          uint64_t* blk_mask, hipStream_t stream, bool defer_fill) {
  using stp::fail;
  if (int rc = stp::check_normalize_args("normalize_indices", topk, top_k, req_id, q_pos, T,
                                         block_table, num_reqs, max_blocks, page_size, window,
                                         num_sinks, cap, tok_out, slot_out, count_out))
    return rc;
  if (T == 0) return STP_OK;
  if (blk_indptr && !defer_fill && (!blk_logical || !blk_page || !blk_mask))
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
    return stp::launch_block_fill({tok_out, slot_out, req_id, q_pos, block_table, num_reqs,
                                   max_blocks, page_size, cap, blk_indptr, blk_logical, blk_page,
                                   blk_mask},
                                  T, stream);
  return STP_OK;
}

namespace stp {

int normalize_deferred(const int32_t* topk, int32_t top_k, const int32_t* req_id,
                       const int32_t* q_pos, int32_t T, const int32_t* block_table,
                       int32_t num_reqs, int32_t max_blocks, int32_t page_size, int32_t window,
                       int32_t num_sinks, int32_t cap, int32_t* tok_out, int32_t* slot_out,
                       int32_t* count_out, int32_t* dropped_out, int32_t* blk_indptr,
                       hipStream_t stream) {
  return normalize_impl(topk, top_k, req_id, q_pos, T, block_table, num_reqs, max_blocks,
                        page_size, window, num_sinks, cap, tok_out, slot_out, count_out,
                        dropped_out, blk_indptr, nullptr, nullptr, nullptr, stream, true);
}

}  // namespace stp

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

extern "C" int stp_block_view_fill(const int32_t* tok_out, const int32_t* slot_out,
                                   const int32_t* req_id, const int32_t* q_pos, int32_t T,
                                   const int32_t* block_table, int32_t num_reqs,
                                   int32_t max_blocks, int32_t page_size, int32_t cap,
                                   int32_t* blk_indptr, int32_t* blk_logical, int32_t* blk_page,
                                   uint64_t* blk_mask, hipStream_t stream) {
  if (int rc = stp::check_block_view_args("block_view_fill", tok_out, slot_out, req_id, q_pos, T,
                                          block_table, num_reqs, max_blocks, page_size, cap,
                                          blk_indptr, blk_logical, blk_page, blk_mask))
    return rc;
  if (T == 0) return STP_OK;
  return stp::launch_block_fill({tok_out, slot_out, req_id, q_pos, block_table, num_reqs,
                                 max_blocks, page_size, cap, blk_indptr, blk_logical, blk_page,
                                 blk_mask},
                                T, stream);
}
