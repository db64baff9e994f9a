// Stage 1: candidate-index normalisation on gfx950.
//
// "5.1.1 · 从索引到 Kernel" §1.1 eq. (1) (S = unique(D ∪ W ∪ A), dedup is
// required), §1.2 eq. (2) (token -> logical block, block union and in-page
// mask), §7.3 (dedup by logical identity with a bitmap; eq. (16)-(17)),
// §7.4 eq. (19) (CSR row pointers); "HiSparse" walkthrough, token -> global
// slot id conversion (slot = table[block] * page + offset, -1 propagation).
//
// Design: one 256-thread workgroup per query token holds a bitmap of the
// token's visible positions in LDS.  D, W and A set bits (an LDS atomicOr per
// candidate, so duplicates collapse for free); a popcount scan over the words
// then emits S in ascending order with its slot ids.  The bitmap bounds the
// work by the context length rather than by k log k.  The CSR block view
// needs a prefix over tokens, so it takes two more small launches: a
// single-workgroup scan of the per-token block counts and a per-token fill.

#include "stp_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxPositions = 1 << 20;     // bitmap of 128 KiB LDS
constexpr int kLdsBudget = 150 * 1024;     // dynamic LDS a normalise workgroup may use
constexpr int kBlockViewMaxCap = 12000;    // block fill keeps 12 bytes per candidate in LDS

struct TokenView {
  const int32_t* table;  // the request's page-table row (LDS copy or global)
  int max_blocks;
  int P;
  int q;
};

// Position t (>= 0) is visible to the query and lies on a mapped page whose
// slot id fits int32.
__device__ __forceinline__ bool visible(const TokenView& v, int t) {
  if (t > v.q) return false;
  const int b = t / v.P;
  if (b >= v.max_blocks) return false;
  const int page = v.table[b];
  if (page < 0) return false;
  const int64_t slot = (int64_t)page * v.P + (t - b * v.P);
  return slot <= INT32_MAX;
}

__device__ __forceinline__ void set_bit(uint64_t* bm, int t) {
  atomicOr((unsigned long long*)&bm[t >> 6], 1ull << (t & 63));
}

// Bits of positions [lo, hi) (hi - lo <= 64) taken from the bitmap.
__device__ __forceinline__ uint64_t bits_in_range(const uint64_t* bm, int lo, int hi, int nwords) {
  uint64_t acc = 0;
  const int w0 = lo >> 6, w1 = (hi - 1) >> 6;
  for (int w = w0; w <= w1 && w < nwords; ++w) {
    const int a = max(lo, w * 64) - w * 64;
    const int b = min(hi, w * 64 + 64) - w * 64;
    const uint64_t m = (b - a == 64) ? ~0ull : (((1ull << (b - a)) - 1) << a);
    acc |= (bm[w] & m);
  }
  return acc;
}

// One workgroup per query token.  LDS: the position bitmap (nwords 64-bit
// words), then, when table_in_lds, the request's page-table row.
__global__ __launch_bounds__(kThreads) void normalize_kernel(
    const int32_t* __restrict__ topk, int top_k, const int32_t* __restrict__ req_id,
    const int32_t* __restrict__ q_pos, const int32_t* __restrict__ block_table, int num_reqs,
    int max_blocks, int P, int window, int num_sinks, int cap, int nwords_alloc, int table_in_lds,
    int32_t* __restrict__ tok_out, int32_t* __restrict__ slot_out, int32_t* __restrict__ count_out,
    int32_t* __restrict__ dropped_out, int32_t* __restrict__ blk_count) {
  extern __shared__ uint64_t bitmap[];
  __shared__ int s_scan[8];
  __shared__ int s_dropped;
  __shared__ int s_blocks;

  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int r = req_id[i];
  const int q = q_pos[i];
  int32_t* tok_row = tok_out + (int64_t)i * cap;
  int32_t* slot_row = slot_out + (int64_t)i * cap;

  if (r < 0 || r >= num_reqs || q < 0) {  // padding row (uniform branch)
    for (int j = tid; j < cap; j += kThreads) {
      tok_row[j] = -1;
      slot_row[j] = -1;
    }
    if (tid == 0) {
      count_out[i] = 0;
      if (dropped_out) dropped_out[i] = 0;
      if (blk_count) blk_count[i] = 0;
    }
    return;
  }

  const int32_t* g_table = block_table + (int64_t)r * max_blocks;
  const int limit = min(q, max_blocks * P - 1);  // last position that can be visible
  const int nwords = (limit >> 6) + 1;
  const int used_blocks = limit / P + 1;           // table entries that can matter
  int32_t* l_table = (int32_t*)(bitmap + nwords_alloc);
  for (int w = tid; w < nwords; w += kThreads) bitmap[w] = 0;
  if (table_in_lds)
    for (int b = tid; b < used_blocks; b += kThreads) l_table[b] = g_table[b];
  if (tid == 0) {
    s_dropped = 0;
    s_blocks = 0;
  }
  __syncthreads();
  const TokenView v{table_in_lds ? l_table : g_table, max_blocks, P, q};

  // D: the dynamic top-k entries, four independent loads in flight per
  // thread; invalid ones are dropped and counted.
  int my_dropped = 0;
  const int32_t* drow = topk + (int64_t)i * top_k;
  for (int j0 = tid; j0 < top_k; j0 += 4 * kThreads) {
    int tv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * kThreads;
      tv[u] = j < top_k ? drow[j] : -1;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = tv[u];
      if (t < 0) continue;
      if (visible(v, t))
        set_bit(bitmap, t);
      else
        ++my_dropped;
    }
  }
  // W: the local window ending at the query's own position.
  if (window > 0) {
    for (int t = max(0, q - window + 1) + tid; t <= q; t += kThreads)
      if (visible(v, t)) set_bit(bitmap, t);
  }
  // A: the sink positions.
  const int na = min(num_sinks, q + 1);
  for (int t = tid; t < na; t += kThreads)
    if (visible(v, t)) set_bit(bitmap, t);
  if (my_dropped) atomicAdd(&s_dropped, my_dropped);
  __syncthreads();

  // Emit S in ascending order: each thread owns a contiguous run of words.
  const int wpt = (nwords + kThreads - 1) / kThreads;
  const int w0 = min(nwords, tid * wpt), w1 = min(nwords, w0 + wpt);
  int c = 0;
  for (int w = w0; w < w1; ++w) c += __popcll(bitmap[w]);
  int total;
  int off = stp::block_exclusive_scan_256(c, s_scan, &total);
  for (int w = w0; w < w1; ++w) {
    uint64_t bits = bitmap[w];
    while (bits) {
      const int t = (w << 6) + __builtin_ctzll(bits);
      bits &= bits - 1;
      const int b = t / P;
      tok_row[off] = t;
      slot_row[off] = v.table[b] * P + (t - b * P);
      ++off;
    }
  }
  for (int j = total + tid; j < cap; j += kThreads) {
    tok_row[j] = -1;
    slot_row[j] = -1;
  }

  // Number of touched logical blocks (for the CSR block view).
  if (blk_count) {
    int nb = 0;
    for (int b = tid; b < used_blocks; b += kThreads) {
      const int lo = b * P, hi = min(lo + P, limit + 1);
      if (bits_in_range(bitmap, lo, hi, nwords)) ++nb;
    }
    if (nb) atomicAdd(&s_blocks, nb);
  }
  __syncthreads();
  if (tid == 0) {
    count_out[i] = total;
    if (dropped_out) dropped_out[i] = s_dropped;
    if (blk_count) blk_count[i] = s_blocks;
  }
}

// In place: indptr[1..T] holds per-token counts; make it the inclusive prefix
// and set indptr[0] = 0.  One workgroup.
__global__ __launch_bounds__(kThreads) void indptr_scan_kernel(int32_t* indptr, int T) {
  __shared__ int s_scan[8];
  int carry = 0;
  for (int base = 0; base < T; base += kThreads) {
    const int j = base + threadIdx.x;
    const int v = j < T ? indptr[1 + j] : 0;
    int total;
    const int ex = stp::block_exclusive_scan_256(v, s_scan, &total);
    if (j < T) indptr[1 + j] = carry + ex + v;
    carry += total;
  }
  if (threadIdx.x == 0) indptr[0] = 0;
}

// Per token: one entry per touched logical block of the sorted S.  The
// token's list is staged in LDS; block k of the token collects its in-page
// bits with LDS atomics, so no thread walks a block serially.
__global__ __launch_bounds__(kThreads) void block_fill_kernel(
    const int32_t* __restrict__ tok_out, const int32_t* __restrict__ count_out,
    const int32_t* __restrict__ req_id, const int32_t* __restrict__ block_table, int max_blocks,
    int P, int cap, const int32_t* __restrict__ indptr, int32_t* __restrict__ blk_logical,
    int32_t* __restrict__ blk_page, uint64_t* __restrict__ blk_mask) {
  extern __shared__ uint64_t lmask[];  // [cap] block masks, then [cap] tokens
  __shared__ int s_scan[8];
  const int i = blockIdx.x;
  const int n = count_out[i];
  if (n == 0) return;
  int32_t* ltok = (int32_t*)(lmask + cap);
  const int32_t* tok = tok_out + (int64_t)i * cap;
  const int32_t* table = block_table + (int64_t)req_id[i] * max_blocks;
  const int out0 = indptr[i];
  const int nb = indptr[i + 1] - out0;
  for (int j = threadIdx.x; j < n; j += kThreads) ltok[j] = tok[j];
  for (int k = threadIdx.x; k < nb; k += kThreads) lmask[k] = 0;
  __syncthreads();
  int carry = 0;  // blocks started before this chunk
  for (int base = 0; base < n; base += kThreads) {
    const int j = base + threadIdx.x;
    int start = 0, t = 0, b = 0;
    if (j < n) {
      t = ltok[j];
      b = t / P;
      start = (j == 0) || (ltok[j - 1] / P != b);
    }
    int total;
    const int ex = stp::block_exclusive_scan_256(start, s_scan, &total);
    if (j < n) {
      const int k = carry + ex + start - 1;  // this token's block
      atomicOr((unsigned long long*)&lmask[k], 1ull << (t - b * P));
      if (start) {
        blk_logical[out0 + k] = b;
        blk_page[out0 + k] = table[b];
      }
    }
    carry += total;
  }
  __syncthreads();
  for (int k = threadIdx.x; k < nb; k += kThreads) blk_mask[out0 + k] = lmask[k];
}

}  // namespace

extern "C" int stp_normalize_indices(const int32_t* topk, int32_t top_k, const int32_t* req_id,
                                     const int32_t* q_pos, int32_t T,
                                     const int32_t* block_table, int32_t num_reqs,
                                     int32_t max_blocks, int32_t page_size, int32_t window,
                                     int32_t num_sinks, int32_t cap, int32_t* tok_out,
                                     int32_t* slot_out, int32_t* count_out, int32_t* dropped_out,
                                     int32_t* blk_indptr, int32_t* blk_logical,
                                     int32_t* blk_page, uint64_t* blk_mask, hipStream_t stream) {
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

  if (blk_indptr && cap > kBlockViewMaxCap)
    return fail(STP_ERR_INVALID_ARG, "normalize_indices: the block view supports cap <= %d",
                kBlockViewMaxCap);

  const int nwords = max(1, (int)(((int64_t)max_blocks * page_size + 63) / 64));
  const size_t bitmap_bytes = (size_t)nwords * sizeof(uint64_t);
  const bool table_in_lds = bitmap_bytes + (size_t)max_blocks * 4 <= (size_t)kLdsBudget;
  const size_t lds = bitmap_bytes + (table_in_lds ? (size_t)max_blocks * 4 : 0);
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)normalize_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget) !=
            hipSuccess ||
        hipFuncSetAttribute((const void*)block_fill_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget) != hipSuccess)
      return fail(STP_ERR_HIP, "normalize_indices: hipFuncSetAttribute failed");
    attr_set = true;
  }
  int32_t* blk_count = blk_indptr ? blk_indptr + 1 : nullptr;
  normalize_kernel<<<T, kThreads, lds, stream>>>(
      topk, top_k, req_id, q_pos, block_table, num_reqs, max_blocks, page_size, window, num_sinks,
      cap, nwords, table_in_lds ? 1 : 0, tok_out, slot_out, count_out, dropped_out, blk_count);
  if (int rc = stp::check_launch("normalize_kernel")) return rc;
  if (blk_indptr) {
    indptr_scan_kernel<<<1, kThreads, 0, stream>>>(blk_indptr, T);
    if (int rc = stp::check_launch("indptr_scan_kernel")) return rc;
    block_fill_kernel<<<T, kThreads, (size_t)cap * 12, stream>>>(
        tok_out, count_out, req_id, block_table, max_blocks, page_size, cap, blk_indptr,
        blk_logical, blk_page, blk_mask);
    if (int rc = stp::check_launch("block_fill_kernel")) return rc;
  }
  return STP_OK;
}
