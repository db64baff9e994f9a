// The block view of a normalised candidate set (internal to libstp): the
// per-token pass that turns the counts left by the normalisation into CSR
// offsets and writes each token's touched blocks.  Shared by the block-view
// kernel of normalize.hip and the merge launch of merge.hip that carries the
// same pass beside the split merge.
//
// "5.1.1 · 从索引到 Kernel" §1.2 eq. (2) (token -> logical block, block union
// and in-page mask), §7.4 eq. (19) (CSR row pointers).
//
// The offset is a prefix over the other tokens' block counts; the
// normalisation stores each count as -(count + 1) in blk_indptr[i + 1] and
// this pass replaces it by the inclusive prefix, so a workgroup reading its
// predecessors sees, for each, either the raw count or an inclusive prefix
// that ends the look-back.  Both are valid whatever the order of the
// workgroups, so nothing waits.
#pragma once

#include "stp_internal.h"

namespace stp {
namespace bv {

constexpr int kFThreads = 1024;  // workgroup of the block-view pass
constexpr int kFWaves = kFThreads / 64;
constexpr int kFDPer = 3;        // entries of S per thread in flight

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

struct FillArgs {
  const int32_t* tok_out;
  const int32_t* slot_out;
  const int32_t* req_id;
  const int32_t* q_pos;
  const int32_t* block_table;
  int num_reqs, max_blocks, P, cap;
  uint64_t pdiv;
  int nwords_alloc;  // bitmap words; the blocks' pages follow them in LDS
  int32_t* blk_indptr;
  int32_t* blk_logical;
  int32_t* blk_page;
  uint64_t* blk_mask;
};

// Per token: CSR offset by look-back, then the touched blocks from a bitmap
// rebuilt out of the token's sorted S.  A block's page is that of any of its
// entries, slot / P (slot = page * P + offset with offset < P), written to
// LDS beside the bitmap (kPageLds) when it fits, else read from the page
// table.  Every load the pass needs is issued in one round trip: its own
// entry, the token's request and position, its entries of S and their slots
// (the rows' tails past the count are -1, so no load waits for the count)
// and the first look-back window.  `bitmap` is the workgroup's dynamic LDS
// (nwords_alloc words, then max_blocks pages when kPageLds); s_red and
// s_scan hold kFWaves ints each.  Called by a whole workgroup of kFThreads
// threads.
template <bool kPageLds>
__device__ __forceinline__ void block_fill_token(const FillArgs& a, int i, uint64_t* bitmap,
                                                 int* s_red, int* s_scan) {
  const int tid = threadIdx.x;
  const int raw = a.blk_indptr[i + 1];
  const int r = a.req_id[i];
  const int q = a.q_pos[i];
  const int32_t* tok = a.tok_out + (int64_t)i * a.cap;
  const int32_t* slot = a.slot_out + (int64_t)i * a.cap;
  int tv[kFDPer], sv[kFDPer];
#pragma unroll
  for (int u = 0; u < kFDPer; ++u) {
    const int j = tid + u * kFThreads;
    tv[u] = j < a.cap ? tok[j] : -1;
    sv[u] = j < a.cap ? slot[j] : -1;
  }
  // the first look-back window's entries (tokens i-1 .. i-kFThreads; never
  // this token's own entry)
  const int k_first = i - 1 - tid;
  const int v_first = k_first >= 0 ? a.blk_indptr[k_first + 1] : -1;

  // written as -(count + 1) by the normalisation; only this workgroup turns it
  // into the inclusive prefix, so a value >= 0 means this token's view is
  // already complete (a repeated fill over the same arrays): nothing to do
  if (raw >= 0) return;
  const int own = -raw - 1;
  const bool pad = r < 0 || r >= a.num_reqs || q < 0;
  const int P = a.P;
  const int limit = pad ? 0 : min(q, a.max_blocks * P - 1);
  const int nwords = (limit >> 6) + 1;
  const int used_blocks = div_p(limit, a.pdiv) + 1;
  int32_t* l_page = (int32_t*)(bitmap + a.nwords_alloc);
  for (int w = tid; w < nwords; w += kFThreads) bitmap[w] = 0;
  __syncthreads();  // every thread has its `own` before thread 0 rewrites the
                    // entry; the bitmap is clear

  // this token's entries into the bitmap (and their blocks' pages), in LDS
  // while the look-back below reads its predecessors
  const uint32_t uP = (uint32_t)P;
  auto set_bits = [&](const int (&v)[kFDPer], const int (&s)[kFDPer]) {
#pragma unroll
    for (int u = 0; u < kFDPer; ++u)
      if (v[u] >= 0) {
        atomicOr((unsigned long long*)&bitmap[v[u] >> 6], 1ull << (v[u] & 63));
        if (kPageLds) l_page[div_p(v[u], a.pdiv)] = (int)((uint32_t)s[u] / uP);
      }
  };
  if (own > 0 && !pad) set_bits(tv, sv);

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

  // entries past the first kFDPer * kFThreads (rows longer than the first batch)
  for (int j0 = kFDPer * kFThreads; j0 < a.cap; j0 += kFDPer * kFThreads) {
#pragma unroll
    for (int u = 0; u < kFDPer; ++u) {
      const int j = j0 + tid + u * kFThreads;
      tv[u] = j < a.cap ? tok[j] : -1;
      sv[u] = j < a.cap ? slot[j] : -1;
    }
    set_bits(tv, sv);
  }
  __syncthreads();

  // Blocks in chunks of kFThreads, one per thread: in-page mask, page,
  // position by a block-wide scan of the flags.
  const int32_t* g_table = a.block_table + (int64_t)r * a.max_blocks;
  int k0 = prefix;
  for (int c0 = 0; c0 < used_blocks; c0 += kFThreads) {
    const int b = c0 + tid;
    uint64_t m = 0;
    if (b < used_blocks) {
      const int lo = b * P, hi = min(lo + P, limit + 1);
      m = bits_in_range(bitmap, lo, hi);
    }
    const int page = m ? (kPageLds ? l_page[b] : g_table[b]) : 0;
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

}  // namespace bv

// Host side: the arrays of one block-view pass (those of a normalisation
// made with the pass deferred) and its launches.
struct BlockViewPass {
  const int32_t* tok_out;
  const int32_t* slot_out;
  const int32_t* req_id;
  const int32_t* q_pos;
  const int32_t* block_table;
  int32_t num_reqs, max_blocks, page_size, cap;
  int32_t* blk_indptr;
  int32_t* blk_logical;
  int32_t* blk_page;
  uint64_t* blk_mask;
};

// Size and pointer checks of a block-view pass over T tokens (`what` names
// the entry point in the error message).
int check_block_view_args(const char* what, const int32_t* tok_out, const int32_t* slot_out,
                          const int32_t* req_id, const int32_t* q_pos, int32_t T,
                          const int32_t* block_table, int32_t num_reqs, int32_t max_blocks,
                          int32_t page_size, int32_t cap, int32_t* blk_indptr,
                          int32_t* blk_logical, int32_t* blk_page, uint64_t* blk_mask);

// The pass on its own launch (normalize.hip).
int launch_block_fill(const BlockViewPass& p, int32_t T, hipStream_t stream);

// The size and pointer checks of stp_normalize_indices (normalize.hip).
int check_normalize_args(const char* what, const int32_t* topk, int32_t top_k,
                         const int32_t* req_id, const int32_t* q_pos, int32_t T,
                         const int32_t* block_table, int32_t num_reqs, int32_t max_blocks,
                         int32_t page_size, int32_t window, int32_t num_sinks, int32_t cap,
                         const int32_t* tok_out, const int32_t* slot_out,
                         const int32_t* count_out);

// The normalisation with its block view deferred (blk_indptr nullable, the
// view's other arrays not needed), after the checks of
// stp_normalize_indices (normalize.hip).
int normalize_deferred(const int32_t* topk, int32_t top_k, const int32_t* req_id,
                       const int32_t* q_pos, int32_t T, const int32_t* block_table,
                       int32_t num_reqs, int32_t max_blocks, int32_t page_size, int32_t window,
                       int32_t num_sinks, int32_t cap, int32_t* tok_out, int32_t* slot_out,
                       int32_t* count_out, int32_t* dropped_out, int32_t* blk_indptr,
                       hipStream_t stream);

// The pass and the normalised split merge of the same T tokens (merge.hip):
// one launch when the wide merge applies and the pass's LDS fits 64 KiB,
// otherwise the pass, then the merge.
int launch_merge_block_view(const uint16_t* o_norm, const float* m_part, const float* l_part,
                            int T, int S, int H, int dv, uint16_t* out, float* lse,
                            const BlockViewPass& bvp, hipStream_t stream);

}  // namespace stp
