// Stage 4: split-KV merge on gfx950.
//
// "5.1.1 · 从索引到 Kernel" §3.2 eq. (7) (rescale every split to the common
// maximum; the partial numerators must be unnormalised), §7.1 eq. (14) (an
// empty split, l_s = 0, takes no part); "PagedAttention 与 RadixAttention：
// 上游机制与海光实现对照" §1.4 part 3 (the combine kernel, one small block per
// head and sequence).
//
// Design: memory-bound.  One 256-thread workgroup covers two heads of one
// token; 128 threads per head each own 4 consecutive output values and read
// the splits' float4 slices (coalesced 2 KiB per split and head).  The merge
// of normalised bf16 outputs with dv % 8 == 0 and up to 8 splits (the
// decode's) covers four heads per workgroup with 16-byte slices, every load
// issued before the first use.

#include "block_view.h"
#include "stp_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kPerHead = 128;

__global__ __launch_bounds__(kThreads) void splitkv_merge_kernel(
    const float* __restrict__ o_part, const float* __restrict__ m_part,
    const float* __restrict__ l_part, int S, int H, int dv, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  const int t = blockIdx.x;
  const int h = blockIdx.y * 2 + (threadIdx.x / kPerHead);
  if (h >= H) return;
  const int c0 = (threadIdx.x % kPerHead) * 4;
  // common maximum over live splits
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) {
    const int64_t k = ((int64_t)t * S + s) * H + h;
    if (l_part[k] > 0.f) M = fmaxf(M, m_part[k]);
  }
  uint16_t* orow = out + ((int64_t)t * H + h) * dv;
  if (M == -INFINITY) {  // no live split
    for (int c = c0; c < dv; c += 4 * kPerHead)
      *(uint2*)(orow + c) = make_uint2(0u, 0u);
    if (lse && c0 == 0) lse[(int64_t)t * H + h] = -INFINITY;
    return;
  }
  float L = 0.f;
  for (int s = 0; s < S; ++s) {
    const int64_t k = ((int64_t)t * S + s) * H + h;
    const float l = l_part[k];
    if (l > 0.f) L += expf(m_part[k] - M) * l;
  }
  const float inv = 1.f / L;
  for (int c = c0; c < dv; c += 4 * kPerHead) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < S; ++s) {
      const int64_t k = ((int64_t)t * S + s) * H + h;
      const float l = l_part[k];
      if (!(l > 0.f)) continue;
      const float w = expf(m_part[k] - M);
      const float4 o = *(const float4*)(o_part + k * dv + c);
      acc.x += w * o.x;
      acc.y += w * o.y;
      acc.z += w * o.z;
      acc.w += w * o.w;
    }
    const uint32_t lo = stp::pack_bf16x2(acc.x * inv, acc.y * inv);
    const uint32_t hi = stp::pack_bf16x2(acc.z * inv, acc.w * inv);
    *(uint2*)(orow + c) = make_uint2(lo, hi);
  }
  if (lse && c0 == 0) lse[(int64_t)t * H + h] = M + logf(L);
}

// Same merge from normalised bf16 split outputs O_s = o_s / l_s: the weight of
// split s is l_s e^(m_s - M) / L (the partition-combine form).  Up to
// eight splits, every split's (m, l) and output slice are loaded before any
// is used, so the loads of one thread overlap.

template <int S>
__device__ __forceinline__ void merge_norm_fixed(const uint16_t* __restrict__ o_norm,
                                                 const float* __restrict__ m_part,
                                                 const float* __restrict__ l_part, int t, int h,
                                                 int H, int dv, int c0, uint16_t* __restrict__ orow,
                                                 float* __restrict__ lse) {
  float m[S], l[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t k = ((int64_t)t * S + s) * H + h;
    m[s] = m_part[k];
    l[s] = l_part[k];
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < S; ++s)
    if (l[s] > 0.f) M = fmaxf(M, m[s]);
  if (M == -INFINITY) {
    for (int c = c0; c < dv; c += 4 * kPerHead) *(uint2*)(orow + c) = make_uint2(0u, 0u);
    if (lse && c0 == 0) lse[(int64_t)t * H + h] = -INFINITY;
    return;
  }
  float w[S], L = 0.f;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    w[s] = l[s] > 0.f ? expf(m[s] - M) * l[s] : 0.f;
    L += w[s];
  }
  const float invL = 1.f / L;
  for (int c = c0; c < dv; c += 4 * kPerHead) {
    uint2 raw[S];
#pragma unroll
    for (int s = 0; s < S; ++s)
      raw[s] = *(const uint2*)(o_norm + (((int64_t)t * S + s) * H + h) * dv + c);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const float ws = w[s] * invL;
      acc.x += ws * __uint_as_float(raw[s].x << 16);
      acc.y += ws * __uint_as_float(raw[s].x & 0xffff0000u);
      acc.z += ws * __uint_as_float(raw[s].y << 16);
      acc.w += ws * __uint_as_float(raw[s].y & 0xffff0000u);
    }
    const uint32_t lo = stp::pack_bf16x2(acc.x, acc.y);
    const uint32_t hi = stp::pack_bf16x2(acc.z, acc.w);
    *(uint2*)(orow + c) = make_uint2(lo, hi);
  }
  if (lse && c0 == 0) lse[(int64_t)t * H + h] = M + logf(L);
}

// The same merge for dv % 8 == 0 and up to eight splits, the form the decode
// uses: four heads per workgroup, 64 threads per head, each owning 8
// consecutive values per 512 (one 16-byte slice per split).  Every split's
// first slice is loaded before (m, l), and both before anything is used, so
// a thread waits for one round trip; the arithmetic and its order are those
// of merge_norm_fixed.
constexpr int kPerHeadWide = 64;
typedef unsigned int uintx4 __attribute__((ext_vector_type(4)));

template <int S>
__device__ __forceinline__ void merge_norm_wide(const uint16_t* __restrict__ o_norm,
                                                const float* __restrict__ m_part,
                                                const float* __restrict__ l_part, int t, int h,
                                                int H, int dv, int c0, uint16_t* __restrict__ orow,
                                                float* __restrict__ lse) {
  const uint16_t* src[S];
  uintx4 raw[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    src[s] = o_norm + (((int64_t)t * S + s) * H + h) * dv;
    raw[s] = *(const uintx4*)(src[s] + c0);
  }
  float m[S], l[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t k = ((int64_t)t * S + s) * H + h;
    m[s] = m_part[k];
    l[s] = l_part[k];
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < S; ++s)
    if (l[s] > 0.f) M = fmaxf(M, m[s]);
  if (M == -INFINITY) {
    for (int c = c0; c < dv; c += 8 * kPerHeadWide) *(uintx4*)(orow + c) = uintx4{0u, 0u, 0u, 0u};
    if (lse && c0 == 0) lse[(int64_t)t * H + h] = -INFINITY;
    return;
  }
  float w[S], L = 0.f;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    w[s] = l[s] > 0.f ? expf(m[s] - M) * l[s] : 0.f;
    L += w[s];
  }
  const float invL = 1.f / L;
  for (int c = c0; c < dv; c += 8 * kPerHeadWide) {
    if (c != c0) {
#pragma unroll
      for (int s = 0; s < S; ++s) raw[s] = *(const uintx4*)(src[s] + c);
    }
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const float ws = w[s] * invL;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += ws * __uint_as_float(raw[s][e] << 16);
        acc[2 * e + 1] += ws * __uint_as_float(raw[s][e] & 0xffff0000u);
      }
    }
    uintx4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = stp::pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
    *(uintx4*)(orow + c) = v;
  }
  if (lse && c0 == 0) lse[(int64_t)t * H + h] = M + logf(L);
}

// merge_norm_wide for a run-time S in [1, 8] (thread: head h of token t,
// values c0 .. c0 + 7 of every 512).
__device__ __forceinline__ void merge_norm_wide_any(const uint16_t* __restrict__ o_norm,
                                                    const float* __restrict__ m_part,
                                                    const float* __restrict__ l_part, int S,
                                                    int t, int h, int H, int dv, int c0,
                                                    uint16_t* __restrict__ out,
                                                    float* __restrict__ lse) {
  uint16_t* orow = out + ((int64_t)t * H + h) * dv;
  switch (S) {
    case 1: return merge_norm_wide<1>(o_norm, m_part, l_part, t, h, H, dv, c0, orow, lse);
    case 2: return merge_norm_wide<2>(o_norm, m_part, l_part, t, h, H, dv, c0, orow, lse);
    case 3: return merge_norm_wide<3>(o_norm, m_part, l_part, t, h, H, dv, c0, orow, lse);
    case 4: return merge_norm_wide<4>(o_norm, m_part, l_part, t, h, H, dv, c0, orow, lse);
    case 5: return merge_norm_wide<5>(o_norm, m_part, l_part, t, h, H, dv, c0, orow, lse);
    case 6: return merge_norm_wide<6>(o_norm, m_part, l_part, t, h, H, dv, c0, orow, lse);
    case 7: return merge_norm_wide<7>(o_norm, m_part, l_part, t, h, H, dv, c0, orow, lse);
    case 8: return merge_norm_wide<8>(o_norm, m_part, l_part, t, h, H, dv, c0, orow, lse);
    default: return;
  }
}

__global__ __launch_bounds__(kThreads) void splitkv_merge_norm_wide_kernel(
    const uint16_t* __restrict__ o_norm, const float* __restrict__ m_part,
    const float* __restrict__ l_part, int S, int H, int dv, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  const int h = blockIdx.y * (kThreads / kPerHeadWide) + (threadIdx.x / kPerHeadWide);
  const int c0 = (threadIdx.x % kPerHeadWide) * 8;
  if (h >= H || c0 >= dv) return;
  merge_norm_wide_any(o_norm, m_part, l_part, S, blockIdx.x, h, H, dv, c0, out, lse);
}

// The wide merge and the block-view pass of the same step in one launch.
// Both follow the decode and neither reads the other's output, so one launch
// pays one ramp and one drain for both.  Workgroups [0, T) run the block-view
// pass of token blockIdx.x; they come first so that their longer chains of
// dependent round trips start first.  Every later workgroup merges 16 heads
// of one token, 64 threads per head as in the wide merge.
constexpr int kMergeHeadsBv = stp::bv::kFThreads / kPerHeadWide;

// One instantiation per split count: the registers of the largest merge
// would otherwise set the occupancy of every launch.
template <int S>
__global__ __launch_bounds__(stp::bv::kFThreads) void merge_block_view_kernel(
    stp::bv::FillArgs fa, int T, const uint16_t* __restrict__ o_norm,
    const float* __restrict__ m_part, const float* __restrict__ l_part, int H, int dv,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  extern __shared__ uint64_t bitmap[];
  __shared__ int s_red[stp::bv::kFWaves];
  __shared__ int s_scan[stp::bv::kFWaves];
  const int b = blockIdx.x;
  if (b < T) {
    stp::bv::block_fill_token<true>(fa, b, bitmap, s_red, s_scan);
    return;
  }
  const int hblocks = (H + kMergeHeadsBv - 1) / kMergeHeadsBv;
  const int t = (b - T) / hblocks;
  const int h = ((b - T) % hblocks) * kMergeHeadsBv + threadIdx.x / kPerHeadWide;
  const int c0 = (threadIdx.x % kPerHeadWide) * 8;
  if (h >= H || c0 >= dv) return;
  merge_norm_wide<S>(o_norm, m_part, l_part, t, h, H, dv, c0, out + ((int64_t)t * H + h) * dv,
                     lse);
}

__global__ __launch_bounds__(kThreads) void splitkv_merge_norm_kernel(
    const uint16_t* __restrict__ o_norm, const float* __restrict__ m_part,
    const float* __restrict__ l_part, int S, int H, int dv, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  const int t = blockIdx.x;
  const int h = blockIdx.y * 2 + (threadIdx.x / kPerHead);
  if (h >= H) return;
  const int c0 = (threadIdx.x % kPerHead) * 4;
  uint16_t* orow = out + ((int64_t)t * H + h) * dv;
  switch (S) {
    case 1: return merge_norm_fixed<1>(o_norm, m_part, l_part, t, h, H, dv, c0, orow, lse);
    case 2: return merge_norm_fixed<2>(o_norm, m_part, l_part, t, h, H, dv, c0, orow, lse);
    case 3: return merge_norm_fixed<3>(o_norm, m_part, l_part, t, h, H, dv, c0, orow, lse);
    case 4: return merge_norm_fixed<4>(o_norm, m_part, l_part, t, h, H, dv, c0, orow, lse);
    case 5: return merge_norm_fixed<5>(o_norm, m_part, l_part, t, h, H, dv, c0, orow, lse);
    case 6: return merge_norm_fixed<6>(o_norm, m_part, l_part, t, h, H, dv, c0, orow, lse);
    case 7: return merge_norm_fixed<7>(o_norm, m_part, l_part, t, h, H, dv, c0, orow, lse);
    case 8: return merge_norm_fixed<8>(o_norm, m_part, l_part, t, h, H, dv, c0, orow, lse);
    default: break;
  }
  // any number of splits: two passes over (m, l), then the weighted sum
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) {
    const int64_t k = ((int64_t)t * S + s) * H + h;
    if (l_part[k] > 0.f) M = fmaxf(M, m_part[k]);
  }
  if (M == -INFINITY) {
    for (int c = c0; c < dv; c += 4 * kPerHead) *(uint2*)(orow + c) = make_uint2(0u, 0u);
    if (lse && c0 == 0) lse[(int64_t)t * H + h] = -INFINITY;
    return;
  }
  float L = 0.f;
  for (int s = 0; s < S; ++s) {
    const int64_t k = ((int64_t)t * S + s) * H + h;
    const float l = l_part[k];
    if (l > 0.f) L += expf(m_part[k] - M) * l;
  }
  const float invL = 1.f / L;
  for (int c = c0; c < dv; c += 4 * kPerHead) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < S; ++s) {
      const int64_t k = ((int64_t)t * S + s) * H + h;
      const float l = l_part[k];
      if (!(l > 0.f)) continue;
      const float w = expf(m_part[k] - M) * l * invL;
      const uint2 raw = *(const uint2*)(o_norm + k * dv + c);
      acc.x += w * __uint_as_float(raw.x << 16);
      acc.y += w * __uint_as_float(raw.x & 0xffff0000u);
      acc.z += w * __uint_as_float(raw.y << 16);
      acc.w += w * __uint_as_float(raw.y & 0xffff0000u);
    }
    const uint32_t lo = stp::pack_bf16x2(acc.x, acc.y);
    const uint32_t hi = stp::pack_bf16x2(acc.z, acc.w);
    *(uint2*)(orow + c) = make_uint2(lo, hi);
  }
  if (lse && c0 == 0) lse[(int64_t)t * H + h] = M + logf(L);
}

}  // namespace

namespace stp {

int launch_merge_normalized(const uint16_t* o_norm, const float* m_part, const float* l_part, int T,
                            int S, int H, int dv, uint16_t* out, float* lse, hipStream_t stream) {
  if (dv % 8 == 0 && S <= 8) {
    dim3 grid(T, (H + kThreads / kPerHeadWide - 1) / (kThreads / kPerHeadWide));
    splitkv_merge_norm_wide_kernel<<<grid, kThreads, 0, stream>>>(o_norm, m_part, l_part, S, H, dv,
                                                                   out, lse);
    return check_launch("splitkv_merge_norm_wide_kernel");
  }
  dim3 grid(T, (H + 1) / 2);
  splitkv_merge_norm_kernel<<<grid, kThreads, 0, stream>>>(o_norm, m_part, l_part, S, H, dv, out,
                                                           lse);
  return check_launch("splitkv_merge_norm_kernel");
}

int launch_merge_block_view(const uint16_t* o_norm, const float* m_part, const float* l_part,
                            int T, int S, int H, int dv, uint16_t* out, float* lse,
                            const BlockViewPass& bvp, hipStream_t stream) {
  const int nwords = max(1, (int)(((int64_t)bvp.max_blocks * bvp.page_size + 63) / 64));
  const size_t lds = (size_t)nwords * sizeof(uint64_t) + (size_t)bvp.max_blocks * 4;
  // one launch when the wide merge applies and the bitmap and the blocks'
  // pages fit the default dynamic LDS; otherwise the two launches one after
  // the other
  if (!(dv % 8 == 0 && S <= 8 && lds <= 64 * 1024)) {
    if (int rc = launch_block_fill(bvp, T, stream)) return rc;
    return launch_merge_normalized(o_norm, m_part, l_part, T, S, H, dv, out, lse, stream);
  }
  const int num_reqs = (bvp.num_reqs == 0 || bvp.max_blocks == 0) ? 0 : bvp.num_reqs;
  const uint64_t pdiv = ((1ull << 32) + (uint64_t)bvp.page_size - 1) / (uint64_t)bvp.page_size;
  bv::FillArgs fa{bvp.tok_out, bvp.slot_out, bvp.req_id, bvp.q_pos, bvp.block_table, num_reqs,
                  bvp.max_blocks, bvp.page_size, bvp.cap, pdiv, nwords, bvp.blk_indptr,
                  bvp.blk_logical, bvp.blk_page, bvp.blk_mask};
  const int hblocks = (H + kMergeHeadsBv - 1) / kMergeHeadsBv;
  const int64_t grid = (int64_t)T + (int64_t)T * hblocks;
  if (grid > INT32_MAX) return fail(STP_ERR_INVALID_ARG, "merge_block_view: grid too large");
  auto go = [&](auto s) {
    merge_block_view_kernel<decltype(s)::value><<<(unsigned)grid, bv::kFThreads, lds, stream>>>(
        fa, T, o_norm, m_part, l_part, H, dv, out, lse);
  };
  switch (S) {
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 3: go(std::integral_constant<int, 3>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    case 5: go(std::integral_constant<int, 5>{}); break;
    case 6: go(std::integral_constant<int, 6>{}); break;
    case 7: go(std::integral_constant<int, 7>{}); break;
    default: go(std::integral_constant<int, 8>{}); break;
  }
  return check_launch("merge_block_view_kernel");
}

int launch_merge(const float* o_part, const float* m_part, const float* l_part, int T, int S,
                 int H, int dv, uint16_t* out, float* lse, hipStream_t stream) {
  dim3 grid(T, (H + 1) / 2);
  splitkv_merge_kernel<<<grid, kThreads, 0, stream>>>(o_part, m_part, l_part, S, H, dv, out, lse);
  return check_launch("splitkv_merge_kernel");
}

}  // namespace stp

extern "C" int stp_splitkv_merge(const float* o_part, const float* m_part, const float* l_part,
                                 int32_t T, int32_t S, int32_t H, int32_t dv, uint16_t* out,
                                 float* lse, hipStream_t stream) {
  using stp::fail;
  if (T < 0 || S < 1 || H < 1 || dv < 1 || dv % 4 != 0)
    return fail(STP_ERR_INVALID_ARG, "splitkv_merge: bad sizes T=%d S=%d H=%d dv=%d", T, S, H, dv);
  if (H > 2 * 65535) return fail(STP_ERR_INVALID_ARG, "splitkv_merge: H %d too large", H);
  if (T == 0) return STP_OK;
  if (!o_part || !m_part || !l_part || !out)
    return fail(STP_ERR_INVALID_ARG, "splitkv_merge: null pointer");
  return stp::launch_merge(o_part, m_part, l_part, T, S, H, dv, out, lse, stream);
}

extern "C" int stp_splitkv_merge_normalized(const uint16_t* o_norm, const float* m_part,
                                            const float* l_part, int32_t T, int32_t S, int32_t H,
                                            int32_t dv, uint16_t* out, float* lse,
                                            hipStream_t stream) {
  using stp::fail;
  if (T < 0 || S < 1 || H < 1 || dv < 1 || dv % 4 != 0)
    return fail(STP_ERR_INVALID_ARG, "splitkv_merge_normalized: bad sizes T=%d S=%d H=%d dv=%d", T,
                S, H, dv);
  if (H > 2 * 65535) return fail(STP_ERR_INVALID_ARG, "splitkv_merge_normalized: H %d too large", H);
  if (T == 0) return STP_OK;
  if (!o_norm || !m_part || !l_part || !out)
    return fail(STP_ERR_INVALID_ARG, "splitkv_merge_normalized: null pointer");
  return stp::launch_merge_normalized(o_norm, m_part, l_part, T, S, H, dv, out, lse, stream);
}

extern "C" int stp_splitkv_merge_with_block_view(
    const uint16_t* o_norm, const float* m_part, const float* l_part, int32_t T, int32_t S,
    int32_t H, int32_t dv, uint16_t* out, float* lse, const int32_t* tok_out,
    const int32_t* slot_out, const int32_t* req_id, const int32_t* q_pos,
    const int32_t* block_table, int32_t num_reqs, int32_t max_blocks, int32_t page_size,
    int32_t cap, int32_t* blk_indptr, int32_t* blk_logical, int32_t* blk_page,
    uint64_t* blk_mask, hipStream_t stream) {
  using stp::fail;
  if (T < 0 || S < 1 || H < 1 || dv < 1 || dv % 4 != 0)
    return fail(STP_ERR_INVALID_ARG, "splitkv_merge_with_block_view: bad sizes T=%d S=%d H=%d dv=%d",
                T, S, H, dv);
  if (H > 2 * 65535)
    return fail(STP_ERR_INVALID_ARG, "splitkv_merge_with_block_view: H %d too large", H);
  if (int rc = stp::check_block_view_args("splitkv_merge_with_block_view", tok_out, slot_out,
                                          req_id, q_pos, T, block_table, num_reqs, max_blocks,
                                          page_size, cap, blk_indptr, blk_logical, blk_page,
                                          blk_mask))
    return rc;
  if (T == 0) return STP_OK;
  if (!o_norm || !m_part || !l_part || !out)
    return fail(STP_ERR_INVALID_ARG, "splitkv_merge_with_block_view: null pointer");
  const stp::BlockViewPass bvp{tok_out,    slot_out,   req_id,      q_pos,    block_table,
                               num_reqs,   max_blocks, page_size,   cap,      blk_indptr,
                               blk_logical, blk_page,  blk_mask};
  return stp::launch_merge_block_view(o_norm, m_part, l_part, T, S, H, dv, out, lse, bvp, stream);
}
