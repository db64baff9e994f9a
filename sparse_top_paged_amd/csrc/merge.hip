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

__global__ __launch_bounds__(kThreads) void splitkv_merge_norm_wide_kernel(
    const uint16_t* __restrict__ o_norm, const float* __restrict__ m_part,
    const float* __restrict__ l_part, int S, int H, int dv, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  const int t = blockIdx.x;
  const int h = blockIdx.y * (kThreads / kPerHeadWide) + (threadIdx.x / kPerHeadWide);
  const int c0 = (threadIdx.x % kPerHeadWide) * 8;
  if (h >= H || c0 >= dv) return;
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
