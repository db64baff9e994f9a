// Stage 3: top-k sparse MLA decode attention on gfx950.
//
// "5.1.1 · 从索引到 Kernel" §2.1 (load candidates straight from the cache
// instead of gathering them to scratch: eq. (3)), §2.2 (whole rows keep the
// transactions full), §3.1 eq. (4)-(6) (tile loop with a running max, sum and
// un-normalised numerator; empty tiles skipped), §3.2 (masks act before the
// exponent; split partial states, eq. (7)); "PagedAttention 与 RadixAttention：
// 上游机制与海光实现对照" §1.4 (exp2 with log2 e folded into the scale; split
// partitions), §1.4 part 4 and §5.2 (load each K/V row once for every query
// head that shares it).
//
// Data: q [T, H, 576] bf16, kv [rows, 576] bf16 (latent 512 first, rope 64
// last; V is the first 512 values of the same row), row_ids [T, cap].
//
// Decomposition.  All H query heads of a token read the same latent rows, so
// a workgroup owns 64 heads of one token and one contiguous range of its
// candidate positions (a split); the two head groups of a (token, split) run
// on the same XCD (blockIdx % 8 picks the XCD) so the second reads the rows
// from that XCD's L2.  Four wave64s per workgroup, one per SIMD:
//   wave w: head half hq = w & 1 (32 heads), dimension half dh = w >> 1.
//   Logits, transposed:  S^T[32 rows x 32 heads] = K[rows x 576] Q^T, each
//     wave contracting its 288 of the 576 dims with v_mfma_f32_32x32x16_bf16
//     (A = K fragment from LDS, B = Q^T fragment kept in 72 VGPRs), the two
//     halves exchanged through LDS and added (a + b == b + a, so both waves
//     hold bit-identical logits).  In this layout a lane owns one head.
//   Online softmax per lane (head) in base 2; the running reference max only
//     moves when a tile's max exceeds it by 2^8, so most tiles skip the
//     128-register rescale.
//   Output, transposed: O^T[256 dims x 32 heads] += V^T P^T over the tile,
//     A = V^T fragments read with ds_read_b64_tr_b16 (the LDS transpose
//     read), B = P^T taken straight from the logit registers: the k-slot to
//     row mapping of the V reads is chosen to match the accumulator layout,
//     so P never moves between lanes.
// Rows are staged in a 3-deep LDS ring of 32-row tiles (36 KiB each) with
// global_load_lds_dwordx4, so no VGPRs hold KV data in flight; chunks are
// XOR-swizzled per row so both the K reads (ds_read_b128) and the V transpose
// reads are free of bank conflicts.  Invalid candidates load a zero row and
// are masked to -inf before the exponent.

#include "stp_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kDQK = 576;
constexpr int kDV = 512;
constexpr int kRowBytes = kDQK * 2;                             // 1152
constexpr int kChunks = kRowBytes / 16;                         // 72 x 16 B
constexpr int kTileRows = 32;
constexpr int kTileBytes = kTileRows * kRowBytes;               // 36 KiB
constexpr int kStages = 3;
constexpr int kSlotsPerThread = kTileRows * kChunks / kThreads; // 9
constexpr int kHeadsPerWG = 64;
constexpr int kIdsMax = 4096;
constexpr int kLdsXchg = kStages * kTileBytes;                  // 110592
constexpr int kXchgBytes = 4 * 64 * 16 * 4;                     // 16 KiB
constexpr int kLdsIds = kLdsXchg + kXchgBytes;                  // 126976
constexpr int kLdsBytes = kLdsIds + kIdsMax * 4;                // 143360
constexpr int kKSteps = kDQK / 2 / 16;                          // 18 per wave
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.0f;

static_assert(kTileRows * kChunks % kThreads == 0, "tile slots per thread");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) char lds_t;
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// Source of every masked-out row: loads stay in bounds and bring zeros.
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[kRowBytes] = {};

// Per-row XOR on the 16-byte chunk index (search over both 32- and 64-bank
// LDS models: conflict-free for the K and the V-transpose read patterns).
__device__ __forceinline__ int swz(int r) {
  return (((r & 3) << 1) | ((r >> 2) & 1)) ^ (((r >> 3) & 1) << 1);
}
__device__ __forceinline__ int tile_off(int r, int c) { return r * kRowBytes + ((c ^ swz(r)) << 4); }

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* kv;
  int64_t kv_rows;
  const int32_t* row_ids;
  const int32_t* counts;
  int cap, T, H;
  float scale_log2;
  int S, G, ntasks;
  float* o_part;   // split mode: [T, S, H, 512], m/l in natural-log units
  float* m_part;
  float* l_part;
  uint16_t* out;   // direct mode: [T, H, 512] bf16
  float* lse;
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every outstanding global load (vmcnt(0)), which would drain the tile ring
// at each barrier; the tile loads are waited for explicitly instead.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool kSplit>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sparse_mla_decode_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) char smem[];
  lds_t* lds = (lds_t*)smem;
  int32_t* ids = (int32_t*)(smem + kLdsIds);
  float* xchg = (float*)(smem + kLdsXchg);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hq = wave & 1;
  const int dh = wave >> 1;

  // XCD-aware task map: the G head groups of one (token, split) get block
  // ids that agree mod 8 and are adjacent in dispatch order.
  const int bid = blockIdx.x;
  const int k8 = bid >> 3;
  const int task = (k8 / a.G) * 8 + (bid & 7);
  const int hg = k8 % a.G;
  if (task >= a.ntasks) return;
  const int t = task / a.S;
  const int s = task - t * a.S;

  int n = a.counts ? a.counts[t] : a.cap;
  n = min(max(n, 0), a.cap);
  const int chunk = (n + a.S - 1) / a.S;
  const int lo = min(n, s * chunk);
  const int len = min(n, lo + chunk) - lo;

  // candidate ids of this split, -1 for invalid ones and up to the tile edge
  const int32_t* src_ids = a.row_ids + (int64_t)t * a.cap + lo;
  const int len_pad = (len + kTileRows - 1) / kTileRows * kTileRows;
  for (int j = tid; j < len_pad; j += kThreads) {
    const int32_t id = j < len ? src_ids[j] : -1;
    ids[j] = (id >= 0 && id < a.kv_rows) ? id : -1;
  }

  // Q^T fragments: lane holds Q[head][288 dh + 16 ks + 8 (lane / 32) + 0..7].
  const int head = hg * kHeadsPerWG + hq * 32 + (lane & 31);
  const bool head_ok = head < a.H;
  bf16x8 qf[kKSteps];
  {
    const uint16_t* qrow =
        a.q + ((int64_t)t * a.H + (head_ok ? head : 0)) * kDQK + 288 * dh + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      shortx8 v = *(const shortx8*)(qrow + 16 * ks);
      if (!head_ok) v = shortx8{0, 0, 0, 0, 0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __syncthreads();  // ids visible

  const int ntiles = (len + kTileRows - 1) / kTileRows;

  // Enqueue the 32 rows of tile i into ring stage st: slot (wave*9+it)*64+lane
  // of the tile holds chunk (slot % 72) ^ swz(row) of row slot / 72.
  auto issue = [&](int i, int st) {
    lds_t* stage = lds + st * kTileBytes;
#pragma unroll
    for (int it = 0; it < kSlotsPerThread; ++it) {
      const int slot = (wave * kSlotsPerThread + it) * 64 + lane;
      const int r = slot / kChunks;
      const int c = (slot - r * kChunks) ^ swz(r);
      const int id = ids[i * kTileRows + r];
      const uint8_t* src = id >= 0 ? (const uint8_t*)a.kv + (int64_t)id * kRowBytes + c * 16
                                   : g_zero_row + c * 16;
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (lds_t*)(stage + (wave * kSlotsPerThread + it) * 1024), 16,
                                       0, 0);
    }
  };

  floatx16 o[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) o[mb] = floatx16{};
  float m_ref = -INFINITY, m_true = -INFINITY, lsum = 0.f;

#pragma unroll
  for (int i = 0; i < kStages - 1; ++i)
    if (i < ntiles) issue(i, i);

  for (int i = 0; i < ntiles; ++i) {
    const int st = i % kStages;
    if (i + 1 < ntiles)
      wait_vmcnt<kSlotsPerThread>();
    else
      wait_vmcnt<0>();
    lds_barrier();  // tile i landed for every wave; stage (i-1) % 3 is free
    if (i + kStages - 1 < ntiles) issue(i + kStages - 1, (i + kStages - 1) % kStages);

    const bool row_valid = ids[i * kTileRows + (lane & 31)] >= 0;
    const uint32_t vmask = (uint32_t)__ballot(row_valid);
    if (vmask == 0) continue;  // same for every wave of the workgroup

    const lds_t* stage = lds + st * kTileBytes;

    // S^T partial = K_tile[:, 288 dh .. +288] Q^T
    floatx16 acc = floatx16{};
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const int c = 36 * dh + 2 * ks + (lane >> 5);
      const shortx8 kraw = *(const __attribute__((address_space(3))) shortx8*)(stage + tile_off(lane & 31, c));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kraw), qf[ks], acc,
                                                    0, 0, 0);
    }
    // exchange halves with the partner wave (same heads, other dims)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *(float4*)(xchg + ((wave * 4 + j) * 64 + lane) * 4) =
          make_float4(acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]);
    lds_barrier();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 p = *(const float4*)(xchg + (((wave ^ 2) * 4 + j) * 64 + lane) * 4);
      acc[4 * j] += p.x;
      acc[4 * j + 1] += p.y;
      acc[4 * j + 2] += p.z;
      acc[4 * j + 3] += p.w;
    }

    // mask, then the online softmax of this lane's head (base 2)
    float sv[16];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rr = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      sv[r] = ((vmask >> rr) & 1u) ? acc[r] * a.scale_log2 : -INFINITY;
      mt = fmaxf(mt, sv[r]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    m_true = fmaxf(m_true, mt);
    const bool need = mt > m_ref + kRescaleLog2;
    if (__ballot(need)) {
      const float m_new = need ? mt : m_ref;
      const float alpha = need ? fast_exp2(m_ref - m_new) : 1.f;
      m_ref = m_new;
      lsum *= alpha;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) o[mb] *= alpha;
    }
    bf16x8 pk[2];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(sv[r] - m_ref);
      psum += p;
      pk[r >> 3][r & 7] = (__bf16)p;
    }
    lsum += psum;

    // O^T[256 dh + 32 mb + m][head] += V^T P^T
    const int g = lane >> 4;
    const int j16 = lane & 15;
#pragma unroll
    for (int kap = 0; kap < 2; ++kap) {
      const int row0 = 16 * kap + 4 * (g >> 1) + (j16 >> 2);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const int dvi = 256 * dh + 32 * mb + 16 * (g & 1) + 4 * (j16 & 3);
        const int cc = dvi >> 3;
        const int boff = (dvi & 7) * 2;
        const shortx4 v0 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(stage + tile_off(row0, cc) + boff));
        const shortx4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_shortx4*)(stage + tile_off(row0 + 8, cc) + boff));
        const shortx8 vv = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pk[kap],
                                                        o[mb], 0, 0, 0);
      }
    }
  }

  const float l_tot = lsum + __shfl_xor(lsum, 32);
  if (!head_ok) return;
  // lane holds O^T[256 dh + 32 mb + 8 (r / 4) + 4 (lane / 32) + r % 4][head]
  const int dv_lane = 256 * dh + 4 * (lane >> 5);
  if (kSplit) {
    const bool live = m_true != -INFINITY;
    const float f = live ? fast_exp2(m_ref - m_true) : 0.f;  // rebase to the true maximum
    float* orow = a.o_part + (((int64_t)t * a.S + s) * a.H + head) * kDV;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *(float4*)(orow + dv_lane + 32 * mb + 8 * rq) =
            make_float4(o[mb][4 * rq] * f, o[mb][4 * rq + 1] * f, o[mb][4 * rq + 2] * f,
                        o[mb][4 * rq + 3] * f);
    if (dh == 0 && lane < 32) {
      const int64_t k = ((int64_t)t * a.S + s) * a.H + head;
      a.m_part[k] = live ? m_true * kLn2 : -INFINITY;
      a.l_part[k] = l_tot * f;
    }
  } else {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = a.out + ((int64_t)t * a.H + head) * kDV;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const uint32_t w0 = stp::f32_to_bf16_rne(o[mb][4 * rq] * inv) |
                            ((uint32_t)stp::f32_to_bf16_rne(o[mb][4 * rq + 1] * inv) << 16);
        const uint32_t w1 = stp::f32_to_bf16_rne(o[mb][4 * rq + 2] * inv) |
                            ((uint32_t)stp::f32_to_bf16_rne(o[mb][4 * rq + 3] * inv) << 16);
        *(uint2*)(orow + dv_lane + 32 * mb + 8 * rq) = make_uint2(w0, w1);
      }
    if (a.lse && dh == 0 && lane < 32)
      a.lse[(int64_t)t * a.H + head] = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

int32_t choose_splits(int32_t T, int32_t H, int32_t cap, int32_t requested) {
  const int G = (H + kHeadsPerWG - 1) / kHeadsPerWG;
  int S;
  if (requested > 0) {
    S = requested;
  } else {
    const int64_t wgs = (int64_t)T * G;
    S = wgs >= 256 ? 1 : (int)((256 + wgs - 1) / wgs);
    S = min(S, max(1, cap / 128));  // keep at least four tiles per split
  }
  S = max(S, (cap + kIdsMax - 1) / kIdsMax);  // a split's ids must fit the LDS list
  return max(S, 1);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int launch_decode(bool split, const uint16_t* q, const uint16_t* kv, int64_t kv_rows,
                  const int32_t* row_ids, const int32_t* counts, int32_t cap, int32_t T, int32_t H,
                  float scale, int32_t S, float* o_part, float* m_part, float* l_part,
                  uint16_t* out, float* lse, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)sparse_mla_decode_kernel<true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes) != hipSuccess ||
        hipFuncSetAttribute((const void*)sparse_mla_decode_kernel<false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes) != hipSuccess)
      return stp::fail(STP_ERR_HIP, "sparse_mla_decode: hipFuncSetAttribute failed");
    attr_set = true;
  }
  DecodeArgs a;
  a.q = q;
  a.kv = kv;
  a.kv_rows = kv_rows;
  a.row_ids = row_ids;
  a.counts = counts;
  a.cap = cap;
  a.T = T;
  a.H = H;
  a.scale_log2 = scale * kLog2e;
  a.S = S;
  a.G = (H + kHeadsPerWG - 1) / kHeadsPerWG;
  a.ntasks = T * S;
  a.o_part = o_part;
  a.m_part = m_part;
  a.l_part = l_part;
  a.out = out;
  a.lse = lse;
  const int64_t blocks = (int64_t)8 * a.G * ((a.ntasks + 7) / 8);
  if (blocks > INT32_MAX) return stp::fail(STP_ERR_INVALID_ARG, "sparse_mla_decode: grid too large");
  if (split)
    sparse_mla_decode_kernel<true><<<(unsigned)blocks, kThreads, kLdsBytes, stream>>>(a);
  else
    sparse_mla_decode_kernel<false><<<(unsigned)blocks, kThreads, kLdsBytes, stream>>>(a);
  return stp::check_launch("sparse_mla_decode_kernel");
}

int check_common(const uint16_t* q, const uint16_t* kv, int64_t kv_rows, const int32_t* row_ids,
                 int32_t cap, int32_t T, int32_t H, float scale) {
  using stp::fail;
  if (T < 0 || H < 1 || cap < 0 || kv_rows <= 0)
    return fail(STP_ERR_INVALID_ARG, "sparse_mla_decode: bad sizes T=%d H=%d cap=%d kv_rows=%lld",
                T, H, cap, (long long)kv_rows);
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
    return fail(STP_ERR_INVALID_ARG, "sparse_mla_decode: scale is not finite");
  if (T > 0 && (!q || !kv || (cap > 0 && !row_ids)))
    return fail(STP_ERR_INVALID_ARG, "sparse_mla_decode: null pointer");
  return STP_OK;
}

}  // namespace

extern "C" int32_t stp_sparse_mla_decode_splits(int32_t T, int32_t H, int32_t cap,
                                                int32_t num_splits) {
  if (T < 0 || H < 1 || cap < 0 || num_splits < 0) return 0;
  return choose_splits(T, H, cap, num_splits);
}

extern "C" size_t stp_sparse_mla_decode_workspace(int32_t T, int32_t H, int32_t cap,
                                                  int32_t num_splits) {
  const int32_t S = stp_sparse_mla_decode_splits(T, H, cap, num_splits);
  if (S <= 1) return 0;
  const size_t n = (size_t)T * S * H;
  return align256(n * kDV * 4) + 2 * align256(n * 4);
}

extern "C" int stp_sparse_mla_decode(const uint16_t* q, const uint16_t* kv, int64_t kv_rows,
                                     const int32_t* row_ids, const int32_t* counts, int32_t cap,
                                     int32_t T, int32_t H, float scale, int32_t num_splits,
                                     void* workspace, size_t workspace_bytes, uint16_t* out,
                                     float* lse, hipStream_t stream) {
  if (int rc = check_common(q, kv, kv_rows, row_ids, cap, T, H, scale)) return rc;
  if (num_splits < 0) return stp::fail(STP_ERR_INVALID_ARG, "sparse_mla_decode: num_splits < 0");
  if (T == 0) return STP_OK;
  if (!out) return stp::fail(STP_ERR_INVALID_ARG, "sparse_mla_decode: null out");
  const int32_t S = choose_splits(T, H, cap, num_splits);
  if (S == 1)
    return launch_decode(false, q, kv, kv_rows, row_ids, counts, cap, T, H, scale, 1, nullptr,
                         nullptr, nullptr, out, lse, stream);
  const size_t need = stp_sparse_mla_decode_workspace(T, H, cap, num_splits);
  if (!workspace || workspace_bytes < need)
    return stp::fail(STP_ERR_WORKSPACE, "sparse_mla_decode: workspace of %zu bytes needed, %zu given",
                     need, workspace_bytes);
  const size_t n = (size_t)T * S * H;
  char* ws = (char*)workspace;
  float* o_part = (float*)ws;
  float* m_part = (float*)(ws + align256(n * kDV * 4));
  float* l_part = (float*)(ws + align256(n * kDV * 4) + align256(n * 4));
  if (int rc = launch_decode(true, q, kv, kv_rows, row_ids, counts, cap, T, H, scale, S, o_part,
                             m_part, l_part, nullptr, nullptr, stream))
    return rc;
  return stp::launch_merge(o_part, m_part, l_part, T, S, H, kDV, out, lse, stream);
}

extern "C" int stp_sparse_mla_decode_partial(const uint16_t* q, const uint16_t* kv,
                                             int64_t kv_rows, const int32_t* row_ids,
                                             const int32_t* counts, int32_t cap, int32_t T,
                                             int32_t H, float scale, int32_t num_splits,
                                             float* o_part, float* m_part, float* l_part,
                                             hipStream_t stream) {
  if (int rc = check_common(q, kv, kv_rows, row_ids, cap, T, H, scale)) return rc;
  if (num_splits < 1)
    return stp::fail(STP_ERR_INVALID_ARG, "sparse_mla_decode_partial: num_splits must be >= 1");
  if ((cap + num_splits - 1) / num_splits > kIdsMax)
    return stp::fail(STP_ERR_INVALID_ARG,
                     "sparse_mla_decode_partial: ceil(cap / num_splits) exceeds %d", kIdsMax);
  if (T == 0) return STP_OK;
  if (!o_part || !m_part || !l_part)
    return stp::fail(STP_ERR_INVALID_ARG, "sparse_mla_decode_partial: null output");
  return launch_decode(true, q, kv, kv_rows, row_ids, counts, cap, T, H, scale, num_splits,
                       o_part, m_part, l_part, nullptr, nullptr, stream);
}
