// Sparse MLA decode over fp8_ds_mla latent rows (656 B) on gfx950.
//
// "HiSparse" walkthrough (the fp8_ds_mla cache shape and row constant: 512 B
// of quantised latent values, 16 B of scales, 128 B of RoPE values);
// "5.1.1 · 从索引到 Kernel" §3.1 eq. (4)-(6) (online softmax), §3.2 (mask
// before the exponent), §7.2 (dequantise right after the tile load, apply the
// scale before QK and AV, never gather the codes to a scratch copy first);
// "PagedAttention 与 RadixAttention" §1.4 (exp2 with log2 e in the scale).
//
// Row: latent value i = e4m3(code_i) * scale_{i / 128} (OCP E4M3, four
// float32 scales at bytes 512..527), RoPE values bf16 at bytes 528..655; the
// key is the 576 values (latent, RoPE), the value vector the first 512.
//
// One 256-thread workgroup per (token, 64-head group, split); wave w owns
// heads 16 w .. 16 w + 15 of the group, the N dimension of its 16x16 MFMAs.
// Rows travel HBM -> LDS as they are stored (656 B, global_load_lds_dwordx4)
// through a 5-stage ring of 32-row tiles, four tiles ahead: 21 KiB per tile
// instead of the 36 KiB of bf16 rows.  Each wave converts what it reads:
//   S^T[32 rows x 16 heads] = K Q^T with v_mfma_f32_16x16x32_bf16, K
//     fragments (8 codes of one row) turned into bf16 by
//     v_cvt_scalef32_pk_bf16_fp8 at scale 1 (every E4M3 value is exact in
//     bf16); the four 128-value groups accumulate separately and are
//     combined with the rows' scales in fp32; the RoPE part is read as bf16.
//   O^T[512 x 16 heads] += V^T P^T with v_mfma_f32_16x16x16_bf16: V^T
//     fragments by ds_read_b64_tr_b8 (one latent column for 8 rows, the two
//     16-row k-steps at once), converted the same way; the group scale goes
//     into P^T instead (P'[row] = P[row] * scale[row][group]), P^T being the
//     lane's own four softmax weights of the S^T accumulator.
// Online softmax in base 2 with the lazy 2^8 rescale; invalid candidates
// load the zero row and are masked.  Splits write normalised bf16 partial
// states merged by the split-KV merge kernel.

#include <algorithm>

#include "stp_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kHeadsPerWG = 64;
constexpr int kRowBytes = 656;
constexpr int kRowChunks = kRowBytes / 16;  // 41
constexpr int kTileRows = 32;
constexpr int kSlots = 6;                   // loads per thread and tile: 6 * 256 >= 32 * 41
constexpr int kStageBytes = kSlots * kThreads * 16;  // 24 KiB (the last 224 slots pad)
constexpr int kStages = 5;
constexpr int kIdsMax = 1024;               // candidate ids of a split, staged in LDS
constexpr int kDQK = 576;
constexpr int kDV = 512;
constexpr int kQKSteps = kDQK / 32;         // 18 k-steps of 16x16x32
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.0f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int uintx2 __attribute__((ext_vector_type(2)));
typedef unsigned int uintx4 __attribute__((ext_vector_type(4)));
typedef int intx2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_t;

struct Fp8Args {
  const uint16_t* q;   // [T, H, 576] bf16
  const uint8_t* kv;   // [kv_rows, 656]
  int64_t kv_rows;
  const int32_t* row_ids;  // [T, cap]
  const int32_t* counts;   // [T] or null
  int cap, T, H, S, G;
  float scale_log2;
  uint16_t* out;     // [T, H, 512] bf16 (S == 1)
  float* lse;        // [T, H] (nullable)
  uint16_t* o_norm;  // S > 1: [T, S, H, 512] bf16, o / l
  float* m_part;     // [T, S, H] natural-log units
  float* l_part;
};

__device__ __attribute__((aligned(16))) uint8_t g_zero_fp8_row[kRowBytes] = {};

// two E4M3 codes (bytes 2 kHi .. 2 kHi + 1 of w) -> two bf16, exactly
template <bool kHi>
__device__ __forceinline__ uint32_t cvt2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sparse_mla_decode_fp8_kernel(Fp8Args a) {
  __shared__ __attribute__((aligned(1024))) char s_ring[kStages * kStageBytes];
  __shared__ int32_t s_ids[kIdsMax];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint8_t* zero_row = g_zero_fp8_row;
  asm volatile("" : "+s"(zero_row));

  // XCD-aware task map, as for the bf16 rows: all workgroups of a token share
  // a block-id residue mod 8, so they run on one XCD and share its L2
  const int bid = blockIdx.x;
  const int xk = bid >> 3;
  const int per_token = a.S * a.G;
  const int t = (xk / per_token) * 8 + (bid & 7);
  const int rem = xk % per_token;
  const int s = rem / a.G;
  const int hg = rem - s * a.G;
  if (t >= a.T) return;

  int n = a.counts ? a.counts[t] : a.cap;
  n = min(max(n, 0), a.cap);
  const int chunk = (n + a.S - 1) / a.S;
  const int lo = min(n, s * chunk);
  const int len = min(n, lo + chunk) - lo;
  const int ntiles = (len + kTileRows - 1) / kTileRows;

  // candidate ids of this split (-1: invalid, or past its end)
  {
    const int32_t* src = a.row_ids + (int64_t)t * a.cap + lo;
    for (int i = tid; i < ntiles * kTileRows; i += kThreads) {
      const int32_t id = i < len ? src[i] : -1;
      s_ids[i] = (id >= 0 && id < a.kv_rows) ? id : -1;
    }
  }
  __syncthreads();

  const uint32_t ring = (uint32_t)(uintptr_t)(lds_t*)s_ring;
  // Tile j into stage j % kStages: slot k * 256 + tid holds chunk q of the
  // tile, row q / 41, column q % 41 (rows as stored, 656 B apart); slots past
  // the tile load the zero row into the padding.
  auto issue = [&](int j) {
    const uint32_t base = ring + (j % kStages) * kStageBytes;
#pragma unroll
    for (int k = 0; k < kSlots; ++k) {
      const int q = k * kThreads + tid;
      const int row = q / kRowChunks, col = q - row * kRowChunks;
      const int32_t id = row < kTileRows ? s_ids[j * kTileRows + row] : -1;
      const uint8_t* p = id >= 0 ? a.kv + (int64_t)id * kRowBytes + 16 * col
                                 : zero_row + (row < kTileRows ? 16 * col : 0);
      stp::load_lds_16<0>(p, __builtin_amdgcn_readfirstlane(base + (k * kThreads + wave * 64) * 16));
    }
  };
  for (int j = 0; j < kStages - 1 && j < ntiles; ++j) issue(j);

  // Q^T fragments (B of S^T = K Q^T): head 16 w + l % 16 of the group, values
  // 32 ks + 8 (l / 16) .. + 7; zero past H.  Kept in AGPRs.
  const int head = hg * kHeadsPerWG + 16 * wave + (lane & 15);
  bf16x8 qf[kQKSteps];
  {
    const uint16_t* qrow = a.q + ((int64_t)t * a.H + min(head, a.H - 1)) * kDQK;
#pragma unroll
    for (int ks = 0; ks < kQKSteps; ++ks) {
      const uintx4 w = head < a.H ? *(const uintx4*)(qrow + 32 * ks + 8 * (lane >> 4))
                                  : uintx4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8, w);
      asm volatile("" : "+a"(qf[ks]));
    }
  }

  floatx4 o[kDV / 16];  // O^T[16 mb + 4 (l / 16) + r][head], AGPRs
#pragma unroll
  for (int mb = 0; mb < kDV / 16; ++mb) o[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, lsum = 0.f;  // lsum: this lane's rows
  const int gq = lane >> 4, j16 = lane & 15;
  // V^T read: lane (gq, j16) points at tile row 4 gq + j16 / 2 (the first four
  // rows of the pair), or 16 + 4 gq + j16 / 2 - 4, bytes 8 (j16 % 2) of a
  // 16-value column block; the transpose hands lane l column l % 16 for the
  // eight rows, which are the rows 4 (l / 16) + r of the two 16-row k-steps.
  const int v_i8 = j16 >> 1;
  const int v_row = v_i8 < 4 ? 4 * gq + v_i8 : 16 + 4 * gq + (v_i8 - 4);
  const uint32_t v_off = v_row * kRowBytes + 8 * (j16 & 1);

  for (int it = 0; it < ntiles; ++it) {
    const int newer = min(kStages - 2, ntiles - 1 - it);
    if (newer >= 3)
      stp::wait_vmcnt<3 * kSlots>();
    else if (newer == 2)
      stp::wait_vmcnt<2 * kSlots>();
    else if (newer == 1)
      stp::wait_vmcnt<kSlots>();
    else
      stp::wait_vmcnt<0>();
    stp::lds_barrier();  // tile it visible; every wave is done with tile it - 1
    if (it + kStages - 1 < ntiles) issue(it + kStages - 1);  // into tile it - 1's stage
    const lds_t* tile = (const lds_t*)s_ring + (it % kStages) * kStageBytes;
    const int r0 = it * kTileRows;

    // scales of this lane's accumulator rows 16 mbk + 4 gq + r, four groups
    float sc[2][4][4];
#pragma unroll
    for (int mbk = 0; mbk < 2; ++mbk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const floatx4 v = *(const __attribute__((address_space(3))) floatx4*)(
            tile + (16 * mbk + 4 * gq + r) * kRowBytes + 512);
#pragma unroll
        for (int g = 0; g < 4; ++g) sc[mbk][r][g] = v[g];
      }

    // S^T, two 16-row blocks
    floatx4 sacc[2];
#pragma unroll
    for (int mbk = 0; mbk < 2; ++mbk) {
      const lds_t* krow = tile + (16 * mbk + j16) * kRowBytes;
      floatx4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int ks = 4 * g + kk;
          const uintx2 w =
              *(const __attribute__((address_space(3))) uintx2*)(krow + 32 * ks + 8 * gq);
          const uintx4 kb = {cvt2<false>(w[0]), cvt2<true>(w[0]), cvt2<false>(w[1]),
                             cvt2<true>(w[1])};
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb), qf[ks],
                                                        acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) st[r] = __builtin_fmaf(sc[mbk][r][g], acc[r], st[r]);
      }
#pragma unroll
      for (int ks = 16; ks < kQKSteps; ++ks) {  // RoPE values, bf16 as stored
        const uintx4 w = *(const __attribute__((address_space(3))) uintx4*)(
            krow + 528 + 2 * (32 * (ks - 16) + 8 * gq));
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), qf[ks], st, 0,
                                                     0, 0);
      }
      sacc[mbk] = st;
    }

    // mask rows past the split or with an invalid id
    float zmax = -INFINITY;
#pragma unroll
    for (int mbk = 0; mbk < 2; ++mbk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * mbk + 4 * gq + r;
        const bool ok = s_ids[r0 + row] >= 0;
        sacc[mbk][r] = ok ? sacc[mbk][r] * a.scale_log2 : -INFINITY;
        zmax = fmaxf(zmax, sacc[mbk][r]);
      }
    zmax = fmaxf(zmax, __shfl_xor(zmax, 16));
    zmax = fmaxf(zmax, __shfl_xor(zmax, 32));
    // the reference maximum moves only when it is beaten by 2^8
    if (__ballot(zmax > m_ref + kRescaleLog2)) {
      const float alpha =
          zmax > m_ref + kRescaleLog2 ? __builtin_amdgcn_exp2f(m_ref - zmax) : 1.f;
      m_ref = zmax > m_ref + kRescaleLog2 ? zmax : m_ref;
      lsum *= alpha;
#pragma unroll
      for (int mb = 0; mb < kDV / 16; ++mb) {
        floatx4 x = o[mb];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] *= alpha;
        o[mb] = x;
      }
    }
    const float neg_m = m_ref == -INFINITY ? 0.f : -m_ref;
    float p[2][4];
#pragma unroll
    for (int mbk = 0; mbk < 2; ++mbk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[mbk][r] = __builtin_amdgcn_exp2f(sacc[mbk][r] + neg_m);
        lsum += p[mbk][r];
      }
    // P'^T per k-step and latent group: P times the row's group scale, bf16
    uintx2 pf[2][4];
#pragma unroll
    for (int mbk = 0; mbk < 2; ++mbk)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        pf[mbk][g] = uintx2{pack_bf16(p[mbk][0] * sc[mbk][0][g], p[mbk][1] * sc[mbk][1][g]),
                            pack_bf16(p[mbk][2] * sc[mbk][2][g], p[mbk][3] * sc[mbk][3][g])};

    // O^T += V^T P'^T: 32 column blocks of 16 latent values
#pragma unroll
    for (int mb = 0; mb < kDV / 16; ++mb) {
      const intx2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) intx2*)(tile + v_off + 16 * mb));
      const uint32_t w0 = (uint32_t)raw[0], w1 = (uint32_t)raw[1];
      const uintx2 v0 = {cvt2<false>(w0), cvt2<true>(w0)};  // rows 4 gq + 0..3
      const uintx2 v1 = {cvt2<false>(w1), cvt2<true>(w1)};  // rows 16 + 4 gq + 0..3
      const int g = mb >> 3;
      o[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, v0),
                                                        __builtin_bit_cast(shortx4, pf[0][g]),
                                                        o[mb], 0, 0, 0);
      o[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(shortx4, v1),
                                                        __builtin_bit_cast(shortx4, pf[1][g]),
                                                        o[mb], 0, 0, 0);
    }
  }

  // this wave's heads: l over the 32 rows of every tile (lanes l ^ 16, l ^ 32)
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (head >= a.H) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const bool split = a.S > 1;
  uint16_t* orow = split ? a.o_norm + (((int64_t)t * a.S + s) * a.H + head) * kDV
                         : a.out + ((int64_t)t * a.H + head) * kDV;
#pragma unroll
  for (int mb = 0; mb < kDV / 16; ++mb) {
    const uintx2 w = {pack_bf16(o[mb][0] * inv, o[mb][1] * inv),
                      pack_bf16(o[mb][2] * inv, o[mb][3] * inv)};
    *(uintx2*)(orow + 16 * mb + 4 * gq) = w;
  }
  if (lane < 16) {
    if (split) {
      const int64_t k = ((int64_t)t * a.S + s) * a.H + head;
      a.m_part[k] = lsum > 0.f ? m_ref * kLn2 : -INFINITY;
      a.l_part[k] = lsum;
    } else if (a.lse) {
      a.lse[(int64_t)t * a.H + head] = lsum > 0.f ? (m_ref + log2f(lsum)) * kLn2 : -INFINITY;
    }
  }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Splits: one workgroup per compute unit in one round when the tokens and
// head groups alone leave units idle, at least 4 tiles per split, and enough
// splits for each one's ids to fit the LDS list.
int fp8_splits(int32_t T, int32_t H, int32_t cap, int32_t requested) {
  const int G = (H + kHeadsPerWG - 1) / kHeadsPerWG;
  const int s_min = std::max(1, (cap + kIdsMax - 1) / kIdsMax);
  if (requested > 0) return std::max(requested, s_min);
  const int64_t wgs = std::max<int64_t>(1, (int64_t)T * G);
  const int64_t cus = stp::device_cus();
  int s = (int)std::max<int64_t>(1, cus / wgs);
  s = std::min(s, std::max(1, (cap + 4 * kTileRows - 1) / (4 * kTileRows)));
  return std::max(std::min(s, 16), s_min);
}

size_t fp8_workspace(int32_t T, int32_t H, int S) {
  if (S <= 1) return 0;
  const size_t n = (size_t)T * S * H;
  return align256(n * kDV * 2) + 2 * align256(n * 4);
}

}  // namespace

extern "C" int32_t stp_sparse_mla_decode_fp8_splits(int32_t T, int32_t H, int32_t cap,
                                                    int32_t num_splits) {
  if (T < 0 || H < 1 || cap < 0 || num_splits < 0) return 0;
  return fp8_splits(T, H, cap, num_splits);
}

extern "C" size_t stp_sparse_mla_decode_fp8_workspace(int32_t T, int32_t H, int32_t cap,
                                                      int32_t num_splits) {
  if (T < 0 || H < 1 || cap < 0 || num_splits < 0) return 0;
  return fp8_workspace(T, H, fp8_splits(T, H, cap, num_splits));
}

extern "C" int stp_sparse_mla_decode_fp8(const uint16_t* q, const uint8_t* kv, int64_t kv_rows,
                                         const int32_t* row_ids, const int32_t* counts,
                                         int32_t cap, int32_t T, int32_t H, float scale,
                                         int32_t num_splits, void* workspace,
                                         size_t workspace_bytes, uint16_t* out, float* lse,
                                         hipStream_t stream) {
  using stp::fail;
  if (T < 0 || H < 1 || cap < 0 || num_splits < 0)
    return fail(STP_ERR_INVALID_ARG, "sparse_mla_decode_fp8: bad sizes T=%d H=%d cap=%d", T, H,
                cap);
  if (kv_rows <= 0) return fail(STP_ERR_INVALID_ARG, "sparse_mla_decode_fp8: kv_rows <= 0");
  if (!(scale > 0.f) || scale == INFINITY)
    return fail(STP_ERR_INVALID_ARG, "sparse_mla_decode_fp8: scale must be positive and finite");
  if (T == 0) return STP_OK;
  if (!q || !kv || !row_ids || !out)
    return fail(STP_ERR_INVALID_ARG, "sparse_mla_decode_fp8: null pointer");
  const int S = fp8_splits(T, H, cap, num_splits);
  const int G = (H + kHeadsPerWG - 1) / kHeadsPerWG;
  const size_t need = fp8_workspace(T, H, S);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(STP_ERR_WORKSPACE, "sparse_mla_decode_fp8: workspace of %zu bytes needed", need);
  if ((cap + S - 1) / S > kIdsMax)
    return fail(STP_ERR_INVALID_ARG, "sparse_mla_decode_fp8: more than %d ids per split", kIdsMax);
  const int64_t blocks = ((int64_t)T + 7) / 8 * 8 * S * G;
  if (blocks > INT32_MAX) return fail(STP_ERR_INVALID_ARG, "sparse_mla_decode_fp8: grid");
  Fp8Args a{};
  a.q = q;
  a.kv = kv;
  a.kv_rows = kv_rows;
  a.row_ids = row_ids;
  a.counts = counts;
  a.cap = cap;
  a.T = T;
  a.H = H;
  a.S = S;
  a.G = G;
  a.scale_log2 = scale * kLog2e;
  a.out = out;
  a.lse = lse;
  if (S > 1) {
    uint8_t* ws = (uint8_t*)workspace;
    const size_t n = (size_t)T * S * H;
    a.o_norm = (uint16_t*)ws;
    a.m_part = (float*)(ws + align256(n * kDV * 2));
    a.l_part = (float*)(ws + align256(n * kDV * 2) + align256(n * 4));
  }
  sparse_mla_decode_fp8_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(a);
  if (int rc = stp::check_launch("sparse_mla_decode_fp8_kernel")) return rc;
  if (S > 1) return stp::launch_merge_normalized(a.o_norm, a.m_part, a.l_part, T, S, H, kDV, out, lse, stream);
  return STP_OK;
}
