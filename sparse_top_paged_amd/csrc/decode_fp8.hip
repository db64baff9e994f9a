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
// through a 3-slot ring of 32-row tiles, three tiles ahead: 21 KiB per tile
// instead of the 36 KiB of bf16 rows.  The workgroup dequantises each tile
// once into a double-buffered bf16 tile (v_cvt_scalef32_pk_bf16_fp8 at scale
// 1: every E4M3 value is a bf16 value, so the codes convert exactly; the
// conversion issues at half rate, so converting per wave would cost four
// times as much) and keeps the rows' scales beside it; then per wave:
//   S^T[32 rows x 16 heads] = K Q^T with v_mfma_f32_16x16x32_bf16; the four
//     128-value latent groups accumulate separately and are combined with the
//     rows' scales in fp32; the RoPE part adds unscaled.
//   O^T[512 x 16 heads] += V^T P^T with one v_mfma_f32_16x16x32_bf16 per 16
//     latent values: V^T by two ds_read_b64_tr_b16 (the 8 rows a lane group
//     holds: 4 of each 16-row block of S^T); the group scale goes into P^T
//     instead (P'[row] = P[row] * scale[row][group]), P^T being the lane's
//     own eight softmax weights of the two S^T blocks, in the same k-slot
//     order as the V^T rows.
// Each tile's MFMA streams are software-pipelined: K and V fragments are read
// eight steps ahead of their MFMAs, and the dequantisation of the next tile
// is spread between the QK MFMAs.  Online softmax in base 2 with the lazy
// 2^8 rescale; invalid candidates load the zero row and are masked.  Splits
// write normalised bf16 partial states merged by the split-KV merge kernel.
// Cost: every wave reads the whole bf16 tile for its 16 heads (about 330 KB
// of LDS traffic per tile and workgroup), which makes the per-tile compute,
// not the row gather, the bound of this kernel.  The MFMAs write VGPRs (a
// build flag of this file), so O^T stays in one register file across the
// tile instead of moving between AGPRs and VGPRs around the QK accumulators;
// bf16 rows are 1184 B apart, so the eight rows a half-wave's transposed V
// read touches fall on distinct banks.

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
constexpr int kStages = 3;                  // raw-row ring (two tiles in flight)
constexpr int kIdsMax = 1024;               // candidate ids of a split, staged in LDS
constexpr int kBfStride = 1184;             // bf16 tile row: 576 values + 32 B of bank offset
constexpr int kBfBytes = kTileRows * kBfStride;
constexpr int kDQK = 576;
constexpr int kDV = 512;
constexpr int kQKSteps = kDQK / 32;         // 18 k-steps of 16x16x32
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleLog2 = 8.0f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
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
  __shared__ __attribute__((aligned(1024))) char s_bf[2 * kBfBytes];
  __shared__ __attribute__((aligned(16))) float s_scale[2][kTileRows][4];
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

  // Q^T fragments (B of S^T = K Q^T): head 16 w + l % 16 of the group, values
  // 32 ks + 8 (l / 16) .. + 7; zero past H.  Loaded together with the
  // candidate ids, before any tile load: a wait for them issued after the
  // tile loads would also wait for the whole ring.
  const int head = hg * kHeadsPerWG + 16 * wave + (lane & 15);
  bf16x8 qf[kQKSteps];
  {
    const uint16_t* qrow = a.q + ((int64_t)t * a.H + min(head, a.H - 1)) * kDQK;
#pragma unroll
    for (int ks = 0; ks < kQKSteps; ++ks) {
      const uintx4 w = head < a.H ? *(const uintx4*)(qrow + 32 * ks + 8 * (lane >> 4))
                                  : uintx4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8, w);
    }
  }
  // candidate ids of this split (-1: invalid, or past its end)
  {
    const int32_t* src = a.row_ids + (int64_t)t * a.cap + lo;
    for (int i = tid; i < ntiles * kTileRows; i += kThreads) {
      const int32_t id = i < len ? src[i] : -1;
      s_ids[i] = (id >= 0 && id < a.kv_rows) ? id : -1;
    }
  }
  __syncthreads();  // ids in LDS, and the Q loads have landed
  // Q^T lives in AGPRs (MFMA reads its B operand there)
#pragma unroll
  for (int ks = 0; ks < kQKSteps; ++ks) asm volatile("" : "+a"(qf[ks]));

  const uint32_t ring = (uint32_t)(uintptr_t)(lds_t*)s_ring;
  // Tile j into raw stage j % kStages: slot k * 256 + tid holds chunk q of
  // the tile, row q / 41, column q % 41 (rows as stored, 656 B apart); slots
  // past the tile load the zero row into the padding.
  auto issue = [&](int j) {
    const uint32_t base = ring + (j % kStages) * kStageBytes;
    // the six ids first (branch-free), so their LDS reads overlap
    int32_t id[kSlots];
    int col[kSlots];
#pragma unroll
    for (int k = 0; k < kSlots; ++k) {
      const int q = k * kThreads + tid;
      const int row = q / kRowChunks;
      col[k] = q - row * kRowChunks;
      const int32_t v = s_ids[j * kTileRows + min(row, kTileRows - 1)];
      id[k] = row < kTileRows ? v : -1;
    }
#pragma unroll
    for (int k = 0; k < kSlots; ++k) {
      const uint8_t* p = id[k] >= 0 ? a.kv + (int64_t)id[k] * kRowBytes + 16 * col[k]
                                    : zero_row + (k * kThreads + tid < kTileRows * kRowChunks
                                                      ? 16 * col[k]
                                                      : 0);
      stp::load_lds_16<0>(p, __builtin_amdgcn_readfirstlane(base + (k * kThreads + wave * 64) * 16));
    }
  };
  // Dequantisation of raw tile j into bf16 buffer j % 2, once per workgroup:
  // the latent codes converted exactly (scale 1; every E4M3 value is a bf16
  // value), the RoPE values copied, the four scales of each row set aside.
  // Thread: latent chunks tid + 256 c (c < 4) of the tile's 32 x 32, RoPE
  // chunk tid (32 x 8), scales of row tid (< 32).
  auto dequant = [&](int j) {
    const lds_t* raw = (const lds_t*)s_ring + (j % kStages) * kStageBytes;
    lds_t* bf = (lds_t*)s_bf + (j & 1) * kBfBytes;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int q = c * kThreads + tid;
      const int row = q >> 5, col = q & 31;
      const uintx4 w =
          *(const __attribute__((address_space(3))) uintx4*)(raw + row * kRowBytes + 16 * col);
      const uintx4 lo4 = {cvt2<false>(w[0]), cvt2<true>(w[0]), cvt2<false>(w[1]), cvt2<true>(w[1])};
      const uintx4 hi4 = {cvt2<false>(w[2]), cvt2<true>(w[2]), cvt2<false>(w[3]), cvt2<true>(w[3])};
      __attribute__((address_space(3))) uintx4* d =
          (__attribute__((address_space(3))) uintx4*)(bf + row * kBfStride + 32 * col);
      d[0] = lo4;
      d[1] = hi4;
    }
    {
      const int row = tid >> 3, col = tid & 7;
      const uintx4 w = *(const __attribute__((address_space(3))) uintx4*)(
          raw + row * kRowBytes + 528 + 16 * col);
      *(__attribute__((address_space(3))) uintx4*)(bf + row * kBfStride + 1024 + 16 * col) = w;
    }
    if (tid < kTileRows)
      *(__attribute__((address_space(3))) floatx4*)&s_scale[j & 1][tid][0] =
          *(const __attribute__((address_space(3))) floatx4*)(raw + tid * kRowBytes + 512);
  };

  floatx4 o[kDV / 16];  // O^T[16 mb + 4 (l / 16) + r][head], AGPRs
#pragma unroll
  for (int mb = 0; mb < kDV / 16; ++mb) o[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, lsum = 0.f;  // lsum: this lane's rows
  const int gq = lane >> 4, j16 = lane & 15;
  // K fragment of QK step k (rows 16 mbk + l % 16, values 32 ks + 8 (l / 16)
  // .. + 7): steps 0 .. 31 cycle through the four latent groups and the two
  // row blocks (k = 8 kk + 2 g + mbk, ks = 4 g + kk) so that consecutive
  // MFMAs feed different accumulators; steps 32 .. 35 are the RoPE values.
  const uint32_t k_off = j16 * kBfStride + 16 * gq;
  auto k_step = [](int k, int& ks, int& mbk, int& g) {
    if (k < 32) {
      mbk = k & 1;
      g = (k >> 1) & 3;
      ks = 4 * g + (k >> 3);
    } else {
      mbk = k & 1;
      g = 4;
      ks = 16 + ((k - 32) >> 1);
    }
  };
  // V^T reads (ds_read_b64_tr_b16) for the A operand of a 16x16x32 step, k-slots
  // 8 gq .. 8 gq + 7 = rows 4 gq + 0..3, then 16 + 4 gq + 0..3: lane (gq, j16)
  // points at row 4 gq + j16 / 4 (+ 16 for the second read), values
  // 16 mb + 4 (j16 % 4) .. + 3; the transpose hands lane l value 16 mb + l % 16.
  const uint32_t v_off = (4 * gq + (j16 >> 2)) * kBfStride + 8 * (j16 & 3);
  // dequantisation work of this thread (see dequant): latent chunks of rows
  // 8 c + tid / 32, column tid % 32; RoPE chunk tid % 8 of row tid / 8; the
  // scales of row tid % 32 (eight threads write the same value)
  const uint32_t dq_raw = (tid >> 5) * kRowBytes + 16 * (tid & 31);
  const uint32_t dq_bf = (tid >> 5) * kBfStride + 32 * (tid & 31);
  const uint32_t rp_raw = (tid >> 3) * kRowBytes + 528 + 16 * (tid & 7);
  const uint32_t rp_bf = (tid >> 3) * kBfStride + 1024 + 16 * (tid & 7);
  const uint32_t sc_raw = (tid & 31) * kRowBytes + 512;

  // Ring: raw tile j is loaded into slot j % 3 in iteration j - 3 (the
  // prologue loads tiles 0, 1, 2), dequantised in iteration j - 1 (tile 0 in
  // the prologue) and its bf16 copy used in iteration j.  In iteration i the
  // slots hold raw tile i + 1 (landed, to dequantise), i + 2 (in flight) and
  // i + 3 (issued into tile i's slot, whose dequantisation every wave finished
  // before the barrier); six loads per thread and tile, completing in order.
  for (int j = 0; j < kStages && j < ntiles; ++j) issue(j);
  if (ntiles > 0) {
    const int newer = min(kStages - 1, ntiles - 1);
    if (newer >= 2)
      stp::wait_vmcnt<2 * kSlots>();
    else if (newer == 1)
      stp::wait_vmcnt<kSlots>();
    else
      stp::wait_vmcnt<0>();
    stp::lds_barrier();
    dequant(0);
  }

  for (int it = 0; it < ntiles; ++it) {
    // raw tile it + 1 must have landed; raw tile it + 2 may still be in flight
    if (it + 1 < ntiles) {
      if (it + 2 < ntiles)
        stp::wait_vmcnt<kSlots>();
      else
        stp::wait_vmcnt<0>();
    }
    // bf16 tile it and raw tile it + 1 visible; every wave is done with tile
    // it - 1 (its bf16 buffer is free again) and with raw tile it
    stp::lds_barrier();
    if (it + kStages < ntiles) issue(it + kStages);
    const lds_t* bf = (const lds_t*)s_bf + (it & 1) * kBfBytes;
    // the next tile's raw rows and bf16 buffer.  In the last iteration there
    // is no next tile: the pass then converts a stale slot that no load
    // targets into the free buffer, which nothing reads (branch-free steps).
    const lds_t* raw = (const lds_t*)s_ring + ((it + 1) % kStages) * kStageBytes;
    lds_t* bfn = (lds_t*)s_bf + ((it + 1) & 1) * kBfBytes;
    const int r0 = it * kTileRows;

    // K fragment ring, eight steps ahead
    uintx4 kf[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int ks, mbk, g;
      k_step(k, ks, mbk, g);
      kf[k] = *(const __attribute__((address_space(3))) uintx4*)(bf + k_off + mbk * 16 * kBfStride +
                                                                  64 * ks);
    }
    // the next tile's raw chunks, its rows' scales; this tile's scales and
    // valid rows
    uintx4 dw[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      dw[c] = *(const __attribute__((address_space(3))) uintx4*)(raw + dq_raw + c * 8 * kRowBytes);
    const uintx4 rope = *(const __attribute__((address_space(3))) uintx4*)(raw + rp_raw);
    const floatx4 nscale = *(const __attribute__((address_space(3))) floatx4*)(raw + sc_raw);
    const uint32_t vmask = (uint32_t)__ballot(s_ids[r0 + (lane & 31)] >= 0);
    __builtin_amdgcn_sched_barrier(0);

    // S^T = K Q^T: 36 MFMA steps, each with the K read eight steps ahead and a
    // share of the next tile's dequantisation (two conversions, or its
    // stores), fenced so that the VALU work issues under the MFMAs
    floatx4 acc[5][2];
#pragma unroll
    for (int g = 0; g < 5; ++g) acc[g][0] = acc[g][1] = floatx4{0.f, 0.f, 0.f, 0.f};
    uint32_t cw[8];
#pragma unroll
    for (int k = 0; k < 36; ++k) {
      int ks, mbk, g;
      k_step(k, ks, mbk, g);
      acc[g][mbk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[k & 7]),
                                                            qf[ks], acc[g][mbk], 0, 0, 0);
      if (k + 8 < 36) {
        int ks2, mbk2, g2;
        k_step(k + 8, ks2, mbk2, g2);
        kf[k & 7] = *(const __attribute__((address_space(3))) uintx4*)(
            bf + k_off + mbk2 * 16 * kBfStride + 64 * ks2);
      }
      // chunk c: conversions in steps 2 + 5 c .. 5 + 5 c, stores in 6 + 5 c
      if (k >= 2 && k < 22) {
        const int c = (k - 2) / 5, ph = (k - 2) % 5;
        if (ph < 4) {
          const uint32_t w = dw[c][ph];
          cw[2 * ph] = cvt2<false>(w);
          cw[2 * ph + 1] = cvt2<true>(w);
        } else {
          __attribute__((address_space(3))) uintx4* d =
              (__attribute__((address_space(3))) uintx4*)(bfn + dq_bf + c * 8 * kBfStride);
          d[0] = uintx4{cw[0], cw[1], cw[2], cw[3]};
          d[1] = uintx4{cw[4], cw[5], cw[6], cw[7]};
        }
      } else if (k == 22) {
        *(__attribute__((address_space(3))) uintx4*)(bfn + rp_bf) = rope;
        *(__attribute__((address_space(3))) floatx4*)&s_scale[(it + 1) & 1][tid & 31][0] = nscale;
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // the S^T accumulators live in VGPRs (the AGPRs hold O^T and Q^T; letting
    // the accumulators take AGPRs makes the compiler move O^T out and back)
#pragma unroll
    for (int g = 0; g < 5; ++g) {
      asm volatile("" : "+v"(acc[g][0]));
      asm volatile("" : "+v"(acc[g][1]));
    }
    // this tile's scales (rows 16 mbk + 4 gq + r of this lane's accumulators),
    // read only now: during the QK steps their registers hold K fragments
    float sc[2][4][4];
#pragma unroll
    for (int mbk = 0; mbk < 2; ++mbk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const floatx4 v = *(const __attribute__((address_space(3))) floatx4*)&s_scale[it & 1]
                                                                                [16 * mbk + 4 * gq + r][0];
#pragma unroll
        for (int g = 0; g < 4; ++g) sc[mbk][r][g] = v[g];
      }
    // V ring for the PV steps, eight steps ahead, read while the softmax runs
    shortx4 vlo[8], vhi[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      vlo[mb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) shortx4*)(bf + v_off + 32 * mb));
      vhi[mb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) shortx4*)(bf + v_off + 16 * kBfStride + 32 * mb));
    }

    // S^T: the latent groups take their rows' scales in fp32, the RoPE part
    // adds unscaled; rows past the split or with an invalid id are masked
    float z[2][4];
    float zmax = -INFINITY;
#pragma unroll
    for (int mbk = 0; mbk < 2; ++mbk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float s = acc[4][mbk][r];
#pragma unroll
        for (int g = 0; g < 4; ++g) s = __builtin_fmaf(sc[mbk][r][g], acc[g][mbk][r], s);
        const int row = 16 * mbk + 4 * gq + r;
        s = (vmask >> row) & 1u ? s * a.scale_log2 : -INFINITY;
        z[mbk][r] = s;
        zmax = fmaxf(zmax, s);
      }
    zmax = fmaxf(zmax, __shfl_xor(zmax, 16));
    zmax = fmaxf(zmax, __shfl_xor(zmax, 32));
    // the reference maximum moves only when it is beaten by 2^8 (a first
    // finite maximum always moves it; O is still zero then)
    {
      const bool move = zmax > m_ref + kRescaleLog2;
      const float alpha = move ? __builtin_amdgcn_exp2f(m_ref - zmax) : 1.f;
      lsum *= alpha;
      if (__ballot(move && m_ref != -INFINITY)) {
#pragma unroll
        for (int mb = 0; mb < kDV / 16; ++mb) {
          floatx4 x = o[mb];
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] *= alpha;
          o[mb] = x;
        }
      }
      m_ref = move ? zmax : m_ref;
    }
    const float neg_m = m_ref == -INFINITY ? 0.f : -m_ref;
    float p[2][4];
#pragma unroll
    for (int mbk = 0; mbk < 2; ++mbk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[mbk][r] = __builtin_amdgcn_exp2f(z[mbk][r] + neg_m);
        lsum += p[mbk][r];
      }
    // P'^T of latent group g, k-slots 8 gq .. + 7 = rows 4 gq + 0..3 of each
    // 16-row block: P times the row's group scale, bf16
    auto p_frag = [&](int g) {
      return uintx4{pack_bf16(p[0][0] * sc[0][0][g], p[0][1] * sc[0][1][g]),
                    pack_bf16(p[0][2] * sc[0][2][g], p[0][3] * sc[0][3][g]),
                    pack_bf16(p[1][0] * sc[1][0][g], p[1][1] * sc[1][1][g]),
                    pack_bf16(p[1][2] * sc[1][2][g], p[1][3] * sc[1][3][g])};
    };
    uintx4 pf = p_frag(0), pf_next = p_frag(1);
    __builtin_amdgcn_sched_barrier(0);

    // O^T += V^T P'^T: one 16x16x32 step per 16 latent values, the V reads
    // eight steps ahead, the next group's P' built under the MFMAs
#pragma unroll
    for (int mb = 0; mb < kDV / 16; ++mb) {
      const shortx8 vf = {vlo[mb & 7][0], vlo[mb & 7][1], vlo[mb & 7][2], vlo[mb & 7][3],
                          vhi[mb & 7][0], vhi[mb & 7][1], vhi[mb & 7][2], vhi[mb & 7][3]};
      o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf),
                                                      __builtin_bit_cast(bf16x8, pf), o[mb], 0, 0,
                                                      0);
      if (mb + 8 < kDV / 16) {
        vlo[mb & 7] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)(bf + v_off + 32 * (mb + 8)));
        vhi[mb & 7] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)(bf + v_off + 16 * kBfStride +
                                                          32 * (mb + 8)));
      }
      if ((mb & 7) == 7 && mb < 31) {
        pf = pf_next;
        if (mb + 9 < kDV / 16) pf_next = p_frag((mb + 9) >> 3);
      }
      __builtin_amdgcn_sched_barrier(0);
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
