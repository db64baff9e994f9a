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
// Rows are staged in a 3-deep LDS ring of 32-row tiles (36.5 KiB each) with
// global_load_lds_dwordx4, so no VGPRs hold KV data in flight.  Invalid
// candidates load a zero row and are masked to -inf before the exponent.

#include "stp_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kDQK = 576;
constexpr int kDV = 512;
constexpr int kRowBytes = kDQK * 2;                             // 1152
constexpr int kChunks = kRowBytes / 16;                         // 72 x 16 B
constexpr int kTileRows = 32;
constexpr int kGroupRows = 8;                                   // rows loaded by one wave
constexpr int kGroupBytes = kGroupRows * kRowBytes + 128;       // 9344 (+128: bank offset)
constexpr int kTileBytes = 4 * kGroupBytes;                     // 37376
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
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) char lds_t;
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// Source of every masked-out row: loads stay in bounds and bring zeros.
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[kRowBytes] = {};

// LDS tile layout: four groups of 8 rows (one group per wave when loading);
// inside a group the 16-byte chunks are chunk-major, so chunk c of group row
// rl sits at group + (c * 8 + rl) * 16.  One load instruction of a wave then
// fills 8 consecutive chunks of its 8 rows (1 KiB of LDS, 8 x 128 B of HBM),
// every lane keeps one row for the whole tile, and every LDS read address
// below is a per-lane base plus a compile-time offset.  Groups are padded by
// 128 B so that rows r and r + 8 fall in different halves of the 64 banks.
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
// The signal fences only stop the compiler from moving memory accesses across
// the barrier; the hardware wait is lgkmcnt(0) (LDS) alone.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left at their maximum
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): global address vaddr + offset, LDS address
// m0 + offset + 16 * lane -- the immediate offset applies to both sides.
// Issued from inline asm so that the compiler's
// wait-count pass does not track these loads: the tile ring waits for them
// explicitly (wait_vmcnt), and the compiler would otherwise drain the ring
// before every LDS access it cannot prove disjoint from the loads in flight.
template <int kOffset>
__device__ __forceinline__ void load_lds_16(const void* gptr, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off offset:%1" ::"v"(gptr), "n"(kOffset),
               "{m0}"(lds_addr));
}

template <int It>
__device__ __forceinline__ void load_row_chunks(const uint8_t* src, uint32_t lds_addr) {
  if constexpr (It < kSlotsPerThread) {
    // chunk column It: global src + 128 It, LDS lds_addr + 1024 It
    load_lds_16<It * 128>(src, lds_addr + It * (1024 - 128));
    load_row_chunks<It + 1>(src, lds_addr);
  }
}

// Output modes of the decode kernel.
enum OutMode : int {
  kOutFinal = 0,       // out = o / l (bf16), lse
  kOutPartialF32 = 1,  // per split: o (unnormalised, fp32), m (natural log), l
  kOutPartialBf16 = 2  // per split: o / l (bf16), m (natural log), l -- the internal split path
};

template <int kMode>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sparse_mla_decode_kernel(DecodeArgs a) {
  // Three separate LDS objects: the compiler can then tell that the exchange
  // buffer and the id list never alias the tile ring.
  __shared__ __attribute__((aligned(16))) char s_tiles[kStages * kTileBytes];
  __shared__ __attribute__((aligned(16))) float s_xchg[kXchgBytes / 4];
  __shared__ __attribute__((aligned(16))) int32_t s_ids[kIdsMax];
  lds_t* lds = (lds_t*)s_tiles;
  int32_t* ids = s_ids;
  float* xchg = s_xchg;

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
  const int ntiles = (len + kTileRows - 1) / kTileRows;

  // candidate ids of this split, -1 for invalid ones and up to the tile edge
  const int32_t* src_ids = a.row_ids + (int64_t)t * a.cap + lo;
  for (int j = tid; j < ntiles * kTileRows; j += kThreads) {
    const int32_t id = j < len ? src_ids[j] : -1;
    ids[j] = (id >= 0 && id < a.kv_rows) ? id : -1;
  }
  __syncthreads();  // ids visible

  // Enqueue the 32 rows of tile i into ring stage st: lane keeps row
  // 8 * wave + lane % 8 and chunks 8 * it + lane / 8, it = 0..8.
  const int ld_row = wave * kGroupRows + (lane & 7);
  const int ld_col = (lane >> 3) * 16;
  auto issue = [&](int i, int st) {
    const int id = ids[i * kTileRows + ld_row];
    const uint8_t* src =
        (id >= 0 ? (const uint8_t*)a.kv + (int64_t)id * kRowBytes : g_zero_row) + ld_col;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds + st * kTileBytes + wave * kGroupBytes));
    load_row_chunks<0>(src, dst);
  };
  // The first two tiles are in flight while Q is fetched.
  if (ntiles > 0) issue(0, 0);
  if (ntiles > 1) issue(1, 1);

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

  // Per-lane LDS read bases (see the layout note above).
  //  K fragment of k-step ks: row lane % 32, chunk 36 dh + 2 ks + lane / 32.
  const int kr = lane & 31;
  const int k_base = (kr >> 3) * kGroupBytes + (kr & 7) * 16 + (36 * dh + (lane >> 5)) * 128;
  //  V^T fragment (transpose read): rows 16 kap + 4 (g / 2) + j / 4 (+ 8),
  //  values 256 dh + 32 mb + 16 (g % 2) + 4 (j % 4) .. + 3, g = lane / 16, j = lane % 16.
  const int vg = lane >> 4, vj = lane & 15;
  const int v_base = (4 * (vg >> 1) + (vj >> 2)) * 16 +
                     (32 * dh + 2 * (vg & 1) + ((vj & 3) >> 1)) * 128 + 8 * (vj & 1);

  floatx16 o[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) o[mb] = floatx16{};
  float m_ref = -INFINITY, m_true = -INFINITY, lsum = 0.f;

  // Pipeline (one barrier per tile).  At the top of iteration i the K
  // fragments of tile i are in registers and tiles i+1, i+2 are in the ring
  // or in flight.  Iteration i: QK MFMAs of tile i under the V transpose
  // reads of tile i; publish the logit half; wait for tile i+1 and barrier
  // (which also frees ring stage i % 3); enqueue tile i+3 there; softmax;
  // PV MFMAs of tile i under the K reads of tile i+1.
  shortx8 kf[kKSteps];
  wait_vmcnt<0>();  // tiles 0 and 1 (and Q)
  lds_barrier();
  if (ntiles > 2) issue(2, 2);
  if (ntiles > 0) {
    const lds_t* kp = lds + k_base;
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      kf[ks] = *(const __attribute__((address_space(3))) shortx8*)(kp + 256 * ks);
  }

  for (int i = 0; i < ntiles; ++i) {
    const int st = i % kStages;
    const lds_t* stage = lds + st * kTileBytes;
    const bool row_valid = ids[i * kTileRows + (lane & 31)] >= 0;
    const uint32_t vmask = (uint32_t)__ballot(row_valid);

    // S^T partial = K_tile[:, 288 dh .. +288] Q^T, with the tile's V^T
    // fragments read meanwhile.
    // two independent accumulator chains (dependent MFMAs issue ~1.5x slower)
    floatx16 acc = floatx16{}, acc2 = floatx16{};
    shortx4 v0[2][8], v1[2][8];
    const lds_t* vp = stage + v_base;
#pragma unroll
    for (int kap = 0; kap < 2; ++kap)
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        v0[kap][mb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_shortx4*)(vp + 2 * kap * kGroupBytes + 512 * mb));
        v1[kap][mb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_shortx4*)(vp + (2 * kap + 1) * kGroupBytes + 512 * mb));
      }
#pragma unroll
    for (int ks = 0; ks < kKSteps; ks += 2) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[ks]), qf[ks], acc,
                                                    0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[ks + 1]),
                                                     qf[ks + 1], acc2, 0, 0, 0);
    }
    // interleave: one MFMA, then two transpose reads
#pragma unroll
    for (int g = 0; g < kKSteps; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
    }
    __builtin_amdgcn_sched_barrier(0);
    acc += acc2;

    // publish this wave's half of the logits
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *(float4*)(xchg + ((wave * 4 + j) * 64 + lane) * 4) =
          make_float4(acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]);
    // tile i+1 must have landed (tile i+2 may still be in flight)
    if (i + 2 < ntiles)
      wait_vmcnt<kSlotsPerThread>();
    else
      wait_vmcnt<0>();
    lds_barrier();  // halves visible; tile i+1 visible; stage i % 3 read by every wave
    if (i + 3 < ntiles) issue(i + 3, st);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 p = *(const float4*)(xchg + (((wave ^ 2) * 4 + j) * 64 + lane) * 4);
      acc[4 * j] += p.x;
      acc[4 * j + 1] += p.y;
      acc[4 * j + 2] += p.z;
      acc[4 * j + 3] += p.w;
    }

    // mask, then the online softmax of this lane's head (base 2).  A tile
    // with no valid row leaves the state untouched (p = 0, no rescale).
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
      const float p = sv[r] == -INFINITY ? 0.f : fast_exp2(sv[r] - m_ref);
      psum += p;
      pk[r >> 3][r & 7] = (__bf16)p;
    }
    lsum += psum;

    // O^T[256 dh + 32 mb + m][head] += V^T P^T, with the next tile's K
    // fragments read meanwhile.
#pragma unroll
    for (int kap = 0; kap < 2; ++kap)
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const shortx8 vv = {v0[kap][mb][0], v0[kap][mb][1], v0[kap][mb][2], v0[kap][mb][3],
                            v1[kap][mb][0], v1[kap][mb][1], v1[kap][mb][2], v1[kap][mb][3]};
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pk[kap],
                                                        o[mb], 0, 0, 0);
      }
    {
      // (on the last tile this reads a stale stage: in bounds and unused)
      const lds_t* kp = lds + ((i + 1) % kStages) * kTileBytes + k_base;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks)
        kf[ks] = *(const __attribute__((address_space(3))) shortx8*)(kp + 256 * ks);
    }
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  const float l_tot = lsum + __shfl_xor(lsum, 32);
  if (!head_ok) return;
  // lane holds O^T[256 dh + 32 mb + 8 (r / 4) + 4 (lane / 32) + r % 4][head]
  const int dv_lane = 256 * dh + 4 * (lane >> 5);
  const bool live = m_true != -INFINITY;
  if (kMode == kOutPartialF32) {
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
    // bf16 o / l: the final output, or a normalised split partial
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = kMode == kOutFinal
                         ? a.out + ((int64_t)t * a.H + head) * kDV
                         : (uint16_t*)a.o_part + (((int64_t)t * a.S + s) * a.H + head) * kDV;
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
    if (dh == 0 && lane < 32) {
      if (kMode == kOutFinal) {
        if (a.lse)
          a.lse[(int64_t)t * a.H + head] = live ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
      } else {
        // normalised partial: l relative to m_ref, m reported as m_ref
        const int64_t k = ((int64_t)t * a.S + s) * a.H + head;
        a.m_part[k] = live ? m_ref * kLn2 : -INFINITY;
        a.l_part[k] = live ? l_tot : 0.f;
      }
    }
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

int launch_decode(int mode, const uint16_t* q, const uint16_t* kv, int64_t kv_rows,
                  const int32_t* row_ids, const int32_t* counts, int32_t cap, int32_t T, int32_t H,
                  float scale, int32_t S, float* o_part, float* m_part, float* l_part,
                  uint16_t* out, float* lse, hipStream_t stream) {
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
  if (mode == kOutPartialF32)
    sparse_mla_decode_kernel<kOutPartialF32><<<(unsigned)blocks, kThreads, 0, stream>>>(a);
  else if (mode == kOutPartialBf16)
    sparse_mla_decode_kernel<kOutPartialBf16><<<(unsigned)blocks, kThreads, 0, stream>>>(a);
  else
    sparse_mla_decode_kernel<kOutFinal><<<(unsigned)blocks, kThreads, 0, stream>>>(a);
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
  return align256(n * kDV * 2) + 2 * align256(n * 4);  // bf16 o / l, then m and l
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
    return launch_decode(kOutFinal, q, kv, kv_rows, row_ids, counts, cap, T, H, scale, 1, nullptr,
                         nullptr, nullptr, out, lse, stream);
  const size_t need = stp_sparse_mla_decode_workspace(T, H, cap, num_splits);
  if (!workspace || workspace_bytes < need)
    return stp::fail(STP_ERR_WORKSPACE, "sparse_mla_decode: workspace of %zu bytes needed, %zu given",
                     need, workspace_bytes);
  // split path: normalised bf16 partial outputs, merged with the
  // partition-combine weights l_s e^(m_s - M) / L
  const size_t n = (size_t)T * S * H;
  char* ws = (char*)workspace;
  uint16_t* o_norm = (uint16_t*)ws;
  float* m_part = (float*)(ws + align256(n * kDV * 2));
  float* l_part = (float*)(ws + align256(n * kDV * 2) + align256(n * 4));
  if (int rc = launch_decode(kOutPartialBf16, q, kv, kv_rows, row_ids, counts, cap, T, H, scale, S,
                             (float*)o_norm, m_part, l_part, nullptr, nullptr, stream))
    return rc;
  return stp::launch_merge_normalized(o_norm, m_part, l_part, T, S, H, kDV, out, lse, stream);
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
  return launch_decode(kOutPartialF32, q, kv, kv_rows, row_ids, counts, cap, T, H, scale, num_splits,
                       o_part, m_part, l_part, nullptr, nullptr, stream);
}
