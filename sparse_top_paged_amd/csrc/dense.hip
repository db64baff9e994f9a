// Dense paged attention with grouped query heads on gfx950: decode over block
// tables and prefix-extend over slot lists.
//
// "PagedAttention 与 RadixAttention：上游机制与海光实现对照": §1.1 (decode
// attention), §1.2 (block table: logical token t lives in slot
// table[t / P] * P + t % P), §1.4 part 4 (the grid runs over KV heads: one
// workgroup loads each KV tile once for every query head of its group), §3.2
// (shifted causal mask j <= i + (Lk - Lq): a fully visible prefix rectangle
// and a lower triangle), §3.3 (qo_indptr, kv_indptr, kv_indices), §3.4 (the
// tile loop stops at the last tile that any query of the block can see), §5
// (the bshd token-pool layout).
//
// Pool: keys and values as [slots, Hkv, 128] fp16, one 256-byte row per slot
// and KV head.  Both kernels stage 64-key tiles in LDS through registers:
// the loads of tile i + 1 are issued before tile i is computed and written
// to LDS after it, so their latency hides behind the compute.  Bad slots
// (unmapped page, outside the pool) load nothing and are masked.
//
// decode: one 256-thread workgroup per (request, KV head).  Lane = token for
// the scores (v_dot2_f32_f16 against the query heads held in registers, one
// or two heads per wave), lane = two output values for the PV sum; online
// softmax in base 2 per head.  At four query heads per KV head there is too
// little width for the matrix cores, and the kernel is bound by the KV bytes.
//
// extend: one 256-thread workgroup per (request, KV head, 64-query block);
// wave w computes query head g * group + w (group <= 4), every wave loads.
// Per 64-key tile and wave: S^T[64 keys x 64 queries] = K Q^T with 32
// v_mfma_f32_32x32x16_f16 (A = K rows from LDS, B = Q^T held in registers),
// the online softmax per query (a lane owns one query column, so its max and
// sum stay in the lane and its partner lane l ^ 32), then O^T[128 x 64] +=
// V^T P^T with 32 more MFMAs (A = V^T from a transposed LDS tile, B = P^T
// built from the S^T accumulators in place).  Tiles wholly inside the prefix
// rectangle skip the mask; the loop ends at the block's last visible key.

#include "stp_internal.h"

namespace {

constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;  // 256
constexpr int kTile = 64;          // keys per tile
constexpr int kThreads = 256;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 halfx2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int uintx4 __attribute__((ext_vector_type(4)));
typedef unsigned int uintx2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_t;

// K (and decode V) tile: 64 keys x 16 chunks of 16 B, chunk c of key t at
// t * 256 + ((c ^ (t % 16)) * 16): a wave reading one chunk of 64 keys, or
// 64 lanes reading 4 bytes each of one key, stays within few banks per pass.
__device__ __forceinline__ int tile_off(int t, int c) { return t * kRowBytes + ((c ^ (t & 15)) << 4); }

// Word e of a 16-byte vector as two halves.  The word is copied to a scalar
// first: hipcc's __builtin_bit_cast applied to a vector component directly
// reads component 0.
__device__ __forceinline__ halfx2 word_h2(uintx4 w, int e) {
  const uint32_t we = w[e];
  return __builtin_bit_cast(halfx2, we);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
using stp::lds_barrier;
using stp::load_lds_16;
using stp::pair_max;
using stp::pair_sum;
using stp::scale_acc;
using stp::wait_vmcnt;

// ---------------------------------------------------------------- decode --

struct DecArgs {
  const uint16_t* q;   // [B, Hq, 128]
  const uint16_t* k;   // [slots, Hkv, 128]
  const uint16_t* v;
  int64_t slots;
  const int32_t* table;  // [B, max_blocks]
  int max_blocks;
  const int32_t* ctx;    // [B]
  int B, Hq, Hkv, P;
  float scale_log2;
  uint16_t* out;  // [B, Hq, 128]
  float* lse;     // [B, Hq] (nullable)
};

__global__ __launch_bounds__(kThreads) void paged_gqa_decode_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(16))) char s_k[kTile * kRowBytes];
  __shared__ __attribute__((aligned(16))) char s_v[kTile * kRowBytes];
  __shared__ uint8_t s_ok[kTile];
  const int b = blockIdx.x / a.Hkv, g = blockIdx.x - (blockIdx.x / a.Hkv) * a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int group = a.Hq / a.Hkv;
  const int n = min(max(a.ctx[b], 0), a.max_blocks * a.P);
  const int ntiles = (n + kTile - 1) / kTile;
  const int32_t* trow = a.table + (int64_t)b * a.max_blocks;
  const int64_t head_stride = (int64_t)a.Hkv * kD;  // elements between slots

  // loader role: chunk lc of tokens lt + 16 u (u = 0..3) of the tile, K and V
  const int lc = tid & 15, lt = tid >> 4;
  auto slot_of = [&](int t) -> int64_t {  // -1 for a token past n or a bad slot
    if (t >= n) return -1;
    const int blk = t / a.P;
    const int page = trow[blk];
    const int64_t s = (int64_t)page * a.P + (t - blk * a.P);
    return (page >= 0 && s < a.slots) ? s : -1;
  };
  int64_t slot_next[4];
  uintx4 kr[4], vr[4];
  auto fetch = [&](const int64_t (&sl)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t e = sl[u] * head_stride + (int64_t)g * kD + lc * 8;
      kr[u] = sl[u] >= 0 ? *(const uintx4*)(a.k + e) : uintx4{0u, 0u, 0u, 0u};
      vr[u] = sl[u] >= 0 ? *(const uintx4*)(a.v + e) : uintx4{0u, 0u, 0u, 0u};
    }
  };
  auto stage = [&](const int64_t (&sl)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = lt + 16 * u;
      *(__attribute__((address_space(3))) uintx4*)((lds_t*)s_k + tile_off(t, lc)) = kr[u];
      *(__attribute__((address_space(3))) uintx4*)((lds_t*)s_v + tile_off(t, lc)) = vr[u];
      if (lc == 0) s_ok[t] = sl[u] >= 0 ? 1 : 0;
    }
  };

  // query heads of this wave: g * group + wave + 4 k, k < 2 (group <= 8)
  halfx2 qv[2][kD / 2];
  bool has[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int hl = wave + 4 * k;
    has[k] = hl < group;
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + g * group + (has[k] ? hl : 0)) * kD;
#pragma unroll
    for (int c = 0; c < kD / 8; ++c) {
      const uintx4 w = *(const uintx4*)(qrow + c * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[k][c * 4 + e] = word_h2(w, e);
    }
  }
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  float o0[2] = {0.f, 0.f}, o1[2] = {0.f, 0.f};

  int64_t sl_cur[4];
  if (ntiles > 0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) sl_cur[u] = slot_of(lt + 16 * u);
    fetch(sl_cur);
    stage(sl_cur);
#pragma unroll
    for (int u = 0; u < 4; ++u) slot_next[u] = slot_of(kTile + lt + 16 * u);
  }
  __syncthreads();
  for (int i = 0; i < ntiles; ++i) {
    // next tile's rows in flight, the one after's page entries too
    int64_t sl_after[4];
    if (i + 1 < ntiles) fetch(slot_next);
#pragma unroll
    for (int u = 0; u < 4; ++u) sl_after[u] = slot_of((i + 2) * kTile + lt + 16 * u);

    const bool ok_t = s_ok[lane] != 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (!has[k]) continue;  // wave-uniform
      // score of this lane's token for head k
      float z = 0.f;
#pragma unroll
      for (int c = 0; c < kD / 8; ++c) {
        const uintx4 w = *(const __attribute__((address_space(3))) uintx4*)((lds_t*)s_k +
                                                                             tile_off(lane, c));
#pragma unroll
        for (int e = 0; e < 4; ++e)
          z = __builtin_amdgcn_fdot2(qv[k][c * 4 + e], word_h2(w, e), z, false);
      }
      z = ok_t ? z * a.scale_log2 : -INFINITY;
      const float m_new = fmaxf(m[k], wave_max(z));
      if (m_new == -INFINITY) continue;  // nothing visible yet (wave-uniform)
      const float alpha = __builtin_amdgcn_exp2f(m[k] - m_new);
      const float p = __builtin_amdgcn_exp2f(z - m_new);
      l[k] = l[k] * alpha + wave_sum(p);
      m[k] = m_new;
      float a0 = o0[k] * alpha, a1 = o1[k] * alpha;
      // PV: lane owns values 2 lane, 2 lane + 1
#pragma unroll 16
      for (int t = 0; t < kTile; ++t) {
        const float pt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), t));
        const halfx2 vv = *(const __attribute__((address_space(3))) halfx2*)(
            (lds_t*)s_v + tile_off(t, lane >> 2) + (lane & 3) * 4);
        a0 = __builtin_fmaf(pt, (float)vv[0], a0);
        a1 = __builtin_fmaf(pt, (float)vv[1], a1);
      }
      o0[k] = a0;
      o1[k] = a1;
    }
    __syncthreads();  // every wave is done with tile i
    if (i + 1 < ntiles) stage(slot_next);
#pragma unroll
    for (int u = 0; u < 4; ++u) slot_next[u] = sl_after[u];
    __syncthreads();  // tile i + 1 visible
  }

#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (!has[k]) continue;
    const int h = g * group + wave + 4 * k;
    const float inv = l[k] > 0.f ? 1.f / l[k] : 0.f;
    const halfx2 ov = {(_Float16)(o0[k] * inv), (_Float16)(o1[k] * inv)};
    *(halfx2*)(a.out + ((int64_t)b * a.Hq + h) * kD + 2 * lane) = ov;
    if (a.lse && lane == 0)
      a.lse[(int64_t)b * a.Hq + h] = l[k] > 0.f ? (m[k] + log2f(l[k])) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------- extend --

constexpr int kQBlock = 64;  // queries per workgroup and head

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

struct ExtArgs {
  const uint16_t* q;  // [N, Hq, 128]
  const uint16_t* k;  // [slots, Hkv, 128]
  const uint16_t* v;
  int64_t slots;
  const int32_t* qo;   // [B + 1]
  const int32_t* kvp;  // [B + 1]
  const int32_t* kvi;  // [kvp[B]]
  int B, Hq, Hkv, qblocks;
  float scale_log2;
  uint16_t* out;  // [N, Hq, 128]
  float* lse;     // [N, Hq] (nullable)
};

// the row a bad key loads: zeros keep P V finite where P = 0
__device__ __attribute__((aligned(16))) uint8_t g_zero_head_row[kRowBytes] = {};

constexpr int kStageBytes = 2 * kTile * kRowBytes;  // K then V, 32 KiB

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void extend_attention_kernel(ExtArgs a) {
  __shared__ __attribute__((aligned(1024))) char s_tiles[2 * kStageBytes];
  __shared__ uint8_t s_ok[2][kTile];
  // all query blocks of one (request, KV head) on one XCD (block id mod 8),
  // so the later ones read the shared K / V tiles from that XCD's L2
  const int bid = blockIdx.x;
  const int xk = bid >> 3;
  const int bg = (xk / a.qblocks) * 8 + (bid & 7);
  const int qb_idx = xk % a.qblocks;
  if (bg >= a.B * a.Hkv) return;
  const int b = bg / a.Hkv, g = bg - (bg / a.Hkv) * a.Hkv;
  const int group = a.Hq / a.Hkv;
  const int q_base = a.qo[b], Lq = a.qo[b + 1] - q_base;
  const int k_base = a.kvp[b], Lk = a.kvp[b + 1] - k_base;
  const int i0 = qb_idx * kQBlock;
  if (i0 >= Lq) return;  // past the request's queries
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int prefix = Lk - Lq;
  // keys that some query of the block may see: j <= i_last + prefix
  const int i_last = min(Lq, i0 + kQBlock) - 1;
  const int jmax = max(0, min(Lk, i_last + prefix + 1));
  const int ntiles = (jmax + kTile - 1) / kTile;
  const bool active = wave < group;
  const int h = g * group + (active ? wave : 0);
  const int64_t head_bytes = (int64_t)a.Hkv * kRowBytes;  // between slots
  const uint8_t* zero_row = g_zero_head_row;
  asm volatile("" : "+s"(zero_row));

  // Tile loads go straight to LDS, 1 KiB (4 keys) per wave instruction:
  // instruction u of wave w fills keys 16 w + 4 u + lane / 16, LDS chunk
  // position lane % 16, so the lane fetches row chunk (lane % 16) ^ (key % 16)
  // -- the swizzled tile layout.
  const int my_key0 = 16 * wave + (lane >> 4);  // + 4 u
  auto slot_of = [&](int j) -> int64_t {
    if (j >= jmax) return -1;
    const int64_t s = a.kvi[k_base + j];
    return (s >= 0 && s < a.slots) ? s : -1;
  };
  auto issue = [&](const int64_t (&sl)[4], int stage) {
    const uint32_t base = (uint32_t)(uintptr_t)(lds_t*)s_tiles + stage * kStageBytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = my_key0 + 4 * u;
      const int c = (lane & 15) ^ (t & 15);
      const uint8_t* kp = sl[u] >= 0 ? (const uint8_t*)a.k + sl[u] * head_bytes + g * kRowBytes + 16 * c
                                     : zero_row + 16 * c;
      const uint8_t* vp = sl[u] >= 0 ? (const uint8_t*)a.v + sl[u] * head_bytes + g * kRowBytes + 16 * c
                                     : zero_row + 16 * c;
      const uint32_t row0 = __builtin_amdgcn_readfirstlane(base + (16 * wave + 4 * u) * kRowBytes);
      load_lds_16<0>(kp, row0);
      load_lds_16<0>(vp, row0 + kTile * kRowBytes);
      if ((lane & 15) == 0) s_ok[stage][t] = sl[u] >= 0 ? 1 : 0;
    }
  };

  // Q^T fragments (B operand of S^T = K Q^T), kept in AGPRs: query
  // 32 qb + lane % 32 of the block, values 16 ks + 8 (lane / 32) .. + 7
  halfx8 qf[2][kD / 16];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = i0 + 32 * qb + (lane & 31);
    const uint16_t* qrow = a.q + ((int64_t)(q_base + min(qi, Lq - 1)) * a.Hq + h) * kD;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      const uintx4 w = qi < Lq ? *(const uintx4*)(qrow + 16 * ks + 8 * (lane >> 5))
                               : uintx4{0u, 0u, 0u, 0u};
      qf[qb][ks] = __builtin_bit_cast(halfx8, w);
      asm volatile("" : "+a"(qf[qb][ks]));
    }
  }
  // LDS addresses.  In the swizzled tile, chunk c of key t sits at
  // t * 256 + ((c ^ (t % 16)) << 4); the stage bases are 32 KiB aligned, so
  // stepping c by a multiple of 2 (or 4) is an XOR on bits 5..7 (6..7) of the
  // address and stepping t by a multiple of 16 an immediate offset.
  //  K fragment (A of S^T): key 32 kb + lane % 32, chunk 2 ks + lane / 32.
  const uint32_t tiles_base = (uint32_t)(uintptr_t)(lds_t*)s_tiles;
  const int kq = lane & 31;
  const uint32_t k_off = kq * kRowBytes + ((((lane >> 5) ^ kq) & 15) << 4);
  //  V^T fragment (ds_read_b64_tr_b16): in each 16-lane group gq of the
  //  wave, lane j16 points at key 4 (gq / 2) + j16 / 4 (+ 8 for the second
  //  read) and values 16 (gq % 2) + 4 (j16 % 4) .. + 3 of a 32-value block;
  //  the transpose hands lane l value l % 32 of the block for keys
  //  4 (l / 32) + 0..3 (and 8 + 4 (l / 32) + 0..3), the keys the S^T
  //  accumulator holds in this lane's registers.  Value block mb: chunk
  //  4 mb + c0, an XOR of mb << 6.
  const int vq = lane >> 4, vj = lane & 15;
  const int v_key = 4 * (vq >> 1) + (vj >> 2);  // < 8
  const int v_c0 = 2 * (vq & 1) + ((vj & 3) >> 1);
  const uint32_t v_off = kTile * kRowBytes + v_key * kRowBytes + ((v_c0 ^ v_key) << 4) +
                         8 * (vj & 1);
  // keys 8 further: chunk XOR 8 more, i.e. bit 7
  const uint32_t v_off_hi = (v_off + 8 * kRowBytes) ^ 128u;

  floatx16 o[4][2];  // O^T[32 mb + row][32 qb + lane % 32]
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) o[mb][qb] = floatx16{};
  float m_ref[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};

  int64_t sl_next[4];
  if (ntiles > 0) {
    int64_t sl0[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) sl0[u] = slot_of(my_key0 + 4 * u);
    issue(sl0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) sl_next[u] = slot_of(kTile + my_key0 + 4 * u);
  }
  wait_vmcnt<0>();
  lds_barrier();  // tile 0 visible
  for (int it = 0; it < ntiles; ++it) {
    const int stage = it & 1;
    // the page entries of tile it + 2, then tile it + 1 into the other stage
    int64_t sl_after[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) sl_after[u] = slot_of((it + 2) * kTile + my_key0 + 4 * u);
    if (it + 1 < ntiles) issue(sl_next, stage ^ 1);
    const int j0 = it * kTile;
    const uint64_t okm = __ballot(s_ok[stage][lane] != 0);
    // no mask needed when every key is real and visible to every query
    const bool full = okm == ~0ull && j0 + kTile - 1 <= i0 + prefix && i0 + kQBlock <= Lq;
    if (active) {
      uint32_t kbase = tiles_base + stage * kStageBytes + k_off;
      uint32_t vbase = tiles_base + stage * kStageBytes + v_off;
      uint32_t vbase_hi = tiles_base + stage * kStageBytes + v_off_hi;
      // this lane's keys are 4 (lane / 32) + (8 (r / 4) + r % 4) of each half
      const uint64_t okl = okm >> (4 * (lane >> 5));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // S^T[key 32 kb + 8 (r / 4) + 4 (lane / 32) + r % 4][query 32 qb + lane % 32]
        floatx16 s[2] = {floatx16{}, floatx16{}};
#pragma unroll
        for (int ks = 0; ks < kD / 16; ++ks) {
          const halfx8 kf = __builtin_bit_cast(
              halfx8, *(const __attribute__((address_space(3))) uintx4*)(
                          (lds_t*)(uintptr_t)((kbase ^ (ks << 5)) + kb * 32 * kRowBytes)));
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[qb][ks], s[qb], 0, 0, 0);
        }
        halfx8 pf[2][2];  // P^T [k-step of 16 keys][qb]
        float alpha[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          // key j0 + 32 kb + 8 (r / 4) + 4 (lane / 32) + r % 4 is visible to
          // query qi iff it is real and 32 kb + 8 (r / 4) + r % 4 <= lim
          const int qi = i0 + 32 * qb + (lane & 31);
          const int lim = qi < Lq ? qi + prefix - j0 - 4 * (lane >> 5) : -1;
          float zmax = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float z = s[qb][r];
            if (!full) {
              const int jl = 32 * kb + 8 * (r >> 2) + (r & 3);
              const bool vis = ((okl >> jl) & 1) && jl <= lim;
              z = vis ? z : -INFINITY;
            }
            s[qb][r] = z;
            zmax = fmaxf(zmax, z);
          }
          const float tmax = pair_max(zmax) * a.scale_log2;
          // the reference maximum moves only when it is beaten by 2^8
          const bool move = tmax > m_ref[qb] + 8.0f;
          alpha[qb] = move ? __builtin_amdgcn_exp2f(m_ref[qb] - tmax) : 1.f;
          m_ref[qb] = move ? tmax : m_ref[qb];
          const float neg_m = m_ref[qb] == -INFINITY ? 0.f : -m_ref[qb];
          float ps = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][r], a.scale_log2, neg_m));
            ps += p;
            pf[r >> 3][qb][r & 7] = (_Float16)p;
          }
          lsum[qb] = lsum[qb] * alpha[qb] + pair_sum(ps);
        }
        if (__ballot(alpha[0] != 1.f || alpha[1] != 1.f)) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) scale_acc(o[mb][qb], alpha[qb]);
        }
        // O^T += V^T P^T over the 32 keys of this half, two k-steps of 16
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const uint32_t koff = (32 * kb + 16 * st) * kRowBytes;
            const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_shortx4*)(uintptr_t)((vbase ^ (mb << 6)) + koff));
            const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_shortx4*)(uintptr_t)((vbase_hi ^ (mb << 6)) + koff));
            const halfx8 vf = __builtin_bit_cast(
                halfx8, (shortx8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              o[mb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[st][qb], o[mb][qb], 0, 0, 0);
          }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) sl_next[u] = sl_after[u];
    wait_vmcnt<0>();  // this wave's loads of tile it + 1
    lds_barrier();    // tile it + 1 visible, stage it & 1 free
  }

  if (!active) return;
  // the exponents were taken against m_ref, so lse = (m_ref + log2 l) ln 2
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = i0 + 32 * qb + (lane & 31);
    if (qi >= Lq) continue;
    const float inv = lsum[qb] > 0.f ? 1.f / lsum[qb] : 0.f;
    uint16_t* orow = a.out + ((int64_t)(q_base + qi) * a.Hq + h) * kD;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const halfx4 w = {(_Float16)(o[mb][qb][4 * rq] * inv), (_Float16)(o[mb][qb][4 * rq + 1] * inv),
                          (_Float16)(o[mb][qb][4 * rq + 2] * inv),
                          (_Float16)(o[mb][qb][4 * rq + 3] * inv)};
        *(halfx4*)(orow + 32 * mb + 8 * rq + 4 * (lane >> 5)) = w;
      }
    if (a.lse && lane < 32)
      a.lse[(int64_t)(q_base + qi) * a.Hq + h] =
          lsum[qb] > 0.f ? (m_ref[qb] + log2f(lsum[qb])) * kLn2 : -INFINITY;
  }
}

int check_dense(const char* what, const void* q, const void* k, const void* v, int64_t slots,
                int32_t B, int32_t Hq, int32_t Hkv, int32_t head_dim, float scale, int max_group) {
  using stp::fail;
  if (B < 0 || Hq < 1 || Hkv < 1 || slots < 0)
    return fail(STP_ERR_INVALID_ARG, "%s: bad sizes B=%d Hq=%d Hkv=%d", what, B, Hq, Hkv);
  if (head_dim != kD) return fail(STP_ERR_INVALID_ARG, "%s: head_dim must be %d", what, kD);
  if (Hq % Hkv != 0 || Hq / Hkv > max_group)
    return fail(STP_ERR_INVALID_ARG, "%s: Hq / Hkv must be a whole number <= %d", what, max_group);
  if (!(scale > 0.f) || scale == INFINITY)
    return fail(STP_ERR_INVALID_ARG, "%s: scale must be positive and finite", what);
  if (B > 0 && (!q || !k || !v)) return fail(STP_ERR_INVALID_ARG, "%s: null pointer", what);
  return STP_OK;
}

}  // namespace

extern "C" int stp_paged_gqa_decode(const uint16_t* q, const uint16_t* k_pool,
                                    const uint16_t* v_pool, int64_t num_slots,
                                    const int32_t* block_table, int32_t max_blocks,
                                    const int32_t* ctx_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                    int32_t head_dim, int32_t page_size, float scale,
                                    uint16_t* out, float* lse, hipStream_t stream) {
  using stp::fail;
  if (int rc = check_dense("paged_gqa_decode", q, k_pool, v_pool, num_slots, B, Hq, Hkv, head_dim,
                           scale, 8))
    return rc;
  if (page_size < 1 || max_blocks < 0)
    return fail(STP_ERR_INVALID_ARG, "paged_gqa_decode: page_size %d / max_blocks %d", page_size,
                max_blocks);
  if ((int64_t)max_blocks * page_size > INT32_MAX)
    return fail(STP_ERR_INVALID_ARG, "paged_gqa_decode: max_blocks * page_size exceeds int32");
  if ((int64_t)B * Hkv > INT32_MAX) return fail(STP_ERR_INVALID_ARG, "paged_gqa_decode: grid");
  if (B == 0) return STP_OK;
  if (!ctx_lens || !out || (max_blocks > 0 && !block_table))
    return fail(STP_ERR_INVALID_ARG, "paged_gqa_decode: null pointer");
  DecArgs a{q, k_pool, v_pool, num_slots, block_table, max_blocks, ctx_lens, B, Hq, Hkv,
            page_size, scale * kLog2e, out, lse};
  paged_gqa_decode_kernel<<<B * Hkv, kThreads, 0, stream>>>(a);
  return stp::check_launch("paged_gqa_decode_kernel");
}

extern "C" int stp_extend_attention(const uint16_t* q, const uint16_t* k_pool,
                                    const uint16_t* v_pool, int64_t num_slots,
                                    const int32_t* qo_indptr, const int32_t* kv_indptr,
                                    const int32_t* kv_indices, int32_t B, int32_t Hq, int32_t Hkv,
                                    int32_t head_dim, int32_t max_extend_len, float scale,
                                    uint16_t* out, float* lse, hipStream_t stream) {
  using stp::fail;
  if (int rc = check_dense("extend_attention", q, k_pool, v_pool, num_slots, B, Hq, Hkv, head_dim,
                           scale, 4))
    return rc;
  if (max_extend_len < 0)
    return fail(STP_ERR_INVALID_ARG, "extend_attention: max_extend_len < 0");
  if (B == 0 || max_extend_len == 0) return STP_OK;
  if (!qo_indptr || !kv_indptr || !kv_indices || !out)
    return fail(STP_ERR_INVALID_ARG, "extend_attention: null pointer");
  const int qblocks = (max_extend_len + kQBlock - 1) / kQBlock;
  const int64_t blocks = ((int64_t)B * Hkv + 7) / 8 * 8 * qblocks;
  if (blocks > INT32_MAX) return fail(STP_ERR_INVALID_ARG, "extend_attention: grid too large");
  ExtArgs a{q, k_pool, v_pool, num_slots, qo_indptr, kv_indptr, kv_indices, B, Hq, Hkv, qblocks,
            scale * kLog2e, out, lse};
  extend_attention_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(a);
  return stp::check_launch("extend_attention_kernel");
}
