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
// and KV head.  Tiles of 64 keys (K and V, 32 KiB) are staged in LDS with a
// 16-byte chunk swizzle; bad slots (unmapped page, outside the pool, past
// the context) load a zero row and are masked before the exponent.
//
// decode: one 256-thread workgroup per (request, KV head, partition), two
// workgroups per compute unit.  Tiles are prefetched two ahead into
// registers and written to a double-buffered LDS tile; each wave takes 16
// keys of a tile for all heads of the group at once: S^T = K Q^T and
// O^T += V^T P^T on 16x16 MFMAs with the query heads as N (up to 16), P^T
// taken from the S^T accumulator registers as they are.  The four waves'
// softmax states are merged at the end; partitions of long contexts write
// partial states merged by a second kernel.  Bound by the KV bytes.
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

#include <algorithm>

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

// K and V tiles: 64 keys x 16 chunks of 16 B, chunk c of key t at
// t * 256 + ((c ^ swz(t)) * 16), swz(t) the two 2-bit halves of t % 16
// swapped.  Rows are 256 B, one full turn of the banks, so the swizzle alone
// spreads a read: 16 consecutive keys of one chunk (the K fragments) land on
// 16 different chunk positions, and so do 4 consecutive keys x 4 consecutive
// chunks (a half-wave of V^T transpose reads).
__device__ __forceinline__ int key_swz(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }
__device__ __forceinline__ int tile_off(int t, int c) { return t * kRowBytes + ((c ^ key_swz(t)) << 4); }

using stp::lds_barrier;
using stp::load_lds_16;
using stp::pair_max;
using stp::pair_sum;
using stp::scale_acc;
using stp::static_for;
using stp::wait_vmcnt;

// the row a bad key loads: zeros keep P V finite where P = 0
__device__ __attribute__((aligned(16))) uint8_t g_zero_head_row[kRowBytes] = {};

constexpr int kStageBytes = 2 * kTile * kRowBytes;  // one tile: K then V, 32 KiB

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// Tile loads go straight to LDS, 1 KiB (4 keys) per wave instruction:
// instruction u of wave w fills keys 16 w + 4 u + lane / 16 of the tile, LDS
// chunk position lane % 16, so the lane fetches row chunk
// (lane % 16) ^ swz(key) -- the swizzled tile layout.  K and V of one key
// share the slot.  slot < 0 loads the zero row.
__device__ __forceinline__ void issue_kv_rows(const uint8_t* kpool, const uint8_t* vpool,
                                              int64_t head_bytes, int g, const uint8_t* zero_row,
                                              uint32_t stage_base, int wave, int lane,
                                              const int64_t (&sl)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int t = 16 * wave + 4 * u + (lane >> 4);
    const int c = (lane & 15) ^ key_swz(t);
    const int64_t off = sl[u] * head_bytes + g * kRowBytes + 16 * c;
    const uint8_t* kp = sl[u] >= 0 ? kpool + off : zero_row + 16 * c;
    const uint8_t* vp = sl[u] >= 0 ? vpool + off : zero_row + 16 * c;
    const uint32_t row0 = __builtin_amdgcn_readfirstlane(stage_base + (16 * wave + 4 * u) * kRowBytes);
    load_lds_16<0>(kp, row0);
    load_lds_16<0>(vp, row0 + kTile * kRowBytes);
  }
}

// ---------------------------------------------------------------- decode --

constexpr int kTabChunk = 2048;    // block-table entries staged in LDS at a time
#ifndef STP_DEC_RING
#define STP_DEC_RING 2
#endif
#ifndef STP_DEC_WAVES
#define STP_DEC_WAVES 2
#endif
constexpr int kDecRing = STP_DEC_RING;    // tiles prefetched into registers
constexpr int kDecWaves = STP_DEC_WAVES;  // waves per SIMD (workgroups per CU)
constexpr int kDecMaxGroup = 16;   // query heads per KV head (the MFMA N width)

struct DecArgs {
  const uint16_t* q;   // [B, Hq, 128]
  const uint16_t* k;   // [slots, Hkv, 128]
  const uint16_t* v;
  int64_t slots;
  const int32_t* table;  // [B, max_blocks]
  int max_blocks;
  const int32_t* ctx;    // [B]
  int B, Hq, Hkv, P;
  int S, part;  // KV partitions per request and their length in tokens (a multiple of 64)
  float scale_log2;
  uint16_t* out;  // [B, Hq, 128]
  float* lse;     // [B, Hq] (nullable)
  float* o_part;  // S > 1: [B, S, Hq, 128] unnormalised, against m_part
  float* m_part;  // [B, S, Hq], base-2 exponent units
  float* l_part;  // [B, S, Hq]
};

struct DecLds {
  char tiles[2 * kStageBytes];  // double buffer; reused for the wave merge at the end
  int32_t tab[kTabChunk];
  uint8_t ok[2][kTile];
};

// One workgroup per (request, KV head, partition), four waves.  Tiles of 64
// keys (32 KiB of K and V) are prefetched kRing tiles ahead into registers
// (thread: 16 B of each of 4 keys, K and V), written to a double-buffered
// LDS tile when their turn comes, one barrier per tile.  Wave w takes keys
// 16 w .. 16 w + 15 of every tile and keeps its own softmax state for the
// group's heads; the four states are merged at the end.  Per tile and wave:
//   S^T[16 keys x 16 heads] = K Q^T with 4 v_mfma_f32_16x16x32_f16 (A = K
//     rows from LDS, B = Q^T in registers, heads past the group are zero);
//   lane l holds head l % 16, keys 4 (l / 16) .. + 3: the column max and sum
//     over the 16 keys take two lane exchanges;
//   O^T[128 x 16 heads] += V^T P^T with 8 v_mfma_f32_16x16x16_f16: A = V^T by
//     ds_read_b64_tr_b16 (lane group gq reads keys 4 gq .. + 3, the keys the
//     accumulator holds), B = P^T, the lane's own four softmax weights.
template <int kRing, int kWaves>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves, kWaves)))
void paged_gqa_decode_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(1024))) DecLds L;
  const int bg = blockIdx.x / a.S, p = blockIdx.x - (blockIdx.x / a.S) * a.S;
  const int b = bg / a.Hkv, g = bg - (bg / a.Hkv) * a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int group = a.Hq / a.Hkv;
  const int n_all = min(max(a.ctx[b], 0), a.max_blocks * a.P);
  // this partition's tokens [t0, n)
  const int t0 = p * a.part;
  const int n = min(n_all, t0 + a.part);
  const int ntiles = n > t0 ? (n - t0 + kTile - 1) / kTile : 0;
  const int nb = (n + a.P - 1) / a.P;  // table entries in use
  const int32_t* trow = a.table + (int64_t)b * a.max_blocks;
  const int64_t head_bytes = (int64_t)a.Hkv * kRowBytes;
  const uint8_t* kpool = (const uint8_t*)a.k + g * kRowBytes;
  const uint8_t* vpool = (const uint8_t*)a.v + g * kRowBytes;
  const uint8_t* zero_row = g_zero_head_row;
  asm volatile("" : "+s"(zero_row));
  const uint32_t tiles_base = (uint32_t)(uintptr_t)(lds_t*)L.tiles;
  const int tab_tokens = kTabChunk * a.P;  // a multiple of the tile size

  int chunk = -1;
  auto load_chunk = [&](int c) {  // all threads; caller brackets with barriers
    for (int i = tid; i < kTabChunk; i += kThreads) {
      const int e = c * kTabChunk + i;
      L.tab[i] = e < nb ? trow[e] : -1;
    }
    chunk = c;
  };
  // the chunk that holds tile j's table entries (a tile never straddles two);
  // called by all threads before they fetch tile j
  auto ensure_chunk = [&](int j) {
    const int c = (t0 + j * kTile) / tab_tokens;
    if (c != chunk) {
      __syncthreads();  // every fetch from the current chunk is done
      load_chunk(c);
      __syncthreads();
    }
  };
  // loader role: chunk lc of keys lt + 16 u (u = 0..3) of a tile
  const int lc = tid & 15, lt = tid >> 4;
  uintx4 kr[kRing][4], vr[kRing][4];
  uint32_t okb[kRing];
  // loads of tile j into register set r; keys past n, unmapped or outside the
  // pool load the zero row and are flagged
  auto fetch = [&](int j, uintx4 (&kk)[4], uintx4 (&vv)[4], uint32_t& ok) {
    ok = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + j * kTile + lt + 16 * u;
      int64_t s = -1;
      if (t < n) {
        const int blk = t / a.P;
        const int e = blk - chunk * kTabChunk;
        const int page = (e >= 0 && e < kTabChunk) ? L.tab[e] : -1;
        s = (int64_t)page * a.P + (t - blk * a.P);
        s = (page >= 0 && s < a.slots) ? s : -1;
      }
      const int64_t off = s * head_bytes + 16 * lc;
      kk[u] = *(const uintx4*)(s >= 0 ? kpool + off : zero_row + 16 * lc);
      vv[u] = *(const uintx4*)(s >= 0 ? vpool + off : zero_row + 16 * lc);
      ok |= (s >= 0 ? 1u : 0u) << u;
    }
  };
  auto stage_write = [&](int st, const uintx4 (&kk)[4], const uintx4 (&vv)[4], uint32_t ok) {
    lds_t* kt = (lds_t*)L.tiles + st * kStageBytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = lt + 16 * u;
      *(__attribute__((address_space(3))) uintx4*)(kt + tile_off(t, lc)) = kk[u];
      *(__attribute__((address_space(3))) uintx4*)(kt + kTile * kRowBytes + tile_off(t, lc)) = vv[u];
      if (lc == 0) L.ok[st][t] = (ok >> u) & 1;
    }
  };

  // Q^T fragments (B of S^T = K Q^T): head l % 16 of the group, values
  // 32 ks + 8 (l / 16) .. + 7; zero past the group
  halfx8 qf[kD / 32];
  {
    const int hl = lane & 15;
    const uint16_t* qrow = a.q + ((int64_t)b * a.Hq + g * group + min(hl, group - 1)) * kD;
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) {
      const uintx4 w = hl < group ? *(const uintx4*)(qrow + 32 * ks + 8 * (lane >> 4))
                                  : uintx4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(halfx8, w);
    }
  }
  // K fragment (A of S^T): key 16 w + l % 16, chunk 4 ks + l / 16; the
  // key's swizzle is swz(l % 16), so ks steps are an XOR of ks << 6.
  const uint32_t k_off = (16 * wave + (lane & 15)) * kRowBytes +
                         (((lane >> 4) ^ key_swz(lane & 15)) << 4);
  // V^T fragment (A of O^T, transpose read): lane (gq, j16) points at key
  // 16 w + 4 gq + j16 / 4, values 16 mb + 4 (j16 % 4) .. + 3, i.e. chunk
  // 2 mb + (j16 % 4) / 2, byte 8 (j16 % 2); mb steps are an XOR of mb << 5.
  const int vq = lane >> 4, vj = lane & 15;
  const int v_tok = 4 * vq + (vj >> 2);
  const uint32_t v_off = kTile * kRowBytes + (16 * wave + v_tok) * kRowBytes +
                         ((((vj & 3) >> 1) ^ key_swz(v_tok)) << 4) + 8 * (vj & 1);

  floatx4 o[kD / 16];
#pragma unroll
  for (int mb = 0; mb < kD / 16; ++mb) o[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, lsum = 0.f;  // head l % 16; lsum over this lane's keys

  auto compute = [&](int st) {
    const uint32_t sbase = tiles_base + st * kStageBytes;
    // S^T for keys 16 w .. + 15
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) {
      const halfx8 kf = __builtin_bit_cast(
          halfx8, *(const __attribute__((address_space(3))) uintx4*)(
                      (lds_t*)(uintptr_t)((sbase + k_off) ^ (ks << 6))));
      s = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[ks], s, 0, 0, 0);
    }
    // mask, column max over the 16 keys (lanes l, l ^ 16, l ^ 32, l ^ 48)
    float zmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = L.ok[st][16 * wave + 4 * (lane >> 4) + r] != 0;
      s[r] = ok ? s[r] * a.scale_log2 : -INFINITY;
      zmax = fmaxf(zmax, s[r]);
    }
    zmax = fmaxf(zmax, __shfl_xor(zmax, 16));
    zmax = fmaxf(zmax, __shfl_xor(zmax, 32));
    // the reference maximum moves only when it is beaten by 2^8
    if (zmax > m_ref + 8.0f) {
      const float alpha = __builtin_amdgcn_exp2f(m_ref - zmax);
      m_ref = zmax;
      lsum *= alpha;
#pragma unroll
      for (int mb = 0; mb < kD / 16; ++mb) o[mb] *= alpha;
    }
    const float neg_m = m_ref == -INFINITY ? 0.f : -m_ref;
    halfx4 pf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pe = __builtin_amdgcn_exp2f(s[r] + neg_m);
      lsum += pe;
      pf[r] = (_Float16)pe;
    }
#pragma unroll
    for (int mb = 0; mb < kD / 16; ++mb) {
      const shortx4 vf = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_shortx4*)(uintptr_t)((sbase + v_off) ^ (mb << 5)));
      o[mb] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(halfx4, vf), pf, o[mb], 0, 0,
                                                    0);
    }
  };

  // prologue: tiles 0 .. kRing - 1 in flight
  static_for<kRing>([&](auto rc) {
    constexpr int r = decltype(rc)::value;
    if (r < ntiles) {
      ensure_chunk(r);
      fetch(r, kr[r], vr[r], okb[r]);
    }
  });
  for (int base = 0; base < ntiles; base += kRing) {
    static_for<kRing>([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      const int i = base + r;
      if (i < ntiles) {
        const int st = i & 1;
        // every wave finished tile i - 2, the last user of this stage, before
        // the barrier of tile i - 1
        stage_write(st, kr[r], vr[r], okb[r]);
        const int jn = i + kRing;
        if (jn < ntiles) {
          ensure_chunk(jn);
          fetch(jn, kr[r], vr[r], okb[r]);
        }
        lds_barrier();  // tile i visible
        compute(st);
      }
    });
  }

  // merge the four waves' states: M = max m_w, out = sum 2^(m_w - M) O_w /
  // sum 2^(m_w - M) l_w
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  __syncthreads();  // every wave is done with the tiles
  float* sm = (float*)L.tiles;           // [4 waves][16 heads]
  float* sl = sm + 4 * kDecMaxGroup;     // [4][16]
  float* so = sl + 4 * kDecMaxGroup;     // [4][16 heads][128]
  if (lane < 16) {
    sm[wave * kDecMaxGroup + lane] = m_ref;
    sl[wave * kDecMaxGroup + lane] = lsum;
  }
#pragma unroll
  for (int mb = 0; mb < kD / 16; ++mb)
    *(floatx4*)&so[(wave * kDecMaxGroup + (lane & 15)) * kD + 16 * mb + 4 * (lane >> 4)] = o[mb];
  __syncthreads();
  for (int x = tid; x < group * (kD / 2); x += kThreads) {
    const int hl = x / (kD / 2), d = 2 * (x % (kD / 2));
    float mw[4], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mw[w] = sm[w * kDecMaxGroup + hl];
      M = fmaxf(M, mw[w]);
    }
    float lt = 0.f, o0 = 0.f, o1 = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = __builtin_amdgcn_exp2f(mw[w] - M);
        lt += f * sl[w * kDecMaxGroup + hl];
        o0 += f * so[(w * kDecMaxGroup + hl) * kD + d];
        o1 += f * so[(w * kDecMaxGroup + hl) * kD + d + 1];
      }
    }
    if (a.S > 1) {  // partial state of this partition
      const int64_t row = ((int64_t)b * a.S + p) * a.Hq + g * group + hl;
      *(float2*)(a.o_part + row * kD + d) = make_float2(o0, o1);
      if (d == 0) {
        a.m_part[row] = M;
        a.l_part[row] = lt;
      }
      continue;
    }
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int64_t row = (int64_t)b * a.Hq + g * group + hl;
    *(halfx2*)(a.out + row * kD + d) = halfx2{(_Float16)(o0 * inv), (_Float16)(o1 * inv)};
    if (a.lse && d == 0) a.lse[row] = lt > 0.f ? (M + log2f(lt)) * kLn2 : -INFINITY;
  }
}

// Merge of the partitions' states, one 64-thread slice per (request, head):
// M = max over partitions with l > 0 of m_p, out = sum 2^(m_p - M) o_p /
// sum 2^(m_p - M) l_p ("PagedAttention 与 RadixAttention" §1.4 part 3).
__global__ __launch_bounds__(kThreads) void paged_gqa_merge_kernel(DecArgs a) {
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (h >= a.Hq) return;
  const int b = blockIdx.x, d = 2 * (threadIdx.x & 63);
  float M = -INFINITY;
  for (int p = 0; p < a.S; ++p) {
    const int64_t row = ((int64_t)b * a.S + p) * a.Hq + h;
    if (a.l_part[row] > 0.f) M = fmaxf(M, a.m_part[row]);
  }
  float lt = 0.f, o0 = 0.f, o1 = 0.f;
  if (M != -INFINITY) {
    for (int p = 0; p < a.S; ++p) {
      const int64_t row = ((int64_t)b * a.S + p) * a.Hq + h;
      const float l = a.l_part[row];
      if (!(l > 0.f)) continue;
      const float f = __builtin_amdgcn_exp2f(a.m_part[row] - M);
      const float2 o = *(const float2*)(a.o_part + row * kD + d);
      lt += f * l;
      o0 += f * o.x;
      o1 += f * o.y;
    }
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int64_t row = (int64_t)b * a.Hq + h;
  *(halfx2*)(a.out + row * kD + d) = halfx2{(_Float16)(o0 * inv), (_Float16)(o1 * inv)};
  if (a.lse && d == 0) a.lse[row] = lt > 0.f ? (M + log2f(lt)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------- extend --

constexpr int kQBlock = 32;      // queries per workgroup and head
constexpr int kExtStages = 2;    // LDS tile double buffer
constexpr int kIdxChunk = 2048;  // slot ids staged in LDS at a time

struct ExtLds {
  char tiles[kExtStages * kStageBytes];
  int32_t idx[kIdxChunk];
};

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

// One workgroup per (request, KV head, 32-query block), two per compute
// unit; wave w computes query head g * group + w (group <= 4) for the 32
// queries, every wave loads.  Per 64-key tile and wave:
//   S^T[64 keys x 32 queries] = K Q^T with 16 v_mfma_f32_32x32x16_f16 (A = K
//     rows from LDS, B = Q^T in registers); lane l owns query l % 32 and
//     keys 8 (r / 4) + 4 (l / 32) + r % 4 of each 32-key half, so a
//     query's max and sum need only the partner lane l ^ 32;
//   O^T[128 x 32] += V^T P^T with 16 more: A = V^T by ds_read_b64_tr_b16,
//     B = P^T made from the S^T registers in place.
// Tiles wholly inside every query's visible range skip the mask; the loop
// ends at the block's last visible key.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void extend_attention_kernel(ExtArgs a) {
  __shared__ __attribute__((aligned(1024))) ExtLds L;
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
  const uint32_t tiles_base = (uint32_t)(uintptr_t)(lds_t*)L.tiles;

  // The request's slot list is staged in LDS a chunk at a time (plain loads
  // of it interleaved with the tile loads would make every use wait for the
  // tile loads in flight).
  const int my_key0 = 16 * wave + (lane >> 4);  // + 4 u, the keys this lane loads
  int chunk = -1;
  auto ensure_chunk = [&](int j) {  // all threads, before tile j's ids are read
    const int c = j * kTile / kIdxChunk;
    if (c != chunk) {
      __syncthreads();  // every read of the current chunk is done
      for (int i = tid; i < kIdxChunk; i += kThreads) {
        const int e = c * kIdxChunk + i;
        L.idx[i] = e < jmax ? a.kvi[k_base + e] : -1;
      }
      chunk = c;
      __syncthreads();
    }
  };
  // Slot ids of tile j, read one iteration before the tile is issued (so
  // that the LDS round trip overlaps a tile's compute): this lane's four
  // keys (sl) and whether key `lane` of the tile is real (ok).
  auto read_ids = [&](int j, int64_t (&sl)[4], bool& ok) {
    ensure_chunk(j);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = j * kTile + my_key0 + 4 * u - chunk * kIdxChunk;
      const int64_t sv = (e >= 0 && e < kIdxChunk) ? L.idx[e] : -1;
      sl[u] = (sv >= 0 && sv < a.slots) ? sv : -1;
    }
    const int e = j * kTile + lane - chunk * kIdxChunk;
    const int64_t sv = (e >= 0 && e < kIdxChunk) ? L.idx[e] : -1;
    ok = sv >= 0 && sv < a.slots;
  };
  auto issue = [&](int j, const int64_t (&sl)[4]) {
    issue_kv_rows((const uint8_t*)a.k, (const uint8_t*)a.v, head_bytes, g, zero_row,
                  tiles_base + (j % kExtStages) * kStageBytes, wave, lane, sl);
  };

  // Q^T fragments (B operand of S^T = K Q^T): query i0 + lane % 32, values
  // 16 ks + 8 (lane / 32) .. + 7
  const int qi = i0 + (lane & 31);
  halfx8 qf[kD / 16];
  {
    const uint16_t* qrow = a.q + ((int64_t)(q_base + min(qi, Lq - 1)) * a.Hq + h) * kD;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) {
      const uintx4 w = qi < Lq ? *(const uintx4*)(qrow + 16 * ks + 8 * (lane >> 5))
                               : uintx4{0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(halfx8, w);
    }
  }
  // LDS addresses.  In the swizzled tile, chunk c of key t sits at
  // t * 256 + ((c ^ swz(t)) << 4); the stage bases are 32 KiB aligned, so
  // stepping c by a multiple of 2 (or 4) is an XOR on bits 5..7 (6..7) of the
  // address and stepping t by a multiple of 16 an immediate offset.
  //  K fragment (A of S^T): key 32 kb + lane % 32, chunk 2 ks + lane / 32.
  const int kq = lane & 31;
  const uint32_t k_off = kq * kRowBytes + (((lane >> 5) ^ key_swz(kq)) << 4);
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
  const uint32_t v_off = kTile * kRowBytes + v_key * kRowBytes + ((v_c0 ^ key_swz(v_key)) << 4) +
                         8 * (vj & 1);
  // keys 8 further: swz(t + 8) = swz(t) ^ 2 for t < 8, i.e. byte bit 5
  const uint32_t v_off_hi = (v_off + 8 * kRowBytes) ^ 32u;

  floatx16 o[kD / 32];  // O^T[32 mb + row][query lane % 32]
#pragma unroll
  for (int mb = 0; mb < kD / 32; ++mb) o[mb] = floatx16{};
  float m_ref = -INFINITY, lsum = 0.f;  // query lane % 32 (lsum: this lane's keys)

  // one tile; `masked` is uniform, so tiles inside every query's visible
  // range skip the mask arithmetic
  auto tile = [&](int stage, int j0, uint64_t okm, bool masked) {
    const uint32_t kbase = tiles_base + stage * kStageBytes + k_off;
    const uint32_t vbase = tiles_base + stage * kStageBytes + v_off;
    const uint32_t vbase_hi = tiles_base + stage * kStageBytes + v_off_hi;
    // S^T[key 32 kb + 8 (r / 4) + 4 (lane / 32) + r % 4][query lane % 32]
    floatx16 s[2] = {floatx16{}, floatx16{}};
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const halfx8 kf = __builtin_bit_cast(
            halfx8, *(const __attribute__((address_space(3))) uintx4*)(
                        (lds_t*)(uintptr_t)((kbase ^ (ks << 5)) + kb * 32 * kRowBytes)));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], s[kb], 0, 0, 0);
      }
    if (masked) {
      // key j0 + 32 kb + 8 (r / 4) + 4 (lane / 32) + r % 4 is visible to
      // query qi iff it is real and 32 kb + 8 (r / 4) + r % 4 <= lim
      const uint64_t okl = okm >> (4 * (lane >> 5));
      const int lim = qi < Lq ? qi + prefix - j0 - 4 * (lane >> 5) : -1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int jl = 32 * kb + 8 * (r >> 2) + (r & 3);
          const bool vis = (jl <= lim) & (((okl >> jl) & 1) != 0);
          s[kb][r] = vis ? s[kb][r] : -INFINITY;
        }
    }
    float zmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) zmax = fmaxf(zmax, fmaxf(s[kb][r], s[kb][r + 1]));
    const float tmax = pair_max(zmax) * a.scale_log2;
    // the reference maximum moves only when it is beaten by 2^8
    if (__ballot(tmax > m_ref + 8.0f)) {
      const float alpha = tmax > m_ref + 8.0f ? __builtin_amdgcn_exp2f(m_ref - tmax) : 1.f;
      m_ref = tmax > m_ref + 8.0f ? tmax : m_ref;
      lsum *= alpha;
#pragma unroll
      for (int mb = 0; mb < kD / 32; ++mb) o[mb] *= alpha;
    }
    const float neg_m = m_ref == -INFINITY ? 0.f : -m_ref;
    halfx8 pf[2][2];  // P^T [kb][k-step of 16 keys]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], a.scale_log2, neg_m));
        lsum += p;
        pf[kb][r >> 3][r & 7] = (_Float16)p;
      }
    // O^T += V^T P^T, four k-steps of 16 keys
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int mb = 0; mb < kD / 32; ++mb) {
          const uint32_t koff = (32 * kb + 16 * st) * kRowBytes;
          const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_shortx4*)(uintptr_t)((vbase ^ (mb << 6)) + koff));
          const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_shortx4*)(uintptr_t)((vbase_hi ^ (mb << 6)) + koff));
          const halfx8 vf = __builtin_bit_cast(
              halfx8, (shortx8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[kb][st], o[mb], 0, 0, 0);
        }
  };

  // prologue: tile 0 in flight, tile 1's ids read
  int64_t sl[4];
  bool ok = false;
  uint64_t okm_next = 0;
  if (ntiles > 0) {
    read_ids(0, sl, ok);
    issue(0, sl);
    okm_next = __ballot(ok);
  }
  if (ntiles > 1) read_ids(1, sl, ok);
  for (int it = 0; it < ntiles; ++it) {
    wait_vmcnt<0>();  // this wave's loads of tile it
    lds_barrier();    // tile it visible; every wave is done with tile it - 1
    const uint64_t okm = okm_next;  // the keys of tile it that are real
    if (it + 1 < ntiles) {
      issue(it + 1, sl);  // into tile it - 1's stage
      okm_next = __ballot(ok);
    }
    if (it + 2 < ntiles) read_ids(it + 2, sl, ok);
    const int stage = it % kExtStages;
    const int j0 = it * kTile;
    // no mask needed when every key is real and visible to every query
    const bool full = okm == ~0ull && j0 + kTile - 1 <= i0 + prefix && i0 + kQBlock <= Lq;
    if (active) tile(stage, j0, okm, !full);
  }

  if (!active || qi >= Lq) return;
  // lane holds O^T[32 mb + 8 (r / 4) + 4 (lane / 32) + r % 4][query]
  const float l_tot = pair_sum(lsum);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* orow = a.out + ((int64_t)(q_base + qi) * a.Hq + h) * kD;
#pragma unroll
  for (int mb = 0; mb < kD / 32; ++mb)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const halfx4 w = {(_Float16)(o[mb][4 * rq] * inv), (_Float16)(o[mb][4 * rq + 1] * inv),
                        (_Float16)(o[mb][4 * rq + 2] * inv), (_Float16)(o[mb][4 * rq + 3] * inv)};
      *(halfx4*)(orow + 32 * mb + 8 * rq + 4 * (lane >> 5)) = w;
    }
  // the exponents were taken against m_ref, so lse = (m_ref + log2 l) ln 2
  if (a.lse && lane < 32)
    a.lse[(int64_t)(q_base + qi) * a.Hq + h] =
        l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
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

// Partitions of the decode: equal token ranges of every request's table.
// Two workgroups share a compute unit (registers and LDS allow two), and a
// workgroup's fixed cost (filling its prefetch ring, the wave merge) makes
// extra partitions a loss once the (request, KV head) workgroups fill about
// two rounds of the device; below that, partitions of at least 8 tiles make
// up the difference.
void dense_split_plan(int32_t B, int32_t Hkv, int64_t max_tokens, int32_t requested, int* S,
                      int* part) {
  const int64_t tiles = std::max<int64_t>(1, (max_tokens + kTile - 1) / kTile);
  int64_t s;
  if (requested > 0) {
    s = std::min<int64_t>(requested, tiles);
  } else {
    const int64_t target = 2 * kDecWaves * (int64_t)stp::device_cus();
    const int64_t wgs = std::max<int64_t>(1, (int64_t)B * Hkv);
    s = wgs >= target ? 1 : std::min((target + wgs - 1) / wgs, (tiles + 7) / 8);
  }
  s = std::max<int64_t>(1, std::min<int64_t>(s, 4096));
  const int64_t p_tiles = (tiles + s - 1) / s;
  *S = (int)((tiles + p_tiles - 1) / p_tiles);
  *part = (int)(p_tiles * kTile);
}

size_t dense_workspace(int32_t B, int32_t Hq, int S) {
  return S > 1 ? (size_t)B * S * Hq * (kD + 2) * sizeof(float) : 0;
}

}  // namespace

extern "C" int32_t stp_paged_gqa_decode_splits(int32_t B, int32_t Hkv, int32_t max_blocks,
                                               int32_t page_size, int32_t num_splits) {
  if (B < 0 || Hkv < 1 || max_blocks < 0 || page_size < 1) return 0;
  int S, part;
  dense_split_plan(B, Hkv, (int64_t)max_blocks * page_size, num_splits, &S, &part);
  return S;
}

extern "C" size_t stp_paged_gqa_decode_workspace(int32_t B, int32_t Hq, int32_t Hkv,
                                                 int32_t max_blocks, int32_t page_size,
                                                 int32_t num_splits) {
  if (B < 0 || Hq < 1 || Hkv < 1 || max_blocks < 0 || page_size < 1) return 0;
  int S, part;
  dense_split_plan(B, Hkv, (int64_t)max_blocks * page_size, num_splits, &S, &part);
  return dense_workspace(B, Hq, S);
}

extern "C" int stp_paged_gqa_decode(const uint16_t* q, const uint16_t* k_pool,
                                    const uint16_t* v_pool, int64_t num_slots,
                                    const int32_t* block_table, int32_t max_blocks,
                                    const int32_t* ctx_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                    int32_t head_dim, int32_t page_size, float scale,
                                    int32_t num_splits, void* workspace, size_t workspace_bytes,
                                    uint16_t* out, float* lse, hipStream_t stream) {
  using stp::fail;
  if (int rc = check_dense("paged_gqa_decode", q, k_pool, v_pool, num_slots, B, Hq, Hkv, head_dim,
                           scale, kDecMaxGroup))
    return rc;
  if (page_size < 1 || page_size > (1 << 20) || max_blocks < 0)
    return fail(STP_ERR_INVALID_ARG, "paged_gqa_decode: page_size %d / max_blocks %d", page_size,
                max_blocks);
  if ((int64_t)max_blocks * page_size > INT32_MAX - kTabChunk * (int64_t)page_size)
    return fail(STP_ERR_INVALID_ARG, "paged_gqa_decode: max_blocks * page_size exceeds int32");
  if (num_splits < 0) return fail(STP_ERR_INVALID_ARG, "paged_gqa_decode: num_splits < 0");
  if (B == 0) return STP_OK;
  if (!ctx_lens || !out || (max_blocks > 0 && !block_table))
    return fail(STP_ERR_INVALID_ARG, "paged_gqa_decode: null pointer");
  int S, part;
  dense_split_plan(B, Hkv, (int64_t)max_blocks * page_size, num_splits, &S, &part);
  const size_t need = dense_workspace(B, Hq, S);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(STP_ERR_WORKSPACE, "paged_gqa_decode: workspace of %zu bytes needed", need);
  if ((int64_t)B * Hkv * S > INT32_MAX) return fail(STP_ERR_INVALID_ARG, "paged_gqa_decode: grid");
  float* ws = (float*)workspace;
  const size_t rows = (size_t)B * S * Hq;
  DecArgs a{q, k_pool, v_pool, num_slots, block_table, max_blocks, ctx_lens, B, Hq, Hkv,
            page_size, S, part, scale * kLog2e, out, lse,
            S > 1 ? ws : nullptr, S > 1 ? ws + rows * kD : nullptr,
            S > 1 ? ws + rows * (kD + 1) : nullptr};
  paged_gqa_decode_kernel<kDecRing, kDecWaves><<<B * Hkv * S, kThreads, 0, stream>>>(a);
  if (int rc = stp::check_launch("paged_gqa_decode_kernel")) return rc;
  if (S > 1) {
    paged_gqa_merge_kernel<<<dim3(B, (Hq + 3) / 4), kThreads, 0, stream>>>(a);
    return stp::check_launch("paged_gqa_merge_kernel");
  }
  return STP_OK;
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
