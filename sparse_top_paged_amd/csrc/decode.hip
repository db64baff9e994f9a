// Stage 3: top-k sparse MLA decode attention on gfx950.
//
// "5.1.1 · 从索引到 Kernel" §2.1 (load candidates straight from the cache
// instead of gathering them to scratch: eq. (3)), §2.2 (whole rows keep the
// transactions full), §3.1 eq. (4)-(6) (tile loop with a running max, sum and
// un-normalised numerator; empty tiles skipped), §3.2 (masks act before the
// exponent; split partial states, eq. (7)); "PagedAttention 与 RadixAttention：
// 上游机制与海光实现对照" §1.4 (exp2 with log2 e folded into the scale; split
// partitions; the normalised partition combine), §1.4 part 4 and §5.2 (load
// each K/V row once for every query head that shares it).
//
// Data: q [T, H, 576] bf16, kv [rows, 576] bf16 (latent 512 first, rope 64
// last; V is the first 512 values of the same row), row_ids [T, cap].
//
// Decomposition.  All H query heads of a token read the same latent rows, so
// a workgroup owns 64 heads of one token and one contiguous range of its
// candidate positions (a split); the two head groups of a (token, split) run
// on the same XCD (blockIdx % 8 picks the XCD) so the second reads the rows
// from that XCD's L2.  Four wave64s per workgroup, one per SIMD, in two roles:
//   score waves (0, 1): wave j owns heads 32 j .. 32 j + 31 of the group and
//     keeps their Q^T for all 576 dims in 144 AGPRs.  Per 32-row tile it
//     forms S^T[32 rows x 32 heads] = K Q^T with 36 v_mfma_f32_32x32x16_bf16
//     (A = K fragment read from LDS), runs the online softmax of its heads
//     (a lane owns one head; base 2; the reference max moves only when a
//     tile beats it by 2^8) and publishes P^T (bf16) and the per-head rescale
//     factor of the tile in LDS.  The softmax of tile i is interleaved with
//     the QK products of tile i + 1, one MFMA per step.
//   output waves (2, 3): wave j owns values 256 j .. 256 j + 255 of all 64
//     heads, O^T[256 x 64] in 256 AGPRs.  One tile behind the score waves it
//     rescales O^T when a factor is not 1 and adds V^T P^T with 32 MFMAs
//     (A = V^T fragments read with ds_read_b64_tr_b16, the LDS transpose
//     read; B = the published P^T, one ds_read_b128 per fragment).
//   The V^T k-slot to row mapping matches the score waves' accumulator
//   layout, so lane l of a score wave writes exactly the P^T fragment that
//   lane l of an output wave reads.  The QK and PV products (576 and 512 MACs
//   per row and head) keep the four SIMDs equally busy, and the softmax of
//   one tile overlaps the PV products of the previous one.
// Rows are staged in a 4-stage LDS ring of 32-row tiles (36.5 KiB each) with
// global_load_lds_dwordx4, so no VGPRs hold KV data in flight; only the
// output waves issue tile loads, three tiles ahead, spread between their
// MFMAs.  One LDS-only workgroup barrier per tile hands over P^T, publishes
// the next tile and frees a ring stage.  Invalid candidates load a zero row
// and are masked to -inf before the exponent.  At the end the output waves
// stage O^T in fp32 through the idle ring, and all four waves scale, round
// and write the rows.

#include <mutex>
#include <type_traits>

#include "block_view.h"
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
constexpr int kStages = 4;
constexpr int kSlotsPerThread = kTileRows * kChunks / kThreads; // 9
constexpr int kHeadsPerWG = 64;
constexpr int kIdsMax = 1120;  // 35 tiles: half of a 2180-candidate list fits (what the LDS has left)
constexpr int kIdTiles = kIdsMax / 32;  // a longer split keeps its ids in a ring of this many tiles
constexpr int kQKSteps = kDQK / 16;                             // 36
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.0f;

static_assert(kTileRows * kChunks % kThreads == 0, "tile slots per thread");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int uintx2 __attribute__((ext_vector_type(2)));
typedef unsigned int uintx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_t;
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef __attribute__((address_space(3))) shortx8 lds_shortx8;

// Source of every masked-out row: loads stay in bounds and bring zeros.
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[kRowBytes] = {};

// fp8_ds_mla rows: 512 E4M3 latent codes, four float32 scales (one per 128
// values), 64 bf16 RoPE values.  The waves stage them through registers and
// write the dequantised row, bf16(f32(code) * scale) for the latent values
// and the RoPE values as they are, into the tile layout of the ring, so that
// every later step is the bf16 path's.  Each wave handles one 8-row group of
// a tile (score wave j group 2 j + 1, output wave j group 2 j): lane l takes
// row l / 8 of the group and, of it, 16-byte chunk l % 8 of each 128-byte
// latent line (codes 128 line + 16 (l % 8) .. + 15), RoPE chunk l % 8 and
// the four scales.
constexpr int kFp8RowBytes = 656;
constexpr int kFp8ScaleOff = 512;
constexpr int kFp8RopeOff = 528;

struct Fp8Rows {
  uintx4 lat[4];  // [line]
  floatx4 scl;
  uintx4 rope;
};

// bf16(f32(code) * scale) of the eight codes in (w0, w1), packed in order
__device__ __forceinline__ uintx4 dequant8(uint32_t w0, uint32_t w1, float sc) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false);
  const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
  const f2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false);
  const f2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
  return uintx4{stp::pack_bf16x2(a.x * sc, a.y * sc), stp::pack_bf16x2(b.x * sc, b.y * sc),
                stp::pack_bf16x2(c.x * sc, c.y * sc), stp::pack_bf16x2(d.x * sc, d.y * sc)};
}

// LDS tile layout: four groups of 8 rows (one group per wave when loading),
// each group nine 1 KiB blocks; block b holds chunks 8 b .. 8 b + 7 (one
// 128-byte line) of each of the 8 rows, row-major, with the chunk position
// XOR-swizzled by the row: chunk c of group row rl sits at
//   group + (c / 8) * 1024 + rl * 128 + ((c % 8) ^ rl) * 16.
// One load instruction of a wave fills one block: each run of 8 consecutive
// lanes reads one row's 128-byte line (the access pattern the vector memory
// path coalesces best), and every LDS read below is a per-lane base plus a
// compile-time offset.  The swizzle keeps both the K reads (ds_read_b128) and
// the V transpose reads free of bank conflicts; groups are padded by 128 B so
// that rows r and r + 8 fall in different halves of the 64 banks.

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* kv;
  int64_t kv_rows;
  const int32_t* row_ids;
  const int32_t* counts;
  int cap, T, H;
  float scale_log2;
  int S, G;
  void* o_part;    // split modes: [T, S, H, 512] fp32 or bf16
  float* m_part;   // [T, S, H], natural-log units
  float* l_part;
  uint16_t* out;   // final mode: [T, H, 512] bf16
  float* lse;
  // task-queue launch: queue x's entries are the first qcount[x] of segment
  // x (qcap entries from qent + 4 qcap x) of (row, start, length, partial
  // slot); queue heads for claiming them
  const int32_t* qcount;
  const int32_t* qent;
  int qcap;
  int32_t* queue;
  // fp8_ds_mla rows (656 B) instead of kv, for the fp8 row format
  const uint8_t* kv8;
  // normalisation in the decode launch (kNorm): token t's candidate list is
  // built from D, W and A as stp_normalize_indices builds it, whose outputs
  // the workgroups also write
  const int32_t* topk;
  const int32_t* req_id;
  const int32_t* q_pos;
  const int32_t* block_table;
  int top_k, num_reqs, max_blocks, P, window, num_sinks, nwords_alloc;
  uint64_t pdiv;
  int32_t* tok_out;
  int32_t* slot_out;
  int32_t* count_out;
  int32_t* dropped_out;
  int32_t* blk_indptr;
};

// Output modes of the decode kernel.
enum OutMode : int {
  kOutFinal = 0,       // out = o / l (bf16), lse
  kOutPartialF32 = 1,  // per split: o (unnormalised, fp32), m, l
  kOutPartialBf16 = 2  // per split: o / l (bf16), m, l
};

using stp::static_for;

using stp::lds_barrier;
using stp::wait_vmcnt;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

using stp::scale_acc;

using stp::load_lds_16;

// 4 bytes per lane from global memory straight into LDS (global_load_lds_dword):
// LDS address m0 + 4 * lane; untracked by the compiler, like load_lds_16.
__device__ __forceinline__ void load_lds_4(const void* gptr, uint32_t lds_addr) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(gptr), "{m0}"(lds_addr));
}
using stp::pair_max;
using stp::pair_sum;

template <int It>
__device__ __forceinline__ void load_row_chunks(const uint8_t* src, uint32_t lds_addr) {
  if constexpr (It < kSlotsPerThread) {
    // chunk column It: global src + 128 It, LDS lds_addr + 1024 It
    load_lds_16<It * 128>(src, lds_addr + It * (1024 - 128));
    load_row_chunks<It + 1>(src, lds_addr);
  }
}

// LDS objects of one workgroup.  Separate variables let the compiler see
// that the hand-off buffers and the id list never alias the tile ring.
struct DecodeLds {
  lds_t* tiles;        // [4][37376]
  lds_t* pbuf;         // [2 buffers][2 head blocks][2 k-steps][64 lanes][16 B]
  float* alpha;        // [2 buffers][64 heads]
  float* stat;         // [3][64]: m_ref, m_true (log2 units), l
  int32_t* ids;        // [kIdsMax]
};

// Score-wave state: online softmax statistics of the wave's 32 heads (log2
// units) and the S^T accumulators of one tile (two MFMA chains).
struct ScoreState {
  float m_ref, m_true, lsum;
};
struct SAcc {
  floatx16 c0, c1;
};

//  K fragment of k-step ks: row lane % 32, chunk 2 ks + lane / 32 of the
//  tile; chunk c = 2 (ks % 4) + lane / 32 + 8 (ks / 4), so four per-lane bases
//  cover every k-step with an immediate offset of 1024 (ks / 4).
__device__ __forceinline__ const lds_t* k_addr(const lds_t* stage, const int (&k_base)[4],
                                               int ks) {
  return stage + k_base[ks & 3] + 1024 * (ks >> 2);
}

constexpr int kKRing = 8;  // K fragments in flight per score wave

// S^T = K Q^T of one tile, on its own (the first tile of a split).
__device__ __forceinline__ void qk_tile(const lds_t* stage, const int (&k_base)[4],
                                        const bf16x8 (&qf)[kQKSteps], SAcc& acc) {
  shortx8 kf[kKRing];
  acc.c0 = floatx16{};
  acc.c1 = floatx16{};
#pragma unroll
  for (int ks = 0; ks < kKRing; ++ks) kf[ks] = *(const lds_shortx8*)k_addr(stage, k_base, ks);
#pragma unroll
  for (int ks = 0; ks < kQKSteps; ++ks) {
    const bf16x8 kfrag = __builtin_bit_cast(bf16x8, kf[ks % kKRing]);
    if (ks & 1)
      acc.c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag, qf[ks], acc.c1, 0, 0, 0);
    else
      acc.c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag, qf[ks], acc.c0, 0, 0, 0);
    if (ks + kKRing < kQKSteps)
      kf[ks % kKRing] = *(const lds_shortx8*)k_addr(stage, k_base, ks + kKRing);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, kKRing, 0);
#pragma unroll
  for (int g = 0; g < kQKSteps - kKRing; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kKRing, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// Online softmax of the tile whose S^T is in `cur`: the reference maximum
// moves only when the tile beats it by 2^8, P^T goes to pbuf[buf] as bf16 and
// the tile's rescale factor to alpha[buf].  With kMasked, rows outside vmask
// are set to -inf before the exponent (only a split's last tile or a tile
// with invalid ids needs it).  With kNext the QK products of the next tile
// (ring stage `next`) are computed into `nxt` at the same time.  The two are
// independent, so the work is laid out as 36 steps, each one MFMA, the K
// fragment read eight steps ahead and about one row's worth of softmax
// arithmetic, fenced so that the compiler keeps that order: the VALU work
// issues while the matrix core runs the MFMA before it.  The softmax is kept
// to a few VALU instructions per row (the scale is applied inside the
// exponent's FMA; exp2(-inf) = 0 covers masked rows), since VALU work beyond
// about four instructions per MFMA slows the MFMA stream.  Branch-free.
// Requires scale_log2 > 0, so that max(z) * scale = max(z * scale).
template <bool kNext, bool kMasked, typename StepFn>
__device__ __forceinline__ void score_step(const DecodeLds& L, const lds_t* next,
                                           const int (&k_base)[4],
                                           const bf16x8 (&qf)[kQKSteps], const SAcc& cur,
                                           SAcc& nxt, uint32_t vmask, float scale_log2, int buf,
                                           int j, int lane, ScoreState& st, StepFn&& step_fn) {
  shortx8 kf[kKRing];
  if constexpr (kNext) {
    nxt.c0 = floatx16{};
    nxt.c1 = floatx16{};
#pragma unroll
    for (int ks = 0; ks < kKRing; ++ks) kf[ks] = *(const lds_shortx8*)k_addr(next, k_base, ks);
  }

  // lane holds rows 8 (r / 4) + 4 (lane / 32) + r % 4 of head lane % 32
  float zv[16];
  float mt = -INFINITY, psum = 0.f, alpha = 1.f, neg_m = 0.f;
  bf16x8 pk[2];
  auto row_max = [&](int r) {
    float z = cur.c0[r] + cur.c1[r];
    if constexpr (kMasked) {
      const int rr = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      z = ((vmask >> rr) & 1u) ? z : -INFINITY;
    }
    zv[r] = z;
    mt = fmaxf(mt, z);
  };
  auto rebase = [&]() {
    mt = pair_max(mt) * scale_log2;
    st.m_true = fmaxf(st.m_true, mt);
    // also taken by the first non-empty tile (m_ref = -inf gives alpha = 0)
    const bool move = mt > st.m_ref + kRescaleLog2;
    alpha = move ? fast_exp2(st.m_ref - mt) : 1.f;
    st.m_ref = move ? mt : st.m_ref;
    neg_m = st.m_ref == -INFINITY ? 0.f : -st.m_ref;  // nothing seen yet: every z is -inf
  };
  auto row_exp = [&](int r) {
    const float p = fast_exp2(__builtin_fmaf(zv[r], scale_log2, neg_m));
    psum += p;
    pk[r >> 3][r & 7] = (__bf16)p;
  };
  auto publish = [&]() {
    st.lsum = st.lsum * alpha + psum;
    // P^T fragments for k-steps 0 and 1 (rows 0-15 and 16-31 of the tile);
    // the lane pair (l, l ^ 32) holds the same alpha, so both may store it.
    lds_t* pb = L.pbuf + ((buf * 2 + j) * 2) * 1024 + lane * 16;
    *(__attribute__((address_space(3))) bf16x8*)(pb) = pk[0];
    *(__attribute__((address_space(3))) bf16x8*)(pb + 1024) = pk[1];
    L.alpha[buf * 64 + 32 * j + (lane & 31)] = alpha;
  };

#pragma unroll
  for (int ks = 0; ks < kQKSteps; ++ks) {
    if constexpr (kNext) {
      const bf16x8 kfrag = __builtin_bit_cast(bf16x8, kf[ks % kKRing]);
      if (ks & 1)
        nxt.c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag, qf[ks], nxt.c1, 0, 0, 0);
      else
        nxt.c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag, qf[ks], nxt.c0, 0, 0, 0);
      if (ks + kKRing < kQKSteps)
        kf[ks % kKRing] = *(const lds_shortx8*)k_addr(next, k_base, ks + kKRing);
    }
    if (ks < 16)
      row_max(ks);
    else if (ks == 16)
      rebase();
    else if (ks < 33)
      row_exp(ks - 17);
    else if (ks == 33)
      publish();
    step_fn(ks);
    if constexpr (kNext) __builtin_amdgcn_sched_barrier(0);
  }
}

// The output waves stage O^T as it is, fp32 rows [64 heads][512] in the
// tile ring (head stride 2064 B, so the 32 heads of a staging store hit
// different banks); all four waves then scale each row by 1 / l of its head,
// round it to bf16 and write it out (the final output, or the split's
// normalised partial): wave w takes heads w, w + 4, ..., one row per step,
// lane c values 8 c .. 8 c + 7, so that a step's store writes the whole
// 1 KiB row.
constexpr int kHeadStrideF = kDV * 4 + 16;
static_assert(kHeadsPerWG * kHeadStrideF <= kStages * kTileBytes, "fp32 staging fits the ring");

__device__ __forceinline__ void copy_out_rows(const DecodeArgs& a, const DecodeLds& L, int t,
                                              int64_t part, int hg, int tid, bool final_out) {
  const int lane = tid & 63, wave = tid >> 6;
  // 1 / l of head `lane` (0 for a head that saw no candidate)
  const float l_lane = L.stat[128 + lane];
  const float inv_lane = l_lane > 0.f ? 1.f / l_lane : 0.f;
#pragma unroll 4
  for (int it = 0; it < kHeadsPerWG / 4; ++it) {
    const int hl = 4 * it + wave;
    const int head = hg * kHeadsPerWG + hl;
    if (head >= a.H) break;  // heads past H come last
    const float inv = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inv_lane), hl));
    const lds_t* row = L.tiles + hl * kHeadStrideF + lane * 32;
    const floatx4 x0 = *(const __attribute__((address_space(3))) floatx4*)(row);
    const floatx4 x1 = *(const __attribute__((address_space(3))) floatx4*)(row + 16);
    uint16_t* orow = final_out ? a.out + ((int64_t)t * a.H + head) * kDV
                               : (uint16_t*)a.o_part + (part * a.H + head) * kDV;
    *(uintx4*)(orow + 8 * lane) =
        uintx4{stp::pack_bf16x2(x0[0] * inv, x0[1] * inv), stp::pack_bf16x2(x0[2] * inv, x0[3] * inv),
               stp::pack_bf16x2(x1[0] * inv, x1[1] * inv), stp::pack_bf16x2(x1[2] * inv, x1[3] * inv)};
  }
}

// The normalisation of token t inside the decode launch ("5.1.1 · 从索引到
// Kernel" §1.1 eq. (1), §1.2 eq. (2); "HiSparse" walkthrough, token -> global
// slot conversion): the same S, slots, count, dropped count and block count
// as stp_normalize_indices, built by each workgroup of the token for itself
// so that no launch stands between the index stage and the attention.
// LDS (ring stages 0 and 1, which the tiles take only after the ids are
// staged): the position bitmap, the request's page-table row, D, and the
// offsets of the bitmap's words and 64-word batches in the list.
//   1. The output waves load the request, the position and D, then the
//      table row; the score waves enqueue the query rows (issue_q) and wait
//      for no load until the bitmap is built, so that no wait of theirs
//      drains the query rows early.
//   2. While the table row is in flight, the output waves set the positions
//      of D, W and A within [0, limit] in an LDS bitmap (atomics); then the
//      positions past each block's last visible slot (all of an unmapped
//      page) are cleared.  One workgroup per token counts D's dropped
//      entries.
//      Then each wave scans its run of 64-word batches, keeping every
//      word's and batch's offset within the run (tagged with the wave; the
//      runs' totals place it in the list).
//   3. The split [lo, lo + len) is the one the static launch cuts for this
//      workgroup.  The batches that meet it go to the four waves in turn,
//      one word per lane; each lane writes its bits' positions into the id
//      list, and words with many bits are emitted by the whole wave.
//   4. The waves turn positions into slots (-1 past the pool), write
//      tok_out / slot_out (head group 0), and pad the list with -1 to the tile
//      edge.  Split 0 of head group 0 writes the count and -(blocks + 1) into
//      blk_indptr (the deferred block view's state), split 0 of the last head
//      group the dropped count, split S - 1 the -1 tail.  An LDS-only barrier
//      hands the ids over.
constexpr int kDenseWord = 16;  // words with more set bits are emitted wave-wide
typedef __attribute__((address_space(3))) uint64_t lds_u64;
typedef __attribute__((address_space(3))) int32_t lds_i32;

// LDS bytes of the normalisation: bitmap, table row, D, word offsets and
// batch offsets.
__host__ __device__ constexpr int64_t norm_lds_bytes(int64_t nwords, int64_t max_blocks,
                                                     int64_t top_k) {
  return nwords * 8 + max_blocks * 4 + top_k * 4 + nwords * 4 + (nwords / 64 + 1) * 4;
}

// Whether the normalisation's LDS fits in ring stage 1 alone, which leaves
// stage 0 free for tile 0 while the list is still being finished.
__device__ __forceinline__ bool norm_in_stage1(const DecodeArgs& a) {
  return norm_lds_bytes(a.nwords_alloc, a.max_blocks, a.top_k) <= kTileBytes;
}

template <class IssueQ, class IssueT0>
__device__ __forceinline__ void normalize_split(const DecodeArgs& a, const DecodeLds& L,
                                                int* s_bad, int t, int sidx, int hg, int& lo_out,
                                                int& len_out, IssueQ&& issue_q,
                                                IssueT0&& issue_tile0) {
  using stp::bv::div_p;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool outw = wave >= 2;  // output waves load; score waves enqueue the query rows
  const int otid = tid - 128;   // thread index among the output waves
  const bool early = norm_in_stage1(a);
  lds_t* nbase = L.tiles + (early ? kTileBytes : 0);
  lds_u64* bm = (lds_u64*)nbase;
  lds_i32* tbl = (lds_i32*)(nbase + (size_t)a.nwords_alloc * 8);
  lds_i32* dl = tbl + a.max_blocks;  // D
  lds_i32* woff = dl + a.top_k;      // each word's offset within its wave's run, tagged
  lds_i32* red = (lds_i32*)L.stat;   // per-wave totals

  // 1. D (output waves: the first 2048 entries in registers), the request
  //    and the position in one round trip (D does not depend on them), then
  //    the table row in flight while the bitmap is cleared
  constexpr int kPer = 16;  // entries per output-wave thread per round (2048)
  // (every wave issues the same loads, with no branch around them, so that
  // the wait for r and q can leave the D loads in flight; the score waves'
  // copies of D go unused)
  const int32_t* drow = a.topk + (int64_t)t * a.top_k;
  const int r_ld = a.req_id[t];
  const int q_ld = a.q_pos[t];
  // (top_k = 0: every load reads the request id, an in-bounds word)
  const int32_t* dsrc = a.top_k > 0 ? drow : a.req_id + t;
  const int dlast = max(a.top_k - 1, 0);
  int dv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) dv[u] = dsrc[min((tid & 127) + 128 * u, dlast)];
  __builtin_amdgcn_sched_barrier(0);  // the D loads go out before the wait for r and q
  const int r = __builtin_amdgcn_readfirstlane(r_ld);
  const int q = __builtin_amdgcn_readfirstlane(q_ld);
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    if (otid + 128 * u >= a.top_k) dv[u] = -1;
  const bool pad = r < 0 || r >= a.num_reqs || q < 0;
  const int P = a.P;
  const int limit = pad ? -1 : min(q, a.max_blocks * P - 1);  // last visible position
  const int nwords = limit >= 0 ? (limit >> 6) + 1 : 0;
  const int used_blocks = limit >= 0 ? div_p(limit, a.pdiv) + 1 : 0;
  const int32_t* g_table = a.block_table + (int64_t)(pad ? 0 : r) * a.max_blocks;
  int tv[kPer];
  if (outw) {
    // no branch per load (used_blocks = 0: the request id again)
    const int32_t* tsrc = used_blocks > 0 ? g_table : a.req_id + t;
    const int tlast = max(used_blocks - 1, 0);
#pragma unroll
    for (int u = 0; u < kPer; ++u) tv[u] = tsrc[min(otid + 128 * u, tlast)];
  } else {
    issue_q();
  }
  // (the whole bitmap: the score waves do not wait for the position, whose
  // load would drain their query rows first)
  for (int w = tid; w < a.nwords_alloc; w += kThreads) bm[w] = 0ull;
  if (tid == 0) {
    s_bad[0] = 0;
    s_bad[1] = 0;
  }
  lds_barrier();  // bitmap clear

  // 2. the output waves set the positions of D, W and A within [0, limit]
  //    in the bitmap while the table row is in flight, then stage the table
  //    row (and D, for the workgroup that counts the dropped entries)
  // (32-bit atomics on the 64-bit words' halves)
  lds_i32* bm32 = (lds_i32*)nbase;
  auto set_bit = [&](int p) {
    __hip_atomic_fetch_or(&bm32[p >> 5], 1 << (p & 31), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  const bool drop_writer = hg == a.G - 1 && sidx == 0;
  if (outw) {
    // (limit < 0 for a padding row: nothing is set)
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (dv[u] >= 0 && dv[u] <= limit) set_bit(dv[u]);
    if (!pad) {
      if (a.window > 0)
        for (int p = max(0, q - a.window + 1) + otid; p <= min(q, limit); p += 128) set_bit(p);
      const int na = min(min(a.num_sinks, q + 1), limit + 1);
      for (int p = otid; p < na; p += 128) set_bit(p);
    }
    if (drop_writer && a.top_k > kPer * 128) {  // (a shorter D stays in registers)
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int k = otid + 128 * u;
        if (k < a.top_k) dl[k] = dv[u];
      }
    }
    for (int k0 = kPer * 128; k0 < a.top_k; k0 += kPer * 128) {  // D past 2048 entries
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int k = k0 + otid + 128 * u;
        dv[u] = k < a.top_k ? drow[k] : -1;
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int k = k0 + otid + 128 * u;
        if (dv[u] >= 0 && dv[u] <= limit) set_bit(dv[u]);
        if (drop_writer && k < a.top_k) dl[k] = dv[u];
      }
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int k = otid + 128 * u;
      if (k < used_blocks) tbl[k] = tv[u];
    }
    for (int k0 = kPer * 128; k0 < used_blocks; k0 += kPer * 128) {  // rows past 2048 blocks
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int k = k0 + otid + 128 * u;
        tv[u] = k < used_blocks ? g_table[k] : -1;
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int k = k0 + otid + 128 * u;
        if (k < used_blocks) tbl[k] = tv[u];
      }
    }
  }
  lds_barrier();  // candidate bitmap, table row and D staged

  // drop the positions that are not visible: block b keeps offsets up to its
  // page's last slot within int32 (none for an unmapped page).  The
  // workgroup that writes the dropped count also counts D's entries >= 0
  // that are not visible.
  // the last visible offset of block b (-1: none)
  auto last_off = [&](int b) {
    const int page = tbl[b];
    if (page < 0) return -1;
    const int64_t room = (int64_t)INT32_MAX - (int64_t)page * P;
    return room >= P - 1 ? P - 1 : (int)max(room, (int64_t)-1);
  };
  for (int b = tid; b < used_blocks; b += kThreads) {
    const int keep = last_off(b);
    if (keep < P - 1) {
      const int c0p = b * P + keep + 1, c1p = min((b + 1) * P, limit + 1);  // [c0p, c1p) dropped
      for (int wd = c0p >> 5; wd <= (c1p - 1) >> 5 && c0p < c1p; ++wd) {
        const int lo32 = max(c0p, wd * 32) - wd * 32, hi32 = min(c1p, wd * 32 + 32) - wd * 32;
        const uint32_t m = (hi32 - lo32 == 32 ? 0xffffffffu : ((1u << (hi32 - lo32)) - 1u)) << lo32;
        __hip_atomic_fetch_and(&bm32[wd], (int)~m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
  }
  lds_barrier();  // bitmap complete

  // D's dropped entries (the workgroup that writes the count): an entry >= 0
  // is kept iff it is at most the limit and its bit survived the clearing
  // above, which removed exactly the positions past their block's last
  // visible slot.  A D of at most 2048 entries is still in the output
  // waves' registers; a longer one was staged in LDS.
  int my_drop = 0;
  if (drop_writer && !pad) {
    auto dropped = [&](int p) {
      if (p < 0) return 0;
      return (p <= limit && ((bm32[p >> 5] >> (p & 31)) & 1) != 0) ? 0 : 1;
    };
    if (a.top_k <= kPer * 128) {
      if (outw) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) my_drop += dropped(dv[u]);
      }
    } else {
      for (int k = tid; k < a.top_k; k += kThreads) my_drop += dropped(dl[k]);
    }
  }

  // counts: each wave scans its run of 64-word batches; a word's (and a
  // batch's) offset is stored within the run, tagged with the wave, and the
  // runs' totals turn it into the list position where it is read
  const bool writer = hg == 0 && sidx == 0;
  const int nbatch = (nwords + 63) >> 6;
  const int bpw = (nbatch + 3) >> 2;
  const int bb0 = min(nbatch, wave * bpw), bb1 = min(nbatch, bb0 + bpw);
  lds_i32* bstart = woff + a.nwords_alloc;  // [nbatch] batch offsets, tagged
  int run = 0;
  for (int bb = bb0; bb < bb1; ++bb) {
    const int w = bb * 64 + lane;
    const int c = w < nwords ? __popcll(bm[w]) : 0;
    const int incl = stp::wave_incl_sum(c);
    if (w < nwords) woff[w] = (run + incl - c) | (wave << 24);
    if (lane == 0) bstart[bb] = run | (wave << 24);
    run += __builtin_amdgcn_readlane(incl, 63);
  }
  int my_blocks = 0;
  if (drop_writer) my_drop = stp::wave_sum(my_drop);
  if (writer) {
    for (int b = tid; b < used_blocks; b += kThreads) {
      const int blo = b * P, bhi = min(blo + P, limit + 1);
      const int w0 = blo >> 6, w1 = (bhi - 1) >> 6, sh = blo & 63;
      uint64_t acc = bm[w0] >> sh;
      if (w1 != w0) acc |= bm[w1] << (64 - sh);
      const int nbits = bhi - blo;
      if (nbits < 64) acc &= (1ull << nbits) - 1;
      my_blocks += acc ? 1 : 0;
    }
    my_blocks = stp::wave_sum(my_blocks);
  }
  if (lane == 0) {
    red[wave] = run;
    red[4 + wave] = my_blocks;
    red[8 + wave] = my_drop;
  }
  lds_barrier();  // word and batch offsets, wave totals
  const int c0 = red[0], c1 = red[1], c2 = red[2];
  const int n = __builtin_amdgcn_readfirstlane(c0 + c1 + c2 + red[3]);
  // a tagged offset -> its position in the list
  auto untag = [&](int e) {
    const int ow = e >> 24;
    return (e & 0xffffff) + (ow > 0 ? c0 : 0) + (ow > 1 ? c1 : 0) + (ow > 2 ? c2 : 0);
  };

  // 3. this workgroup's split, as the static launch cuts the list: the
  //    positions of the batches that meet it go into the id list, batch
  //    bb_first + i to wave i % 4, one word per lane
  const int chunk = (n + a.S - 1) / a.S;
  const int lo = min(n, sidx * chunk);
  const int len = min(n, lo + chunk) - lo;
  const int hi_pos = lo + len;
  const int ntiles = (len + kTileRows - 1) / kTileRows;
  int bb_first = 0;  // the last batch that starts at or before lo
  for (int b0 = 0; b0 < nbatch; b0 += 64) {
    const int bb = b0 + lane;
    bb_first += __popcll(__ballot(bb < nbatch && untag(bstart[bb]) <= lo));
  }
  bb_first = max(0, bb_first - 1);
  for (int bb = bb_first + wave; len > 0 && bb < nbatch; bb += 4) {
    const int w = bb * 64 + lane;
    const uint64_t x = w < nwords ? (uint64_t)bm[w] : 0ull;
    const int e = w < nwords ? woff[w] : 0;
    if (untag(__builtin_amdgcn_readfirstlane(bstart[bb])) >= hi_pos) break;
    int off = w < nwords ? untag(e) : n;
    const int c = __popcll(x);
    const bool meets = c > 0 && off < hi_pos && off + c > lo;
    // sparse words: the owning lane walks the bits of both halves at once
    // (two independent chains), writing to a scratch slot past the list for
    // a position outside the split
    if (__ballot(meets && c < kDenseWord)) {
      const bool sparse = meets && c < kDenseWord;
      uint32_t blo = sparse ? (uint32_t)x : 0u, bhi = sparse ? (uint32_t)(x >> 32) : 0u;
      int olo = off - lo, ohi = off - lo + __popc((uint32_t)x);
      const int plo = w * 64, phi = w * 64 + 32;
      lds_i32* ids = (lds_i32*)L.ids;
      while (blo | bhi) {  // branch-free body: an empty half writes the scratch slot
        const bool vlo = blo != 0, vhi = bhi != 0;
        ids[vlo && (unsigned)olo < (unsigned)len ? olo : kIdsMax] = plo + (int)__ffs(blo) - 1;
        ids[vhi && (unsigned)ohi < (unsigned)len ? ohi : kIdsMax] = phi + (int)__ffs(bhi) - 1;
        blo &= blo - 1;
        bhi &= bhi - 1;
        olo += vlo ? 1 : 0;
        ohi += vhi ? 1 : 0;
      }
    }
    // dense words: one lane per bit
    uint64_t dense = __ballot(meets && c >= kDenseWord);
    while (dense) {
      const int src = __builtin_ctzll(dense);
      dense &= dense - 1;
      const uint32_t xlo = __builtin_amdgcn_readlane((uint32_t)x, src);
      const uint32_t xhi = __builtin_amdgcn_readlane((uint32_t)(x >> 32), src);
      const int woff0 = __builtin_amdgcn_readlane(off, src);
      const uint32_t below = __builtin_amdgcn_mbcnt_hi(xhi, __builtin_amdgcn_mbcnt_lo(xlo, 0u));
      const bool mine = ((lane < 32 ? xlo >> lane : xhi >> (lane - 32)) & 1u) != 0;
      const int pos = woff0 + (int)below;
      if (mine && pos >= lo && pos < hi_pos) L.ids[pos - lo] = (bb * 64 + src) * 64 + lane;
    }
  }
  lds_barrier();  // positions of the split in the id list

  // 4. positions -> slots, the lists and the token's scalars
  {
    int32_t* tok_row = a.tok_out + (int64_t)t * a.cap;
    int32_t* slot_row = a.slot_out + (int64_t)t * a.cap;
    int bad = 0;
    // (normalisation in stage 1) tile 0 first: output wave j turns rows
    // 16 j .. 16 j + 15 into slots and enqueues them into stage 0 at once,
    // so that the gather of the first tile overlaps the rest of the list;
    // the same wave then writes those entries (no other wave touches them)
    const bool first_done = early && len > 0;
    if (first_done && outw)
      issue_tile0([&](int k) {
        int id = -1;
        if (k < len) {
          const int p = L.ids[k];
          const int b = div_p(p, a.pdiv);
          const int slot = tbl[b] * P + (p - b * P);
          const bool valid = slot < a.kv_rows;
          id = valid ? slot : -1;
          if ((lane & 7) == 0) {  // one lane per row
            bad |= valid ? 0 : 1;
            if (hg == 0) {
              tok_row[lo + k] = p;
              slot_row[lo + k] = slot;
            }
          }
        }
        if ((lane & 7) == 0) L.ids[k] = id;
        return id;
      });
    const int k_from = first_done ? kTileRows : 0;  // entries this loop still converts
    constexpr int kCB = 3;  // entries per thread with their LDS reads together
    for (int k0 = 0; k0 < ntiles * kTileRows; k0 += kCB * kThreads) {
      int pv[kCB], bv[kCB], pg[kCB];
#pragma unroll
      for (int u = 0; u < kCB; ++u) {
        const int k = k0 + tid + kThreads * u;
        pv[u] = k < len && k >= k_from ? L.ids[k] : 0;
      }
#pragma unroll
      for (int u = 0; u < kCB; ++u) {
        bv[u] = div_p(pv[u], a.pdiv);
        pg[u] = tbl[bv[u]];
      }
#pragma unroll
      for (int u = 0; u < kCB; ++u) {
        const int k = k0 + tid + kThreads * u;
        if (k < ntiles * kTileRows && k >= k_from) {
          int id = -1;
          if (k < len) {
            const int slot = pg[u] * P + (pv[u] - bv[u] * P);
            const bool valid = slot < a.kv_rows;
            id = valid ? slot : -1;
            bad |= valid ? 0 : 1;
            if (hg == 0) {
              tok_row[lo + k] = pv[u];
              slot_row[lo + k] = slot;
            }
          }
          L.ids[k] = id;
        }
      }
    }
    if (__ballot(bad) != 0 && lane == 0) s_bad[0] = 1;
    if (hg == 0 && sidx == a.S - 1)
      for (int k = n + tid; k < a.cap; k += kThreads) {
        tok_row[k] = -1;
        slot_row[k] = -1;
      }
    if (writer && tid == 0) {
      int nb = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) nb += red[4 + w];
      a.count_out[t] = n;
      if (a.blk_indptr) a.blk_indptr[t + 1] = -(nb + 1);
    }
    if (drop_writer && tid == 0 && a.dropped_out) {
      int dropped = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) dropped += red[8 + w];
      a.dropped_out[t] = dropped;
    }
  }
  lo_out = __builtin_amdgcn_readfirstlane(lo);
  len_out = __builtin_amdgcn_readfirstlane(len);
  lds_barrier();  // ids and s_bad visible; stages 0 and 1 free for the tiles
}

// One work item: token t, candidate positions lo .. lo + len - 1 of its list,
// head group hg; split partials go to slot `part` ([part][H][512]).  kFp8:
// the rows are fp8_ds_mla rows (a.kv8), dequantised on their way into the
// ring.  kLong: the split may hold more candidates than the LDS id list
// (kIdsMax): the list is then a ring of kIdTiles tiles, tile t in slot
// t % kIdTiles; the first kIdTiles tiles are staged as usual, and in output
// iteration i the slot of tile i - 1 (whose ids every wave is done with after
// B(i)) takes tile i + kIdTiles - 1's ids by LDS DMA, as they are in
// memory: position and range checks then happen where ids are read.
// final_out (kOutFinal / kOutPartialBf16 epilogues only): the final output
// and lse rather than the split's normalised partial and (m, l); a run-time
// flag, so that a launch that writes both kinds (the queue launch) holds one
// copy of the item.
template <int kMode, bool kFp8 = false, bool kLong = false, bool kNorm = false,
          bool kPeel = true>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, const DecodeLds& L, int* s_bad,
                                            const uint8_t* zero_row, int t, int lo, int len,
                                            int hg, int64_t part, int sidx = 0,
                                            bool final_out = kMode == kOutFinal) {
  // opaque per call, so that nothing derived from the thread index is hoisted
  // out of the queue launch's item loop (it would stay live across the whole
  // item and push the registers into spills)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool score = wave < 2;
  const int j = wave & 1;

  // Row loads go straight to LDS (global_load_lds), one 8-row group per wave
  // instruction sequence: lane keeps row lane / 8 of the group and, in block
  // it = 0..8, chunk 8 it + ((lane % 8) ^ (lane / 8)).
  const int ld_col = ((lane & 7) ^ (lane >> 3)) * 16;
  auto group_dst = [&](int st, int grp) {
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(L.tiles + st * kTileBytes + grp * kGroupBytes));
  };
  // Score wave j's 32 query rows go to ring stage 2 + j, in the tile layout
  // (coalesced like any tile; read back as MFMA fragments before B(0), after
  // which the stage carries tiles again).
  auto issue_q = [&]() {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int head = hg * kHeadsPerWG + 32 * j + grp * kGroupRows + (lane >> 3);
      const uint8_t* src =
          (head < a.H ? (const uint8_t*)(a.q + ((int64_t)t * a.H + head) * kDQK) : zero_row) +
          ld_col;
      load_row_chunks<0>(src, group_dst(2 + j, grp));
    }
  };
  // kNorm: the split's range and ids come from the token's normalisation,
  // which enqueues the query rows itself
  // (kNorm, normalisation in stage 1) tile 0's rows from their ids, given
  // by row
  auto issue_tile0 = [&](auto&& id_of_row) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int grp = 2 * j + g;
      const int id = id_of_row(grp * kGroupRows + (lane >> 3));
      load_row_chunks<0>((id >= 0 ? (const uint8_t*)a.kv + (int64_t)id * kRowBytes : zero_row) +
                             ld_col,
                         group_dst(0, grp));
    }
  };
  bool tile0_issued = false;
  if constexpr (kNorm) {
    normalize_split(a, L, s_bad, t, sidx, hg, lo, len, issue_q, issue_tile0);
    tile0_issued = norm_in_stage1(a);
  } else if (score) {
    issue_q();
  }
  const int ntiles = (len + kTileRows - 1) / kTileRows;

  // candidate ids of this split, -1 for invalid ones and up to the tile edge;
  // read by the output waves, whose load queue is empty here (the score
  // waves' queue holds the query rows), and handed over with an LDS-only
  // barrier so that nobody waits for the query rows yet
  if (!kNorm && !score) {
    // every load first, then the stores: one round trip instead of one per
    // 128 ids
    constexpr int kPer = (kIdsMax + 127) / 128;
    const int32_t* src_ids = a.row_ids + (int64_t)t * a.cap + lo;
    int32_t v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = tid - 128 + 128 * k;
      v[k] = i < len ? src_ids[i] : -1;
    }
    int bad = 0;
    const int staged = kLong ? min(ntiles * kTileRows, kIdsMax) : ntiles * kTileRows;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = tid - 128 + 128 * k;
      const bool valid = v[k] >= 0 && v[k] < a.kv_rows;
      if (i < staged) L.ids[i] = valid ? v[k] : -1;
      bad |= (i < len && !valid) ? 1 : 0;
    }
    const int wbad = __ballot(bad) != 0 ? 1 : 0;
    if (lane == 0) s_bad[j] = wbad;
  }
  if constexpr (!kNorm) lds_barrier();
  // a split with an invalid id masks every tile, otherwise only its last tile
  // (the rows past its end) needs a mask (a long split: every tile, its later
  // ids are not seen before their turn)
  const bool mask_all = kLong || (s_bad[0] | s_bad[1]) != 0;

  // id of row r of tile i, -1 for an invalid candidate or a row past the end
  auto id_at = [&](int i, int r) {
    if constexpr (kLong) {
      const int id = L.ids[(i % kIdTiles) * kTileRows + r];
      return (i * kTileRows + r < len && id >= 0 && id < a.kv_rows) ? id : -1;
    } else {
      return L.ids[i * kTileRows + r];
    }
  };
  // kLong: in output iteration i, load tile i + kIdTiles - 1's ids into the
  // slot of tile i - 1 (output wave 0, one id per lane)
  auto refill_ids = [&](int i) {
    if constexpr (kLong) {
      const int tn = i + kIdTiles - 1;
      if (j == 0 && lane < kTileRows && tn * kTileRows + lane < len) {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)(L.ids + (tn % kIdTiles) * kTileRows));
        load_lds_4(a.row_ids + (int64_t)t * a.cap + lo + tn * kTileRows + lane, dst);
      }
    }
  };

  // source of this lane's row of group grp of tile i (the zero row for an
  // invalid candidate)
  auto row_src = [&](int i, int grp) {
    const int id = id_at(i, grp * kGroupRows + (lane >> 3));
    return (id >= 0 ? (const uint8_t*)a.kv + (int64_t)id * kRowBytes : zero_row) + ld_col;
  };
  auto issue_group = [&](int i, int st, int grp) {
    load_row_chunks<0>(row_src(i, grp), group_dst(st, grp));
  };
  // Only the output waves load tiles (two row groups each); the score waves'
  // QK MFMAs and softmax stay free of load issue (one group from every wave
  // measured no faster).
  auto issue = [&](int i, int st) {
    issue_group(i, st, 2 * j);
    issue_group(i, st, 2 * j + 1);
  };
  auto tile_mask = [&](int i) { return (uint32_t)__ballot(id_at(i, lane & 31) >= 0); };
  if constexpr (!kFp8) {
    if (!score) {
      if (ntiles > 0 && !tile0_issued) issue(0, 0);
      if (ntiles > 1) issue(1, 1);
    }
  }

  // fp8 rows: each wave stages one row group of every tile through its
  // registers (score wave j group 2 j + 1, output wave j group 2 j): lane l
  // takes row l / 8 of the group and, of it, 16-byte chunk l % 8 of each
  // 128-byte latent line, its RoPE chunk and the four scales.  Tile t is
  // loaded one iteration before it is dequantised into its ring stage (in
  // the window between B(t - 2) and B(t - 1); stage (t - 2) % 4 is then
  // free: tile t - 4's V^T was read in iteration t - 4 and its K before);
  // tiles 0 and 1 are written before B(0).  Past the last tile the zero row
  // is loaded, so every iteration does the same work.
  const int f8_grp = score ? 2 * j + 1 : 2 * j;
  const int rl = lane >> 3, u8 = lane & 7;
  auto fp8_row = [&](int tile) {
    const int id = tile < ntiles ? id_at(tile, f8_grp * kGroupRows + rl) : -1;
    return id >= 0 ? a.kv8 + (int64_t)id * kFp8RowBytes : zero_row;
  };
  // LDS offsets in a stage: latent chunk 16 line + 2 u + half of group row
  // rl sits in block 2 line + u / 4 at position ((2 u + half) % 8) ^ rl;
  // RoPE chunk u in block 8 at position u ^ rl
  int lat_off[2];
#pragma unroll
  for (int half = 0; half < 2; ++half)
    lat_off[half] = f8_grp * kGroupBytes + (u8 >> 2) * 1024 + rl * 128 +
                    ((((2 * u8 + half) & 7) ^ rl) << 4);
  const int rope_off = f8_grp * kGroupBytes + 8 * 1024 + rl * 128 + ((u8 ^ rl) << 4);
  // global (not flat) loads: a flat load also counts against the LDS
  // counter, so every LDS wait would wait for the rows in flight too
  typedef const __attribute__((address_space(1))) uintx4 g_uintx4;
  typedef const __attribute__((address_space(1))) floatx4 g_floatx4;
  auto load_latent = [&](Fp8Rows& b, int line, const uint8_t* p) {
    b.lat[line] = *(g_uintx4*)(p + 128 * line + 16 * u8);
  };
  auto load_rope = [&](Fp8Rows& b, const uint8_t* p) {
    b.rope = *(g_uintx4*)(p + kFp8RopeOff + 16 * u8);
  };
  auto load_scales = [&](floatx4& sc, const uint8_t* p) { sc = *(g_floatx4*)(p + kFp8ScaleOff); };
  auto load_all = [&](Fp8Rows& b, int tile) {
    const uint8_t* p = fp8_row(tile);
    load_scales(b.scl, p);
#pragma unroll
    for (int line = 0; line < 4; ++line) load_latent(b, line, p);
    load_rope(b, p);
  };
  auto store_half = [&](const Fp8Rows& b, int line, int half, lds_t* stage) {
    const uintx4 d = b.lat[line];
    const uintx4 w = half ? dequant8(d[2], d[3], b.scl[line]) : dequant8(d[0], d[1], b.scl[line]);
    *(__attribute__((address_space(3))) uintx4*)(stage + 2 * line * 1024 + lat_off[half]) = w;
  };
  auto store_rope = [&](const Fp8Rows& b, lds_t* stage) {
    *(__attribute__((address_space(3))) uintx4*)(stage + rope_off) = b.rope;
  };
  auto store_all = [&](const Fp8Rows& b, lds_t* stage) {
#pragma unroll
    for (int line = 0; line < 4; ++line) {
      store_half(b, line, 0, stage);
      store_half(b, line, 1, stage);
    }
    store_rope(b, stage);
  };
  Fp8Rows fb;  // (fp8) the tile being staged
  // tiles 0 and 1 into stages 0 and 1, tile 2 loaded (before B(0))
  auto fp8_prologue = [&]() {
    Fp8Rows f0;
    load_all(f0, 0);
    load_all(fb, 1);
    store_all(f0, L.tiles);
    store_all(fb, L.tiles + kTileBytes);
    load_all(fb, 2);
  };

  // Pipeline over the ring of kStages = 4 tiles, with P(i) the published P^T
  // of tile i (pbuf[i % 2]) and B(i) the i-th workgroup barrier:
  //   prologue: query rows (stages 2, 3) and tiles 0, 1 enqueued and landed;
  //     the score waves move Q^T into registers; B(0).
  //   score waves, iteration i (0 <= i < ntiles): softmax of tile i, whose
  //     S^T was computed in iteration i-1 (tile 0: right after B(0)),
  //     together with the QK products of tile i+1; ends with B(i+1), which
  //     publishes P(i).
  //   output waves, iteration i (1 <= i <= ntiles): see below; V(0) is read
  //     between B(0) and B(1).
  if (score) {
    const int kr = lane & 31;
    int k_base[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      k_base[q4] = (kr >> 3) * kGroupBytes + (kr & 7) * 128 +
                   (((2 * q4 + (lane >> 5)) ^ (kr & 7)) << 4);
    // Q^T fragments: the query rows sit in stage 2 + j in the tile layout, so
    // the B fragment of k-step ks is read like a K fragment.  Q^T then lives
    // in AGPRs (MFMA takes its B operand from there), leaving the VGPRs to
    // the K fragment ring and the softmax.
    bf16x8 qf[kQKSteps];
    {
      wait_vmcnt<0>();  // this wave's query rows
      const lds_t* qstage = L.tiles + (2 + j) * kTileBytes;
      shortx8 qv[kQKSteps];
#pragma unroll
      for (int ks = 0; ks < kQKSteps; ++ks)
        qv[ks] = *(const lds_shortx8*)k_addr(qstage, k_base, ks);
      __builtin_amdgcn_sched_barrier(0);  // all 36 reads in flight before the first use
#pragma unroll
      for (int ks = 0; ks < kQKSteps; ++ks) {
        qf[ks] = __builtin_bit_cast(bf16x8, qv[ks]);
        asm volatile("" : "+a"(qf[ks]));
      }
    }
    ScoreState st{-INFINITY, -INFINITY, 0.f};
    SAcc acc_a, acc_b;
    if constexpr (kFp8) fp8_prologue();  // (stages 0 and 1; Q^T is in registers)
    lds_barrier();  // B(0): tiles 0 and 1 visible, Q^T read out of stages 2 and 3
    if (ntiles > 0) qk_tile(L.tiles, k_base, qf, acc_a);
    // iteration i: softmax of tile i (S^T in registers) with the QK of tile
    // i+1; P(i) is published by the barrier B(i+1) that ends it.  Unrolled by
    // two so that the accumulator sets swap roles without copies, with the
    // last tile peeled off, so that the loop body holds one straight-line
    // variant of the step (a branch between variants would let the compiler
    // hoist their common softmax arithmetic out of the MFMA stream).
    // (fp8 rows) iteration i also dequantises this wave's group of tile
    // i + 2 into its stage and loads tile i + 3 into the same registers: a
    // half line every fourth MFMA (the line reloaded after its second half),
    // the RoPE chunk after, the new scales into registers of their own
    auto full = [&](auto masked, int i, const SAcc& cur, SAcc& nxt) {
      constexpr bool kMasked = decltype(masked)::value;
      lds_t* stage = L.tiles + ((i + 2) % kStages) * kTileBytes;
      const uint8_t* pn = kFp8 ? fp8_row(i + 3) : zero_row;
      floatx4 nscl;
      if constexpr (kFp8) load_scales(nscl, pn);
      score_step<true, kMasked>(L, L.tiles + ((i + 1) % kStages) * kTileBytes, k_base, qf, cur,
                                nxt, kMasked ? tile_mask(i) : ~0u, a.scale_log2, i & 1, j, lane,
                                st, [&](int ks) {
                                  if constexpr (kFp8) {
                                    if (ks >= 2 && ks <= 30 && (ks & 3) == 2) {
                                      const int n = (ks - 2) >> 2, line = n >> 1, half = n & 1;
                                      store_half(fb, line, half, stage);
                                      if (half) load_latent(fb, line, pn);
                                    } else if (ks == 34) {
                                      store_rope(fb, stage);
                                      load_rope(fb, pn);
                                    }
                                  }
                                });
      if constexpr (kFp8) fb.scl = nscl;
      lds_barrier();
    };
    auto last = [&](int i, const SAcc& cur) {
      SAcc none;
      score_step<false, true>(L, L.tiles, k_base, qf, cur, none, tile_mask(i), a.scale_log2,
                              i & 1, j, lane, st, [](int) {});
      lds_barrier();
    };
    auto run = [&](auto masked) {
      int i = 0;
      for (; i + 2 < ntiles; i += 2) {
        full(masked, i, acc_a, acc_b);
        full(masked, i + 1, acc_b, acc_a);
      }
      if (ntiles - i == 2) {
        full(masked, i, acc_a, acc_b);
        last(i + 1, acc_b);
      } else if (ntiles - i == 1) {
        last(i, acc_a);
      }
    };
    if (mask_all)
      run(std::true_type{});
    else
      run(std::false_type{});
    const float l_tot = pair_sum(st.lsum);
    if (lane < 32) {
      L.stat[0 * 64 + 32 * j + lane] = st.m_ref;
      L.stat[1 * 64 + 32 * j + lane] = st.m_true;
      L.stat[2 * 64 + 32 * j + lane] = l_tot;
    }
    lds_barrier();  // statistics published
    if (kMode == kOutPartialF32) return;
    lds_barrier();  // output rows staged by the output waves
    copy_out_rows(a, L, t, part, hg, tid, final_out);
    return;
  }

  // ---- output waves ----
  //  V^T fragment (transpose read): rows 16 kap + 4 (g / 2) + j16 / 4 (+ 8),
  //  values 256 j + 32 mb + 16 (g % 2) + 4 (j16 % 4) .. + 3, g = lane / 16.
  //  Chunk cc = 32 j + 4 mb + cc0 with cc0 = 2 (g % 2) + (j16 % 4) / 2 < 4, so
  //  two per-lane bases (mb parity) plus immediates cover every read.
  const int vg = lane >> 4, vj = lane & 15;
  const int v_rl = 4 * (vg >> 1) + (vj >> 2);
  const int v_cc0 = 2 * (vg & 1) + ((vj & 3) >> 1);
  int v_base[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    v_base[par] = 4 * j * 1024 + v_rl * 128 + (((v_cc0 + 4 * par) ^ v_rl) << 4) + 8 * (vj & 1);
  auto vaddr = [&](const lds_t* stage, int kap, int half, int mb) {
    return (lds_shortx4*)(stage + v_base[mb & 1] + (2 * kap + half) * kGroupBytes +
                          1024 * (mb >> 1));
  };
  auto read_v = [&](const lds_t* stage, shortx4 (&v0)[2][8], shortx4 (&v1)[2][8]) {
#pragma unroll
    for (int kap = 0; kap < 2; ++kap)
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        v0[kap][mb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vaddr(stage, kap, 0, mb));
        v1[kap][mb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vaddr(stage, kap, 1, mb));
      }
  };
  floatx16 o[2][8];  // O^T[256 j + 32 mb + m][32 hb + head]
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) o[hb][mb] = floatx16{};
  shortx4 v0[2][8], v1[2][8];

  // One output iteration i (1 <= i <= ntiles) but for the work on the tile
  // after next: apply P(i-1) to V(i-1), read V(i) for the next iteration; the
  // 18 steps of the next tile's loads (bf16 rows) or of the row staging (fp8
  // rows), step(k), sit between the MFMA pairs and after the last one.
  // Returns whether tile i was the last.
  auto pv_iteration = [&](int i, auto&& step) {
    const int buf = (i - 1) & 1;
    const float a0 = L.alpha[buf * 64 + (lane & 31)];
    const float a1 = L.alpha[buf * 64 + 32 + (lane & 31)];
    bf16x8 pf[2][2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int kap = 0; kap < 2; ++kap)
        pf[hb][kap] = *(const __attribute__((address_space(3))) bf16x8*)(
            L.pbuf + ((buf * 2 + hb) * 2 + kap) * 1024 + lane * 16);
    // alpha = 0 only while nothing has been accumulated (O^T is still zero)
    if (__ballot((a0 != 1.f && a0 != 0.f) || (a1 != 1.f && a1 != 0.f))) {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        scale_acc(o[0][mb], a0);
        scale_acc(o[1][mb], a1);
      }
    }
    // PV MFMAs of tile i-1; each V^T fragment register pair is refilled from
    // tile i right after its last use (after the last tile the reads hit a
    // stale stage: in bounds and unused).
    const lds_t* vn = L.tiles + (i % kStages) * kTileBytes;
    auto pv_pair = [&](auto kc, auto mc) {
      constexpr int kap = decltype(kc)::value, mb = decltype(mc)::value;
      const shortx8 vv = {v0[kap][mb][0], v0[kap][mb][1], v0[kap][mb][2], v0[kap][mb][3],
                          v1[kap][mb][0], v1[kap][mb][1], v1[kap][mb][2], v1[kap][mb][3]};
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
        o[hb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv),
                                                            pf[hb][kap], o[hb][mb], 0, 0, 0);
      v0[kap][mb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vaddr(vn, kap, 0, mb));
      v1[kap][mb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(vaddr(vn, kap, 1, mb));
      step(std::integral_constant<int, kap * 8 + mb>{});
      __builtin_amdgcn_sched_barrier(0);
    };
    static_for<2>([&](auto kc) { static_for<8>([&](auto mc) { pv_pair(kc, mc); }); });
    step(std::integral_constant<int, 16>{});
    step(std::integral_constant<int, 17>{});
    return i == ntiles;
  };

  if constexpr (!kFp8) {
    // ids of this lane's two rows of the tile that the next iteration
    // enqueues (clamped to the last tile), read one iteration ahead: the
    // loop's first MFMA then waits for P^T and the factors only, not for
    // two id round trips before them
    int nid[2];
    auto read_next_ids = [&](int tile) {
      const int tc = min(tile, ntiles - 1);
      nid[0] = id_at(tc, 2 * j * kGroupRows + (lane >> 3));
      nid[1] = id_at(tc, (2 * j + 1) * kGroupRows + (lane >> 3));
    };
    auto id_src = [&](int id) {
      return (id >= 0 ? (const uint8_t*)a.kv + (int64_t)id * kRowBytes : zero_row) + ld_col;
    };
    wait_vmcnt<0>();  // tiles 0 and 1
    lds_barrier();    // B(0): stages 2 and 3 are free again
    if (ntiles > 0) {
      if (ntiles > 2) issue(2, 2);
      read_next_ids(4);
      read_v(L.tiles, v0, v1);
      // tile 2 must have landed before B(1) (tile 3 may stay in flight)
      if (ntiles > 3) {
        issue(3, 3);
        wait_vmcnt<2 * kSlotsPerThread>();
      } else {
        wait_vmcnt<0>();
      }
      lds_barrier();  // B(1): P(0) published
    }
    // iteration i (1 <= i <= ntiles): enqueue tile i+3 into the stage of tile
    // i-1 (its V^T is in registers, its K was read two iterations ago); apply
    // P(i-1) to V(i-1); read V(i) for the next iteration; tile i+2 lands before
    // the barrier B(i+1) (the score waves read it in iteration i+1).  The 18
    // load instructions of tile i+3 are spread between the MFMAs, one per MFMA
    // pair, so that the wave never stalls on a full load queue.  Past the last
    // tile nothing is loaded (and the wait before the barrier drains the queue).
    // kPeel: the iterations that load (i + 3 < ntiles) and the last three,
    // which do not, run as two loops (kLoads 1 and 0); otherwise one loop
    // loads the zero row past the last tile (kLoads 2, into the free stage:
    // fewer registers where the item itself sits in a loop).  Either way no
    // load sits behind a branch.
    auto iteration = [&](int i, auto loads) {
      constexpr int kLoads = decltype(loads)::value;
      refill_ids(i);  // (kLong) lands before B(i+1): the wait below leaves only tile i+3's loads
      const bool real = kLoads == 1 || (kLoads == 2 && i + 3 < ntiles);
      // tile i+3's ids (kLoads 2: past the end those of the last tile, not
      // used)
      const uint8_t* src0 = kLoads == 0 ? zero_row : id_src(nid[0]);
      const uint8_t* src1 = kLoads == 0 ? zero_row : id_src(nid[1]);
      if (kLoads == 2 && !real) {
        src0 = zero_row + ld_col;
        src1 = zero_row + ld_col;
      }
      const int st3 = (i + 3) % kStages;
      const uint32_t dst0 = group_dst(st3, 2 * j), dst1 = group_dst(st3, 2 * j + 1);
      auto load_chunk = [&](auto c) {
        constexpr int kC = decltype(c)::value;
        if constexpr (kLoads != 0 && kC == 1) read_next_ids(i + 4);
        if constexpr (kLoads == 0)
          return;
        else if constexpr (kC < kSlotsPerThread)
          load_lds_16<kC * 128>(src0, dst0 + kC * (1024 - 128));
        else
          load_lds_16<(kC - kSlotsPerThread) * 128>(src1,
                                                    dst1 + (kC - kSlotsPerThread) * (1024 - 128));
      };
      if (pv_iteration(i, load_chunk)) return true;
      // tile i+2 must have landed before B(i+1) (tile i+3 may stay in flight)
      if constexpr (kLoads == 0)
        wait_vmcnt<0>();
      else
        wait_vmcnt<2 * kSlotsPerThread>();
      lds_barrier();  // B(i+1)
      return false;
    };
    int i = 1;
    if constexpr (kPeel) {
      for (; i + 3 < ntiles; ++i) iteration(i, std::integral_constant<int, 1>{});
      for (; i <= ntiles; ++i)
        if (iteration(i, std::integral_constant<int, 0>{})) break;
    } else {
      for (; i <= ntiles; ++i)
        if (iteration(i, std::integral_constant<int, 2>{})) break;
    }
  } else {
    // fp8 rows (this wave's group 2 j, see above)
    fp8_prologue();
    lds_barrier();  // B(0): tiles 0 and 1 written, stages 2 and 3 free again
    if (ntiles > 0) {
      store_all(fb, L.tiles + 2 * kTileBytes);
      load_all(fb, 3);
      read_v(L.tiles, v0, v1);
      lds_barrier();  // B(1): P(0) published, tile 2 written
    }
    // iteration i: dequantise tile i+2 into its stage while loading tile i+3
    // into the same registers: the scales first (into registers of their
    // own, taken over at the end), then a half line on every other MFMA
    // pair (the line reloaded after its second half), the RoPE chunk after
    // the last pair
    for (int i = 1; i <= ntiles; ++i) {
      refill_ids(i);
      lds_t* stage = L.tiles + ((i + 2) % kStages) * kTileBytes;
      const uint8_t* pn = fp8_row(i + 3);
      floatx4 nscl;
      load_scales(nscl, pn);
      auto step = [&](auto kc) {
        constexpr int k = decltype(kc)::value;
        if constexpr (k < 16 && k % 2 == 0) {
          constexpr int n = k / 2, line = n >> 1, half = n & 1;
          store_half(fb, line, half, stage);
          if constexpr (half == 1) load_latent(fb, line, pn);
        } else if constexpr (k == 16) {
          store_rope(fb, stage);
          load_rope(fb, pn);
        }
      };
      const bool last = pv_iteration(i, step);
      fb.scl = nscl;
      if (last) break;
      // (kLong) the id refill of the previous iteration has landed: only this
      // iteration's six row loads may still be in flight
      if constexpr (kLong) wait_vmcnt<6>();
      lds_barrier();  // B(i+1): tile i+2 written
    }
  }
  wait_vmcnt<0>();  // nothing left in flight before the ring is reused below
  lds_barrier();  // statistics published

  // lane holds O^T[256 j + 32 mb + 8 (r / 4) + 4 (lane / 32) + r % 4][32 hb + lane % 32]
  const int dv_lane = 256 * j + 4 * (lane >> 5);
  if (kMode == kOutPartialF32) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int hl = 32 * hb + (lane & 31);
      const int head = hg * kHeadsPerWG + hl;
      if (head >= a.H) continue;
      const float m_ref = L.stat[hl], m_true = L.stat[64 + hl], l_tot = L.stat[128 + hl];
      const bool live = m_true != -INFINITY;
      const float f = live ? fast_exp2(m_ref - m_true) : 0.f;  // rebase to the true maximum
      float* orow = (float*)a.o_part + (part * a.H + head) * kDV;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          *(float4*)(orow + dv_lane + 32 * mb + 8 * rq) =
              make_float4(o[hb][mb][4 * rq] * f, o[hb][mb][4 * rq + 1] * f,
                          o[hb][mb][4 * rq + 2] * f, o[hb][mb][4 * rq + 3] * f);
      if (j == 0 && lane < 32) {
        const int64_t k = part * a.H + head;
        a.m_part[k] = live ? m_true * kLn2 : -INFINITY;
        a.l_part[k] = l_tot * f;
      }
    }
    return;
  }

  // bf16 o / l (the final output, or a normalised split partial): O^T staged
  // in fp32 through the idle tile ring, then scaled, rounded and written out
  // by all four waves.
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int hl = 32 * hb + (lane & 31);
    lds_t* hrow = L.tiles + hl * kHeadStrideF + dv_lane * 4;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *(__attribute__((address_space(3))) floatx4*)(hrow + (32 * mb + 8 * rq) * 4) =
            floatx4{o[hb][mb][4 * rq], o[hb][mb][4 * rq + 1], o[hb][mb][4 * rq + 2],
                    o[hb][mb][4 * rq + 3]};
  }
  lds_barrier();  // output rows staged
  copy_out_rows(a, L, t, part, hg, tid, final_out);
  if (lane < 32) {
    // lse / (m, l): output wave j covers heads 32 j .. 32 j + 31, one lane each
    const int hl = 32 * j + (lane & 31);
    const int head = hg * kHeadsPerWG + hl;
    if (head < a.H) {
      const float m_ref = L.stat[hl], m_true = L.stat[64 + hl], l_tot = L.stat[128 + hl];
      const bool live = m_true != -INFINITY;
      if (final_out) {
        if (a.lse)
          a.lse[(int64_t)t * a.H + head] = live ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
      } else {
        // m = the split's max logit, l = sum of exp(z - m)
        const int64_t k = part * a.H + head;
        a.m_part[k] = live ? m_true * kLn2 : -INFINITY;
        a.l_part[k] = live ? l_tot * fast_exp2(m_ref - m_true) : 0.f;
      }
    }
  }
}

// Kernel.  Static launch: one workgroup per (token, split, head group) in an
// XCD-aware order; every workgroup of one token (all splits, all head groups)
// gets a block id of the same residue mod 8, i.e. runs on the same XCD, so
// the token's query rows and the KV rows its head groups share are fetched
// into one L2.  Queue launch (kQueue): a persistent grid takes work items
// (task, head group) from eight queues, one per XCD: queue x holds the tasks
// of rows x, x + 8, ... (the plan's queue entries), so all splits of a row run
// on one XCD and share its query rows there, and both head groups of a task
// sit next to each other, so the pair shares the KV rows in that L2.  Each workgroup's first item is
// assigned by its block id; later items are claimed with the queue heads,
// the workgroup's own XCD queue first, then the others.  A task that covers
// its whole row writes the row's final output and lse itself (its entry's
// slot is -1); the others write partial states for the merge.  A workgroup ends
// when no queue has an unclaimed item (every queue is finite and its head
// only grows, so every workgroup exits).
template <int kMode, bool kQueue, bool kFp8 = false, bool kLong = false, bool kNorm = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sparse_mla_decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) char s_tiles[kStages * kTileBytes];
  __shared__ __attribute__((aligned(16))) char s_pbuf[2 * 2 * 2 * 1024];
  __shared__ __attribute__((aligned(16))) float s_alpha[2 * 64];
  __shared__ __attribute__((aligned(16))) float s_stat[3 * 64];
  __shared__ __attribute__((aligned(16))) int32_t s_ids[kIdsMax + 4];  // + a scratch slot
  __shared__ int s_bad[2];
  const DecodeLds L{(lds_t*)s_tiles, (lds_t*)s_pbuf, s_alpha, s_stat, s_ids};
  // the zero row's address, fetched once: inside the loops its GOT load (a
  // scalar load, which only a full lgkmcnt(0) wait covers) would drain the
  // LDS reads in flight
  const uint8_t* zero_row = g_zero_row;
  asm volatile("" : "+s"(zero_row));

  if constexpr (!kQueue) {
    const int bid = blockIdx.x;
    const int xk = bid >> 3;
    const int per_token = a.S * a.G;
    const int t = (xk / per_token) * 8 + (bid & 7);
    const int rem = xk % per_token;
    const int s = rem / a.G;
    const int hg = rem - s * a.G;
    if (t >= a.T) return;
    if constexpr (kNorm) {
      decode_item<kMode, false, false, true, kMode != kOutPartialF32>(
          a, L, s_bad, zero_row, t, 0, 0, hg, (int64_t)t * a.S + s, s);
    } else {
      int n = a.counts ? a.counts[t] : a.cap;
      n = min(max(n, 0), a.cap);
      const int chunk = (n + a.S - 1) / a.S;
      const int lo = min(n, s * chunk);
      const int len = min(n, lo + chunk) - lo;
      decode_item<kMode, kFp8, kLong, false, kMode != kOutPartialF32>(a, L, s_bad, zero_row, t,
                                                                     lo, len, hg,
                                      (int64_t)t * a.S + s);
    }
  } else {
    const int grid = gridDim.x;
    const int x = blockIdx.x & 7;
    // queue q: items i = 0 .. items(q) - 1 over its entries (item i is entry
    // i / G of segment q, head group i % G); the first pre(q) of them are
    // pre-assigned, one to each workgroup of block id = q (mod 8) (no atomic
    // for a workgroup's first item), the rest are claimed with the queue head
    // (an atomic counter from 0) as item pre(q) + head
    const int idx = blockIdx.x >> 3;  // the pre-assigned item in queue x
    int4 e0 = make_int4(-1, 0, 0, 0);
    if (threadIdx.x == 0 && idx / a.G < a.qcap)  // read together with the counts
      e0 = *(const int4*)(a.qent + 4 * ((int64_t)x * a.qcap + idx / a.G));
    // the queue counts are read where they are used (by the claiming thread),
    // so that nothing of them stays live across an item
    auto items = [&](int q) { return a.G * a.qcount[q]; };
    auto pre = [&](int q) { return (grid - q + 7) >> 3; };
    bool dynamic = false;  // does any queue hold items beyond the pre-assigned ones?
#pragma unroll
    for (int y = 0; y < 8; ++y) dynamic |= items(y) > pre(y);
    dynamic = __builtin_amdgcn_readfirstlane(dynamic ? 1 : 0) != 0;
    int qi = 0;  // queues x, x + 1, ... (mod 8) before qi are exhausted
    bool first = true;
    __shared__ int s_ent[5];
    for (;;) {
      __syncthreads();  // the previous item is done with LDS and s_ent
      if (threadIdx.x == 0) {
        int q = x, i = -1;
        int4 e = e0;
        if (first && idx < items(x)) {
          i = idx;
        } else if (dynamic) {
          // own queue first, then the others: their heads read in one go, an
          // atomic only where items remain (so leaving costs at most one
          // atomic and one read when every queue is drained)
          if (qi == 0) {
            if (pre(x) < items(x)) {
              const int k = pre(x) + atomicAdd(a.queue + x, 1);
              if (k < items(x)) i = k;
            }
            if (i < 0) qi = 1;
          }
          if (i < 0 && qi < 8) {
            int head[8];
#pragma unroll
            for (int y = 0; y < 8; ++y)
              head[y] = __hip_atomic_load(a.queue + y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (; qi < 8; ++qi) {
              q = (x + qi) & 7;
              int hq = head[0];
#pragma unroll
              for (int y = 1; y < 8; ++y) hq = y == q ? head[y] : hq;
              if (pre(q) + hq >= items(q)) continue;
              const int k = pre(q) + atomicAdd(a.queue + q, 1);
              if (k < items(q)) {
                i = k;
                break;
              }
            }
          }
          if (i >= 0) e = *(const int4*)(a.qent + 4 * ((int64_t)q * a.qcap + i / a.G));
        }
        first = false;
        if (i >= 0) {
          s_ent[0] = e.x;  // row
          s_ent[1] = e.y;  // start
          s_ent[2] = e.z;  // length
          s_ent[3] = e.w;  // partial slot
          s_ent[4] = i - (i / a.G) * a.G;
        } else {
          s_ent[0] = -1;
        }
      }
      __syncthreads();
      // the item is the same for the whole workgroup: keep it (and all that
      // derives from it) in scalar registers, as the static launch does
      const int row = __builtin_amdgcn_readfirstlane(s_ent[0]);
      if (row < 0) break;
      const int lo = __builtin_amdgcn_readfirstlane(s_ent[1]);
      const int len = __builtin_amdgcn_readfirstlane(s_ent[2]);
      const int part = __builtin_amdgcn_readfirstlane(s_ent[3]);
      const int hg = __builtin_amdgcn_readfirstlane(s_ent[4]);
      // a row's only task (slot -1) writes the row's final output itself
      decode_item<kMode, false, false, false, false>(a, L, s_bad, zero_row, row, lo, len, hg,
                                                     part < 0 ? 0 : (int64_t)part, 0,
                         part < 0);
    }
  }
}

using stp::device_cus;

// Automatic split count: one workgroup per compute unit at a time, so the
// launch takes ceil(workgroups / CUs) rounds of (fixed per-workgroup cost +
// tiles of its split), and splitting adds the merge launch plus partial
// states for it to read.  Costs in tile units: about four tiles of prologue
// and epilogue per workgroup; the merge three tiles plus about 0.9 tile per
// split per 32 query tokens.  The automatic count keeps a split's ids within
// the LDS list (kIdsMax); a requested count is taken as it is (longer splits
// run with the id ring).  The count depends on the current device's compute
// units.
int32_t choose_splits(int32_t T, int32_t H, int32_t cap, int32_t requested) {
  const int G = (H + kHeadsPerWG - 1) / kHeadsPerWG;
  const int s_min = max(1, (cap + kIdsMax - 1) / kIdsMax);
  if (requested > 0) return requested;
  const int64_t cus = device_cus();
  int best = s_min;
  double best_cost = 1e300;
  for (int S = s_min; S <= max(s_min, 16); ++S) {
    const int64_t wgs = (int64_t)T * G * S;
    const int64_t rounds = (wgs + cus - 1) / cus;
    const int tiles = ((cap + S - 1) / S + kTileRows - 1) / kTileRows;
    const double cost = (double)rounds * (4.0 + tiles) + (S > 1 ? 3.0 + 0.9 * S * T / 32.0 : 0.0);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = S;
    }
  }
  return best;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int launch_decode(int mode, const uint16_t* q, const uint16_t* kv, int64_t kv_rows,
                  const int32_t* row_ids, const int32_t* counts, int32_t cap, int32_t T, int32_t H,
                  float scale, int32_t S, float* o_part, float* m_part, float* l_part,
                  uint16_t* out, float* lse, hipStream_t stream, const uint8_t* kv8 = nullptr) {
  DecodeArgs a{};
  a.q = q;
  a.kv = kv;
  a.kv8 = kv8;
  a.kv_rows = kv_rows;
  a.row_ids = row_ids;
  a.counts = counts;
  a.cap = cap;
  a.T = T;
  a.H = H;
  a.scale_log2 = scale * kLog2e;
  a.S = S;
  a.G = (H + kHeadsPerWG - 1) / kHeadsPerWG;
  a.o_part = o_part;
  a.m_part = m_part;
  a.l_part = l_part;
  a.out = out;
  a.lse = lse;
  const int64_t blocks = (int64_t)8 * ((T + 7) / 8) * S * a.G;
  if (blocks > INT32_MAX) return stp::fail(STP_ERR_INVALID_ARG, "sparse_mla_decode: grid too large");
  // a split longer than the LDS id list takes the id ring (kLong)
  const bool lng = (cap + S - 1) / S > kIdsMax;
  auto go = [&](auto kern) { kern<<<(unsigned)blocks, kThreads, 0, stream>>>(a); };
  if (kv8) {  // fp8_ds_mla rows: the final output or normalised partials
    if (mode == kOutPartialBf16)
      lng ? go(sparse_mla_decode_kernel<kOutPartialBf16, false, true, true>)
          : go(sparse_mla_decode_kernel<kOutPartialBf16, false, true, false>);
    else
      lng ? go(sparse_mla_decode_kernel<kOutFinal, false, true, true>)
          : go(sparse_mla_decode_kernel<kOutFinal, false, true, false>);
  } else if (mode == kOutPartialF32) {
    lng ? go(sparse_mla_decode_kernel<kOutPartialF32, false, false, true>)
        : go(sparse_mla_decode_kernel<kOutPartialF32, false, false, false>);
  } else if (mode == kOutPartialBf16) {
    lng ? go(sparse_mla_decode_kernel<kOutPartialBf16, false, false, true>)
        : go(sparse_mla_decode_kernel<kOutPartialBf16, false, false, false>);
  } else {
    lng ? go(sparse_mla_decode_kernel<kOutFinal, false, false, true>)
        : go(sparse_mla_decode_kernel<kOutFinal, false, false, false>);
  }
  return stp::check_launch("sparse_mla_decode_kernel");
}

// The normalisation's arguments for the launches that carry it.
struct NormCall {
  const int32_t* topk;
  int32_t top_k;
  const int32_t* req_id;
  const int32_t* q_pos;
  const int32_t* block_table;
  int32_t num_reqs, max_blocks, page_size, window, num_sinks;
  int32_t* tok_out;
  int32_t* slot_out;
  int32_t* count_out;
  int32_t* dropped_out;
  int32_t* blk_indptr;
  int32_t* blk_logical;
  int32_t* blk_page;
  uint64_t* blk_mask;
};

// Whether the normalisation fits in the decode launch: splits within the
// LDS id list, the bitmap and the page-table row within ring stages 0 and 1.
bool norm_fits(const NormCall& nc, int32_t cap, int32_t S) {
  const int64_t nwords = max((int64_t)1, ((int64_t)nc.max_blocks * nc.page_size + 63) / 64);
  return (cap + S - 1) / S <= kIdsMax &&
         norm_lds_bytes(nwords, nc.max_blocks, nc.top_k) <= 2 * (int64_t)kTileBytes;
}

// The normalisation of T tokens and the decode of their lists in one launch
// (norm_fits must hold): mode kOutFinal (S = 1) or kOutPartialBf16.  The
// block view is left deferred (blk_indptr holds the per-token state).
int launch_norm_decode(int mode, const NormCall& nc, const uint16_t* q, const uint16_t* kv,
                       int64_t kv_rows, int32_t cap, int32_t T, int32_t H, float scale, int32_t S,
                       void* o_part, float* m_part, float* l_part, uint16_t* out, float* lse,
                       hipStream_t stream) {
  DecodeArgs a{};
  a.q = q;
  a.kv = kv;
  a.kv_rows = kv_rows;
  a.cap = cap;
  a.T = T;
  a.H = H;
  a.scale_log2 = scale * kLog2e;
  a.S = S;
  a.G = (H + kHeadsPerWG - 1) / kHeadsPerWG;
  a.o_part = o_part;
  a.m_part = m_part;
  a.l_part = l_part;
  a.out = out;
  a.lse = lse;
  a.topk = nc.topk;
  a.top_k = nc.top_k;
  a.req_id = nc.req_id;
  a.q_pos = nc.q_pos;
  a.block_table = nc.block_table;
  a.num_reqs = (nc.num_reqs == 0 || nc.max_blocks == 0) ? 0 : nc.num_reqs;
  a.max_blocks = nc.max_blocks;
  a.P = nc.page_size;
  a.window = nc.window;
  a.num_sinks = nc.num_sinks;
  a.nwords_alloc = max(1, (int)(((int64_t)nc.max_blocks * nc.page_size + 63) / 64));
  a.pdiv = ((1ull << 32) + (uint64_t)nc.page_size - 1) / (uint64_t)nc.page_size;
  a.tok_out = nc.tok_out;
  a.slot_out = nc.slot_out;
  a.count_out = nc.count_out;
  a.dropped_out = nc.dropped_out;
  a.blk_indptr = nc.blk_indptr;
  const int64_t blocks = (int64_t)8 * ((T + 7) / 8) * S * a.G;
  if (blocks > INT32_MAX) return stp::fail(STP_ERR_INVALID_ARG, "normalize_and_decode: grid too large");
  if (mode == kOutFinal)
    sparse_mla_decode_kernel<kOutFinal, false, false, false, true>
        <<<(unsigned)blocks, kThreads, 0, stream>>>(a);
  else
    sparse_mla_decode_kernel<kOutPartialBf16, false, false, false, true>
        <<<(unsigned)blocks, kThreads, 0, stream>>>(a);
  return stp::check_launch("sparse_mla_decode_kernel (with normalisation)");
}

int check_common(const uint16_t* q, const uint16_t* kv, int64_t kv_rows, const int32_t* row_ids,
                 int32_t cap, int32_t T, int32_t H, float scale) {
  using stp::fail;
  if (T < 0 || H < 1 || cap < 0 || kv_rows <= 0)
    return fail(STP_ERR_INVALID_ARG, "sparse_mla_decode: bad sizes T=%d H=%d cap=%d kv_rows=%lld",
                T, H, cap, (long long)kv_rows);
  if (!(scale > 0.f) || scale == INFINITY)
    return fail(STP_ERR_INVALID_ARG, "sparse_mla_decode: scale must be positive and finite");
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

namespace {

// The split path of stp_sparse_mla_decode over a workspace of at least
// stp_sparse_mla_decode_workspace() bytes: normalised bf16 partial outputs,
// merged with the partition-combine weights l_s e^(m_s - M) / L.
int decode_split_path(const uint16_t* q, const uint16_t* kv, int64_t kv_rows,
                      const int32_t* row_ids, const int32_t* counts, int32_t cap, int32_t T,
                      int32_t H, float scale, int32_t S, void* workspace, uint16_t* out,
                      float* lse, hipStream_t stream) {
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

// Scratch of stp_sparse_mla_decode_noalloc: the split partials of one call in
// device memory the library owns (each GPU holds its own copy until the
// process ends).  Host code never uses the array's name as an address: its
// device address is looked up once per device (scratch_address) and passed
// to the kernels like a caller's workspace.
constexpr size_t kScratchBytes = (size_t)36 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up on the first
// call on that device (with that device current).
int scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return stp::fail(STP_ERR_HIP, "sparse_mla_decode_noalloc: no current device (or id >= %d)",
                     kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return stp::fail(STP_ERR_HIP, "sparse_mla_decode_noalloc: hipGetSymbolAddress failed: %s",
                       hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return STP_OK;
}

}  // namespace

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
  return decode_split_path(q, kv, kv_rows, row_ids, counts, cap, T, H, scale, S, workspace, out,
                           lse, stream);
}

extern "C" size_t stp_sparse_mla_decode_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" int stp_sparse_mla_decode_noalloc(const uint16_t* q, const uint16_t* kv,
                                             int64_t kv_rows, const int32_t* row_ids,
                                             const int32_t* counts, int32_t cap, int32_t T,
                                             int32_t H, float scale, int32_t num_splits,
                                             uint16_t* out, float* lse, hipStream_t stream) {
  if (int rc = check_common(q, kv, kv_rows, row_ids, cap, T, H, scale)) return rc;
  if (num_splits < 0)
    return stp::fail(STP_ERR_INVALID_ARG, "sparse_mla_decode_noalloc: num_splits < 0");
  if (T == 0) return STP_OK;
  if (!out) return stp::fail(STP_ERR_INVALID_ARG, "sparse_mla_decode_noalloc: null out");
  const int32_t S = choose_splits(T, H, cap, num_splits);
  if (S == 1)
    return launch_decode(kOutFinal, q, kv, kv_rows, row_ids, counts, cap, T, H, scale, 1, nullptr,
                         nullptr, nullptr, out, lse, stream);
  const size_t need = stp_sparse_mla_decode_workspace(T, H, cap, num_splits);
  if (need > kScratchBytes)
    return stp::fail(STP_ERR_WORKSPACE,
                     "sparse_mla_decode_noalloc: %d splits of T=%d H=%d need %zu bytes of scratch, "
                     "more than its %zu (ask for fewer splits or split the batch)",
                     S, T, H, need, kScratchBytes);
  void* ws = nullptr;
  if (int rc = scratch_address(&ws)) return rc;
  return decode_split_path(q, kv, kv_rows, row_ids, counts, cap, T, H, scale, S, ws, out, lse,
                           stream);
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
  if (T == 0) return STP_OK;
  if (!o_part || !m_part || !l_part)
    return stp::fail(STP_ERR_INVALID_ARG, "sparse_mla_decode_partial: null output");
  return launch_decode(kOutPartialF32, q, kv, kv_rows, row_ids, counts, cap, T, H, scale, num_splits,
                       o_part, m_part, l_part, nullptr, nullptr, stream);
}

extern "C" int stp_sparse_mla_decode_partial_normalized(
    const uint16_t* q, const uint16_t* kv, int64_t kv_rows, const int32_t* row_ids,
    const int32_t* counts, int32_t cap, int32_t T, int32_t H, float scale, int32_t num_splits,
    uint16_t* o_norm, float* m_part, float* l_part, hipStream_t stream) {
  if (int rc = check_common(q, kv, kv_rows, row_ids, cap, T, H, scale)) return rc;
  if (num_splits < 1)
    return stp::fail(STP_ERR_INVALID_ARG,
                     "sparse_mla_decode_partial_normalized: num_splits must be >= 1");
  if (T == 0) return STP_OK;
  if (!o_norm || !m_part || !l_part)
    return stp::fail(STP_ERR_INVALID_ARG, "sparse_mla_decode_partial_normalized: null output");
  return launch_decode(kOutPartialBf16, q, kv, kv_rows, row_ids, counts, cap, T, H, scale,
                       num_splits, (float*)o_norm, m_part, l_part, nullptr, nullptr, stream);
}

// Normalisation and decode in one call.  The decode launch builds each
// token's list itself when norm_fits holds; otherwise the normalisation runs
// first as its own launch.  The block view (when asked for) is completed by
// the merge launch, or by its own launch after a single-pass decode.
namespace {

int check_norm_call(const char* what, const NormCall& nc, int32_t T, int32_t cap) {
  return stp::check_normalize_args(what, nc.topk, nc.top_k, nc.req_id, nc.q_pos, T,
                                   nc.block_table, nc.num_reqs, nc.max_blocks, nc.page_size,
                                   nc.window, nc.num_sinks, cap, nc.tok_out, nc.slot_out,
                                   nc.count_out);
}

// Normalisation (block view deferred) and a decode of mode kOutFinal or
// kOutPartialBf16 over the lists it writes: one launch or two.
int norm_then_decode(int mode, const NormCall& nc, const uint16_t* q, const uint16_t* kv,
                     int64_t kv_rows, int32_t cap, int32_t T, int32_t H, float scale, int32_t S,
                     void* o_part, float* m_part, float* l_part, uint16_t* out, float* lse,
                     hipStream_t stream) {
  if (norm_fits(nc, cap, S))
    return launch_norm_decode(mode, nc, q, kv, kv_rows, cap, T, H, scale, S, o_part, m_part,
                              l_part, out, lse, stream);
  if (int rc = stp::normalize_deferred(nc.topk, nc.top_k, nc.req_id, nc.q_pos, T, nc.block_table,
                                       nc.num_reqs, nc.max_blocks, nc.page_size, nc.window,
                                       nc.num_sinks, cap, nc.tok_out, nc.slot_out, nc.count_out,
                                       nc.dropped_out, nc.blk_indptr, stream))
    return rc;
  return launch_decode(mode, q, kv, kv_rows, nc.slot_out, nc.count_out, cap, T, H, scale, S,
                       (float*)o_part, m_part, l_part, out, lse, stream);
}

stp::BlockViewPass block_view_pass(const NormCall& nc, int32_t cap) {
  return {nc.tok_out,    nc.slot_out,    nc.req_id,   nc.q_pos,      nc.block_table,
          nc.num_reqs,   nc.max_blocks,  nc.page_size, cap,          nc.blk_indptr,
          nc.blk_logical, nc.blk_page,   nc.blk_mask};
}

}  // namespace

extern "C" int stp_normalize_and_decode(
    const int32_t* topk, int32_t top_k, const int32_t* req_id, const int32_t* q_pos, int32_t T,
    const int32_t* block_table, int32_t num_reqs, int32_t max_blocks, int32_t page_size,
    int32_t window, int32_t num_sinks, int32_t cap, int32_t* tok_out, int32_t* slot_out,
    int32_t* count_out, int32_t* dropped_out, int32_t* blk_indptr, int32_t* blk_logical,
    int32_t* blk_page, uint64_t* blk_mask, const uint16_t* q, const uint16_t* kv,
    int64_t kv_rows, int32_t H, float scale, int32_t num_splits, void* workspace,
    size_t workspace_bytes, uint16_t* out, float* lse, hipStream_t stream) {
  using stp::fail;
  const NormCall nc{topk,       top_k,     req_id,    q_pos,     block_table, num_reqs,
                    max_blocks, page_size, window,    num_sinks, tok_out,     slot_out,
                    count_out,  dropped_out, blk_indptr, blk_logical, blk_page, blk_mask};
  if (int rc = check_norm_call("normalize_and_decode", nc, T, cap)) return rc;
  if (int rc = check_common(q, kv, kv_rows, slot_out, cap, T, H, scale)) return rc;
  if (num_splits < 0) return fail(STP_ERR_INVALID_ARG, "normalize_and_decode: num_splits < 0");
  if (T == 0) return STP_OK;
  if (!out) return fail(STP_ERR_INVALID_ARG, "normalize_and_decode: null out");
  if (blk_indptr && (!blk_logical || !blk_page || !blk_mask))
    return fail(STP_ERR_INVALID_ARG, "normalize_and_decode: block view arrays missing");
  const int32_t S = choose_splits(T, H, cap, num_splits);
  if (S == 1) {
    if (int rc = norm_then_decode(kOutFinal, nc, q, kv, kv_rows, cap, T, H, scale, 1, nullptr,
                                  nullptr, nullptr, out, lse, stream))
      return rc;
    return blk_indptr ? stp::launch_block_fill(block_view_pass(nc, cap), T, stream) : STP_OK;
  }
  const size_t need = stp_sparse_mla_decode_workspace(T, H, cap, num_splits);
  if (!workspace || workspace_bytes < need)
    return fail(STP_ERR_WORKSPACE, "normalize_and_decode: workspace of %zu bytes needed, %zu given",
                need, workspace_bytes);
  const size_t n = (size_t)T * S * H;
  char* ws = (char*)workspace;
  uint16_t* o_norm = (uint16_t*)ws;
  float* m_part = (float*)(ws + align256(n * kDV * 2));
  float* l_part = (float*)(ws + align256(n * kDV * 2) + align256(n * 4));
  if (int rc = norm_then_decode(kOutPartialBf16, nc, q, kv, kv_rows, cap, T, H, scale, S, o_norm,
                                m_part, l_part, nullptr, nullptr, stream))
    return rc;
  if (blk_indptr)
    return stp::launch_merge_block_view(o_norm, m_part, l_part, T, S, H, kDV, out, lse,
                                        block_view_pass(nc, cap), stream);
  return stp::launch_merge_normalized(o_norm, m_part, l_part, T, S, H, kDV, out, lse, stream);
}

extern "C" int stp_normalize_and_decode_partial_normalized(
    const int32_t* topk, int32_t top_k, const int32_t* req_id, const int32_t* q_pos, int32_t T,
    const int32_t* block_table, int32_t num_reqs, int32_t max_blocks, int32_t page_size,
    int32_t window, int32_t num_sinks, int32_t cap, int32_t* tok_out, int32_t* slot_out,
    int32_t* count_out, int32_t* dropped_out, int32_t* blk_indptr, const uint16_t* q,
    const uint16_t* kv, int64_t kv_rows, int32_t H, float scale, int32_t num_splits,
    uint16_t* o_norm, float* m_part, float* l_part, hipStream_t stream) {
  using stp::fail;
  const NormCall nc{topk,       top_k,     req_id,    q_pos,     block_table, num_reqs,
                    max_blocks, page_size, window,    num_sinks, tok_out,     slot_out,
                    count_out,  dropped_out, blk_indptr, nullptr, nullptr,    nullptr};
  if (int rc = check_norm_call("normalize_and_decode_partial_normalized", nc, T, cap)) return rc;
  if (int rc = check_common(q, kv, kv_rows, slot_out, cap, T, H, scale)) return rc;
  if (num_splits < 1)
    return fail(STP_ERR_INVALID_ARG,
                "normalize_and_decode_partial_normalized: num_splits must be >= 1");
  if (T == 0) return STP_OK;
  if (!o_norm || !m_part || !l_part)
    return fail(STP_ERR_INVALID_ARG, "normalize_and_decode_partial_normalized: null output");
  return norm_then_decode(kOutPartialBf16, nc, q, kv, kv_rows, cap, T, H, scale, num_splits,
                          o_norm, m_part, l_part, nullptr, nullptr, stream);
}

// fp8_ds_mla rows: the same launch and split path, the rows dequantised on
// their way into the ring.
extern "C" int32_t stp_sparse_mla_decode_fp8_splits(int32_t T, int32_t H, int32_t cap,
                                                    int32_t num_splits) {
  return stp_sparse_mla_decode_splits(T, H, cap, num_splits);
}

extern "C" size_t stp_sparse_mla_decode_fp8_workspace(int32_t T, int32_t H, int32_t cap,
                                                      int32_t num_splits) {
  return stp_sparse_mla_decode_workspace(T, H, cap, num_splits);
}

extern "C" int stp_sparse_mla_decode_fp8(const uint16_t* q, const uint8_t* kv, int64_t kv_rows,
                                         const int32_t* row_ids, const int32_t* counts,
                                         int32_t cap, int32_t T, int32_t H, float scale,
                                         int32_t num_splits, void* workspace,
                                         size_t workspace_bytes, uint16_t* out, float* lse,
                                         hipStream_t stream) {
  using stp::fail;
  if (int rc = check_common(q, (const uint16_t*)kv, kv_rows, row_ids, cap, T, H, scale)) return rc;
  if (num_splits < 0)
    return fail(STP_ERR_INVALID_ARG, "sparse_mla_decode_fp8: num_splits < 0");
  if (T == 0) return STP_OK;
  if (!out) return fail(STP_ERR_INVALID_ARG, "sparse_mla_decode_fp8: null out");
  if ((uintptr_t)kv % 16 != 0)
    return fail(STP_ERR_INVALID_ARG, "sparse_mla_decode_fp8: kv must be 16-byte aligned");
  const int32_t S = choose_splits(T, H, cap, num_splits);
  if (S == 1)
    return launch_decode(kOutFinal, q, nullptr, kv_rows, row_ids, counts, cap, T, H, scale, 1,
                         nullptr, nullptr, nullptr, out, lse, stream, kv);
  const size_t need = stp_sparse_mla_decode_workspace(T, H, cap, num_splits);
  if (!workspace || workspace_bytes < need)
    return fail(STP_ERR_WORKSPACE, "sparse_mla_decode_fp8: workspace of %zu bytes needed, %zu given",
                need, workspace_bytes);
  const size_t n = (size_t)T * S * H;
  char* ws = (char*)workspace;
  uint16_t* o_norm = (uint16_t*)ws;
  float* m_part = (float*)(ws + align256(n * kDV * 2));
  float* l_part = (float*)(ws + align256(n * kDV * 2) + align256(n * 4));
  if (int rc = launch_decode(kOutPartialBf16, q, nullptr, kv_rows, row_ids, counts, cap, T, H,
                             scale, S, (float*)o_norm, m_part, l_part, nullptr, nullptr, stream, kv))
    return rc;
  return stp::launch_merge_normalized(o_norm, m_part, l_part, T, S, H, kDV, out, lse, stream);
}

namespace stp {

int decode_ids_max() { return kIdsMax; }

int decode_head_groups(int32_t H) { return (H + kHeadsPerWG - 1) / kHeadsPerWG; }

int decode_choose_splits(int32_t T, int32_t H, int32_t cap) { return choose_splits(T, H, cap, 0); }

int launch_decode_tasks(const uint16_t* q, const uint16_t* kv, int64_t kv_rows,
                        const int32_t* row_ids, int32_t cap, int32_t T, int32_t H, float scale,
                        const int32_t* qcount, const int32_t* qent, int32_t qcap, int32_t* queue,
                        int32_t grid, uint16_t* o_norm, float* m_part, float* l_part,
                        uint16_t* out, float* lse, hipStream_t stream) {
  DecodeArgs a{};
  a.q = q;
  a.kv = kv;
  a.kv_rows = kv_rows;
  a.row_ids = row_ids;
  a.cap = cap;
  a.T = T;
  a.H = H;
  a.scale_log2 = scale * kLog2e;
  a.S = 1;
  a.G = decode_head_groups(H);
  a.o_part = o_norm;
  a.m_part = m_part;
  a.l_part = l_part;
  a.out = out;
  a.lse = lse;
  a.qcount = qcount;
  a.qent = qent;
  a.qcap = qcap;
  a.queue = queue;
  sparse_mla_decode_kernel<kOutPartialBf16, true><<<(unsigned)grid, kThreads, 0, stream>>>(a);
  return check_launch("sparse_mla_decode_kernel (task queue)");
}

}  // namespace stp
