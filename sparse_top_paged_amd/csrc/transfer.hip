// Staged bulk host <-> device KV transfer on gfx950.
//
// "[HiCache] TMA-staged host<->device KV transfer kernel (sm_90+)",
// Motivation (a cached prefix is brought back from the pinned host pool into
// the device pool layer by layer while the forward pass runs; what matters
// is the bytes per second per compute unit taken from it, and bandwidth =
// bytes in flight / round trip) and Modifications 1, 3 and 5 (deep loads
// with no registers holding data, index prefetch, any row size that is a
// multiple of 16 B).
//
// What it computes: for every buffer b and list position i,
//   dst[b] + dst_idx[i] * dst_stride  <-  src[b] + src_idx[i] * src_stride,
// row_bytes bytes each; a row whose source or destination index falls
// outside its pool is skipped.  Either side may be pinned host memory (its
// device-visible address) or device memory.
//
// Design.  gfx950 has no TMA; the counterpart of a bulk copy into shared
// memory is global_load_lds_dwordx4, which moves 16 B per lane straight into
// LDS.  A 256-thread workgroup keeps a ring of three 32 KiB stages: two
// loader waves keep two stages in flight (64 KiB) with no VGPR holding data,
// two storer waves write the third out.  (A fourth stage, 96 KiB in flight,
// measured the same: about 12.8 GB/s of host reads per workgroup, a limit of
// the compute unit's outstanding requests rather than of the ring.)  Loads and stores sit on different
// waves, so a loader's wait counts only its own loads, which complete in
// order.  The work of a call is the flat list of (buffer, position) rows cut
// into equal contiguous ranges, one per workgroup; a range is processed in
// chunks of up to 4096 rows of one buffer whose validated row indices are
// staged in LDS first (no index load then sits between the tile loads, whose
// completion the compiler cannot see).  Within a chunk the rows are a flat
// sequence of 16-B units, 2048 per stage: lane l of loader (or storer) wave w
// takes unit 128 k + 64 w + l of a stage (k < 16), whatever row it falls in,
// so page runs and scattered rows cost the same instructions and one load
// instruction moves 1 KiB of consecutive units.  A loader lane issues every
// load (a skipped unit loads the zero row), so its count per stage is fixed.

#include <algorithm>

#include "stp_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnitsPerStage = 2048;  // 16-B units: 32 KiB
constexpr int kStages = 3;
constexpr int kPerLane = kUnitsPerStage / 128;  // units per loader / storer lane and stage
constexpr int kChunkRows = 4096;      // row indices staged in LDS at a time
constexpr int kMaxBufs = 32;

typedef unsigned int uintx4 __attribute__((ext_vector_type(4)));

struct TransferArgs {
  const uint8_t* src[kMaxBufs];
  uint8_t* dst[kMaxBufs];
  int nbufs;
  int row_units;  // row_bytes / 16
  float inv_row_units;
  int64_t src_stride, dst_stride;
  int64_t src_rows, dst_rows;
  const int32_t* src_idx;
  const int32_t* dst_idx;
  int n;
  int64_t total_rows;  // nbufs * n
};

__device__ __attribute__((aligned(16))) uint8_t g_transfer_zero[16] = {};

__global__ __launch_bounds__(kThreads) void kv_transfer_kernel(TransferArgs a) {
  __shared__ __attribute__((aligned(1024))) char s_ring[kStages * kUnitsPerStage * 16];
  __shared__ int32_t s_src[kChunkRows];
  __shared__ int32_t s_dst[kChunkRows];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool loader = wave < 2;
  const int w2 = wave & 1;
  const int64_t r0 = a.total_rows * blockIdx.x / gridDim.x;
  const int64_t r1 = a.total_rows * (blockIdx.x + 1) / gridDim.x;
  const uint8_t* zero = g_transfer_zero;
  asm volatile("" : "+s"(zero));
  const uint32_t ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)s_ring;

  for (int64_t c0 = r0; c0 < r1;) {
    // a chunk: rows of one buffer, at most kChunkRows of them
    const int b = (int)(c0 / a.n);
    const int p0 = (int)(c0 - (int64_t)b * a.n);
    const int64_t left = r1 - c0;
    int rows = left < kChunkRows ? (int)left : kChunkRows;
    rows = rows < a.n - p0 ? rows : a.n - p0;
    __syncthreads();  // the previous chunk is done with its indices and ring
    for (int i = tid; i < rows; i += kThreads) {
      const int32_t si = a.src_idx[p0 + i], di = a.dst_idx[p0 + i];
      const bool ok = si >= 0 && si < a.src_rows && di >= 0 && di < a.dst_rows;
      s_src[i] = ok ? si : -1;
      s_dst[i] = ok ? di : -1;
    }
    __syncthreads();
    const uint8_t* src = a.src[b];
    uint8_t* dst = a.dst[b];
    const int units = rows * a.row_units;
    const int nst = (units + kUnitsPerStage - 1) / kUnitsPerStage;

    // unit u of the chunk: row u / row_units, 16-B column u % row_units (u
    // < 2^24, so the float quotient is off by at most one)
    auto row_of = [&](int u) {
      int r = (int)((float)u * a.inv_row_units);
      r -= r * a.row_units > u ? 1 : 0;
      r += (r + 1) * a.row_units <= u ? 1 : 0;
      return r;
    };
    auto load_stage = [&](int s) {
      const uint32_t base = ring + (s % kStages) * (kUnitsPerStage * 16);
#pragma unroll
      for (int k = 0; k < kPerLane; ++k) {
        const int u = s * kUnitsPerStage + k * 128 + w2 * 64 + lane;
        const uint8_t* p = zero;
        if (u < units) {
          const int r = row_of(u), c = u - r * a.row_units;
          const int32_t si = s_src[r];
          if (si >= 0) p = src + (int64_t)si * a.src_stride + 16 * c;
        }
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(base + (k * 128 + w2 * 64) * 16);
        stp::load_lds_16<0>(p, m0);
      }
    };
    auto store_stage = [&](int s) {
      const __attribute__((address_space(3))) char* base =
          (const __attribute__((address_space(3))) char*)s_ring + (s % kStages) * (kUnitsPerStage * 16);
#pragma unroll
      for (int k = 0; k < kPerLane; ++k) {
        const int u = s * kUnitsPerStage + k * 128 + w2 * 64 + lane;
        const uintx4 v = *(const __attribute__((address_space(3))) uintx4*)(
            base + (k * 128 + w2 * 64 + lane) * 16);
        if (u < units) {
          const int r = row_of(u), c = u - r * a.row_units;
          const int32_t di = s_dst[r];
          if (di >= 0) *(uintx4*)(dst + (int64_t)di * a.dst_stride + 16 * c) = v;
        }
      }
    };

    // Ring: stage s is loaded in iteration s - (S - 1) (the prologue loads
    // 0 .. S - 2) into slot s % S and stored in iteration s.  A loader wave
    // issues, in order, L(0) .. L(S - 2) and then L(i + S - 1) per iteration
    // i, kPerLane loads each, so in iteration i at most the S - 2 stages after
    // L(i) may still be in flight once L(i) has landed.  The LDS-only barrier
    // then hands stage i to the storers; it also follows their reads of stage
    // i - 1, whose slot L(i + S - 1) refills.
    if (loader)
      for (int s = 0; s < kStages - 1 && s < nst; ++s) load_stage(s);
    for (int i = 0; i < nst; ++i) {
      if (loader) {
        const int newer = min(kStages - 2, nst - 1 - i);
        if (newer >= 2)
          stp::wait_vmcnt<2 * kPerLane>();
        else if (newer == 1)
          stp::wait_vmcnt<kPerLane>();
        else
          stp::wait_vmcnt<0>();
      }
      stp::lds_barrier();
      if (loader) {
        if (i + kStages - 1 < nst) load_stage(i + kStages - 1);
      } else {
        store_stage(i);
      }
    }
    c0 += rows;
  }
}

}  // namespace

extern "C" int stp_kv_transfer(const void* const* src_bufs, void* const* dst_bufs, int32_t num_bufs,
                               int64_t row_bytes, int64_t src_stride, int64_t src_rows,
                               int64_t dst_stride, int64_t dst_rows, const int32_t* src_idx,
                               const int32_t* dst_idx, int32_t n, int32_t num_blocks,
                               hipStream_t stream) {
  using stp::fail;
  if (num_bufs < 1 || num_bufs > kMaxBufs)
    return fail(STP_ERR_INVALID_ARG, "kv_transfer: num_bufs %d outside [1, %d]", num_bufs, kMaxBufs);
  if (row_bytes <= 0 || row_bytes % 16 != 0 || row_bytes > 65536)
    return fail(STP_ERR_INVALID_ARG, "kv_transfer: row_bytes must be a multiple of 16 in [16, 65536]");
  if (src_stride < row_bytes || dst_stride < row_bytes || src_stride % 16 || dst_stride % 16)
    return fail(STP_ERR_INVALID_ARG, "kv_transfer: strides must be multiples of 16, >= row_bytes");
  if (src_rows < 0 || dst_rows < 0 || n < 0 || num_blocks < 1)
    return fail(STP_ERR_INVALID_ARG, "kv_transfer: negative size or num_blocks < 1");
  if ((int64_t)kChunkRows * (row_bytes / 16) > INT32_MAX)
    return fail(STP_ERR_INVALID_ARG, "kv_transfer: row too large");
  if (n == 0) return STP_OK;
  if (!src_bufs || !dst_bufs || !src_idx || !dst_idx)
    return fail(STP_ERR_INVALID_ARG, "kv_transfer: null pointer");
  TransferArgs a{};
  for (int b = 0; b < num_bufs; ++b) {
    if (!src_bufs[b] || !dst_bufs[b]) return fail(STP_ERR_INVALID_ARG, "kv_transfer: null buffer");
    a.src[b] = (const uint8_t*)src_bufs[b];
    a.dst[b] = (uint8_t*)dst_bufs[b];
  }
  a.nbufs = num_bufs;
  a.row_units = (int)(row_bytes / 16);
  a.inv_row_units = 1.0f / (float)a.row_units;
  a.src_stride = src_stride;
  a.dst_stride = dst_stride;
  a.src_rows = src_rows;
  a.dst_rows = dst_rows;
  a.src_idx = src_idx;
  a.dst_idx = dst_idx;
  a.n = n;
  a.total_rows = (int64_t)num_bufs * n;
  const int64_t blocks = std::min<int64_t>(num_blocks, a.total_rows);
  kv_transfer_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(a);
  return stp::check_launch("kv_transfer_kernel");
}
