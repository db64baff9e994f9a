// Internal helpers shared by the HIP sources of libstp (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "stp.h"

namespace stp {

// Records the message returned by stp_last_error() and passes the status through.
int fail(int status, const char* fmt, ...);

// Checks the launch that was just enqueued.
int check_launch(const char* what);

// Compute units of the current device (queried once per device; 256 if the
// query fails).
int device_cus();

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Inclusive prefix sum across the 64 lanes of a wave with DPP row moves
// (no LDS round trips): shifts by 1, 2, 4, 8 inside each 16-lane row, then
// the row totals broadcast forward (row_bcast:15 into rows 1 and 3,
// row_bcast:31 into rows 2 and 3).
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Sum over the wave, in every lane.
__device__ __forceinline__ int wave_sum(int x) {
  return __builtin_amdgcn_readlane(wave_incl_sum(x), 63);
}

// Block-wide exclusive scan of one int per thread over a workgroup of kW
// waves; `scratch` holds kW ints.  Returns the exclusive prefix and writes
// the block total.
template <int kW>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_incl_sum(v);
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const int sw = scratch[w];
    off += w < wave ? sw : 0;
    tot += sw;
  }
  __syncthreads();
  *total = tot;
  return off + x - v;
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), unrolled.
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that orders LDS only (__syncthreads() would also wait
// for every tile load in flight).  The signal fences stop the compiler from
// moving memory accesses across it; the hardware wait is lgkmcnt(0) alone.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left at their maximum
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// max / sum of x over the lane pair (l, l ^ 32), identical in both lanes.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): global address vaddr + offset, LDS address
// m0 + offset + 16 * lane -- the immediate offset applies to both sides.
// Issued from inline asm so that the compiler's wait-count pass does not
// track these loads: the tile ring waits for them explicitly (wait_vmcnt),
// and the compiler would otherwise drain the ring before every LDS access it
// cannot prove disjoint from the loads in flight.
template <int kOffset>
__device__ __forceinline__ void load_lds_16(const void* gptr, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off offset:%1" ::"v"(gptr), "n"(kOffset),
               "{m0}"(lds_addr));
}

typedef float floatx16 __attribute__((ext_vector_type(16)));

// acc *= f for an MFMA accumulator kept in AGPRs.  Written as inline asm on
// AGPR operands so that the compiler keeps the accumulators in AGPRs (a plain
// VALU multiply makes it move all 256 of them through VGPRs).
__device__ __forceinline__ void scale_acc(floatx16& acc, float f) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float t;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "v_mul_f32 %1, %1, %2\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(acc[r]), "=&v"(t)
        : "v"(f));
  }
}

// Two fp32 values -> a packed bf16 pair (a in the low half), round to
// nearest even, by the hardware conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Split-KV merge launchers (merge.hip).  launch_merge takes un-normalised
// fp32 numerators; launch_merge_normalized takes bf16 o_s / l_s, the form the
// decode entry point's split path writes.
int launch_merge(const float* o_part, const float* m_part, const float* l_part, int T, int S,
                 int H, int dv, uint16_t* out, float* lse, hipStream_t stream);
int launch_merge_normalized(const uint16_t* o_norm, const float* m_part, const float* l_part, int T,
                            int S, int H, int dv, uint16_t* out, float* lse, hipStream_t stream);

// Sparse MLA decode over a plan's queues (decode.hip): a persistent grid of
// `grid` workgroups takes (entry, head group) items from eight queues (the
// first qcount[x] entries of segment x, qcap entries from qent + 4 qcap x,
// each (row, start, length, slot), claimed with the queue heads) and writes
// normalised bf16 partials to their slots, or, for slot -1 (a task that
// covers its whole row), the row's final out and lse.
int launch_decode_tasks(const uint16_t* q, const uint16_t* kv, int64_t kv_rows,
                        const int32_t* row_ids, int32_t cap, int32_t T, int32_t H, float scale,
                        const int32_t* qcount, const int32_t* qent, int32_t qcap, int32_t* queue,
                        int32_t grid, uint16_t* o_norm, float* m_part, float* l_part,
                        uint16_t* out, float* lse, hipStream_t stream);
int decode_ids_max();                 // candidate positions one work item may hold
int decode_head_groups(int32_t H);    // work items per task
int decode_choose_splits(int32_t T, int32_t H, int32_t cap);

}  // namespace stp
