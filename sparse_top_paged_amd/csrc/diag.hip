// Diagnostics: bandwidth ceilings of the decode's row gather and of a plain
// streaming read.
//
// "5.1.1 · 从索引到 Kernel" §2 and eq. (8)-(9): at decode the time of the
// sparse attention step is set by the bytes of the candidate rows it has to
// bring in, which are scattered across the cache by slot id.  The gather
// kernel reads exactly those rows, with the work split and the XCD placement
// of the decode kernel, and does nothing else, so its rate is the most the
// decode can reach for the same access pattern on this GPU; the streaming
// read gives what HBM delivers to sequential reads on the same device (§6.1:
// rates are set against what the hardware sustains, not nominal peaks).
//
// Gather grid: per query token, `parts` contiguous ranges of its candidate
// list (split as the decode splits them), each read by `replicas` workgroups
// (the decode reads every range once per group of query heads).  All
// workgroups of a token get block ids of one residue mod 8, as in the decode.
// A workgroup stages its ids in LDS; each of its four waves then streams its
// own groups of 8 rows (groups w, w + 4, ...) through a ring in LDS with
// global_load_lds_dwordx4 -- one instruction per 128-byte line of the 8
// rows, each run of 8 lanes on one row's line, the decode's tile layout --
// keeping a fixed number of groups in flight, and xor-folds every word it
// loaded once its group has landed.  A lane only reads back the 16 bytes it
// loaded itself, so the waves never wait for each other.  Row sizes whose
// line count has no ring variant use a register pipeline (eight 16-byte
// loads per thread in flight).

#include "stp_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kIdsMax = 4096;
constexpr int kDepth = 8;        // register pipeline: loads in flight per thread
constexpr int kRingLines = 27;   // ring: 128-byte-line instructions in flight per wave

typedef unsigned int uintx4 __attribute__((ext_vector_type(4)));

struct GatherArgs {
  const uint8_t* rows;
  int64_t num_rows;
  int row_bytes;  // multiple of 16
  const int32_t* row_ids;
  const int32_t* counts;
  int cap, T, parts, replicas;
  uint32_t* checksum;
};

// This workgroup's token and candidate range (the decode's split of it), the
// ids staged in LDS (-1 for invalid ones).  Returns false past the last token.
__device__ __forceinline__ bool stage_range(const GatherArgs& a, int32_t* s_ids, int* len_out) {
  const int bid = blockIdx.x;
  const int xk = bid >> 3;
  const int per_token = a.parts * a.replicas;
  const int t = (xk / per_token) * 8 + (bid & 7);
  const int part = (xk % per_token) / a.replicas;
  if (t >= a.T) return false;
  int n = a.counts ? a.counts[t] : a.cap;
  n = min(max(n, 0), a.cap);
  const int chunk = (n + a.parts - 1) / a.parts;
  const int lo = min(n, part * chunk);
  const int len = min(n, lo + chunk) - lo;  // <= kIdsMax (checked on the host)
  for (int i = threadIdx.x; i < len; i += kThreads) {
    const int32_t id = a.row_ids[(int64_t)t * a.cap + lo + i];
    s_ids[i] = (id >= 0 && id < a.num_rows) ? id : -1;
  }
  *len_out = len;
  return true;
}

__device__ __forceinline__ void write_checksum(const GatherArgs& a, uint32_t acc) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t s_acc[kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s_acc[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) a.checksum[blockIdx.x] = s_acc[0] ^ s_acc[1] ^ s_acc[2] ^ s_acc[3];
}

// Ring variant for rows of kLines 128-byte lines (the last one possibly
// partial): kDepthG = kRingLines / kLines groups of 8 rows in flight per
// wave, kDepthG * kLines KiB of LDS per wave.
template <int kLines>
__global__ __launch_bounds__(kThreads) void row_gather_ring_kernel(GatherArgs a) {
  constexpr int kDepthG = kRingLines / kLines;
  static_assert(kDepthG >= 2, "at least two groups in flight");
  __shared__ int32_t s_ids[kIdsMax];
  __shared__ __attribute__((aligned(16))) char s_ring[4 * kDepthG * kLines * 1024];
  int len = 0;
  if (!stage_range(a, s_ids, &len)) return;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cpr = a.row_bytes >> 4;                 // 16-byte chunks per row
  const int groups = (len + 7) / 8;
  const int mine = groups > wave ? (groups - wave + 3) / 4 : 0;  // groups wave, wave + 4, ...
  const int rl = lane >> 3, cl = lane & 7;
  const uint32_t ring = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(s_ring + wave * kDepthG * kLines * 1024));
  // group k of this wave (k < mine) into ring slot k % kDepthG; for rows
  // past the range, invalid ids and chunks beyond the row the lane reads the
  // row's first chunk or row 0, in bounds, and its words are left out of the
  // fold
  auto issue = [&](int k) {
    const int r = (wave + 4 * k) * 8 + rl;
    const int id = r < len ? s_ids[r] : -1;
    const uint8_t* row = a.rows + (int64_t)max(id, 0) * a.row_bytes;
    const uint32_t dst = ring + (uint32_t)((k % kDepthG) * kLines * 1024);
#pragma unroll
    for (int l = 0; l < kLines; ++l) {
      const int c = 8 * l + cl;
      const uint8_t* src = row + (c < cpr ? c : 0) * 16;
      asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(dst + l * 1024));
    }
  };
  auto fold = [&](int k) {
    const int r = (wave + 4 * k) * 8 + rl;
    const bool valid_row = k < mine && r < len && s_ids[r] >= 0;
    const __attribute__((address_space(3))) uintx4* p =
        (const __attribute__((address_space(3))) uintx4*)(uintptr_t)(ring + (k % kDepthG) * kLines * 1024 + lane * 16);
    uint32_t acc = 0;
#pragma unroll
    for (int l = 0; l < kLines; ++l) {
      const uintx4 v = p[l * 64];
      const bool use = valid_row && 8 * l + cl < cpr;
      acc ^= use ? (v.x ^ v.y ^ v.z ^ v.w) : 0u;
    }
    return acc;
  };
  uint32_t acc = 0;
#pragma unroll
  for (int k = 0; k < kDepthG; ++k)
    if (k < mine) issue(k);
  for (int k = 0; k < mine; ++k) {
    // group k has landed: with groups k + 1 .. k + kDepthG - 1 all issued,
    // they may stay in flight; near the end everything is drained
    if (k + kDepthG <= mine)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kDepthG - 1) * kLines) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    acc ^= fold(k);
    if (k + kDepthG < mine) issue(k + kDepthG);  // refills slot k % kDepthG
  }
  write_checksum(a, acc);
}

__global__ __launch_bounds__(kThreads) void row_gather_kernel(GatherArgs a) {
  __shared__ int32_t s_ids[kIdsMax];
  int len = 0;
  if (!stage_range(a, s_ids, &len)) return;
  __syncthreads();

  // Wave instruction s covers 8 rows x one 128-byte line (group s / lines,
  // line s % lines): each run of 8 lanes reads one row's line.  Wave w takes
  // instructions w, w + 4, w + 8, ... and keeps kDepth of them in flight,
  // refilling each register set right after folding it.
  const int cpr = a.row_bytes / 16;          // chunks per row
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lines = (cpr + 7) / 8;           // 128-byte lines per row
  const int groups = (len + 7) / 8;          // groups of 8 rows
  const int steps = groups * lines;          // wave instructions for all rows
  const int mine = steps > wave ? (steps - wave + 3) / 4 : 0;
  // Every lane loads (branch-free, so the compiler keeps kDepth loads in
  // flight): entries past the end or with an invalid id read row 0 or the
  // last valid instruction again, and their words are masked out of the fold.
  auto load = [&](int k, bool& use) -> uintx4 {
    const int kk = min(k, mine - 1);
    const int s = wave + 4 * kk;
    const int g = s / lines, l = s - g * lines;
    const int r = g * 8 + (lane >> 3);
    const int c = l * 8 + (lane & 7);
    const int id = s_ids[min(r, len - 1)];
    use = k < mine && r < len && c < cpr && id >= 0;
    const int64_t off = (int64_t)max(id, 0) * a.row_bytes + (int64_t)min(c, cpr - 1) * 16;
    return *(const uintx4*)(a.rows + off);
  };
  uint32_t acc = 0;
  if (mine > 0) {
    uintx4 v[kDepth];
    bool use[kDepth];
#pragma unroll
    for (int u = 0; u < kDepth; ++u) v[u] = load(u, use[u]);
    for (int k0 = 0; k0 < mine; k0 += kDepth) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        const uint32_t w = v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        acc ^= use[u] ? w : 0u;
        v[u] = load(k0 + kDepth + u, use[u]);
        __builtin_amdgcn_sched_barrier(0);  // keep fold u and its refill together
      }
    }
  }
  write_checksum(a, acc);
}

// Streaming read of [0, n16) 16-byte units: grid-stride, four independent
// loads in flight per thread, one xor per workgroup.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uintx4* __restrict__ src,
                                                              int64_t n16,
                                                              uint32_t* __restrict__ checksum) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uintx4 a0 = src[i], a1 = src[i + stride], a2 = src[i + 2 * stride],
                 a3 = src[i + 3 * stride];
    acc ^= a0.x ^ a0.y ^ a0.z ^ a0.w ^ a1.x ^ a1.y ^ a1.z ^ a1.w ^ a2.x ^ a2.y ^ a2.z ^ a2.w ^
           a3.x ^ a3.y ^ a3.z ^ a3.w;
  }
  for (; i < n16; i += stride) {
    const uintx4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t s_acc[kThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s_acc[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) checksum[blockIdx.x] = s_acc[0] ^ s_acc[1] ^ s_acc[2] ^ s_acc[3];
}

}  // namespace

extern "C" int32_t stp_row_gather_blocks(int32_t T, int32_t parts, int32_t replicas) {
  if (T < 0 || parts < 1 || replicas < 1) return 0;
  const int64_t b = (int64_t)8 * ((T + 7) / 8) * parts * replicas;
  return b > INT32_MAX ? 0 : (int32_t)b;
}

extern "C" int stp_row_gather(const void* rows, int64_t num_rows, int64_t row_bytes,
                              const int32_t* row_ids, const int32_t* counts, int32_t cap, int32_t T,
                              int32_t parts, int32_t replicas, uint32_t* checksum,
                              hipStream_t stream) {
  using stp::fail;
  if (T < 0 || cap < 0 || num_rows <= 0 || parts < 1 || replicas < 1)
    return fail(STP_ERR_INVALID_ARG, "row_gather: bad sizes");
  if (row_bytes < 16 || row_bytes % 16 != 0 || row_bytes > (1 << 20))
    return fail(STP_ERR_INVALID_ARG, "row_gather: row_bytes must be a positive multiple of 16");
  if ((cap + parts - 1) / parts > kIdsMax)
    return fail(STP_ERR_INVALID_ARG, "row_gather: ceil(cap / parts) exceeds %d", kIdsMax);
  const int32_t blocks = stp_row_gather_blocks(T, parts, replicas);
  if (T == 0) return STP_OK;
  if (blocks == 0) return fail(STP_ERR_INVALID_ARG, "row_gather: grid too large");
  if (!rows || !checksum || (cap > 0 && !row_ids))
    return fail(STP_ERR_INVALID_ARG, "row_gather: null pointer");
  GatherArgs a{(const uint8_t*)rows, num_rows, (int)row_bytes, row_ids, counts, cap, T, parts,
               replicas, checksum};
  const int lines = (int)((row_bytes / 16 + 7) / 8);
  switch (lines) {
    case 2: row_gather_ring_kernel<2><<<blocks, kThreads, 0, stream>>>(a); break;
    case 6: row_gather_ring_kernel<6><<<blocks, kThreads, 0, stream>>>(a); break;
    case 9: row_gather_ring_kernel<9><<<blocks, kThreads, 0, stream>>>(a); break;
    default: row_gather_kernel<<<blocks, kThreads, 0, stream>>>(a); break;
  }
  return stp::check_launch("row_gather_kernel");
}

extern "C" int stp_stream_read(const void* src, int64_t bytes, int32_t blocks, uint32_t* checksum,
                               hipStream_t stream) {
  using stp::fail;
  if (bytes < 0 || bytes % 16 != 0 || blocks < 1)
    return fail(STP_ERR_INVALID_ARG, "stream_read: bytes must be a multiple of 16, blocks >= 1");
  if (bytes == 0) return STP_OK;
  if (!src || !checksum) return fail(STP_ERR_INVALID_ARG, "stream_read: null pointer");
  stream_read_kernel<<<blocks, kThreads, 0, stream>>>((const uintx4*)src, bytes / 16, checksum);
  return stp::check_launch("stream_read_kernel");
}
