// Diagnostic: bandwidth ceiling of the decode's row gather.
//
// "5.1.1 · 从索引到 Kernel" §2 and eq. (8)-(9): at decode the time of the
// sparse attention step is set by the bytes of the candidate rows it has to
// bring in, which are scattered across the cache by slot id.  This kernel
// reads exactly those rows, with the work split and the XCD placement of the
// decode kernel, and does nothing else, so its rate is the most the decode
// can reach for the same access pattern on this GPU.
//
// Grid: per query token, `parts` contiguous ranges of its candidate list
// (split as the decode splits them), each read by `replicas` workgroups (the
// decode reads every range once per group of query heads).  All workgroups
// of a token get block ids of one residue mod 8, as in the decode.  A
// workgroup stages its ids in LDS, then streams its rows with 16-byte loads,
// eight per thread always in flight, each run of 8 lanes covering one
// 128-byte line of a row, and xor-folds the words into one checksum per
// workgroup.

#include "stp_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kIdsMax = 4096;
constexpr int kDepth = 8;  // loads in flight per thread

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

__global__ __launch_bounds__(kThreads) void row_gather_kernel(GatherArgs a) {
  __shared__ int32_t s_ids[kIdsMax];
  const int bid = blockIdx.x;
  const int xk = bid >> 3;
  const int per_token = a.parts * a.replicas;
  const int t = (xk / per_token) * 8 + (bid & 7);
  const int part = (xk % per_token) / a.replicas;
  if (t >= a.T) return;
  int n = a.counts ? a.counts[t] : a.cap;
  n = min(max(n, 0), a.cap);
  const int chunk = (n + a.parts - 1) / a.parts;
  const int lo = min(n, part * chunk);
  const int len = min(n, lo + chunk) - lo;  // <= kIdsMax (checked on the host)
  for (int i = threadIdx.x; i < len; i += kThreads) {
    const int32_t id = a.row_ids[(int64_t)t * a.cap + lo + i];
    s_ids[i] = (id >= 0 && id < a.num_rows) ? id : -1;
  }
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
  // xor over the workgroup
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t s_acc[4];
  if (lane == 0) s_acc[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) a.checksum[bid] = s_acc[0] ^ s_acc[1] ^ s_acc[2] ^ s_acc[3];
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
  row_gather_kernel<<<blocks, kThreads, 0, stream>>>(a);
  return stp::check_launch("row_gather_kernel");
}
