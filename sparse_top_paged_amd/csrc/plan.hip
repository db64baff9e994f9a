// Plan / run for the sparse MLA decode: fixed-capacity task tables, a
// persistent work queue and graph-stable launches on gfx950.
//
// "5.1.1 · 从索引到 Kernel" §5.1 (plan once per step from the row lengths,
// run per layer; the caller provides the workspace, sized for a capacity
// tier, and an over-capacity request is refused rather than written out of
// bounds), §7.1 (graph capture: every device address and every grid shape
// stays fixed; contents and valid counts change in place; the grid is sized
// for the tier's capacity and reads the number of valid tasks), §7.4 (a
// ragged row of k candidates becomes ceil(k / R) tasks (row, start, end,
// split), numbered by a prefix sum -- here cut evenly, task i of a row of n
// candidates and k tasks covering floor(i n / k) .. floor((i + 1) n / k) - 1;
// long rows split so no workgroup carries a
// tail; each task keeps its row, and its partial goes to the slot of
// (row, split), whatever order the tasks run in).
//
// Device-side plan.  The row lengths are produced on the device (the
// normalisation's counts), so the plan is one small kernel rather than a
// host inspector: planning costs no device-to-host copy, and plan + run can
// be captured in one HIP graph per tier and replayed with new counts and
// candidates.  A tier is (T, cap, R): T rows (a smaller batch pads with
// empty rows, which plan to no task), at most cap candidates per row, R
// candidate positions per task.  Its fixed sizes:
//   max_tasks = T * ceil(cap / R),
//   qcap = ceil(T / 8) * ceil(cap / R) (entries one queue may hold),
//   plan buffer (int32): [0] tasks, [1] T, [2] R, [3] max_tasks,
//     [4 .. 11] the eight queue heads, [12 .. 19] qcount, [20] qcap,
//     [32 .. 32 + T] row_first, then from the next multiple of four the
//     tasks, 4 int32 each, then eight queue segments of qcap entries of 4
//     int32 each,
//   workspace: bf16 o / l [max_tasks][H][512], then fp32 m and l
//     [max_tasks][H], each 256-byte aligned.
// Queue x of the run holds the tasks of rows x, x + 8, x + 16, ... (all
// splits of a row on one XCD, so its query rows are fetched once there):
// the first qcount[x] entries of segment x, row by row, each a task in the
// form the run consumes: (row, start, length, slot = row_first[row] +
// split, or -1 when the task is the row's only one: the run then writes the
// row's output directly and the merge leaves the row alone), so one 16-byte
// read starts a work item, and a segment's place does
// not depend on the counts (a workgroup fetches its first entry together
// with the queue lengths).
// The queue heads start at zero: the plan kernel clears them, and each run's
// merge kernel clears them again after the decode has drained the queues, so
// one plan serves any number of runs (the layers of a step).

#include <algorithm>

#include "stp_internal.h"

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kHeader = 32;
constexpr int kQCount = 12;
constexpr int kQCap = 20;
constexpr int kQueues = 8;
constexpr int kDV = 512;
constexpr int kMergeThreads = 256;
constexpr int kPerHead = 128;  // merge threads per head: 4 values each

__host__ __device__ int64_t max_tasks_of(int32_t T, int32_t cap, int32_t R) {
  return cap > 0 ? (int64_t)T * ((cap + R - 1) / R) : 0;
}
__host__ __device__ int64_t tasks_offset(int32_t T) { return ((int64_t)kHeader + T + 1 + 3) / 4 * 4; }
__host__ __device__ int64_t queue_cap(int32_t T, int32_t cap, int32_t R) {
  return cap > 0 ? (int64_t)((T + 7) / 8) * ((cap + R - 1) / R) : 0;
}
size_t plan_bytes_of(int32_t T, int32_t cap, int32_t R) {
  return (size_t)(tasks_offset(T) + 4 * max_tasks_of(T, cap, R) + 32 * queue_cap(T, cap, R)) * 4;
}
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t workspace_of(int32_t T, int32_t H, int32_t cap, int32_t R) {
  const size_t n = (size_t)max_tasks_of(T, cap, R) * H;
  return align256(n * kDV * 2) + 2 * align256(n * 4);
}

// One workgroup: rows in chunks of 1024, a wave scan plus a scan of the
// sixteen wave totals per chunk, carried across chunks.
__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(const int32_t* counts, int T,
                                                                   int cap, int R,
                                                                   int32_t* plan) {
  __shared__ int s_wave[kPlanThreads / 64];
  __shared__ int s_carry;
  __shared__ int s_qbase[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t* row_first = plan + kHeader;
  int32_t* tasks = plan + tasks_offset(T);
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int r0 = 0; r0 < T; r0 += kPlanThreads) {
    const int r = r0 + tid;
    int n = 0;
    if (r < T) n = min(max(counts ? counts[r] : cap, 0), cap);
    const int k = (n + R - 1) / R;
    int v = k;  // inclusive scan within the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(v, d);
      if (lane >= d) v += u;
    }
    if (lane == 63) s_wave[wave] = v;
    __syncthreads();
    int before = s_carry;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
    const int first = before + v - k;
    if (r < T) {
      row_first[r] = first;
      for (int i = 0; i < k; ++i) {
        int32_t* e = tasks + 4 * (int64_t)(first + i);
        e[0] = r;
        e[1] = (int)((int64_t)i * n / k);
        e[2] = (int)((int64_t)(i + 1) * n / k);
        e[3] = i;
      }
    }
    __syncthreads();  // every thread has read s_carry and s_wave
    if (tid == kPlanThreads - 1) s_carry = before + v;
    __syncthreads();
  }
  // queue order: rows by (r % 8, r / 8); a second scan in that order gives
  // each row's place in its queue (its offset from the queue's first row)
  const int total = s_carry;
  const int64_t qcap = queue_cap(T, cap, R);
  int32_t* qent = tasks + 4 * max_tasks_of(T, cap, R);
  const int cT = (T + 7) / 8;
  __syncthreads();  // row_first visible to the workgroup; s_carry read by all
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int j0 = 0; j0 < 8 * cT; j0 += kPlanThreads) {
    const int j = j0 + tid;
    const int x = j / cT;
    const int r = (j - x * cT) * 8 + x;
    const bool valid = j < 8 * cT && r < T;
    int n = 0;
    if (valid) n = min(max(counts ? counts[r] : cap, 0), cap);
    const int k = (n + R - 1) / R;
    int v = k;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(v, d);
      if (lane >= d) v += u;
    }
    if (lane == 63) s_wave[wave] = v;
    __syncthreads();
    int before = s_carry;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
    const int first = before + v - k;
    if (j < 8 * cT && j == x * cT) s_qbase[x] = first;  // row x opens queue x
    __syncthreads();
    if (valid) {
      const int f = row_first[r];
      int32_t* seg = qent + 4 * ((int64_t)x * qcap + (first - s_qbase[x]));
      for (int i = 0; i < k; ++i) {
        int32_t* e = seg + 4 * i;
        const int lo = (int)((int64_t)i * n / k);
        e[0] = r;
        e[1] = lo;
        e[2] = (int)((int64_t)(i + 1) * n / k) - lo;
        e[3] = k == 1 ? -1 : f + i;  // a whole row: the run writes its output
      }
    }
    __syncthreads();
    if (tid == kPlanThreads - 1) s_carry = before + v;
    __syncthreads();
  }
  if (tid == 0) {
    row_first[T] = total;
    plan[0] = total;
    plan[1] = T;
    plan[2] = R;
    plan[3] = (int)max_tasks_of(T, cap, R);
    plan[kQCap] = (int)qcap;
  }
  if (tid < kQueues) plan[4 + tid] = 0;
  if (tid < 8)
    plan[kQCount + tid] = T == 0 ? 0 : (tid < 7 ? s_qbase[tid + 1] : total) - s_qbase[tid];
}

// Merge of each row's partial slots row_first[t] .. row_first[t + 1] - 1
// (rows with exactly one task already hold their output and are skipped)
// (the partition combine of normalised outputs: weights l_p e^(m_p - M) / L
// over the slots with l_p > 0), in one pass over chunks of four (rows of at
// most four slots) or eight slots whose loads are all issued together;
// across chunks the running maximum moves and rescales the sums, as in the
// online softmax.  A row without a live
// slot gets out = 0 and lse = -inf.  Block (0, 0) also clears the queue
// heads for the next run.
// One chunk of up to N slots pb .. min(pb + N, p1) - 1 folded into the
// running (M, L, acc); every load of the chunk is issued before any use.
template <int N>
__device__ __forceinline__ void merge_chunk(const uint16_t* __restrict__ o_norm,
                                            const float* __restrict__ m_part,
                                            const float* __restrict__ l_part, int pb, int p1,
                                            int H, int h, int c, float& M, float& L,
                                            float4& acc) {
  float mv[N], lv[N];
  uint2 ov[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const bool in = pb + i < p1;
    const int64_t k = (int64_t)(in ? pb + i : pb) * H + h;  // in bounds either way
    mv[i] = m_part[k];
    lv[i] = in ? l_part[k] : 0.f;
    ov[i] = *(const uint2*)(o_norm + k * kDV + c);
  }
  float Mc = M;
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (lv[i] > 0.f) Mc = fmaxf(Mc, mv[i]);
  if (Mc == -INFINITY) return;  // no live slot yet
  const float f = expf(M - Mc);   // 0 while nothing was live
  L *= f;
  acc.x *= f;
  acc.y *= f;
  acc.z *= f;
  acc.w *= f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (!(lv[i] > 0.f)) continue;
    const float w = expf(mv[i] - Mc) * lv[i];
    L += w;
    acc.x += w * __uint_as_float(ov[i].x << 16);
    acc.y += w * __uint_as_float(ov[i].x & 0xffff0000u);
    acc.z += w * __uint_as_float(ov[i].y << 16);
    acc.w += w * __uint_as_float(ov[i].y & 0xffff0000u);
  }
  M = Mc;
}

__global__ __launch_bounds__(kMergeThreads) void task_merge_kernel(
    const uint16_t* __restrict__ o_norm, const float* __restrict__ m_part,
    const float* __restrict__ l_part, const int32_t* __restrict__ row_first, int H,
    uint16_t* __restrict__ out, float* __restrict__ lse, int32_t* queue) {
  const int t = blockIdx.x;
  if (t == 0 && blockIdx.y == 0 && threadIdx.x < kQueues) queue[threadIdx.x] = 0;
  const int h = blockIdx.y * 2 + (int)threadIdx.x / kPerHead;
  if (h >= H) return;
  const int c = ((int)threadIdx.x % kPerHead) * 4;
  const int p0 = row_first[t], p1 = row_first[t + 1];
  if (p1 - p0 == 1) return;  // written by its task
  uint16_t* orow = out + ((int64_t)t * H + h) * kDV;
  float M = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (p1 - p0 <= 4) {  // the common case: one short chunk
    if (p1 > p0) merge_chunk<4>(o_norm, m_part, l_part, p0, p1, H, h, c, M, L, acc);
  } else {
    for (int pb = p0; pb < p1; pb += 8)
      merge_chunk<8>(o_norm, m_part, l_part, pb, p1, H, h, c, M, L, acc);
  }
  if (M == -INFINITY) {
    *(uint2*)(orow + c) = make_uint2(0u, 0u);
    if (lse && c == 0) lse[(int64_t)t * H + h] = -INFINITY;
    return;
  }
  const float invL = 1.f / L;
  *(uint2*)(orow + c) = make_uint2(stp::pack_bf16x2(acc.x * invL, acc.y * invL),
                                   stp::pack_bf16x2(acc.z * invL, acc.w * invL));
  if (lse && c == 0) lse[(int64_t)t * H + h] = M + logf(L);
}

int check_tier(const char* what, int32_t T, int32_t cap, int32_t R) {
  if (T < 0 || cap < 0)
    return stp::fail(STP_ERR_INVALID_ARG, "%s: T=%d cap=%d must be >= 0", what, T, cap);
  if (R < 1 || R > stp::decode_ids_max())
    return stp::fail(STP_ERR_INVALID_ARG, "%s: rows_per_task %d outside [1, %d]", what, R,
                     stp::decode_ids_max());
  if (max_tasks_of(T, cap, R) > (int64_t)INT32_MAX / 16)
    return stp::fail(STP_ERR_INVALID_ARG, "%s: tier too large", what);
  return STP_OK;
}

}  // namespace

extern "C" int32_t stp_decode_plan_rows_per_task(int32_t T, int32_t H, int32_t cap) {
  if (T < 0 || H < 1 || cap < 0) return 0;
  // the static split count's task size, rounded up to whole 32-row tiles
  const int S = stp::decode_choose_splits(std::max(T, 1), H, cap);
  const int per = (std::max(cap, 1) + S - 1) / S;
  return std::min(stp::decode_ids_max(), std::max(32, (per + 31) / 32 * 32));
}

extern "C" size_t stp_decode_plan_bytes(int32_t T, int32_t cap, int32_t rows_per_task) {
  if (T < 0 || cap < 0 || rows_per_task < 1) return 0;
  return plan_bytes_of(T, cap, rows_per_task);
}

extern "C" size_t stp_decode_run_workspace(int32_t T, int32_t H, int32_t cap,
                                           int32_t rows_per_task) {
  if (T < 0 || H < 1 || cap < 0 || rows_per_task < 1) return 0;
  return workspace_of(T, H, cap, rows_per_task);
}

extern "C" int stp_decode_plan(const int32_t* counts, int32_t T, int32_t cap,
                               int32_t rows_per_task, int32_t* plan, size_t plan_bytes,
                               hipStream_t stream) {
  if (int rc = check_tier("decode_plan", T, cap, rows_per_task)) return rc;
  if (!plan) return stp::fail(STP_ERR_INVALID_ARG, "decode_plan: null plan buffer");
  const size_t need = plan_bytes_of(T, cap, rows_per_task);
  if (plan_bytes < need)
    return stp::fail(STP_ERR_WORKSPACE, "decode_plan: plan buffer of %zu bytes needed, %zu given",
                     need, plan_bytes);
  decode_plan_kernel<<<1, kPlanThreads, 0, stream>>>(counts, T, cap, rows_per_task, plan);
  return stp::check_launch("decode_plan_kernel");
}

extern "C" int stp_decode_run(const uint16_t* q, const uint16_t* kv, int64_t kv_rows,
                              const int32_t* row_ids, int32_t cap, int32_t T, int32_t H,
                              float scale, int32_t rows_per_task, int32_t* plan,
                              size_t plan_bytes, void* workspace, size_t workspace_bytes,
                              uint16_t* out, float* lse, hipStream_t stream) {
  using stp::fail;
  if (int rc = check_tier("decode_run", T, cap, rows_per_task)) return rc;
  if (H < 1 || kv_rows <= 0)
    return fail(STP_ERR_INVALID_ARG, "decode_run: H=%d kv_rows=%lld", H, (long long)kv_rows);
  if (!(scale > 0.f) || scale == INFINITY)
    return fail(STP_ERR_INVALID_ARG, "decode_run: scale must be positive and finite");
  if (T == 0) return STP_OK;
  if (!q || !kv || !out || !plan || (cap > 0 && !row_ids))
    return fail(STP_ERR_INVALID_ARG, "decode_run: null pointer");
  if (plan_bytes < plan_bytes_of(T, cap, rows_per_task))
    return fail(STP_ERR_WORKSPACE, "decode_run: plan buffer of %zu bytes needed, %zu given",
                plan_bytes_of(T, cap, rows_per_task), plan_bytes);
  const size_t need = workspace_of(T, H, cap, rows_per_task);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(STP_ERR_WORKSPACE, "decode_run: workspace of %zu bytes needed, %zu given", need,
                workspace_bytes);
  const int64_t mt = max_tasks_of(T, cap, rows_per_task);
  const size_t n = (size_t)mt * H;
  char* ws = (char*)workspace;
  uint16_t* o_norm = (uint16_t*)ws;
  float* m_part = (float*)(ws + align256(n * kDV * 2));
  float* l_part = (float*)(ws + align256(n * kDV * 2) + align256(n * 4));
  int32_t* queue = plan + 4;
  const int32_t* row_first = plan + kHeader;
  if (mt > 0) {
    const int64_t items = mt * stp::decode_head_groups(H);
    const int grid = (int)std::min<int64_t>(stp::device_cus(), items);
    if (int rc = stp::launch_decode_tasks(q, kv, kv_rows, row_ids, cap, T, H, scale,
                                          plan + kQCount, plan + tasks_offset(T) + 4 * mt,
                                          (int32_t)queue_cap(T, cap, rows_per_task), queue, grid,
                                          o_norm, m_part, l_part, out, lse, stream))
      return rc;
  }
  const dim3 mgrid((unsigned)T, (unsigned)((H + 1) / 2));
  task_merge_kernel<<<mgrid, kMergeThreads, 0, stream>>>(o_norm, m_part, l_part, row_first, H, out,
                                                         lse, queue);
  return stp::check_launch("task_merge_kernel");
}
