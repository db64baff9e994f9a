/*
 * stp.h -- C ABI of the top-k sparse MLA decode path on MI355X (gfx950).
 *
 * The path has four stages, each one call (or a pair) below:
 *   1. stp_normalize_indices   candidate sets S = unique(D ∪ W ∪ A), token ->
 *                              logical block -> physical slot id, block view;
 *   2. stp_hot_lookup_swapin   per-request hot buffer with LRU eviction and
 *      stp_hot_reset           row-by-row swap-in from a pinned host pool,
 *      stp_backup_rows         and the back-up of each step's new rows;
 *   3. stp_sparse_mla_decode   attention over the selected latent rows with an
 *                              online softmax (optionally split);
 *      stp_sparse_mla_decode_fp8   the same over 656-byte fp8_ds_mla rows;
 *      stp_decode_plan / stp_decode_run   the same as a plan (task table of a
 *                              capacity tier) and a graph-stable run over it;
 *   4. stp_splitkv_merge       merge of split partial states.
 * Beside it, dense paged attention with grouped query heads over a token pool:
 *      stp_paged_gqa_decode    decode over block tables;
 *      stp_extend_attention    prefill of new tokens over a cached prefix;
 * and the staged bulk transfer of KV rows between host and device pools:
 *      stp_kv_transfer.
 *
 * Sources: "HiSparse" hot-buffer walkthrough (devpress.csdn.net); "5.1.1 · 从
 * 索引到 Kernel" (PaperTrace); "PagedAttention 与 RadixAttention：上游机制与海光
 * 实现对照"; "[HiCache] TMA-staged host<->device KV transfer kernel (sm_90+)".
 *
 * Conventions shared by every call
 *  - Ownership: the caller owns every buffer (device memory, pinned host
 *    memory, workspace) and every stream.  No call allocates, frees or
 *    synchronises; each only enqueues kernels on `stream` and returns.
 *  - Pointers are device pointers unless stated otherwise.  A "host pool"
 *    pointer is the device-visible address of pinned host memory
 *    (hipHostMalloc + hipHostGetDevicePointer, or torch pin_memory()).
 *  - bf16 data is passed as uint16_t bit patterns.  Row-major layouts.
 *  - Padding / invalid ids are -1 everywhere.
 *  - Data anomalies found on the device (ids out of range, causally invalid
 *    candidates, unmapped pages) are not errors: they are dropped, and
 *    counted where an output exists for it.  Argument errors are detected on
 *    the host before anything is launched and return a non-zero status; the
 *    message of the last error of the calling thread is stp_last_error().
 *  - Calls on one stream run in order; calls that share state (hot-buffer
 *    dgi/lru, outputs) on different streams must be ordered by the caller.
 */
#ifndef STP_H_
#define STP_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  STP_OK = 0,
  STP_ERR_INVALID_ARG = 1, /* bad pointer / size / unsupported shape */
  STP_ERR_WORKSPACE = 2,   /* workspace missing or too small: nothing launched */
  STP_ERR_HIP = 3          /* a HIP launch or attribute call failed */
};

/* Human-readable message of the last non-zero status returned on this thread. */
const char* stp_last_error(void);

/* Library version string. */
const char* stp_version(void);

/*
 * Device-visible address of pinned host memory (hipHostGetDevicePointer):
 * what the host-pool arguments below expect.  STP_ERR_HIP if `host` is not
 * pinned host memory.
 */
int stp_host_device_pointer(const void* host, void** dev);

/*
 * ---- Stage 1: candidate normalisation -------------------------------------
 * "5.1.1 · 从索引到 Kernel" §1.1 eq. (1), §1.2 eq. (2), §7.3 eq. (16)-(17),
 * §7.4 eq. (19); "HiSparse" walkthrough, token -> global slot id conversion.
 *
 * For every query token i (request r = req_id[i], position q = q_pos[i]):
 *   D = entries >= 0 of topk[i, 0:top_k]      (entries < 0 are padding)
 *   W = [max(0, q - window + 1), q]           (empty when window == 0)
 *   A = [0, min(num_sinks, q + 1))
 *   S = ascending unique t of D ∪ W ∪ A with t <= q, t / page_size < max_blocks
 *       and block_table[r, t / page_size] >= 0 (and a slot that fits int32).
 *   tok_out[i, j]  = j-th element of S, j < |S|; -1 for j >= |S|
 *   slot_out[i, j] = block_table[r, t / P] * P + t % P for t = tok_out[i, j]
 *   count_out[i]   = |S|
 *   dropped_out[i] = number of D entries (with multiplicity) >= 0 that fail
 *                    the filter (beyond q, outside the table, unmapped page).
 *   A token whose req_id is outside [0, num_reqs) or whose q_pos < 0 is a
 *   padding row: count 0, dropped 0, all -1.
 * Block view (optional; pass blk_indptr == NULL to skip; then the three other
 * block arrays are ignored):
 *   blk_indptr[T + 1]: CSR row pointers over tokens (blk_indptr[0] = 0);
 *   for k in [blk_indptr[i], blk_indptr[i+1]): blk_logical[k] = ascending
 *   unique t / P over S_i, blk_page[k] = its physical page, blk_mask[k] = the
 *   in-page membership bits (bit t % P set for each t of S_i in the block).
 *   The block arrays must hold T * cap entries (the worst case).
 *
 * Layouts: topk [T, top_k] int32; req_id, q_pos [T] int32; block_table
 * [num_reqs, max_blocks] int32 (-1 = unmapped); tok_out, slot_out [T, cap].
 * Requirements: T >= 0, top_k >= 0, 1 <= page_size <= 64, window >= 0,
 * num_sinks >= 0, cap >= top_k + window + num_sinks (so |S| <= cap always),
 * max_blocks * page_size <= 1,048,576 positions (the per-token bitmap lives in
 * LDS).  dropped_out may be NULL.
 */
int stp_normalize_indices(const int32_t* topk, int32_t top_k, const int32_t* req_id,
                          const int32_t* q_pos, int32_t T, const int32_t* block_table,
                          int32_t num_reqs, int32_t max_blocks, int32_t page_size, int32_t window,
                          int32_t num_sinks, int32_t cap, int32_t* tok_out, int32_t* slot_out,
                          int32_t* count_out, int32_t* dropped_out, int32_t* blk_indptr,
                          int32_t* blk_logical, int32_t* blk_page, uint64_t* blk_mask,
                          hipStream_t stream);

/*
 * The same normalisation in two calls, so that the block view, which the
 * decode does not read, can run on another stream (after the decode, beside
 * the merge: the decode's workgroups hold every compute unit's LDS).
 * stp_normalize_indices_deferred takes the arguments of stp_normalize_indices
 * and writes everything but the block view's logical / page / mask arrays;
 * blk_indptr then holds per-token intermediate values.  stp_block_view_fill,
 * enqueued after it with the same tok_out, slot_out, req_id, q_pos,
 * block_table, sizes and block-view arrays, completes the view; until it has
 * run, blk_indptr is not the CSR index.  It takes each block's page from the
 * slot ids (slot / page_size) and reads the page table only when the
 * per-token bitmap and pages do not fit in LDS.  The pair's results equal one
 * stp_normalize_indices call.  A second fill over arrays it has already
 * completed changes nothing (tokens whose entry is final are skipped); run
 * it once per deferred normalisation.  Errors as stp_normalize_indices.
 */
int stp_normalize_indices_deferred(const int32_t* topk, int32_t top_k, const int32_t* req_id,
                                   const int32_t* q_pos, int32_t T, const int32_t* block_table,
                                   int32_t num_reqs, int32_t max_blocks, int32_t page_size,
                                   int32_t window, int32_t num_sinks, int32_t cap,
                                   int32_t* tok_out, int32_t* slot_out, int32_t* count_out,
                                   int32_t* dropped_out, int32_t* blk_indptr,
                                   int32_t* blk_logical, int32_t* blk_page, uint64_t* blk_mask,
                                   hipStream_t stream);
int stp_block_view_fill(const int32_t* tok_out, const int32_t* slot_out, const int32_t* req_id,
                        const int32_t* q_pos, int32_t T, const int32_t* block_table,
                        int32_t num_reqs, int32_t max_blocks, int32_t page_size, int32_t cap,
                        int32_t* blk_indptr, int32_t* blk_logical, int32_t* blk_page,
                        uint64_t* blk_mask, hipStream_t stream);

/*
 * ---- Stage 2: hot buffer ----------------------------------------------------
 * "HiSparse" walkthrough: overview (SwapIn / BackUp), hot cache
 * initialisation (per-request region of hot_size + 1 rows, 16-byte rows),
 * sections "Phase 1" .. "Phase 5" of the swap-in kernel.
 *
 * Per request row r in [0, num_rows) with base = r * region_stride and
 * G = global_ids[r, 0:cap] (unique slot ids, -1 padded -- as produced by
 * stp_normalize_indices' slot_out):
 *   Phase 1: G[i] < 0 -> hot_rows_out = -1; G[i] == newest_global[r] ->
 *            hot_rows_out = base + hot_size (the reserved newest-token row);
 *            otherwise pending.
 *   Phase 2: walk lru[r, 0..hot_size) (least recent first); a slot s whose
 *            dgi[r, s] is pending is a hit: hot_rows_out = base + s.
 *   Phase 3: pending entries left are misses; in ascending i the m-th miss
 *            takes the m-th evictable slot of the walk; dgi[r, slot] = G[i];
 *            hot_rows_out = base + slot; miss_mask = 1.
 *   Phase 4: lru[r] = [evictables not taken] + [slots loaded] + [hits].
 *   Phase 5: each miss copies host_pool row G[i] (row_bytes bytes) into
 *            hot_cache row base + slot, reading the pinned host memory from
 *            the GPU; if G[i] >= host_rows the hot row is zeroed and
 *            dgi[r, slot] = -1 (ownership revoked), hot_rows_out unchanged.
 *   stats[0] += hits, stats[1] += misses (newest and -1 entries are neither).
 *   Rows r >= num_real_rows are padding: hot_rows_out = -1, miss_mask = 0,
 *   state untouched.
 * Layouts: global_ids, hot_rows_out [num_rows, cap] int32; miss_mask
 * [num_rows, cap] uint8 (nullable); newest_global [num_rows] int32; dgi
 * [num_rows, hot_size] int32; lru [num_rows, hot_size] int16; hot_cache
 * [num_rows * region_stride, row_bytes] bytes (device); host_pool
 * [host_rows, row_bytes] bytes (device-visible pinned host memory); stats
 * [2] int64 (nullable, accumulated, caller zeroes it).
 * Requirements: row_bytes > 0 and row_bytes % 16 == 0 (else INVALID_ARG, as
 * the coordinator's 16-byte row check); 1 <= hot_size <= 32767 (int16 LRU);
 * region_stride >= hot_size + 1; 0 <= cap <= hot_size (so misses never
 * exceed the evictable slots); 0 <= num_real_rows <= num_rows;
 * num_rows * region_stride <= INT32_MAX; stp_hot_lds_bytes(cap, hot_size) > 0
 * (the per-row LDS working set fits).  The ids of a row must be
 * unique (stage 1 guarantees it); duplicates give unspecified slot choices.
 * State starts as stp_hot_reset leaves it.
 */
int stp_hot_lookup_swapin(const void* host_pool, int64_t host_rows, void* hot_cache,
                          int64_t row_bytes, const int32_t* global_ids, int32_t cap,
                          const int32_t* newest_global, int32_t* dgi, int16_t* lru, int32_t hot_size,
                          int32_t region_stride, int32_t num_real_rows, int32_t num_rows,
                          int32_t* hot_rows_out, uint8_t* miss_mask, int64_t* stats,
                          hipStream_t stream);

/* LDS bytes stp_hot_lookup_swapin needs for (cap, hot_size); 0 if unsupported. */
size_t stp_hot_lds_bytes(int32_t cap, int32_t hot_size);

/*
 * Drop the cached state of request rows before they are reused ("HiSparse"
 * walkthrough, HiSparseCoordinator: a recycled slot's stale state must be
 * dropped first): dgi[r, :] = -1, lru[r, :] = 0 .. hot_size-1 for every r in
 * rows[0:n] (rows == NULL: r = 0 .. n-1, and n <= num_rows).  dgi / lru are
 * [num_rows, hot_size]; row indices outside [0, num_rows) are skipped.
 */
int stp_hot_reset(int32_t* dgi, int16_t* lru, int32_t hot_size, int32_t num_rows,
                  const int32_t* rows, int32_t n, hipStream_t stream);

/*
 * BackUp ("HiSparse" walkthrough, overview): copy n rows of row_bytes bytes,
 * host_pool[dst_ids[j]] <- hot_cache[src_rows[j]], writing pinned host memory
 * from the GPU.  Entries with src_rows[j] outside [0, hot_rows) or dst_ids[j]
 * outside [0, host_rows) are skipped.  Two entries with the same destination
 * race.  Requirements: row_bytes > 0, row_bytes % 16 == 0, n >= 0.
 */
int stp_backup_rows(const void* hot_cache, int64_t hot_rows, void* host_pool, int64_t host_rows,
                    int64_t row_bytes, const int32_t* src_rows, const int32_t* dst_ids, int32_t n,
                    hipStream_t stream);

/*
 * ---- Stage 3: sparse MLA decode attention -----------------------------------
 * "5.1.1 · 从索引到 Kernel" §3.1 eq. (4)-(6), §3.2 (mask before exp, empty
 * sets), §7.3 (sets); "PagedAttention 与 RadixAttention" §1.1 (decode
 * attention), §1.4 (exp2 with log2 e folded into the scale; partitions).
 *
 * For token t and head h, over the rows R_t = { row_ids[t, j] : j < n_t,
 * 0 <= row_ids[t, j] < kv_rows } with n_t = counts[t] (counts == NULL: n_t =
 * cap):
 *   z_j  = scale * <q[t, h, 0:576], kv[row_j, 0:576]>
 *   out[t, h, :] = sum_j softmax(z)_j * kv[row_j, 0:512]     (bf16, RNE)
 *   lse[t, h]    = log(sum_j exp(z_j))                        (natural log)
 * Empty R_t: out = 0, lse = -inf.  Entries are a set: a repeated row id is
 * counted twice (callers pass stage 1's unique lists).
 * Layouts: q [T, H, 576] bf16; kv [kv_rows, 576] bf16 (the paged latent pool
 * addressed by slot id, or the hot cache addressed by hot row); row_ids
 * [T, cap] int32; counts [T] int32 (nullable); out [T, H, 512] bf16; lse
 * [T, H] float (nullable).
 * num_splits: 0 = choose automatically (from T, H, cap and the current
 * device's compute-unit count, so that the workgroups fill whole rounds of
 * the device), otherwise the number of contiguous position ranges of
 * ceil(n_t / num_splits) each (a performance hint: the result does not
 * depend on it beyond float rounding).  Splits > 1 need a
 * workspace of stp_sparse_mla_decode_workspace() bytes (STP_ERR_WORKSPACE if
 * smaller); the workspace may be reused once the call's work has completed
 * on `stream`.
 * num_splits = 1 is a single pass per token: no partial states, no merge.
 * A split of more than 1120 candidates (the ids a workgroup stages in LDS at
 * once) keeps them in a ring of 35 32-row tiles refilled as it goes; the
 * automatic count stays within 1120 per split.
 * Requirements: T >= 0, H >= 1, cap >= 0, 0 < kv_rows, 0 < scale < inf.
 */
int stp_sparse_mla_decode(const uint16_t* q, const uint16_t* kv, int64_t kv_rows,
                          const int32_t* row_ids, const int32_t* counts, int32_t cap, int32_t T,
                          int32_t H, float scale, int32_t num_splits, void* workspace,
                          size_t workspace_bytes, uint16_t* out, float* lse, hipStream_t stream);

/*
 * stp_sparse_mla_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * stp_sparse_mla_decode minus (workspace, workspace_bytes); the split
 * partials live in a scratch array the library holds in device memory, one
 * copy per GPU, kept until the process ends
 * (stp_sparse_mla_decode_noalloc_max_bytes() bytes, 36 MiB).  Nothing is
 * allocated or freed.  A shape whose split path needs more scratch
 * (stp_sparse_mla_decode_workspace() > the maximum) returns STP_ERR_WORKSPACE
 * before anything is launched.  The scratch of the current device is used:
 * call it with the stream's device current.  Every call on a GPU shares that
 * GPU's scratch: calls that overlap in time on one GPU (other streams,
 * other threads) race, so order them on one stream or by events.
 */
int stp_sparse_mla_decode_noalloc(const uint16_t* q, const uint16_t* kv, int64_t kv_rows,
                                  const int32_t* row_ids, const int32_t* counts, int32_t cap,
                                  int32_t T, int32_t H, float scale, int32_t num_splits,
                                  uint16_t* out, float* lse, hipStream_t stream);
size_t stp_sparse_mla_decode_noalloc_max_bytes(void);

/*
 * Stage 3 over fp8_ds_mla rows ("HiSparse" walkthrough: the 656-byte
 * FP8_DS_MLA row, 512 B quantised latent + 16 B scales + 128 B RoPE;
 * "5.1.1 · 从索引到 Kernel" §7.2: dequantise at tile load).  As
 * stp_sparse_mla_decode, with kv [kv_rows, 656] uint8 rows: latent value i =
 * e4m3(byte i) * scale[i / 128] (OCP FP8 E4M3; scale = float32 at bytes
 * 512 + 4 (i / 128)), RoPE values bf16 at bytes 528..655; the key is the 576
 * values, the value vector the first 512.  Each latent value is
 * reconstructed right after the row is loaded as bf16(f32(code) * scale)
 * (both roundings to nearest even), the RoPE values taken as they are, and
 * attention runs over the reconstructed rows exactly as stp_sparse_mla_decode
 * over bf16 rows ("5.1.1 · 从索引到 Kernel" §7.2: apply the scale at tile load
 * and check against the same reconstructed values).  num_splits 0 =
 * automatic (the bf16 rule); more than one split needs
 * stp_sparse_mla_decode_fp8_workspace() bytes.  Splits of any length, as
 * for bf16 rows.  kv must be 16-byte aligned.
 * Requirements: T >= 0, H >= 1, cap >= 0, kv_rows > 0, 0 < scale < inf.
 */
int stp_sparse_mla_decode_fp8(const uint16_t* q, const uint8_t* kv, int64_t kv_rows,
                              const int32_t* row_ids, const int32_t* counts, int32_t cap,
                              int32_t T, int32_t H, float scale, int32_t num_splits,
                              void* workspace, size_t workspace_bytes, uint16_t* out, float* lse,
                              hipStream_t stream);
int32_t stp_sparse_mla_decode_fp8_splits(int32_t T, int32_t H, int32_t cap, int32_t num_splits);
size_t stp_sparse_mla_decode_fp8_workspace(int32_t T, int32_t H, int32_t cap,
                                           int32_t num_splits);

/*
 * Plan / run ("5.1.1 · 从索引到 Kernel" §5.1: plan once from the row lengths,
 * run per layer, caller-provided workspace sized for a capacity tier; §7.1:
 * for graph capture every address and grid shape is fixed by the tier and
 * the kernels read the valid task count; §7.4: a row of n candidates becomes
 * ceil(n / R) tasks (row, start, end, split) numbered by a prefix sum, and
 * each task's partial goes to the slot of its (row, split)).
 *
 * A tier is (T, cap, rows_per_task = R): T rows (pad a smaller batch with
 * rows whose count is 0: they get no task, out = 0 and lse = -inf), at most
 * cap candidates per row, at most R (1 <= R <= 1120) candidate positions per
 * task.  max_tasks = T * ceil(cap / R).
 *
 * stp_decode_plan reads counts [T] (nullable: every row has cap candidates;
 * each count is clamped to [0, cap]) on the device and writes the plan
 * buffer (int32, stp_decode_plan_bytes() bytes, caller-owned device memory):
 *   [0] number of tasks, [1] T, [2] R, [3] max_tasks, [4..11] queue heads
 *   (set to 0), [12..19] qcount, [20] qcap = ceil(T / 8) * ceil(cap / R),
 *   [32 .. 32 + T] row_first (row_first[r] = tasks before row r), then, from
 *   int32 index ceil((33 + T) / 4) * 4, the tasks as 4 int32 (row, start,
 *   end, split), row by row in split order (task i of a row of n candidates
 *   and k tasks covers floor(i n / k) .. floor((i + 1) n / k) - 1), then
 *   eight queue segments of qcap entries of 4 int32 (row, start,
 *   end - start, slot = row_first[row] + split, or -1 for a row's only task,
 *   whose output the run writes directly): queue x (run on XCD x) is
 *   the first qcount[x] entries of segment x, the tasks of rows x, x + 8,
 *   x + 16, ... in order.
 * stp_decode_run computes, for every row t, the attention of
 * stp_sparse_mla_decode over row_ids[t, 0 : count_t] (the counts the plan
 * was made from): a persistent grid pops (task, head group) work items from
 * the eight queues (each workgroup's first item by its block id, later ones
 * claimed with the queue heads), writes each task's normalised partial to slot
 * row_first[row] + split of the workspace (stp_decode_run_workspace() bytes:
 * bf16 o/l [max_tasks][H][512], then fp32 m and l [max_tasks][H], each
 * 256-byte aligned), and a merge writes out [T, H, 512] bf16 and lse [T, H]
 * (nullable); a row's only task writes that row's out and lse itself.  The
 * run reads only the queue entries; their order, within a queue or across
 * queues, does not change the result (each entry carries its row and slot),
 * so a caller may reorder them.  The run leaves the queue heads at 0, so
 * one plan serves any number of runs; runs over one plan buffer must not
 * overlap in time (they share the queue heads).  Grids depend only on the
 * tier and the device, so plan + run (or run alone) can be captured in a HIP
 * graph and replayed after the counts and candidates change in place.
 * Errors: STP_ERR_INVALID_ARG for bad sizes, R outside [1, 1120] or null
 * pointers; STP_ERR_WORKSPACE when the plan buffer or workspace is smaller
 * than the tier needs.
 */
int stp_decode_plan(const int32_t* counts, int32_t T, int32_t cap, int32_t rows_per_task,
                    int32_t* plan, size_t plan_bytes, hipStream_t stream);
int stp_decode_run(const uint16_t* q, const uint16_t* kv, int64_t kv_rows, const int32_t* row_ids,
                   int32_t cap, int32_t T, int32_t H, float scale, int32_t rows_per_task,
                   int32_t* plan, size_t plan_bytes, void* workspace, size_t workspace_bytes,
                   uint16_t* out, float* lse, hipStream_t stream);
/* Bytes of the plan buffer and of the run workspace of a tier (0 for bad
 * sizes), and a task size R for (T, H, cap): the static split's range
 * rounded up to whole 32-row tiles, at most 1120. */
size_t stp_decode_plan_bytes(int32_t T, int32_t cap, int32_t rows_per_task);
size_t stp_decode_run_workspace(int32_t T, int32_t H, int32_t cap, int32_t rows_per_task);
int32_t stp_decode_plan_rows_per_task(int32_t T, int32_t H, int32_t cap);

/* Splits stp_sparse_mla_decode uses for num_splits (0 = auto) at this shape, on
 * the current device (query it, and the workspace size, on the device the
 * decode will run on). */
int32_t stp_sparse_mla_decode_splits(int32_t T, int32_t H, int32_t cap, int32_t num_splits);

/* Workspace bytes stp_sparse_mla_decode needs for this shape and num_splits. */
size_t stp_sparse_mla_decode_workspace(int32_t T, int32_t H, int32_t cap, int32_t num_splits);

/*
 * Split partial states only ("5.1.1 · 从索引到 Kernel" §3.2 eq. (7) inputs):
 * for split s covering positions [s*c, min(n_t, (s+1)*c)), c = ceil(n_t / S):
 *   m_part[t, s, h] = max_j z_j (natural-log units), l_part = sum_j exp(z_j - m),
 *   o_part[t, s, h, :] = sum_j exp(z_j - m) * kv[row_j, 0:512]  (unnormalised);
 *   an empty split has m = -inf, l = 0, o = 0.
 * Layouts: o_part [T, S, H, 512] float, m_part / l_part [T, S, H] float.
 * Requirements as stp_sparse_mla_decode with num_splits = S >= 1.
 */
int stp_sparse_mla_decode_partial(const uint16_t* q, const uint16_t* kv, int64_t kv_rows,
                                  const int32_t* row_ids, const int32_t* counts, int32_t cap,
                                  int32_t T, int32_t H, float scale, int32_t num_splits,
                                  float* o_part, float* m_part, float* l_part, hipStream_t stream);

/*
 * Split partial states in normalised form (the partition outputs of
 * "PagedAttention 与 RadixAttention" §1.4, what stp_sparse_mla_decode's own
 * split path writes): for split s of token t and head h,
 *   o_norm[t, s, h, :] = (sum_j exp(z_j - m) kv[row_j, 0:512]) / l  (bf16, RNE)
 *   m_part, l_part as in stp_sparse_mla_decode_partial; an empty split has
 *   o_norm = 0, m = -inf, l = 0.
 * Layouts: o_norm [T, S, H, 512] bf16, m_part / l_part [T, S, H] float.
 */
int stp_sparse_mla_decode_partial_normalized(const uint16_t* q, const uint16_t* kv,
                                             int64_t kv_rows, const int32_t* row_ids,
                                             const int32_t* counts, int32_t cap, int32_t T,
                                             int32_t H, float scale, int32_t num_splits,
                                             uint16_t* o_norm, float* m_part, float* l_part,
                                             hipStream_t stream);

/*
 * ---- Normalisation and decode in one call -------------------------------------
 * "5.1.1 · 从索引到 Kernel" §4.2 eq. (10): the index stage's time adds to
 * every decode step, so the decode launch can build the candidate lists
 * itself.  stp_normalize_and_decode equals stp_normalize_indices(topk ...
 * blk_mask) followed by stp_sparse_mla_decode(q, kv, kv_rows, slot_out,
 * count_out, cap, T, H, scale, num_splits, workspace, workspace_bytes, out,
 * lse): the same normalisation outputs (block view included when blk_indptr
 * is given) and the same attention output, bit for bit.  Arguments, layouts,
 * requirements and errors are those of the two calls; the workspace is
 * stp_sparse_mla_decode_workspace(T, H, cap, num_splits) bytes.
 * When every split fits the decode's LDS id list (ceil(cap / S) <= 1120) and
 * the per-token bitmap, page-table row, top-k list and word offsets fit two
 * of the decode's LDS ring stages (12 * nw + 4 * max_blocks + 4 * top_k +
 * 4 * (nw / 64 + 1) <= 74,752 bytes, nw = ceil(max_blocks * page_size / 64);
 * within one stage, 37,376 bytes, the first tile's rows load while the list
 * is finished), each decode
 * workgroup builds its token's list in LDS and stages its split's slots
 * directly (head group 0 also writes tok_out / slot_out for its split), so
 * no launch stands between the two stages; otherwise the normalisation runs
 * as its own launch first.  The split path then runs the merge, and the
 * block view in the merge's launch (stp_splitkv_merge_with_block_view); a
 * single pass completes the block view in a launch of its own.
 *
 * stp_normalize_and_decode_partial_normalized stops before the merge: it
 * equals stp_normalize_indices_deferred (blk_indptr nullable, left in the
 * deferred state) followed by stp_sparse_mla_decode_partial_normalized with
 * num_splits = S >= 1.  stp_splitkv_merge_with_block_view completes both.
 */
int stp_normalize_and_decode(const int32_t* topk, int32_t top_k, const int32_t* req_id,
                             const int32_t* q_pos, int32_t T, const int32_t* block_table,
                             int32_t num_reqs, int32_t max_blocks, int32_t page_size,
                             int32_t window, int32_t num_sinks, int32_t cap, int32_t* tok_out,
                             int32_t* slot_out, int32_t* count_out, int32_t* dropped_out,
                             int32_t* blk_indptr, int32_t* blk_logical, int32_t* blk_page,
                             uint64_t* blk_mask, const uint16_t* q, const uint16_t* kv,
                             int64_t kv_rows, int32_t H, float scale, int32_t num_splits,
                             void* workspace, size_t workspace_bytes, uint16_t* out, float* lse,
                             hipStream_t stream);
int stp_normalize_and_decode_partial_normalized(
    const int32_t* topk, int32_t top_k, const int32_t* req_id, const int32_t* q_pos, int32_t T,
    const int32_t* block_table, int32_t num_reqs, int32_t max_blocks, int32_t page_size,
    int32_t window, int32_t num_sinks, int32_t cap, int32_t* tok_out, int32_t* slot_out,
    int32_t* count_out, int32_t* dropped_out, int32_t* blk_indptr, const uint16_t* q,
    const uint16_t* kv, int64_t kv_rows, int32_t H, float scale, int32_t num_splits,
    uint16_t* o_norm, float* m_part, float* l_part, hipStream_t stream);

/*
 * ---- Stage 4: split-KV merge -------------------------------------------------
 * "5.1.1 · 从索引到 Kernel" §3.2 eq. (7) for any number of splits, §7.1 (an
 * empty split, l_s = 0, takes no part); "PagedAttention 与 RadixAttention"
 * §1.4 part 3 (combine).  With m = max over live splits of m_part:
 *   out[t, h, :] = sum_s e^(m_s - m) o_s / sum_s e^(m_s - m) l_s   (bf16, RNE)
 *   lse[t, h]    = m + log(sum_s e^(m_s - m) l_s);  no live split: 0 and -inf.
 * Layouts as stp_sparse_mla_decode_partial (dv values per head instead of
 * 512); lse nullable.  Requirements: T >= 0, S >= 1, H >= 1, 1 <= dv, dv % 4 == 0.
 */
int stp_splitkv_merge(const float* o_part, const float* m_part, const float* l_part, int32_t T,
                      int32_t S, int32_t H, int32_t dv, uint16_t* out, float* lse,
                      hipStream_t stream);

/*
 * The same merge from normalised bf16 split outputs O_s = o_s / l_s: with
 * M = max over live splits of m_s and w_s = l_s e^(m_s - M) / sum_s' (...),
 *   out = sum_s w_s O_s (bf16, RNE), lse = M + log(sum_s l_s e^(m_s - M))
 * ("PagedAttention 与 RadixAttention" §1.4 part 3, the combine derivation).
 * Layouts: o_norm [T, S, H, dv] bf16, m_part / l_part [T, S, H] float.
 */
int stp_splitkv_merge_normalized(const uint16_t* o_norm, const float* m_part,
                                 const float* l_part, int32_t T, int32_t S, int32_t H, int32_t dv,
                                 uint16_t* out, float* lse, hipStream_t stream);

/*
 * stp_splitkv_merge_normalized and stp_block_view_fill of the same T tokens
 * in one call.  Both run after the decode and neither reads the other's
 * output ("5.1.1 · 从索引到 Kernel" §4.2 eq. (10): the index stage's time is
 * part of every step), so when the merge's slices are 16 bytes wide
 * (dv % 8 == 0, S <= 8) and the block view's per-token LDS (the position
 * bitmap, 8 * ceil(max_blocks * page_size / 64) bytes, and the blocks'
 * pages, 4 * max_blocks bytes) fits in 64 KiB, a single launch carries both: the
 * first T workgroups complete the block view, the others merge.  Otherwise
 * the call enqueues the fill and then the merge.  The results are those of
 * the two calls.  Arguments, layouts, requirements and errors are those of
 * the two calls (the block-view arrays as left by
 * stp_normalize_indices_deferred); T counts both the merge's tokens and the
 * normalised tokens.
 */
int stp_splitkv_merge_with_block_view(const uint16_t* o_norm, const float* m_part,
                                      const float* l_part, int32_t T, int32_t S, int32_t H,
                                      int32_t dv, uint16_t* out, float* lse,
                                      const int32_t* tok_out, const int32_t* slot_out,
                                      const int32_t* req_id, const int32_t* q_pos,
                                      const int32_t* block_table, int32_t num_reqs,
                                      int32_t max_blocks, int32_t page_size, int32_t cap,
                                      int32_t* blk_indptr, int32_t* blk_logical,
                                      int32_t* blk_page, uint64_t* blk_mask, hipStream_t stream);

/*
 * ---- Dense paged attention with grouped query heads -------------------------
 * "PagedAttention 与 RadixAttention：上游机制与海光实现对照" §1.1 (decode
 * attention), §1.2 (block table), §1.4 part 4 (grouped query heads: the grid
 * runs over KV heads), §3.1-§3.4 (extend attention, the shifted causal mask,
 * the ragged metadata arrays, the tile loop with early exit), §5 (the bshd
 * token-pool layout).
 *
 * Token pool: k_pool, v_pool [num_slots, Hkv, head_dim] fp16 (uint16_t bit
 * patterns), one row per slot and KV head.  Query head h reads KV head
 * h / (Hq / Hkv).  Outputs are fp16 (round to nearest even) and the natural
 * log-sum-exp of the scaled scores as float; a query with no visible key gets
 * out = 0 and lse = -inf.  Keys whose slot is unmapped or outside the pool
 * are data, not errors: they take no part.
 * Requirements: head_dim == 128, Hq % Hkv == 0, 0 < scale < inf.
 */

/*
 * Decode, one query token per request: for request b with n = ctx_lens[b]
 * (values < 0 read as 0), token t < n lives in slot
 * block_table[b, t / page_size] * page_size + t % page_size (a table entry
 * < 0, or t / page_size >= max_blocks, is an unmapped page), and
 *   out[b, h, :] = softmax_t(scale * <q[b, h], K[slot_t, h / group]>) V[slot_t, h / group]
 * Layouts: q, out [B, Hq, 128]; block_table [B, max_blocks] int32; ctx_lens
 * [B] int32; lse [B, Hq] (nullable).  Hq / Hkv <= 16, page_size <= 2^20.
 * One workgroup per (request, KV head, partition) reads each K / V tile once
 * for every query head of its group.  num_splits: 0 = choose automatically
 * (from B, Hkv, max_blocks * page_size and the current device's compute
 * units), otherwise the number of equal token ranges (partitions, the
 * vLLM v2 PARTITION_SIZE idea of §1.4) each request's table is cut into; a
 * performance hint that changes the result only by float rounding.  More
 * than one partition needs stp_paged_gqa_decode_workspace() bytes of
 * workspace (STP_ERR_WORKSPACE if smaller), reusable once the call's work
 * has completed on `stream`.
 */
int stp_paged_gqa_decode(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                         int64_t num_slots, const int32_t* block_table, int32_t max_blocks,
                         const int32_t* ctx_lens, int32_t B, int32_t Hq, int32_t Hkv,
                         int32_t head_dim, int32_t page_size, float scale, int32_t num_splits,
                         void* workspace, size_t workspace_bytes, uint16_t* out, float* lse,
                         hipStream_t stream);

/* Partitions stp_paged_gqa_decode uses for num_splits (0 = auto) at this
 * shape on the current device, and the workspace bytes it then needs. */
int32_t stp_paged_gqa_decode_splits(int32_t B, int32_t Hkv, int32_t max_blocks, int32_t page_size,
                                    int32_t num_splits);
size_t stp_paged_gqa_decode_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t max_blocks,
                                      int32_t page_size, int32_t num_splits);

/*
 * Extend (prefill over a cached prefix): request b has Lq = qo_indptr[b+1] -
 * qo_indptr[b] new queries, rows qo_indptr[b] .. of the packed q, and Lk =
 * kv_indptr[b+1] - kv_indptr[b] keys at slots kv_indices[kv_indptr[b] ..
 * kv_indptr[b+1]) (the cached prefix first, then the new tokens).  Query i
 * sees key j iff j <= i + (Lk - Lq):
 *   out[qo_indptr[b] + i, h, :] = softmax_{j visible}(scale * <q, K_j>) V_j
 * Layouts: q, out [N, Hq, 128] with N = qo_indptr[B]; qo_indptr, kv_indptr
 * [B + 1] int32 ascending; kv_indices [kv_indptr[B]] int32; lse [N, Hq]
 * (nullable).  max_extend_len >= every Lq (it sizes the grid: queries of a
 * request beyond it are not computed).  Hq / Hkv <= 4.  Key tiles past the
 * last one any query of a 64-query block can see are not read.
 */
int stp_extend_attention(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                         int64_t num_slots, const int32_t* qo_indptr, const int32_t* kv_indptr,
                         const int32_t* kv_indices, int32_t B, int32_t Hq, int32_t Hkv,
                         int32_t head_dim, int32_t max_extend_len, float scale, uint16_t* out,
                         float* lse, hipStream_t stream);

/*
 * ---- Staged bulk host <-> device KV transfer --------------------------------
 * "[HiCache] TMA-staged host<->device KV transfer kernel (sm_90+)",
 * Motivation and Modifications (cached prefixes brought back from the pinned
 * host pool layer by layer on a side stream; any row size that is a multiple
 * of 16 B; layer-first and page-first host views).
 *
 * For every buffer b < num_bufs and list position i < n:
 *   dst_bufs[b] + dst_idx[i] * dst_stride  <-  src_bufs[b] + src_idx[i] * src_stride
 * row_bytes bytes each.  A position whose src_idx is outside [0, src_rows) or
 * whose dst_idx is outside [0, dst_rows) is skipped (data, not an error).
 * Two positions with the same destination race.
 * src_bufs / dst_bufs: host arrays of num_bufs device-visible addresses
 * (device memory, or pinned host memory through stp_host_device_pointer);
 * one call per direction, H2D or D2H or device to device.  A page-first host
 * view (rows of all layers interleaved) is a per-layer base with stride
 * layers * row_bytes.  src_idx, dst_idx: device arrays [n] int32.
 * num_blocks: workgroups (256 threads, 128 KiB of LDS each) the transfer may
 * occupy; each keeps 64 KiB of loads in flight (about 12.8 GB/s of host
 * reads per workgroup on MI355X; five saturate a PCIe 5.0 x16 link).
 * Requirements: 1 <= num_bufs <= 32; row_bytes a multiple of 16 in
 * [16, 65536]; strides multiples of 16 and >= row_bytes; n >= 0;
 * num_blocks >= 1.
 */
int stp_kv_transfer(const void* const* src_bufs, void* const* dst_bufs, int32_t num_bufs,
                    int64_t row_bytes, int64_t src_stride, int64_t src_rows, int64_t dst_stride,
                    int64_t dst_rows, const int32_t* src_idx, const int32_t* dst_idx, int32_t n,
                    int32_t num_blocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* STP_H_ */
