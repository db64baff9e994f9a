// Stage 2: per-request hot buffer with LRU eviction, swap-in from a pinned host
// pool, reset and back-up, on gfx950.
//
// "HiSparse" walkthrough (devpress.csdn.net): overview (SwapIn / BackUp),
// hot cache initialisation (regions of hot_size + 1 rows, 16-byte rows, the
// last row reserved for the newest token), "swap_in 方法流程详解" (padded rows
// come out -1), the single fused swap-in kernel with one block per request
// and its five phases, and the 16-byte vector row copy.
// "[HiCache] TMA-staged host<->device KV transfer kernel (sm_90+)",
// Motivation: host-link bandwidth = bytes in flight / round trip.
//
// Design for wave64: one 1024-thread workgroup per request row.  The
// request's candidate ids and, when they fit, its LRU order and stored ids
// are staged in LDS in one round trip; phase 1 enters the pending entries in
// an open-addressing table of entry indices (a cell's key is read through the
// staged candidate list); phase 2 walks the LRU order in 1024-slot chunks
// (LDS reads only when staged), and a block-wide scan keeps hits and
// evictables in walk order (hits from the front of an LDS array, evictables
// from the back); phase 3 lists the misses with a scan in entry order and
// gives the m-th the m-th evictable; phase 4 rewrites the order; phase 5
// streams the missing rows from host memory with every thread of the
// workgroup issuing several independent 16-byte loads before its stores, so
// that enough bytes are in flight to cover the PCIe round trip.  Order is
// decided by positions, never by lane timing, so the result is bit-exact
// and independent of the wave width.

#include "stp_internal.h"

namespace {

constexpr int kThreads = 256;       // reset and back-up kernels
constexpr int kSwapThreads = 1024;  // swap-in kernel
constexpr int kSwapWaves = kSwapThreads / 64;

__device__ __forceinline__ uint32_t hash_of(int32_t g, int bits) {
  return ((uint32_t)g * 2654435761u) >> (32 - bits);
}

struct HotLds {
  int32_t* tab;     // [HS] entry index of a pending id (-1 = empty); after phase 2: miss ids
  int32_t* cand;    // [cap] the request's candidate ids
  int32_t* dgi;     // [H] staged stored ids (when staged)
  int16_t* order;   // [H]: hits at the front, evictables reversed at the back
  int16_t* lru;     // [H] staged LRU order (when staged)
  int16_t* misses;  // [cap] entry index of the m-th miss
  uint8_t* pend;    // [cap]
};

// LDS layout: tab, cand, (dgi), order, (lru), misses, pend -- every array
// aligned to its element size.
__device__ __forceinline__ HotLds carve(char* smem, int hash_bits, int cap, int H, bool staged) {
  const int HS = 1 << hash_bits;
  HotLds s;
  s.tab = (int32_t*)smem;
  s.cand = s.tab + HS;
  s.dgi = s.cand + cap;
  s.order = (int16_t*)(s.dgi + (staged ? H : 0));
  s.lru = s.order + H;
  s.misses = s.lru + (staged ? H : 0);
  s.pend = (uint8_t*)(s.misses + cap);
  return s;
}

// Entry index of pending id g in the table, or -1.  The table holds entry
// indices only; a cell's key is the staged candidate id it points at.
__device__ __forceinline__ int find_pending(const HotLds& s, int32_t g, int hash_bits, int hmask) {
  for (uint32_t h = hash_of(g, hash_bits);; h = (h + 1) & hmask) {
    const int e = s.tab[h];
    if (e < 0) return -1;
    if (s.cand[e] == g) return e;
  }
}

template <bool kStaged>
__global__ __launch_bounds__(kSwapThreads) void hot_swapin_kernel(
    const uint8_t* __restrict__ host_pool, int64_t host_rows, uint8_t* __restrict__ hot_cache,
    int64_t row_bytes, const int32_t* __restrict__ global_ids, int cap,
    const int32_t* __restrict__ newest_global, int32_t* __restrict__ dgi,
    int16_t* __restrict__ lru, int H, int region_stride, int num_real_rows,
    int32_t* __restrict__ out, uint8_t* __restrict__ miss_mask,
    unsigned long long* __restrict__ stats, int hash_bits) {
  extern __shared__ __align__(16) char smem[];
  __shared__ int s_scan[kSwapWaves];
  __shared__ int s_bad_order;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* G = global_ids + (int64_t)r * cap;
  int32_t* row_out = out + (int64_t)r * cap;
  uint8_t* row_miss = miss_mask ? miss_mask + (int64_t)r * cap : nullptr;

  if (r >= num_real_rows) {  // padding row: outputs -1, state untouched
    for (int i = tid; i < cap; i += kSwapThreads) {
      row_out[i] = -1;
      if (row_miss) row_miss[i] = 0;
    }
    return;
  }

  const HotLds s = carve(smem, hash_bits, cap, H, kStaged);
  const int HS = 1 << hash_bits;
  const int hmask = HS - 1;
  const int64_t base = (int64_t)r * region_stride;
  const int32_t newest = newest_global[r];
  int32_t* row_dgi = dgi + (int64_t)r * H;
  int16_t* row_lru = lru + (int64_t)r * H;

  // The request's candidate ids, and (when they fit) its LRU order and stored
  // ids, all in flight together.
  for (int k = tid; k < HS; k += kSwapThreads) s.tab[k] = -1;
  for (int i = tid; i < cap; i += kSwapThreads) s.cand[i] = G[i];
  if (kStaged) {
    for (int p = tid; p < H; p += kSwapThreads) {
      s.lru[p] = row_lru[p];
      s.dgi[p] = row_dgi[p];
    }
  }
  if (tid == 0) s_bad_order = 0;
  __syncthreads();

  // Phase 1.  An entry is a padding id (< 0: no row), the request's newest
  // token (its reserved row base + H), or pending; pending entries are
  // entered in the table for the walk to find, and their outputs are written
  // by phase 2 (hits) or phase 3 (misses).
  for (int i = tid; i < cap; i += kSwapThreads) {
    const int32_t g = s.cand[i];
    const bool pending = g >= 0 && g != newest;
    if (!pending) row_out[i] = g < 0 ? -1 : (int32_t)(base + H);
    if (row_miss) row_miss[i] = 0;
    s.pend[i] = pending ? 1 : 0;
    if (pending) {
      // ids are unique, so an occupied cell holds another id: move on
      uint32_t h = hash_of(g, hash_bits);
      while (atomicCAS(&s.tab[h], -1, i) >= 0) h = (h + 1) & hmask;
    }
  }
  __syncthreads();

  // Phase 2: walk the LRU order, least recent first.  Every slot the walk
  // meets must be a slot of the region (the order is a permutation of
  // [0, H) as stp_hot_reset and this kernel leave it); if one is not, the
  // row's state is not ours to read and the row is left untouched.
  int hits = 0, evicts = 0;
  for (int p0 = 0; p0 < H; p0 += kSwapThreads) {
    const int p = p0 + tid;
    const bool in_range = p < H;
    const int slot = in_range ? (kStaged ? s.lru[p] : row_lru[p]) : 0;
    const bool slot_ok = slot >= 0 && slot < H;
    if (in_range && !slot_ok) s_bad_order = 1;
    const int32_t cached = (in_range && slot_ok) ? (kStaged ? s.dgi[slot] : row_dgi[slot]) : -1;
    const int found = cached >= 0 ? find_pending(s, cached, hash_bits, hmask) : -1;
    const bool hit = found >= 0;
    const bool evict = in_range && !hit;
    if (hit) {
      row_out[found] = (int32_t)(base + slot);
      s.pend[found] = 0;
    }
    int total;
    const int pre = stp::block_exclusive_scan<kSwapWaves>((hit ? 1 << 16 : 0) | (evict ? 1 : 0),
                                                           s_scan, &total);
    if (hit) s.order[hits + (pre >> 16)] = (int16_t)slot;
    if (evict) s.order[H - 1 - (evicts + (pre & 0xffff))] = (int16_t)slot;
    hits += total >> 16;
    evicts += total & 0xffff;
  }
  __syncthreads();
  if (s_bad_order) {
    for (int i = tid; i < cap; i += kSwapThreads) {
      row_out[i] = -1;
      if (row_miss) row_miss[i] = 0;
    }
    return;
  }

  // Phase 3: the entries still pending are the misses; the scan lists them
  // in entry order, and the m-th takes the m-th evictable of the walk (least
  // recent first).
  int misses = 0;
  for (int i0 = 0; i0 < cap; i0 += kSwapThreads) {
    const int i = i0 + tid;
    const bool miss = i < cap && s.pend[i];
    int total;
    const int pre = stp::block_exclusive_scan<kSwapWaves>(miss ? 1 : 0, s_scan, &total);
    if (miss) s.misses[misses + pre] = (int16_t)i;
    misses += total;
  }
  __syncthreads();
  for (int m = tid; m < misses; m += kSwapThreads) {
    const int i = s.misses[m];
    const int slot = s.order[H - 1 - m];
    const int32_t g = s.cand[i];
    s.tab[m] = g;  // the table is no longer needed: the copy's source ids
    row_out[i] = (int32_t)(base + slot);
    if (row_miss) row_miss[i] = 1;
    row_dgi[slot] = g;
  }
  __syncthreads();

  // Phase 4: [evictables not taken] + [slots just loaded] + [hits].
  const int E = H - hits;
  for (int p = tid; p < H; p += kSwapThreads) {
    int slot;
    if (p < E - misses)
      slot = s.order[H - 1 - (p + misses)];
    else if (p < E)
      slot = s.order[H - 1 - (p - (E - misses))];
    else
      slot = s.order[p - E];
    row_lru[p] = (int16_t)slot;
  }

  // Phase 5: host -> hot row copies, 16-byte vectors, 4 in flight per thread
  // (64 KiB per workgroup).
  const int64_t nvec = row_bytes >> 4;
  const int64_t total_vec = (int64_t)misses * nvec;
  const int4* host4 = (const int4*)host_pool;
  int4* hot4 = (int4*)hot_cache;
  const int4 zero = make_int4(0, 0, 0, 0);
  for (int64_t k0 = tid; k0 < total_vec; k0 += 4 * kSwapThreads) {
    int4 v[4];
    int64_t dst[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t k = k0 + (int64_t)u * kSwapThreads;
      dst[u] = -1;
      if (k < total_vec) {
        const int m = (int)(k / nvec);
        const int64_t e = k - (int64_t)m * nvec;
        const int32_t g = s.tab[m];
        dst[u] = (base + s.order[H - 1 - m]) * nvec + e;
        v[u] = (g < host_rows) ? host4[(int64_t)g * nvec + e] : zero;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (dst[u] >= 0) hot4[dst[u]] = v[u];
  }
  __syncthreads();
  for (int m = tid; m < misses; m += kSwapThreads)
    if (s.tab[m] >= host_rows) row_dgi[s.order[H - 1 - m]] = -1;  // ownership revoked
  if (tid == 0 && stats) {
    atomicAdd(&stats[0], (unsigned long long)hits);
    atomicAdd(&stats[1], (unsigned long long)misses);
  }
}

__global__ __launch_bounds__(kThreads) void hot_reset_kernel(int32_t* dgi, int16_t* lru, int H,
                                                             int num_rows, const int32_t* rows) {
  const int r = rows ? rows[blockIdx.x] : blockIdx.x;
  if (r < 0 || r >= num_rows) return;
  for (int p = threadIdx.x; p < H; p += kThreads) {
    dgi[(int64_t)r * H + p] = -1;
    lru[(int64_t)r * H + p] = (int16_t)p;
  }
}

// One wave per row; each lane moves 16-byte vectors.
__global__ __launch_bounds__(kThreads) void backup_kernel(const int4* __restrict__ hot,
                                                          int64_t hot_rows, int4* __restrict__ host,
                                                          int64_t host_rows, int64_t nvec,
                                                          const int32_t* __restrict__ src,
                                                          const int32_t* __restrict__ dst, int n) {
  const int j = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (j >= n) return;
  const int32_t s = src[j], d = dst[j];
  if (s < 0 || s >= hot_rows || d < 0 || d >= host_rows) return;
  const int4* a = hot + (int64_t)s * nvec;
  int4* b = host + (int64_t)d * nvec;
  for (int64_t e = threadIdx.x & 63; e < nvec; e += 64) b[e] = a[e];
}

int hash_bits_for(int cap) {
  int bits = 6;
  while ((1 << bits) < 2 * cap) ++bits;
  return bits;
}

size_t lds_bytes_for(int cap, int H, bool staged = false) {
  const int HS = 1 << hash_bits_for(cap);
  return (size_t)HS * 4 + (size_t)cap * 4 + (size_t)H * 2 + (size_t)cap * 2 + (size_t)cap +
         (staged ? (size_t)H * 6 : 0);
}

constexpr size_t kLdsLimit = 160 * 1024 - 256;

}  // namespace

extern "C" size_t stp_hot_lds_bytes(int32_t cap, int32_t hot_size) {
  if (cap < 0 || hot_size < 1 || hot_size > 32767 || cap > hot_size) return 0;
  const size_t b = lds_bytes_for(cap, hot_size);
  return b <= kLdsLimit ? b : 0;
}

extern "C" int stp_hot_lookup_swapin(const void* host_pool, int64_t host_rows, void* hot_cache,
                                     int64_t row_bytes, const int32_t* global_ids, int32_t cap,
                                     const int32_t* newest_global, int32_t* dgi, int16_t* lru,
                                     int32_t hot_size, int32_t region_stride,
                                     int32_t num_real_rows, int32_t num_rows,
                                     int32_t* hot_rows_out, uint8_t* miss_mask, int64_t* stats,
                                     hipStream_t stream) {
  using stp::fail;
  if (row_bytes <= 0 || row_bytes % 16 != 0)
    return fail(STP_ERR_INVALID_ARG, "hot_lookup_swapin: row_bytes %lld is not a positive "
                "multiple of 16", (long long)row_bytes);
  if (hot_size < 1 || hot_size > 32767)
    return fail(STP_ERR_INVALID_ARG, "hot_lookup_swapin: hot_size %d not in [1, 32767]", hot_size);
  if (region_stride < hot_size + 1)
    return fail(STP_ERR_INVALID_ARG, "hot_lookup_swapin: region_stride %d < hot_size + 1",
                region_stride);
  if (cap < 0 || cap > hot_size)
    return fail(STP_ERR_INVALID_ARG, "hot_lookup_swapin: cap %d not in [0, hot_size]", cap);
  if (num_rows < 0 || num_real_rows < 0 || num_real_rows > num_rows || host_rows < 0)
    return fail(STP_ERR_INVALID_ARG, "hot_lookup_swapin: bad row counts");
  if ((int64_t)num_rows * region_stride > INT32_MAX)
    return fail(STP_ERR_INVALID_ARG, "hot_lookup_swapin: hot rows exceed int32 ids");
  const size_t lds = stp_hot_lds_bytes(cap, hot_size);
  if (lds == 0)
    return fail(STP_ERR_INVALID_ARG, "hot_lookup_swapin: cap %d / hot_size %d exceed LDS", cap,
                hot_size);
  if (num_rows == 0) return STP_OK;
  if (!hot_rows_out || (cap > 0 && !global_ids) ||
      (num_real_rows > 0 && (!newest_global || !dgi || !lru || !hot_cache)) ||
      (num_real_rows > 0 && host_rows > 0 && !host_pool))
    return fail(STP_ERR_INVALID_ARG, "hot_lookup_swapin: null pointer");
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)hot_swapin_kernel<true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit) !=
            hipSuccess ||
        hipFuncSetAttribute((const void*)hot_swapin_kernel<false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit) !=
            hipSuccess)
      return fail(STP_ERR_HIP, "hot_lookup_swapin: hipFuncSetAttribute failed");
    attr_set = true;
  }
  // stage the LRU order and stored ids in LDS when they fit beside the hash
  const size_t staged_lds = lds_bytes_for(cap, hot_size, true);
  if (staged_lds <= kLdsLimit)
    hot_swapin_kernel<true><<<num_rows, kSwapThreads, staged_lds, stream>>>(
        (const uint8_t*)host_pool, host_rows, (uint8_t*)hot_cache, row_bytes, global_ids, cap,
        newest_global, dgi, lru, hot_size, region_stride, num_real_rows, hot_rows_out, miss_mask,
        (unsigned long long*)stats, hash_bits_for(cap));
  else
    hot_swapin_kernel<false><<<num_rows, kSwapThreads, lds, stream>>>(
        (const uint8_t*)host_pool, host_rows, (uint8_t*)hot_cache, row_bytes, global_ids, cap,
        newest_global, dgi, lru, hot_size, region_stride, num_real_rows, hot_rows_out, miss_mask,
        (unsigned long long*)stats, hash_bits_for(cap));
  return stp::check_launch("hot_swapin_kernel");
}

extern "C" int stp_hot_reset(int32_t* dgi, int16_t* lru, int32_t hot_size, int32_t num_rows,
                             const int32_t* rows, int32_t n, hipStream_t stream) {
  using stp::fail;
  if (hot_size < 1 || hot_size > 32767 || n < 0 || num_rows < 0)
    return fail(STP_ERR_INVALID_ARG, "hot_reset: bad hot_size, num_rows or n");
  if (!rows && n > num_rows) return fail(STP_ERR_INVALID_ARG, "hot_reset: n > num_rows");
  if (n == 0 || num_rows == 0) return STP_OK;
  if (!dgi || !lru) return fail(STP_ERR_INVALID_ARG, "hot_reset: null pointer");
  hot_reset_kernel<<<n, kThreads, 0, stream>>>(dgi, lru, hot_size, num_rows, rows);
  return stp::check_launch("hot_reset_kernel");
}

extern "C" int stp_backup_rows(const void* hot_cache, int64_t hot_rows, void* host_pool,
                               int64_t host_rows, int64_t row_bytes, const int32_t* src_rows,
                               const int32_t* dst_ids, int32_t n, hipStream_t stream) {
  using stp::fail;
  if (row_bytes <= 0 || row_bytes % 16 != 0)
    return fail(STP_ERR_INVALID_ARG, "backup_rows: row_bytes %lld is not a positive multiple "
                "of 16", (long long)row_bytes);
  if (n < 0 || hot_rows < 0 || host_rows < 0)
    return fail(STP_ERR_INVALID_ARG, "backup_rows: negative size");
  if (n == 0) return STP_OK;
  if (!hot_cache || !host_pool || !src_rows || !dst_ids)
    return fail(STP_ERR_INVALID_ARG, "backup_rows: null pointer");
  const int rows_per_block = kThreads / 64;
  backup_kernel<<<(n + rows_per_block - 1) / rows_per_block, kThreads, 0, stream>>>(
      (const int4*)hot_cache, hot_rows, (int4*)host_pool, host_rows, row_bytes / 16, src_rows,
      dst_ids, n);
  return stp::check_launch("backup_kernel");
}
