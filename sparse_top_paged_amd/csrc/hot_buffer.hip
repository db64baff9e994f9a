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
// Design for wave64: one 1024-thread workgroup per request row.  Phase 1
// builds an open-addressing hash (key = global id, value = entry index) in
// LDS and, when they fit, stages the request's LRU order and stored ids in
// LDS with the same round trip; phase 2 walks the LRU order in 1024-slot
// chunks (LDS reads only when staged), and a block-wide scan
// keeps hits and evictables in walk order (hits from the front of an LDS
// array, evictables from the back); phase 3 gives misses, in entry order,
// the evictables from least recent on; phase 4 rewrites the order; phase 5
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
constexpr int kEmpty = -1;

__device__ __forceinline__ uint32_t hash_of(int32_t g, int bits) {
  return ((uint32_t)g * 2654435761u) >> (32 - bits);
}

struct HotLds {
  int32_t* keys;    // [HS]; after phase 2: global ids of the misses, in miss order
  int32_t* dgi;     // [H] staged stored ids (when staged)
  int16_t* vals;    // [HS]
  int16_t* order;   // [H]: hits at the front, evictables reversed at the back
  int16_t* lru;     // [H] staged LRU order (when staged)
  uint8_t* pend;    // [cap]
};

// LDS layout: keys, (dgi), vals, order, (lru), pend -- every array aligned to
// its element size.
__device__ __forceinline__ HotLds carve(char* smem, int hash_bits, int H, bool staged) {
  const int HS = 1 << hash_bits;
  HotLds s;
  s.keys = (int32_t*)smem;
  s.dgi = s.keys + HS;
  s.vals = (int16_t*)(s.dgi + (staged ? H : 0));
  s.order = s.vals + HS;
  s.lru = s.order + H;
  s.pend = (uint8_t*)(s.lru + (staged ? H : 0));
  return s;
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

  const HotLds s = carve(smem, hash_bits, H, kStaged);
  const int HS = 1 << hash_bits;
  const int hmask = HS - 1;
  const int64_t base = (int64_t)r * region_stride;
  const int32_t newest = newest_global[r];
  int32_t* row_dgi = dgi + (int64_t)r * H;
  int16_t* row_lru = lru + (int64_t)r * H;

  for (int k = tid; k < HS; k += kSwapThreads) s.keys[k] = kEmpty;
  if (kStaged) {
    // the LRU order and stored ids, all loads in flight with phase 1's
    for (int p = tid; p < H; p += kSwapThreads) {
      s.lru[p] = row_lru[p];
      s.dgi[p] = row_dgi[p];
    }
  }
  __syncthreads();

  // Phase 1: classify entries; pending ones go into the hash.
  for (int i = tid; i < cap; i += kSwapThreads) {
    const int32_t g = G[i];
    if (row_miss) row_miss[i] = 0;
    uint8_t p = 0;
    if (g < 0) {
      row_out[i] = -1;
    } else if (g == newest) {
      row_out[i] = (int32_t)(base + H);
    } else {
      uint32_t h = hash_of(g, hash_bits);
      while (true) {
        const int32_t old = atomicCAS(&s.keys[h], kEmpty, g);
        if (old == kEmpty || old == g) {
          s.vals[h] = (int16_t)i;
          break;
        }
        h = (h + 1) & hmask;
      }
      p = 1;
    }
    s.pend[i] = p;
  }
  __syncthreads();

  // Phase 2: walk the LRU order, least recent first.
  int hits = 0, evicts = 0;
  for (int p0 = 0; p0 < H; p0 += kSwapThreads) {
    const int p = p0 + tid;
    const bool in_range = p < H;
    const int slot = in_range ? (kStaged ? s.lru[p] : row_lru[p]) : -1;
    const int32_t cached =
        (slot >= 0 && slot < H) ? (kStaged ? s.dgi[slot] : row_dgi[slot]) : -1;
    int found = -1;
    if (cached >= 0) {
      uint32_t h = hash_of(cached, hash_bits);
      while (true) {
        const int32_t k = s.keys[h];
        if (k == cached) {
          found = s.vals[h];
          break;
        }
        if (k == kEmpty) break;
        h = (h + 1) & hmask;
      }
    }
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

  // Phase 3: misses, in entry order, take evictables from least recent on.
  int misses = 0;
  for (int i0 = 0; i0 < cap; i0 += kSwapThreads) {
    const int i = i0 + tid;
    const bool miss = i < cap && s.pend[i];
    int total;
    const int pre = stp::block_exclusive_scan<kSwapWaves>(miss ? 1 : 0, s_scan, &total);
    if (miss) {
      const int m = misses + pre;
      const int slot = s.order[H - 1 - m];
      const int32_t g = G[i];
      s.keys[m] = g;  // the hash is no longer needed: reuse it as the miss list
      if (slot < 0 || slot >= H) {  // only reachable from a corrupted LRU state
        row_out[i] = -1;
      } else {
        row_out[i] = (int32_t)(base + slot);
        if (row_miss) row_miss[i] = 1;
        row_dgi[slot] = g;
      }
    }
    misses += total;
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
        const int32_t g = s.keys[m];
        const int slot = s.order[H - 1 - m];
        if (slot >= 0 && slot < H) {
          dst[u] = (base + slot) * nvec + e;
          v[u] = (g < host_rows) ? host4[(int64_t)g * nvec + e] : zero;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (dst[u] >= 0) hot4[dst[u]] = v[u];
  }
  __syncthreads();
  for (int m = tid; m < misses; m += kSwapThreads) {
    const int slot = s.order[H - 1 - m];
    if (s.keys[m] >= host_rows && slot >= 0 && slot < H) row_dgi[slot] = -1;  // ownership revoked
  }
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
  return (size_t)HS * 4 + (size_t)HS * 2 + (size_t)H * 2 + (size_t)cap +
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
