"""Per-request hot buffer with LRU eviction, swap-in and back-up (oracle).

TEST INFRASTRUCTURE ONLY -- see the package header.

The hot buffer is a cache policy, so the oracle replays the algorithm's
steps in the order the "HiSparse" walkthrough (devpress.csdn.net) gives them,
sections "Phase 1" to "Phase 5" of the swap-in kernel, written from the
prose and the worked example rather than from the printed listing:

  1. classify each entry g of the request's (unique) global-id list:
     g < 0 -> output -1; g == newest -> the reserved row base + hot_size;
     otherwise the entry is pending;
  2. walk the request's LRU order from least to most recently used; a slot
     whose stored global id is pending is a hit (output base + slot), every
     other slot is evictable;
  3. pending entries left after the walk are misses; in ascending entry
     order the m-th miss takes the m-th evictable slot (least recent first)
     and the slot's stored id becomes g;
  4. new LRU order = [evictables not taken] + [slots just loaded, in miss
     order] + [hit slots, in walk order];
  5. each miss copies host row g into hot row base + slot; when g is not a
     row of the host pool the hot row is zeroed and the slot's stored id
     revoked (-1), while the entry's output keeps base + slot.

Rows at or beyond num_real_rows are padding: every output is -1 and the
request's state is untouched ("Padded rows are skipped by the kernel and must
come out as -1", section "swap_in 方法流程详解").

Readings (listed in the design notes): initial state is stored id -1 with the
identity LRU order; stats accumulate (hits, misses) where the newest and
invalid entries count as neither; the id list of a row must be unique.

Pins (tests/test_oracle_hot_buffer.py): the complete worked example of the
walkthrough (initial state, every intermediate array, final state; stored
under tests/golden/), the closed form of a cold start on an identity LRU
order, idempotence of re-applying the same set, and the invariants "LRU stays
a permutation", "stored ids >= 0 stay distinct", "every resolved entry's hot
row equals its host row byte for byte".  hot_reset: after a multi-step run
it restores the initial state exactly, a reset row then replays the
cold-start closed form, and rows left out of a subset keep their state.
"""

import numpy as np


class HotState:
    """Device state of the hot buffer: stored global ids and LRU order."""

    def __init__(self, num_rows, hot_size):
        self.hot_size = hot_size
        self.dgi = np.full((num_rows, hot_size), -1, dtype=np.int32)
        self.lru = np.tile(np.arange(hot_size, dtype=np.int16), (num_rows, 1))

    def copy(self):
        c = HotState.__new__(HotState)
        c.hot_size = self.hot_size
        c.dgi = self.dgi.copy()
        c.lru = self.lru.copy()
        return c


def hot_reset(state, rows=None):
    """Drop every stale slot of the given rows (all rows when None).

    The walkthrough's coordinator relies on a recycled slot's stale state
    being dropped before reuse (HiSparseCoordinator docstring): the row goes
    back to the initial state (stored id -1 everywhere, identity LRU order).
    A row index outside the state is data, not an error, and is skipped.
    """
    num_rows = state.dgi.shape[0]
    rows = range(num_rows) if rows is None else rows
    for r in rows:
        r = int(r)
        if not 0 <= r < num_rows:
            continue
        state.dgi[r, :] = -1
        state.lru[r, :] = np.arange(state.hot_size, dtype=np.int16)


def _one_row(state, r, G, newest, host_pool, hot_cache, region_stride):
    H = state.hot_size
    base = r * region_stride
    n = len(G)
    out = np.full(n, -1, dtype=np.int32)
    miss = np.zeros(n, dtype=np.uint8)
    valid = [int(g) for g in G if g >= 0]
    assert len(valid) == len(set(valid)), "global ids of a row must be unique"

    # Phase 1: classify.
    pending = {}
    for i, g in enumerate(G):
        g = int(g)
        if g < 0:
            out[i] = -1
        elif g == newest:
            out[i] = base + H
        else:
            pending[g] = i

    # Phase 2: LRU walk, least recent first.
    dgi = state.dgi[r]
    lru = state.lru[r]
    hits, evict = [], []
    for p in range(H):
        s = int(lru[p])
        cached = int(dgi[s]) if 0 <= s < H else -1
        if cached >= 0 and cached in pending:
            i = pending.pop(cached)
            out[i] = base + s
            hits.append(s)
        else:
            evict.append(s)

    # Phase 3: misses in entry order take evictable slots, least recent first.
    miss_list = sorted(pending.items(), key=lambda kv: kv[1])
    assert len(miss_list) <= len(evict)
    loaded = []
    for m, (g, i) in enumerate(miss_list):
        s = evict[m]
        out[i] = base + s
        miss[i] = 1
        dgi[s] = g
        loaded.append((g, s))

    # Phase 4: new LRU order.
    M = len(miss_list)
    new_lru = evict[M:] + evict[:M] + hits
    state.lru[r, :] = np.asarray(new_lru, dtype=np.int16)

    # Phase 5: host -> hot copies.
    host_rows = host_pool.shape[0]
    for g, s in loaded:
        if 0 <= g < host_rows:
            hot_cache[base + s, :] = host_pool[g, :]
        else:
            hot_cache[base + s, :] = 0
            dgi[s] = -1
    return out, miss, len(hits), M


def hot_lookup_swapin(state, host_pool, hot_cache, global_ids, newest,
                      region_stride, num_real_rows):
    """Run lookup, LRU update and swap-in for every request row.

    host_pool [host_rows, row_bytes] uint8, hot_cache [rows*stride, row_bytes]
    uint8 (updated in place), global_ids [R, cap] int, newest [R] int.
    Returns (hot_rows_out [R, cap] int32, miss_mask [R, cap] uint8,
    stats = np.array([hits, misses], int64)).
    """
    R, cap = global_ids.shape
    assert region_stride >= state.hot_size + 1
    out = np.full((R, cap), -1, dtype=np.int32)
    miss = np.zeros((R, cap), dtype=np.uint8)
    stats = np.zeros(2, dtype=np.int64)
    for r in range(R):
        if r >= num_real_rows:
            continue
        o, m, h, nm = _one_row(state, r, global_ids[r], int(newest[r]),
                               host_pool, hot_cache, region_stride)
        out[r] = o
        miss[r] = m
        stats += (h, nm)
    return out, miss, stats


def backup_rows(hot_cache, host_pool, src_rows, dst_ids):
    """BackUp: copy each new hot row to its host-pool row, byte for byte.

    "HiSparse" walkthrough, overview (the BackUp interface).  Entries with a
    negative or out-of-range index on either side are skipped.
    """
    for s, d in zip(src_rows, dst_ids):
        s, d = int(s), int(d)
        if 0 <= s < hot_cache.shape[0] and 0 <= d < host_pool.shape[0]:
            host_pool[d, :] = hot_cache[s, :]
