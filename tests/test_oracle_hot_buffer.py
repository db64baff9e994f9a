"""Pins for the hot-buffer oracle (CPU only).

Fixed by the pages: the complete worked swap-in example of the "HiSparse"
walkthrough (initial state, every phase, final state).  Fixed by closed form:
a cold start on the identity LRU order and idempotent re-application.
Invariants: LRU stays a permutation, stored ids stay distinct, every resolved
hot row equals its host row, padded rows stay untouched.
"""

import numpy as np
import pytest

import oracle
import workloads


def _bytes_pool(rows, row_bytes, seed):
    return np.random.default_rng(seed).integers(0, 256, size=(rows, row_bytes), dtype=np.uint8)


def test_worked_example(golden):
    g = golden("hisparse_swapin_example.txt")
    H = g["hot_size"][0]
    st = oracle.HotState(1, H)
    st.lru[0] = np.asarray(g["lru_before"], np.int16)
    st.dgi[0] = np.asarray(g["dgi_before"], np.int32)
    host = _bytes_pool(2000, 32, 1)
    hot = np.zeros((H + 1 + 15, 32), np.uint8)  # region_stride 32 (>= H + 1)
    out, miss, stats = oracle.hot_lookup_swapin(st, host, hot, np.asarray([g["global_ids"]]),
                                               np.asarray(g["newest"]), 32, 1)
    assert list(out[0]) == g["out"]
    assert list(miss[0]) == g["miss_mask"]
    assert list(st.lru[0]) == g["lru_after"]
    assert list(st.dgi[0]) == g["dgi_after"]
    assert list(stats) == g["stats"]
    for src, slot in g["copies"]:
        assert np.array_equal(hot[slot], host[src])
    # hits followed by reversed evictables: the phase-2 compaction printed on the page
    hits = g["hits"]
    evict = [s for s in g["lru_before"] if s not in hits]
    assert hits + evict[::-1] == g["s_lru_out"]
    # the m-th miss takes s_lru_out[H - 1 - m]
    for m, slot in enumerate(g["miss_slots"]):
        assert g["s_lru_out"][H - 1 - m] == slot


def test_cold_start_closed_form():
    H, M = 64, 23
    st = oracle.HotState(2, H)
    host = _bytes_pool(500, 16, 2)
    hot = np.zeros((2 * 128, 16), np.uint8)
    ids = np.full((2, 30), -1, np.int32)
    ids[0, :M] = np.arange(100, 100 + M)
    out, miss, stats = oracle.hot_lookup_swapin(st, host, hot, ids, np.asarray([-5, -5]), 128, 1)
    assert list(out[0, :M]) == list(range(M))            # slots 0..M-1 in entry order
    assert list(st.lru[0]) == list(range(M, H)) + list(range(M))
    assert list(stats) == [0, M]
    assert np.all(out[1] == -1) and list(st.lru[1]) == list(range(H))  # padded row untouched


def test_idempotent_reapply():
    H = 32
    st = oracle.HotState(1, H)
    host = _bytes_pool(300, 16, 3)
    hot = np.zeros((64, 16), np.uint8)
    ids = np.asarray([[7, 50, 3, -1, 120, 9]], np.int32)
    out1, _, _ = oracle.hot_lookup_swapin(st, host, hot, ids, np.asarray([-1]), 64, 1)
    lru1 = st.lru.copy()
    out2, miss2, stats2 = oracle.hot_lookup_swapin(st, host, hot, ids, np.asarray([-1]), 64, 1)
    assert np.array_equal(out1, out2)
    assert miss2.sum() == 0 and list(stats2) == [5, 0]
    # all hits: evictables keep their order, then the hits in walk order
    assert sorted(st.lru[0].tolist()) == list(range(H))
    assert list(st.lru[0][-5:]) == [s for s in lru1[0] if s in set(out1[0][out1[0] >= 0].tolist())]


def test_out_of_range_source_revokes():
    H = 16
    st = oracle.HotState(1, H)
    host = _bytes_pool(10, 16, 4)
    hot = np.full((32, 16), 9, np.uint8)
    ids = np.asarray([[2, 15]], np.int32)          # 15 is not a host row
    out, miss, _ = oracle.hot_lookup_swapin(st, host, hot, ids, np.asarray([-1]), 32, 1)
    s_bad = out[0, 1]
    assert miss[0, 1] == 1 and st.dgi[0, s_bad] == -1 and np.all(hot[s_bad] == 0)
    assert np.array_equal(hot[out[0, 0]], host[2])


def test_multistep_invariants():
    c = workloads.hot_steps_case(seed=11, batch=3, ctx0=600, steps=6, top_k=40, window=6, sinks=2,
                                 page_size=16, heads=1)
    st = oracle.HotState(c.batch, c.hot_size)
    row_bytes = 32
    host = _bytes_pool(c.host_rows, row_bytes, 5)
    hot = np.zeros((c.batch * c.region_stride, row_bytes), np.uint8)
    total = np.zeros(2, np.int64)
    for t in range(c.steps):
        res = oracle.normalize(c.topk[t], np.arange(c.batch, dtype=np.int32), c.q_pos(t), c.window,
                               c.num_sinks, c.block_table, c.page_size, c.cap)
        newest = np.asarray([c.block_table[r][c.q_pos(t)[r] // c.page_size] * c.page_size
                             + c.q_pos(t)[r] % c.page_size for r in range(c.batch)], np.int32)
        out, miss, stats = oracle.hot_lookup_swapin(st, host, hot, res["slot"], newest,
                                                   c.region_stride, c.batch)
        total += stats
        for r in range(c.batch):
            assert sorted(st.lru[r].tolist()) == list(range(c.hot_size))
            held = st.dgi[r][st.dgi[r] >= 0]
            assert len(set(held.tolist())) == len(held)
            for j in range(res["count"][r]):
                g = res["slot"][r, j]
                if g == newest[r]:
                    assert out[r, j] == r * c.region_stride + c.hot_size
                else:
                    assert np.array_equal(hot[out[r, j]], host[g])
                    assert st.dgi[r][out[r, j] - r * c.region_stride] == g
    assert total[0] > 0 and total[1] > 0


def test_backup():
    hot = _bytes_pool(20, 16, 6)
    host = np.zeros((10, 16), np.uint8)
    oracle.backup_rows(hot, host, [3, 7, -1, 19], [1, 4, 2, 99])
    assert np.array_equal(host[1], hot[3]) and np.array_equal(host[4], hot[7])
    assert np.all(host[[0, 2, 3, 5, 6, 7, 8, 9]] == 0)


def test_duplicate_ids_rejected():
    st = oracle.HotState(1, 8)
    with pytest.raises(AssertionError):
        oracle.hot_lookup_swapin(st, np.zeros((10, 16), np.uint8), np.zeros((16, 16), np.uint8),
                                 np.asarray([[1, 1]], np.int32), np.asarray([-1]), 16, 1)


def _run_some_steps(st, c, host, hot, steps):
    for t in range(steps):
        res = oracle.normalize(c.topk[t], np.arange(c.batch, dtype=np.int32), c.q_pos(t), c.window,
                               c.num_sinks, c.block_table, c.page_size, c.cap)
        oracle.hot_lookup_swapin(st, host, hot, res["slot"], np.full(c.batch, -1, np.int32),
                                 c.region_stride, c.batch)


def test_reset_restores_initial_state():
    # "HiSparse" walkthrough, HiSparseCoordinator: a recycled request slot's
    # stale state is dropped before reuse.  The initial state (stored id -1,
    # identity LRU order) is fixed independently by the cold-start closed form.
    c = workloads.hot_steps_case(seed=21, batch=4, ctx0=500, steps=4, top_k=24, window=4, sinks=2,
                                 page_size=16, heads=1)
    st = oracle.HotState(c.batch, c.hot_size)
    host = _bytes_pool(c.host_rows, 16, 7)
    hot = np.zeros((c.batch * c.region_stride, 16), np.uint8)
    _run_some_steps(st, c, host, hot, c.steps)
    assert np.any(st.dgi >= 0) and np.any(st.lru != np.arange(c.hot_size))
    before = st.copy()
    oracle.hot_reset(st, rows=np.asarray([2, 0], np.int32))
    for r in (0, 2):
        assert np.all(st.dgi[r] == -1)
        assert list(st.lru[r]) == list(range(c.hot_size))
    for r in (1, 3):  # rows outside the subset keep their state bit for bit
        assert np.array_equal(st.dgi[r], before.dgi[r])
        assert np.array_equal(st.lru[r], before.lru[r])
    oracle.hot_reset(st)
    fresh = oracle.HotState(c.batch, c.hot_size)
    assert np.array_equal(st.dgi, fresh.dgi) and np.array_equal(st.lru, fresh.lru)


def test_reset_row_replays_cold_start():
    # after a reset, the next lookup of M distinct ids is the cold-start
    # closed form: entries take slots 0 .. M-1 in order, LRU = [M..H-1, 0..M-1]
    H, M = 32, 9
    st = oracle.HotState(2, H)
    host = _bytes_pool(400, 16, 8)
    hot = np.zeros((2 * 64, 16), np.uint8)
    ids = np.full((2, 12), -1, np.int32)
    ids[:, :M] = np.arange(200, 200 + M)
    oracle.hot_lookup_swapin(st, host, hot, ids[:, ::-1].copy(), np.asarray([-1, -1]), 64, 2)
    ids2 = np.full((2, 12), -1, np.int32)
    ids2[:, :M] = np.arange(300, 300 + M)
    oracle.hot_reset(st, rows=[1])
    out, miss, stats = oracle.hot_lookup_swapin(st, host, hot, ids2, np.asarray([-1, -1]), 64, 2)
    assert list(out[1, :M]) == [64 + s for s in range(M)]
    assert list(st.lru[1]) == list(range(M, H)) + list(range(M))
    assert miss[1, :M].sum() == M
    # row 0 kept its state: its new misses skip the slots the first call filled
    assert set(out[0, :M].tolist()).isdisjoint(set(range(M)))


def test_reset_skips_rows_outside_state():
    st = oracle.HotState(2, 8)
    st.dgi[:] = 5
    st.lru[:] = 3
    oracle.hot_reset(st, rows=[-1, 2, 7])
    assert np.all(st.dgi == 5) and np.all(st.lru == 3)
