"""Pins for the normalisation oracle (CPU only).

Fixed by the pages: the two worked index examples of "5.1.1 · 从索引到 Kernel"
§1.2.  Fixed by construction: a brute-force scan over every position on tiny
random inputs (a different construction from the oracle's set union), and
the invariants of eq. (1) (dedup, ordering) and eq. (17) (slot injectivity).
"""

import numpy as np
import pytest

import oracle
import workloads


def _one_row_normalize(cands, table, page_size, q, window=0, sinks=0):
    topk = np.asarray([cands], dtype=np.int32)
    bt = np.asarray([table], dtype=np.int32)
    return oracle.normalize(topk, np.zeros(1, np.int32), np.asarray([q], np.int32), window, sinks,
                            bt, page_size, cap=len(cands) + window + sinks)


@pytest.mark.parametrize("name", ["index_example_page64.txt", "index_example_page16.txt"])
def test_worked_index_examples(golden, name):
    g = golden(name)
    P = g["page_size"][0]
    cands = g["candidates"]
    q = max(cands)  # w = a = 0 and q at the last candidate: nothing is filtered
    res = _one_row_normalize(cands, g["table"], P, q)
    n = res["count"][0]
    assert n == len(cands)
    assert list(res["tok"][0, :n]) == sorted(cands)
    assert list(res["slot"][0, :n]) == g["slots"]
    assert list(res["blk_logical"]) == g["indices"]
    assert list(res["blk_page"]) == g["pages"]
    if "indptr" in g:
        assert list(res["blk_indptr"]) == g["indptr"]
    for b, key in enumerate(["offsets_block0", "offsets_block1"]):
        mask = int(res["blk_mask"][b])
        assert [o for o in range(64) if mask >> o & 1] == g[key]
    assert res["dropped"][0] == 0


def _brute_force(topk_row, q, window, sinks, table_row, P):
    """Scan every position 0..q and keep it if it is a member and mapped."""
    D = [int(t) for t in topk_row]
    S = []
    for t in range(0, q + 1):
        member = (t in D) or (window > 0 and q - window < t) or (t < sinks)
        b = t // P
        mapped = b < len(table_row) and table_row[b] >= 0
        if member and mapped:
            S.append(t)
    dropped = 0
    for t in D:
        if t < 0:
            continue
        b = t // P
        if t > q or b >= len(table_row) or table_row[b] < 0:
            dropped += 1
    return S, dropped


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_small(seed):
    c = workloads.random_small_case(seed, T=4, R=3, ctx=90 + seed * 7, top_k=24, window=seed % 6,
                                    sinks=seed % 4, page_size=[1, 4, 15, 16, 17, 64][seed % 6])
    res = oracle.normalize(c.topk, c.req_id, c.q_pos, c.window, c.num_sinks, c.block_table,
                           c.page_size, c.cap)
    for i in range(c.T):
        r = c.req_id[i]
        S, nd = _brute_force(c.topk[i], int(c.q_pos[i]), c.window, c.num_sinks, c.block_table[r],
                             c.page_size)
        n = res["count"][i]
        assert list(res["tok"][i, :n]) == S
        assert res["dropped"][i] == nd
        assert np.all(res["tok"][i, n:] == -1) and np.all(res["slot"][i, n:] == -1)
        for j, t in enumerate(S):
            assert res["slot"][i, j] == c.block_table[r][t // c.page_size] * c.page_size + t % c.page_size


def _brute_force_int32(topk_row, q, window, sinks, table_row, P):
    """Positions 0..q that are members, mapped, and whose slot page * P +
    offset is at most 2^31 - 1; D entries >= 0 failing any of those count as
    dropped."""
    def visible(t):
        b = t // P
        if t > q or b >= len(table_row) or table_row[b] < 0:
            return False
        return int(table_row[b]) * P + t % P <= 2**31 - 1
    D = [int(t) for t in topk_row]
    S = [t for t in range(q + 1)
         if ((t in D) or (window > 0 and q - window < t) or (t < sinks)) and visible(t)]
    dropped = sum(1 for t in D if t >= 0 and not visible(t))
    return S, dropped


def test_slots_past_int32_are_dropped():
    c = workloads.int32_edge_case()
    res = oracle.normalize(c.topk, c.req_id, c.q_pos, c.window, c.num_sinks, c.block_table,
                           c.page_size, c.cap)
    lost = 0
    for i in range(c.T):
        r = c.req_id[i]
        S, nd = _brute_force_int32(c.topk[i], int(c.q_pos[i]), c.window, c.num_sinks,
                                   c.block_table[r], c.page_size)
        n = res["count"][i]
        assert list(res["tok"][i, :n]) == S
        assert res["dropped"][i] == nd
        slots = [int(c.block_table[r][t // 48]) * 48 + t % 48 for t in S]
        assert list(res["slot"][i, :n]) == slots and max(slots, default=0) <= 2**31 - 1
        if r == 0:  # the sinks sit in page 0's kept offsets; page 1 contributes nothing
            assert all(t < 32 or t >= 96 for t in S) and {0, 1, 2} <= set(S)
            lost += sum(1 for t in range(32, min(96, int(c.q_pos[i]) + 1))
                        if t in set(int(x) for x in c.topk[i]))
    assert lost > 0  # the case does exercise the rule


def test_duplicates_count_once_and_order_free():
    c = workloads.random_small_case(5, T=2, R=2, ctx=200, top_k=30)
    base = oracle.normalize(c.topk, c.req_id, c.q_pos, c.window, c.num_sinks, c.block_table,
                            c.page_size, c.cap)
    rng = np.random.default_rng(0)
    # appending every entry a second time and shuffling must not change S
    doubled = np.concatenate([c.topk, c.topk], axis=1)
    doubled = np.stack([rng.permutation(r) for r in doubled])
    res = oracle.normalize(doubled, c.req_id, c.q_pos, c.window, c.num_sinks, c.block_table,
                           c.page_size, c.cap)
    assert np.array_equal(res["tok"], base["tok"])
    assert np.array_equal(res["slot"], base["slot"])
    assert np.array_equal(res["dropped"], 2 * base["dropped"])  # dropped counts entries


def test_invariants_deepseek_shape():
    c = workloads.deepseek_case(batch=3, ctx=4096, heads=2, top_k=256, window=128, sinks=4)
    res = oracle.normalize(c.topk, c.req_id, c.q_pos, c.window, c.num_sinks, c.block_table,
                           c.page_size, c.cap)
    ip = res["blk_indptr"]
    for i in range(c.T):
        n = res["count"][i]
        tok = res["tok"][i, :n]
        assert np.all(np.diff(tok) > 0)                          # strictly ascending
        assert len(set(res["slot"][i, :n].tolist())) == n       # injective
        # every window and sink position is present
        q = int(c.q_pos[i])
        assert set(range(q - 127, q + 1)) <= set(tok.tolist())
        assert set(range(4)) <= set(tok.tolist())
        # block view covers exactly S
        masks = res["blk_mask"][ip[i]:ip[i + 1]]
        assert sum(bin(int(m)).count("1") for m in masks) == n
        assert np.all(np.diff(res["blk_logical"][ip[i]:ip[i + 1]]) > 0)


def test_padding_rows_and_empty():
    topk = np.asarray([[3, 4], [1, 2], [5, -1]], dtype=np.int32)
    bt = np.asarray([[0, 1]], dtype=np.int32)
    res = oracle.normalize(topk, np.asarray([-1, 0, 5], np.int32), np.asarray([10, -1, 10], np.int32),
                           2, 1, bt, 8, cap=5)
    assert list(res["count"]) == [0, 0, 0]
    assert list(res["dropped"]) == [0, 0, 0]
    assert list(res["blk_indptr"]) == [0, 0, 0, 0]


def test_cap_overflow_raises():
    topk = np.arange(10, dtype=np.int32)[None, :]
    bt = np.asarray([[0, 1]], dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.normalize(topk, np.zeros(1, np.int32), np.asarray([15], np.int32), 0, 0, bt, 8, cap=5)
