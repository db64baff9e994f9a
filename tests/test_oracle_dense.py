"""Pins for the dense paged attention oracle (CPU only).

Fixed by the pages: the three-request ragged extend batch of the
PagedAttention page §3.3 (its metadata arrays), and the shifted causal mask
of §3.2 (pinned in test_oracle_attention.py).  Fixed by mathematics: a
pure-Python math.fsum loop over rows gathered by an independent position
loop, for decode and extend; identical keys give the mean of the values and
lse = z + ln n; a single key gives its value row; no prefix reduces the
extend to causal prefill (lower-triangular mask); one query per request
reduces it to the decode over the same slots.
"""

import math

import numpy as np

import oracle


def _pool(rng, slots, hkv, d):
    k = rng.standard_normal((slots, hkv, d)).astype(np.float16)
    v = rng.standard_normal((slots, hkv, d)).astype(np.float16)
    return k, v


def _fsum_attend(q_rows, K_rows, V_rows, scale):
    """Per query row: math.fsum softmax attention over the given key rows."""
    out, lse = oracle.attend_fsum([list(map(float, q)) for q in q_rows],
                                  [list(map(float, k)) for k in K_rows],
                                  [list(map(float, v)) for v in V_rows], scale)
    return np.asarray(out), np.asarray(lse)


def test_ragged_example_metadata(golden):
    g = golden("extend_ragged_example.txt")
    md = oracle.extend_metadata(g["extend_seq_lens"], g["seq_lens"])
    for key in ["qo_indptr", "kv_indptr", "extend_prefix_lens", "extend_start_loc"]:
        assert md[key].tolist() == g[key], key
    # the slots of each request are the printed slice of kv_indices
    kv = np.asarray(g["kv_indices"])
    assert kv[md["kv_indptr"][0]:md["kv_indptr"][1]].tolist() == [108, 109, 110, 111, 42, 43]
    assert kv[md["kv_indptr"][1]:md["kv_indptr"][2]].tolist() == [201, 202, 203]
    assert kv[md["kv_indptr"][2]:md["kv_indptr"][3]].tolist() == [80, 81, 82, 83, 84, 99]


def test_ragged_example_against_fsum(golden):
    g = golden("extend_ragged_example.txt")
    md = oracle.extend_metadata(g["extend_seq_lens"], g["seq_lens"])
    rng = np.random.default_rng(5)
    hq, hkv, d = 4, 2, 8
    k, v = _pool(rng, 256, hkv, d)
    N = md["qo_indptr"][-1]
    q = rng.standard_normal((N, hq, d)).astype(np.float16)
    out, lse = oracle.extend_attention(q, k, v, md["qo_indptr"], md["kv_indptr"],
                                       g["kv_indices"], 0.3)
    # independent: per request, per query row i, the keys j <= prefix + i by a loop
    kv = g["kv_indices"]
    for b in range(3):
        q0, pre = g["extend_start_loc"][b], g["extend_prefix_lens"][b]
        k0 = md["kv_indptr"][b]
        for i in range(g["extend_seq_lens"][b]):
            visible = [kv[k0 + j] for j in range(pre + i + 1)]
            for h in range(hq):
                grp = h // (hq // hkv)
                o_ref, l_ref = _fsum_attend([q[q0 + i, h]], [k[s, grp] for s in visible],
                                            [v[s, grp] for s in visible], 0.3)
                assert np.max(np.abs(out[q0 + i, h] - o_ref[0])) < 1e-12
                assert abs(lse[q0 + i, h] - l_ref[0]) < 1e-12


def test_decode_against_fsum_gather():
    rng = np.random.default_rng(6)
    B, hq, hkv, d, P = 3, 8, 2, 16, 4
    table = np.asarray([[5, 2, 9, 0], [7, 1, 3, 8], [4, 6, 11, 10]], np.int32)
    k, v = _pool(rng, 12 * P, hkv, d)
    ctx = np.asarray([13, 1, 16], np.int32)
    q = rng.standard_normal((B, hq, d)).astype(np.float16)
    out, lse = oracle.paged_gqa_decode(q, k, v, table, ctx, P, 0.25)
    for b in range(B):
        slots = []
        for t in range(ctx[b]):  # independent position loop
            slots.append(int(table[b][t // P]) * P + t % P)
        for h in range(hq):
            grp = h // (hq // hkv)
            o_ref, l_ref = _fsum_attend([q[b, h]], [k[s, grp] for s in slots],
                                        [v[s, grp] for s in slots], 0.25)
            assert np.max(np.abs(out[b, h] - o_ref[0])) < 1e-12
            assert abs(lse[b, h] - l_ref[0]) < 1e-12


def test_closed_forms():
    rng = np.random.default_rng(7)
    d, n = 16, 5
    krow = rng.standard_normal(d).astype(np.float16)
    k = np.tile(krow, (n, 1, 1))                        # n identical keys, one KV head
    v = rng.standard_normal((n, 1, d)).astype(np.float16)
    q = rng.standard_normal((1, 1, d)).astype(np.float16)
    out, lse = oracle.paged_gqa_decode(q, k, v, np.asarray([[0]], np.int32),
                                       np.asarray([n], np.int32), 8, 0.5)
    z = 0.5 * float(np.dot(q[0, 0].astype(np.float64), krow.astype(np.float64)))
    assert np.allclose(out[0, 0], v[:, 0].astype(np.float64).mean(axis=0), atol=1e-13)
    assert abs(lse[0, 0] - (z + math.log(n))) < 1e-12
    out1, lse1 = oracle.paged_gqa_decode(q, k, v, np.asarray([[0]], np.int32),
                                         np.asarray([1], np.int32), 8, 0.5)
    assert np.array_equal(out1[0, 0], v[0, 0].astype(np.float64))
    assert abs(lse1[0, 0] - z) < 1e-13
    out0, lse0 = oracle.paged_gqa_decode(q, k, v, np.asarray([[0]], np.int32),
                                         np.asarray([0], np.int32), 8, 0.5)
    assert np.all(out0 == 0) and np.isneginf(lse0[0, 0])


def test_no_prefix_is_causal_prefill_and_one_query_is_decode():
    rng = np.random.default_rng(8)
    hq, hkv, d, P = 4, 4, 8, 4
    k, v = _pool(rng, 64, hkv, d)
    # no prefix: the mask is the lower triangle
    assert np.array_equal(oracle.shifted_causal_mask(6, 6), np.tril(np.ones((6, 6), bool)))
    # one query per request: extend == decode over the same slots
    table = np.asarray([[3, 0, 7, 1], [2, 9, 4, 5]], np.int32)
    ctx = np.asarray([11, 6], np.int32)
    q = rng.standard_normal((2, hq, d)).astype(np.float16)
    dec, dlse = oracle.paged_gqa_decode(q, k, v, table, ctx, P, 0.4)
    slots = [oracle.decode_slots(table[b], ctx[b], P) for b in range(2)]
    md = oracle.extend_metadata([1, 1], ctx)
    ext, else_ = oracle.extend_attention(q, k, v, md["qo_indptr"], md["kv_indptr"],
                                         np.concatenate(slots), 0.4)
    assert np.max(np.abs(dec - ext)) < 1e-14 and np.max(np.abs(dlse - else_)) < 1e-14


def test_bad_ids_take_no_part():
    """Unmapped pages (entry < 0), blocks past the end of the table, slots
    outside the pool (decode) and kv_indices outside the pool (extend) drop
    out: the result equals an fsum over the remaining rows only."""
    rng = np.random.default_rng(9)
    hq, hkv, d, P = 4, 2, 8, 4
    slots_n = 40
    k, v = _pool(rng, slots_n, hkv, d)
    # request 0: page 1 unmapped, page 3 = 12 -> slots 48..51 outside the pool;
    # request 1: ctx 14 with a 3-entry table -> tokens 12, 13 past the table
    table = np.asarray([[2, -1, 5, 12], [0, 7, 3, 0]], np.int32)[:, :4]
    table_short = table[:, :3]
    ctx = np.asarray([16, 14], np.int32)
    q = rng.standard_normal((2, hq, d)).astype(np.float16)
    out, lse = oracle.paged_gqa_decode(q, k, v, table_short, ctx, P, 0.3)
    out4, lse4 = oracle.paged_gqa_decode(q, k, v, table, ctx, P, 0.3)
    for b, tab in ((0, table_short[0]), (1, table_short[1])):
        live = []
        for t in range(ctx[b]):
            blk = t // P
            if blk < len(tab) and tab[blk] >= 0 and tab[blk] * P + t % P < slots_n:
                live.append(int(tab[blk]) * P + t % P)
        for h in range(hq):
            g = h // (hq // hkv)
            o_ref, l_ref = _fsum_attend([q[b, h]], [k[s, g] for s in live],
                                        [v[s, g] for s in live], 0.3)
            assert np.max(np.abs(out[b, h] - o_ref[0])) < 1e-12
            assert abs(lse[b, h] - l_ref[0]) < 1e-12
    # request 0's fourth page maps outside the pool: the same result
    assert np.max(np.abs(out4[0] - out[0])) < 1e-14
    # extend: kv slots -1 and 45 drop out of request 0's keys
    kvi = np.asarray([3, -1, 17, 45, 8, 9, 30], np.int32)
    qo, kvp = np.asarray([0, 3]), np.asarray([0, 7])
    qe = rng.standard_normal((3, hq, d)).astype(np.float16)
    oe, le = oracle.extend_attention(qe, k, v, qo, kvp, kvi, 0.3)
    for i in range(3):
        live = [int(kvi[j]) for j in range(i + 4 + 1) if 0 <= kvi[j] < slots_n]
        for h in range(hq):
            g = h // (hq // hkv)
            o_ref, l_ref = _fsum_attend([qe[i, h]], [k[s, g] for s in live],
                                        [v[s, g] for s in live], 0.3)
            assert np.max(np.abs(oe[i, h] - o_ref[0])) < 1e-12
            assert abs(le[i, h] - l_ref[0]) < 1e-12
