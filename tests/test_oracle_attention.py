"""Pins for the attention oracle (CPU only).

Fixed by mathematics: a pure-Python math.fsum triple loop; dense masked
softmax over all positions with -inf outside S ("5.1.1 · 从索引到 Kernel"
§1.2: masking the block union back to S); one-candidate and q = 0 closed
forms; S = all positions gives textbook decode attention; a doubled key
shifts its logit by exactly ln 2 (§7.3).  Fixed by the pages: the shifted
causal mask matrix of the PagedAttention page §3.2.
"""

import math

import numpy as np
import pytest

import oracle
import workloads


def _tiny():
    c = workloads.tiny_case()
    kv = workloads.pool_bits(c.kv_rows, c.pool_seed)
    res = oracle.normalize(c.topk, c.req_id, c.q_pos, c.window, c.num_sinks, c.block_table,
                           c.page_size, c.cap)
    return c, kv, res


def test_fsum_triple_loop_agrees():
    c, kv, res = _tiny()
    out, lse = oracle.attend_sparse(c.q_bits, kv, res["slot"], res["count"], c.scale)
    n = res["count"][0]
    rows = res["slot"][0, :n]
    qf = oracle.bf16_bits_to_f64(c.q_bits[0])
    K = oracle.bf16_bits_to_f64(kv[rows])
    heads = [0, 5, 15]
    o_ref, l_ref = oracle.attend_fsum([list(qf[h]) for h in heads], [list(k) for k in K],
                                      [list(k[:512]) for k in K], c.scale)
    for j, h in enumerate(heads):
        assert np.max(np.abs(out[0, h] - np.asarray(o_ref[j]))) < 1e-12
        assert abs(lse[0, h] - l_ref[j]) < 1e-12


def test_dense_masked_equals_sparse():
    c, kv, res = _tiny()
    out, lse = oracle.attend_sparse(c.q_bits, kv, res["slot"], res["count"], c.scale)
    # all 256 positions of the request, in logical order, masked to S
    table = c.block_table[0]
    slots_all = np.asarray([table[t // 64] * 64 + t % 64 for t in range(256)])
    K = oracle.bf16_bits_to_f64(kv[slots_all])
    member = np.zeros((1, 256), bool)
    member[0, res["tok"][0, :res["count"][0]]] = True
    Q = oracle.bf16_bits_to_f64(c.q_bits[0])
    o2, l2 = oracle.attend_dense_masked(Q, K, K[:, :512], np.repeat(member, c.H, axis=0), c.scale)
    assert np.max(np.abs(out[0] - o2)) < 1e-12
    assert np.max(np.abs(lse[0] - l2)) < 1e-12


def test_single_candidate_and_zero_query():
    rng = np.random.default_rng(3)
    kv = workloads.normal_bf16(rng, (50, 576))
    q = workloads.normal_bf16(rng, (2, 4, 576))
    q[1] = 0  # bf16 zero bits
    ids = np.full((2, 6), -1, np.int32)
    ids[0, 0] = 17
    ids[1, :5] = [1, 4, 9, 16, 25]
    out, lse = oracle.attend_sparse(q, kv, ids, None, 0.1)
    v = oracle.bf16_bits_to_f64(kv)
    z = 0.1 * oracle.bf16_bits_to_f64(q[0]) @ v[17]
    assert np.allclose(out[0], np.broadcast_to(v[17, :512], (4, 512)), atol=0, rtol=1e-15)
    assert np.allclose(lse[0], z, atol=1e-13)
    assert np.allclose(out[1], np.broadcast_to(v[[1, 4, 9, 16, 25], :512].mean(axis=0), (4, 512)),
                       atol=1e-14)
    assert np.allclose(lse[1], math.log(5))


def test_full_set_is_textbook_decode():
    rng = np.random.default_rng(4)
    L, H = 40, 3
    kv = workloads.normal_bf16(rng, (L, 576))
    q = workloads.normal_bf16(rng, (1, H, 576))
    out, _ = oracle.attend_sparse(q, kv, np.arange(L, dtype=np.int32)[None, :], None, 1 / 24)
    Q = oracle.bf16_bits_to_f64(q[0])
    K = oracle.bf16_bits_to_f64(kv)
    logits = Q @ K.T / 24
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    assert np.max(np.abs(out[0] - w @ K[:, :512])) < 1e-13


def test_doubled_key_shifts_logit_by_ln2():
    """A multiset that repeats key t equals the set with z_t + ln 2 (§7.3)."""
    rng = np.random.default_rng(5)
    kv = workloads.normal_bf16(rng, (8, 576))
    q = workloads.normal_bf16(rng, (1, 2, 576))
    dup = np.asarray([[0, 1, 2, 3, 3]], np.int32)
    out_dup, lse_dup = oracle.attend_sparse(q, kv, dup, None, 0.05)
    out_set, lse_set = oracle.attend_sparse(q, kv, dup[:, :4], None, 0.05)
    Q = oracle.bf16_bits_to_f64(q[0])
    K = oracle.bf16_bits_to_f64(kv[:4])
    z = 0.05 * Q @ K.T
    z[:, 3] += math.log(2)
    w = np.exp(z - z.max(axis=1, keepdims=True))
    ref = (w / w.sum(axis=1, keepdims=True)) @ K[:, :512]
    assert np.max(np.abs(out_dup[0] - ref)) < 1e-13
    assert np.max(np.abs(out_dup - out_set)) > 1e-3   # dedup changes the result


def test_shifted_causal_mask(golden):
    g = golden("shifted_mask_example.txt")
    m = oracle.shifted_causal_mask(g["Lq"][0], g["Lk"][0])
    assert m.astype(int).tolist() == [g["row0"], g["row1"], g["row2"]]
    # decode (Lq = 1) sees every position up to and including its own
    assert oracle.shifted_causal_mask(1, 9).all()


def test_empty_set():
    q = np.zeros((1, 2, 576), np.uint16)
    kv = np.zeros((4, 576), np.uint16)
    out, lse = oracle.attend_sparse(q, kv, np.full((1, 3), -1, np.int32), None, 1.0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("splits", [1, 2, 3, 8, 50])
def test_partial_then_merge_equals_single_pass(splits):
    c, kv, res = _tiny()
    out, lse = oracle.attend_sparse(c.q_bits, kv, res["slot"], res["count"], c.scale)
    o, m, l = oracle.attend_partial(c.q_bits, kv, res["slot"], res["count"], c.scale, splits)
    out2, lse2 = oracle.merge(o, m, l)
    assert np.max(np.abs(out - out2)) < 1e-13
    assert np.max(np.abs(lse - lse2)) < 1e-13
    if splits > res["count"][0]:
        assert np.any(l == 0)  # some splits are empty and must be ignored


def test_split_ranges():
    assert oracle.split_ranges(10, 3) == [(0, 4), (4, 8), (8, 10)]
    assert oracle.split_ranges(2, 4) == [(0, 1), (1, 2), (2, 2), (2, 2)]
    assert oracle.split_ranges(0, 2) == [(0, 0), (0, 0)]
