"""GPU parity: sparse MLA decode (stage 3), its partial states and the merge (stage 4).

The oracle computes in fp64 from the same bf16 inputs; the GPU output is bf16.
Tolerance (helpers.assert_attention_close): |err| <= 2e-2 per element, per
(token, head) max error <= 1e-2 of the reference's largest magnitude, and
|lse err| <= 1e-2.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_attention_close, bf16_bits_of, bf16_dev, dev, to_dev

pytestmark = pytest.mark.gpu


def _decode(q_bits, kv, ids, counts, scale, splits):
    import sparse_top_paged_amd as stp
    out, lse = stp.sparse_mla_decode(bf16_dev(q_bits), kv, to_dev(ids),
                                     None if counts is None else to_dev(counts), scale, splits)
    torch.cuda.synchronize()
    return out, lse


def _tiny():
    c = workloads.tiny_case()
    kv_bits = workloads.pool_bits(c.kv_rows, c.pool_seed)
    ref = oracle.normalize(c.topk, c.req_id, c.q_pos, c.window, c.num_sinks, c.block_table,
                           c.page_size, c.cap)
    return c, kv_bits, ref


@pytest.mark.parametrize("splits", [0, 1, 2, 3, 7])
def test_tiny_case(splits):
    c, kv_bits, ref = _tiny()
    out, lse = _decode(c.q_bits, bf16_dev(kv_bits), ref["slot"], ref["count"], c.scale, splits)
    o_ref, l_ref = oracle.attend_sparse(c.q_bits, kv_bits, ref["slot"], ref["count"], c.scale)
    assert_attention_close(out, lse, o_ref, l_ref, f"tiny splits={splits}")


@pytest.mark.parametrize("H", [8, 16, 64, 80, 128, 192])
@pytest.mark.parametrize("cap", [1, 31, 33, 100])
def test_head_counts_and_ragged_tiles(H, cap):
    rng = np.random.default_rng(H * 1000 + cap)
    T, rows = 3, 500
    kv_bits = workloads.normal_bf16(rng, (rows, 576))
    q_bits = workloads.normal_bf16(rng, (T, H, 576))
    ids = np.full((T, cap), -1, np.int32)
    counts = np.zeros(T, np.int32)
    for t in range(T):
        n = [cap, max(1, cap // 2), max(0, cap - 7)][t]
        ids[t, :n] = rng.choice(rows, size=n, replace=False)
        counts[t] = n
    for splits in (1, 2):
        out, lse = _decode(q_bits, bf16_dev(kv_bits), ids, counts, 1 / 24, splits)
        o_ref, l_ref = oracle.attend_sparse(q_bits, kv_bits, ids, counts, 1 / 24)
        assert_attention_close(out, lse, o_ref, l_ref, f"H={H} cap={cap} splits={splits}")


def test_invalid_ids_and_no_counts():
    rng = np.random.default_rng(5)
    rows = 300
    kv_bits = workloads.normal_bf16(rng, (rows, 576))
    q_bits = workloads.normal_bf16(rng, (4, 16, 576))
    ids = rng.integers(-3, rows + 40, size=(4, 70)).astype(np.int32)  # -ids, out of range
    ids[2] = -1                                                        # an all-invalid row
    for splits in (1, 3):
        out, lse = _decode(q_bits, bf16_dev(kv_bits), ids, None, 0.05, splits)
        o_ref, l_ref = oracle.attend_sparse(q_bits, kv_bits, ids, None, 0.05)
        assert_attention_close(out, lse, o_ref, l_ref, f"invalid ids splits={splits}")
        assert torch.all(out[2] == 0) and torch.all(torch.isneginf(lse[2]))


def test_empty_single_and_equal_logits():
    rng = np.random.default_rng(6)
    rows = 64
    kv_bits = workloads.normal_bf16(rng, (rows, 576))
    q_bits = workloads.normal_bf16(rng, (3, 32, 576))
    q_bits[2] = 0                                      # every logit equal -> mean of V rows
    ids = np.full((3, 40), -1, np.int32)
    ids[1, 0] = 17                                     # a single candidate
    ids[2, :40] = np.arange(40)
    counts = np.asarray([0, 1, 40], np.int32)          # row 0 is empty
    out, lse = _decode(q_bits, bf16_dev(kv_bits), ids, counts, 1 / 24, 1)
    o_ref, l_ref = oracle.attend_sparse(q_bits, kv_bits, ids, counts, 1 / 24)
    assert_attention_close(out, lse, o_ref, l_ref, "edge rows")
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    # one candidate: the output is its V row exactly (bf16 in, bf16 out)
    v = kv_bits[17, :512]
    assert np.array_equal(bf16_bits_of(out[1]), np.broadcast_to(v, (32, 512)))
    assert abs(float(lse[2, 0]) - math.log(40)) < 1e-5


@pytest.mark.parametrize("gain", [8.0, 40.0])
def test_extreme_logits(gain):
    """Large logits: the online max must move by far more than the rescale threshold."""
    rng = np.random.default_rng(int(gain))
    rows = 400
    kv_bits = workloads.normal_bf16(rng, (rows, 576))
    q = rng.standard_normal((2, 64, 576)).astype(np.float32) * gain
    q_bits = workloads.bf16_bits(q)
    ids = np.stack([rng.permutation(rows)[:300] for _ in range(2)]).astype(np.int32)
    # token 0 lists its rows by ascending head-0 logit, so that head's running
    # max rises tile after tile (input construction only)
    z0 = workloads.bf16_bits(q[0, 0:1]).astype(np.uint32) << 16
    qv = z0.view(np.float32).astype(np.float64)[0]
    kvf = (kv_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ids[0] = ids[0][np.argsort(kvf[ids[0]] @ qv)]
    for splits in (1, 4):
        out, lse = _decode(q_bits, bf16_dev(kv_bits), ids, None, 1 / 24, splits)
        o_ref, l_ref = oracle.attend_sparse(q_bits, kv_bits, ids, None, 1 / 24)
        assert_attention_close(out, lse, o_ref, l_ref, f"gain={gain} splits={splits}")


@pytest.mark.parametrize("splits", [1, 2, 5, 8])
def test_partial_states(splits):
    import sparse_top_paged_amd as stp
    c, kv_bits, ref = _tiny()
    o, m, l = stp.sparse_mla_decode_partial(bf16_dev(c.q_bits), bf16_dev(kv_bits),
                                            to_dev(ref["slot"]), to_dev(ref["count"]), c.scale,
                                            splits)
    torch.cuda.synchronize()
    o_r, m_r, l_r = oracle.attend_partial(c.q_bits, kv_bits, ref["slot"], ref["count"], c.scale,
                                          splits)
    o, m, l = (x.cpu().numpy().astype(np.float64) for x in (o, m, l))
    live = l_r > 0
    assert np.array_equal(l > 0, live)
    assert np.all(np.isneginf(m[~live])) and np.all(o[~live] == 0)
    assert np.max(np.abs(m[live] - m_r[live])) < 1e-4           # the split's max logit
    assert np.max(np.abs(np.log(l[live]) - np.log(l_r[live]))) < 1e-2
    norm = o[live] / l[live][:, None]
    norm_r = o_r[live] / l_r[live][:, None]
    assert np.max(np.abs(norm - norm_r)) < 2e-2
    # the library merge of these states equals the single pass
    out, lse = stp.splitkv_merge(*(torch.from_numpy(x.astype(np.float32)).to(dev()) for x in (o, m, l)))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attend_sparse(c.q_bits, kv_bits, ref["slot"], ref["count"], c.scale)
    assert_attention_close(out, lse, o_ref, l_ref, f"partial+merge splits={splits}")


@pytest.mark.parametrize("splits", [1, 3, 8])
def test_partial_states_normalized(splits):
    """The split path of sparse_mla_decode: bf16 o / l per split, then the
    partition-combine merge."""
    import sparse_top_paged_amd as stp
    c, kv_bits, ref = _tiny()
    o, m, l = stp.sparse_mla_decode_partial_normalized(bf16_dev(c.q_bits), bf16_dev(kv_bits),
                                                       to_dev(ref["slot"]), to_dev(ref["count"]),
                                                       c.scale, splits)
    torch.cuda.synchronize()
    o_r, m_r, l_r = oracle.attend_partial(c.q_bits, kv_bits, ref["slot"], ref["count"], c.scale,
                                          splits)
    on = o.float().cpu().numpy().astype(np.float64)
    m, l = (x.cpu().numpy().astype(np.float64) for x in (m, l))
    live = l_r > 0
    assert np.array_equal(l > 0, live)
    assert np.all(np.isneginf(m[~live])) and np.all(on[~live] == 0)
    assert np.max(np.abs(m[live] - m_r[live])) < 1e-4
    assert np.max(np.abs(np.log(l[live]) - np.log(l_r[live]))) < 1e-2
    norm_r = o_r[live] / l_r[live][:, None]
    assert np.max(np.abs(on[live] - norm_r)) < 2e-2
    out, lse = stp.splitkv_merge_normalized(
        o, *(torch.from_numpy(x.astype(np.float32)).to(dev()) for x in (m, l)))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attend_sparse(c.q_bits, kv_bits, ref["slot"], ref["count"], c.scale)
    assert_attention_close(out, lse, o_ref, l_ref, f"normalized partial+merge splits={splits}")


@pytest.mark.parametrize("S,dv", [(1, 512), (2, 512), (8, 512), (33, 512), (3, 36), (5, 1024),
                                  (4, 8)])
def test_merge_normalized_against_oracle(S, dv):
    # dv % 8 == 0 with S <= 8: 16-byte slices, four heads per workgroup
    # (dv 1024: two slices per thread; dv 8: one thread per head); dv 36 and
    # S 33: two heads per workgroup, 8-byte slices
    import sparse_top_paged_amd as stp
    rng = np.random.default_rng(100 + S + dv)
    T, H = 3, 20
    m = (rng.standard_normal((T, S, H)) * 4).astype(np.float32)
    l = rng.uniform(0.5, 30, size=(T, S, H)).astype(np.float32)
    on_bits = workloads.normal_bf16(rng, (T, S, H, dv))
    l[0, 0, :] = 0.0
    m[0, 0, :] = 1e30
    on_bits[0, 0] = 0
    l[2, :, 3] = 0.0
    on_bits[2, :, 3] = 0
    out, lse = stp.splitkv_merge_normalized(bf16_dev(on_bits),
                                            *(torch.from_numpy(x).to(dev()) for x in (m, l)))
    torch.cuda.synchronize()
    on = oracle.bf16_bits_to_f64(on_bits)
    o_ref, l_ref = oracle.merge_normalized(on, m.astype(np.float64), l.astype(np.float64))
    assert_attention_close(out, lse, o_ref, l_ref, f"merge normalized S={S} dv={dv}")
    assert torch.all(out[2, 3] == 0) and torch.isneginf(lse[2, 3])


@pytest.mark.parametrize("S", [1, 2, 8, 33])
def test_merge_against_oracle(S):
    import sparse_top_paged_amd as stp
    rng = np.random.default_rng(S)
    T, H, dv = 3, 20, 512
    m = (rng.standard_normal((T, S, H)) * 4).astype(np.float32)
    l = rng.uniform(0.5, 30, size=(T, S, H)).astype(np.float32)
    o = (rng.standard_normal((T, S, H, dv)) * l[..., None] * 0.1).astype(np.float32)
    l[0, 0, :] = 0.0                     # an empty split: its m must be ignored
    m[0, 0, :] = 1e30
    o[0, 0] = 0.0
    l[2, :, 3] = 0.0                     # a head with no live split
    o[2, :, 3] = 0.0
    out, lse = stp.splitkv_merge(*(torch.from_numpy(x).to(dev()) for x in (o, m, l)))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.merge(o.astype(np.float64), m.astype(np.float64), l.astype(np.float64))
    assert_attention_close(out, lse, o_ref, l_ref, f"merge S={S}")
    assert torch.all(out[2, 3] == 0) and torch.isneginf(lse[2, 3])


def _full_check(case, kv, out, lse, tokens, where):
    """Oracle over the given tokens at full size (every (token, head) element), from rows
    copied back from the pool."""
    ref = oracle.normalize(case.topk[tokens], case.req_id[tokens], case.q_pos[tokens], case.window,
                           case.num_sinks, case.block_table, case.page_size, case.cap)
    print(f"[{where}] comparing {len(tokens)} tokens with the oracle", flush=True)
    for j, t in enumerate(tokens):
        n = ref["count"][j]
        rows = ref["slot"][j, :n]
        kv_rows = bf16_bits_of(kv[torch.from_numpy(rows.astype(np.int64)).to(kv.device)])
        o_ref, l_ref = oracle.attend_sparse(case.q_bits[t:t + 1], kv_rows,
                                            np.arange(n, dtype=np.int32)[None, :], None, case.scale)
        assert_attention_close(out[t:t + 1], lse[t:t + 1], o_ref, l_ref, f"{where} token {t}")


def test_deepseek_shape_full_size():
    """Batch 32, 128 heads, context 32768, top-k 2048 + window 128 + 4 sinks, page 64, in the
    benchmark's launch configuration (normalise, then decode with automatic splits)."""
    import sparse_top_paged_amd as stp
    c = workloads.deepseek_case()
    kv = workloads.pool_torch(c.kv_rows, c.pool_seed, dev())
    norm = stp.normalize_indices(to_dev(c.topk), to_dev(c.req_id), to_dev(c.q_pos),
                                 to_dev(c.block_table), c.page_size, c.window, c.num_sinks, c.cap,
                                 block_view=False)
    out, lse = stp.sparse_mla_decode(bf16_dev(c.q_bits), kv, norm["slot"], norm["count"], c.scale)
    torch.cuda.synchronize()
    # every token: the kernel places token t on XCD t % 8 and its split edges vary by token
    _full_check(c, kv, out, lse, list(range(c.T)), "deepseek")
    del kv


@pytest.mark.parametrize("clustered", [False, True])
def test_long_context_eight_splits(clustered):
    """Batch 64, context 131072 (9.7 GB pool), top-k only, 8-way split then merge."""
    import sparse_top_paged_amd as stp
    c = workloads.locality_case(4002 if clustered else 4001, clustered)
    kv = workloads.pool_torch(c.kv_rows, c.pool_seed, dev())
    norm = stp.normalize_indices(to_dev(c.topk), to_dev(c.req_id), to_dev(c.q_pos),
                                 to_dev(c.block_table), c.page_size, c.window, c.num_sinks, c.cap,
                                 block_view=False)
    out, lse = stp.sparse_mla_decode(bf16_dev(c.q_bits), kv, norm["slot"], norm["count"], c.scale,
                                     num_splits=8)
    torch.cuda.synchronize()
    _full_check(c, kv, out, lse, list(range(c.T)), "long context")
    del kv
    torch.cuda.empty_cache()


def _long_lists(rng, T, H, cap, rows):
    """Lists longer than the 1120 ids a workgroup stages at once: full, ragged
    and short counts, valid ids left in the list past each count (they must
    not be read), and invalid ids (negative, past the pool) in later tiles."""
    kv_bits = workloads.normal_bf16(rng, (rows, 576))
    q_bits = workloads.normal_bf16(rng, (T, H, 576))
    ids = np.stack([rng.choice(rows, size=cap, replace=False) for _ in range(T)]).astype(np.int32)
    counts = np.asarray([cap, cap - 1, 1121, 1120, 1119, 35 * 32 * 2 + 17, 40, 0][:T], np.int32)
    for t in range(T):
        if counts[t] > 1500:
            ids[t, 1500] = -7                 # invalid ids past the first ring turn
            ids[t, counts[t] - 2] = rows + 3
    return q_bits, kv_bits, ids, counts


@pytest.mark.parametrize("splits", [1, 2])
def test_long_splits_single_pass(splits):
    """num_splits = 1 is one pass per token over all 3000 candidates (no merge);
    2 splits give 1500 each: both longer than the LDS id list, so the ids go
    through the ring (35 tiles) and are range-checked where they are read."""
    import sparse_top_paged_amd as stp
    rng = np.random.default_rng(77 + splits)
    T, H, cap, rows = 8, 64, 3000, 6000
    q_bits, kv_bits, ids, counts = _long_lists(rng, T, H, cap, rows)
    assert stp.decode_splits(T, H, cap, splits) == splits
    assert stp.decode_workspace_bytes(T, H, cap, 1) == 0
    out, lse = _decode(q_bits, bf16_dev(kv_bits), ids, counts, 0.04, splits)
    o_ref, l_ref = oracle.attend_sparse(q_bits, kv_bits, ids, counts, 0.04)
    assert_attention_close(out, lse, o_ref, l_ref, f"long lists, {splits} split(s)")
    assert torch.all(out[7] == 0) and torch.all(torch.isneginf(lse[7]))


def test_long_split_partial_states():
    """The unnormalised partial states of two 1500-candidate splits, merged,
    against the oracle's partials and the single pass."""
    import sparse_top_paged_amd as stp
    rng = np.random.default_rng(78)
    T, H, cap, rows = 6, 64, 3000, 6000
    q_bits, kv_bits, ids, counts = _long_lists(rng, T, H, cap, rows)
    q, kv = bf16_dev(q_bits), bf16_dev(kv_bits)
    o_p, m_p, l_p = stp.sparse_mla_decode_partial(q, kv, to_dev(ids), to_dev(counts), 0.04, 2)
    out, lse = stp.splitkv_merge(o_p, m_p, l_p)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attend_sparse(q_bits, kv_bits, ids, counts, 0.04)
    assert_attention_close(out, lse, o_ref, l_ref, "long partial states, merged")


def test_deepseek_shape_single_pass():
    """The 32-token, 2180-candidate decode with num_splits = 1: one pass per
    (token, head group) over the whole list, every token against the oracle."""
    import sparse_top_paged_amd as stp
    c = workloads.deepseek_case()
    kv = workloads.pool_torch(c.kv_rows, c.pool_seed, dev())
    norm = stp.normalize_indices(to_dev(c.topk), to_dev(c.req_id), to_dev(c.q_pos),
                                 to_dev(c.block_table), c.page_size, c.window, c.num_sinks, c.cap,
                                 block_view=False)
    out, lse = stp.sparse_mla_decode(bf16_dev(c.q_bits), kv, norm["slot"], norm["count"], c.scale,
                                     num_splits=1)
    torch.cuda.synchronize()
    _full_check(c, kv, out, lse, list(range(c.T)), "single pass")
    del kv
