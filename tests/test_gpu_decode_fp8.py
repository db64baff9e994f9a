"""GPU parity: sparse MLA decode over fp8_ds_mla rows (656 B) against the fp64 oracle.

The oracle reconstructs the rows as the kernel does (each latent value
bf16(f32(code) * scale), "5.1.1 · 从索引到 Kernel" §7.2: the correctness
baseline uses the same reconstructed KV) and attends in fp64; the GPU output
is bf16, compared with the bf16 decode's bar (helpers.assert_attention_close).
A candidate set of one row returns that row's value vector exactly (weight 1,
one term, and the reconstructed values are bf16 already), so those cases check
the reconstruction of every latent value through the kernel (all 254 finite
codes, subnormals and signed zeros included) bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_attention_close, bf16_dev, dev, to_dev

pytestmark = pytest.mark.gpu


def _decode(q_bits, rows, ids, counts, scale, splits):
    import sparse_top_paged_amd as stp
    out, lse = stp.sparse_mla_decode_fp8(bf16_dev(q_bits), to_dev(rows), to_dev(ids),
                                         None if counts is None else to_dev(counts), scale,
                                         splits)
    torch.cuda.synchronize()
    return out, lse


def _all_code_rows(rng, n):
    """Rows whose latent codes run through every finite E4M3 code."""
    rows = workloads.fp8_rows(rng, n)
    finite = np.asarray([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    for r in range(n):
        rows[r, :512] = np.roll(np.resize(finite, 512), 37 * r)
    return rows


@pytest.mark.parametrize("splits", [1, 3])
def test_single_row_returns_dequantised_values(splits):
    rng = np.random.default_rng(21)
    rows = _all_code_rows(rng, 6)
    rows[:, 512:528] = np.asarray([[2.0 ** -8, 0.37, 1.0, 3.5]] * 6, "<f4").view(np.uint8)
    T, H = 6, 64
    q = workloads.normal_bf16(rng, (T, H, 576))
    ids = np.full((T, 40), -1, np.int32)
    ids[:, 7] = np.arange(T)                 # one valid id per token, elsewhere in the list
    out, lse = _decode(q, rows, ids, None, 576 ** -0.5, splits)
    # out = the reconstructed V exactly: softmax weight 1 on one row, and the
    # reconstructed values are bf16 numbers already
    V = oracle.dequant_rows(rows)[:, :512]
    o = out.float().cpu().numpy().astype(np.float64)
    for t in range(T):
        assert np.array_equal(o[t], np.broadcast_to(V[t], o[t].shape)), f"token {t}"


@pytest.mark.parametrize("splits", [0, 1, 2, 5])
@pytest.mark.parametrize("H,cap", [(16, 1), (64, 31), (80, 33), (128, 100), (128, 700)])
def test_random_ragged(H, cap, splits):
    rng = np.random.default_rng(H * 1000 + cap)
    kv_rows = 3000
    rows = workloads.fp8_rows(rng, kv_rows)
    T = 3
    q = workloads.normal_bf16(rng, (T, H, 576))
    ids = rng.integers(-5, kv_rows + 5, size=(T, cap)).astype(np.int32)
    counts = np.asarray([cap, max(0, cap - 7), cap // 2], np.int32)
    out, lse = _decode(q, rows, ids, counts, 576 ** -0.5, splits)
    o_ref, l_ref = oracle.attend_sparse_fp8(q, rows, ids, counts, 576 ** -0.5)
    assert_attention_close(out, lse, o_ref, l_ref, f"H {H} cap {cap} splits {splits}")


@pytest.mark.parametrize("splits", [1, 2])
def test_long_splits(splits):
    """Splits longer than the 1120 ids staged at once (the id ring): one pass
    over 2600 candidates, or two of 1300; ids out of range in later tiles,
    counts short of the list (valid ids left past them)."""
    rng = np.random.default_rng(90 + splits)
    kv_rows, T, H, cap = 4000, 4, 64, 2600
    rows = workloads.fp8_rows(rng, kv_rows)
    q = workloads.normal_bf16(rng, (T, H, 576))
    ids = np.stack([rng.choice(kv_rows, size=cap, replace=False) for _ in range(T)]).astype(np.int32)
    ids[:, 1700] = -3
    ids[:, 2300] = kv_rows + 9
    counts = np.asarray([cap, 2301, 1121, 700], np.int32)
    out, lse = _decode(q, rows, ids, counts, 576 ** -0.5, splits)
    o_ref, l_ref = oracle.attend_sparse_fp8(q, rows, ids, counts, 576 ** -0.5)
    assert_attention_close(out, lse, o_ref, l_ref, f"fp8 long splits {splits}")


def test_empty_sets():
    rng = np.random.default_rng(5)
    rows = workloads.fp8_rows(rng, 50)
    q = workloads.normal_bf16(rng, (2, 64, 576))
    ids = np.full((2, 64), -1, np.int32)
    out, lse = _decode(q, rows, ids, np.asarray([0, 64], np.int32), 576 ** -0.5, 0)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_deepseek_shape_full_size():
    """Batch 32, 128 heads, context 32768, top-k 2048 + window 128 + 4 sinks, page
    64, over a 1,048,576-row fp8 pool (688 MB), normalise then decode with
    automatic splits; every token against the oracle."""
    import sparse_top_paged_amd as stp
    c = workloads.deepseek_case()
    kv = workloads.fp8_pool_torch(c.kv_rows, c.pool_seed, dev())
    norm = stp.normalize_indices(to_dev(c.topk), to_dev(c.req_id), to_dev(c.q_pos),
                                 to_dev(c.block_table), c.page_size, c.window, c.num_sinks, c.cap,
                                 block_view=False)
    out, lse = stp.sparse_mla_decode_fp8(bf16_dev(c.q_bits), kv, norm["slot"], norm["count"],
                                         c.scale)
    torch.cuda.synchronize()
    slots = norm["slot"].cpu().numpy()
    counts = norm["count"].cpu().numpy()
    for t in range(c.T):  # every token
        sl = slots[t, :counts[t]]
        rows = kv[torch.from_numpy(sl.astype(np.int64)).to(dev())].cpu().numpy()
        o_ref, l_ref = oracle.attend_sparse_fp8(c.q_bits[t:t + 1], rows,
                                                np.arange(len(sl), dtype=np.int32)[None, :], None,
                                                c.scale)
        assert_attention_close(out[t:t + 1], lse[t:t + 1], o_ref, l_ref, f"token {t}")
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
