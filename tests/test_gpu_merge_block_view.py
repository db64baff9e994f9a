"""GPU parity: stp_splitkv_merge_with_block_view, the split merge and the
block view of the same tokens in one call.  Its block view equals the
one-call normalisation's and the oracle's bit for bit, and its merge equals
stp_splitkv_merge_normalized bit for bit (and the oracle's merge within the
attention bar).  Covered: the single launch (wide merge, LDS within 64 KiB) at
the DeepSeek-shaped size and with a 600-token look-back, and the two-launch
forms (more than eight splits, dv not a multiple of 8, a bitmap and table
row past 64 KiB)."""

import numpy as np
import pytest

import oracle
import workloads
from helpers import assert_attention_close, bf16_dev, bf16_bits_of, dev, to_dev

pytestmark = pytest.mark.gpu

KEYS = ["tok", "slot", "count", "dropped", "blk_indptr"]


def _case(name):
    if name == "deepseek":
        return workloads.deepseek_case(), 4, 128, 512
    if name == "lookback":
        return workloads.random_small_case(77, T=600, R=5, ctx=900, top_k=60, window=7, sinks=3,
                                           page_size=16), 3, 20, 512
    if name == "many_splits":
        return workloads.random_small_case(81, T=9, R=3, ctx=700, top_k=50, window=5, sinks=2,
                                           page_size=32), 9, 20, 512
    if name == "narrow":
        return workloads.random_small_case(82, T=9, R=3, ctx=700, top_k=50, window=5, sinks=2,
                                           page_size=32), 3, 20, 36
    if name == "global_table":
        return workloads.random_small_case(79, T=4, R=2, ctx=300000, top_k=500, window=100,
                                           sinks=2, page_size=1, unmapped_frac=0.01), 2, 20, 512
    return workloads.random_small_case(80, T=0, R=1, ctx=100, top_k=8, window=2, sinks=1,
                                       page_size=16), 2, 20, 512


def _partials(rng, T, S, H, dv):
    m = (rng.standard_normal((T, S, H)) * 4).astype(np.float32)
    l = rng.uniform(0.5, 30, size=(T, S, H)).astype(np.float32)
    on_bits = workloads.normal_bf16(rng, (T, S, H, dv))
    if T > 1:
        l[0, 0, :] = 0.0      # an empty split: its m must be ignored
        m[0, 0, :] = 1e30
        on_bits[0, 0] = 0
        l[1, :, 3] = 0.0      # a head with no live split
        on_bits[1, :, 3] = 0
    return m, l, on_bits


@pytest.mark.parametrize("name", ["deepseek", "lookback", "many_splits", "narrow", "global_table",
                                  "empty"])
def test_merge_with_block_view(name):
    import torch
    import sparse_top_paged_amd as stp
    c, S, H, dv = _case(name)
    T = c.topk.shape[0]
    print(f"[merge_with_block_view] {name}: T={T} S={S} H={H} dv={dv}", flush=True)
    args = [to_dev(np.asarray(a, np.int32)) for a in (c.topk, c.req_id, c.q_pos, c.block_table)]
    want = stp.normalize_indices(*args, c.page_size, c.window, c.num_sinks, c.cap)
    m, l, on_bits = _partials(np.random.default_rng(500 + T + S + dv), T, S, H, dv)
    on, md, ld = bf16_dev(on_bits), to_dev(m), to_dev(l)
    want_out, want_lse = stp.splitkv_merge_normalized(on, md, ld)
    torch.cuda.synchronize()
    want = {k: v.cpu().numpy() for k, v in want.items()}
    want_out, want_lse = bf16_bits_of(want_out), want_lse.cpu().numpy()
    for rep in range(2):
        got = stp.normalize_indices(*args, c.page_size, c.window, c.num_sinks, c.cap,
                                    defer_block_view=True)
        out, lse = stp.splitkv_merge_with_block_view(on, md, ld, got, args[1], args[2], args[3],
                                                     c.page_size)
        if rep == 1:
            # a repeated call over the completed arrays: the view is unchanged
            stp.splitkv_merge_with_block_view(on, md, ld, got, args[1], args[2], args[3],
                                              c.page_size, out=out, lse=lse)
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy() for k, v in got.items()}
        for k in KEYS:
            assert np.array_equal(got[k], want[k]), k
        nnz = int(want["blk_indptr"][-1]) if T else 0
        for k in ("blk_logical", "blk_page", "blk_mask"):
            assert np.array_equal(got[k][:nnz], want[k][:nnz]), k
        assert np.array_equal(bf16_bits_of(out), want_out)
        assert np.array_equal(lse.cpu().numpy(), want_lse, equal_nan=True)
    if T == 0:
        return
    # against the oracle: the block view exactly, the merge at the attention bar
    o = oracle.normalize(c.topk, c.req_id, c.q_pos, c.window, c.num_sinks, c.block_table,
                         c.page_size, c.cap)
    assert np.array_equal(got["blk_indptr"], o["blk_indptr"])
    nnz = int(o["blk_indptr"][-1])
    assert np.array_equal(got["blk_logical"][:nnz], o["blk_logical"])
    assert np.array_equal(got["blk_page"][:nnz], o["blk_page"])
    assert np.array_equal(got["blk_mask"][:nnz].view(np.uint64), o["blk_mask"])
    o_ref, l_ref = oracle.merge_normalized(oracle.bf16_bits_to_f64(on_bits), m.astype(np.float64),
                                           l.astype(np.float64))
    assert_attention_close(out, lse, o_ref, l_ref, f"merge with block view {name}")
    assert torch.all(out[1, 3] == 0) and torch.isneginf(lse[1, 3])
