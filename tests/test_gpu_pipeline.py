"""GPU parity of the whole decode step with the hot buffer (all four stages).

Per step: normalise -> hot lookup / swap-in from pinned host memory ->
sparse decode over the hot cache -> back-up of the new rows.  The oracle
attends over the full host pool by slot id, so a wrong hit, a missed copy or
a stale row shows up as an attention error as well as a state mismatch.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_attention_close, bf16_dev, dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("splits", [1, 0])
def test_hot_decode_steps(splits):
    import sparse_top_paged_amd as stp
    c = workloads.hot_steps_case(seed=3100, batch=4, ctx0=3000, steps=5, top_k=128, window=16,
                                 sinks=4, page_size=64, heads=32)
    H, stride, P = c.hot_size, c.region_stride, c.page_size
    pool_bits = workloads.pool_bits(c.host_rows, c.pool_seed)          # full KV, bf16 bits
    host_np = pool_bits.view(np.uint8).reshape(c.host_rows, 1152).copy()
    host = torch.from_numpy(host_np.copy()).pin_memory()
    hot = torch.zeros((c.batch * stride, 1152), dtype=torch.uint8, device=dev())
    dgi = torch.empty((c.batch, H), dtype=torch.int32, device=dev())
    lru = torch.empty((c.batch, H), dtype=torch.int16, device=dev())
    stp.hot_reset(dgi, lru)
    table = to_dev(c.block_table)
    req = np.arange(c.batch, dtype=np.int32)
    for t in range(c.steps):
        q_pos = c.q_pos(t)
        newest = np.asarray([c.block_table[r][q_pos[r] // P] * P + q_pos[r] % P
                             for r in range(c.batch)], np.int32)
        # the step's new KV row (already in the host pool's bits) lands in the reserved row
        hot[torch.arange(c.batch, device=dev()) * stride + H] = to_dev(host_np[newest])
        norm = stp.normalize_indices(to_dev(c.topk[t]), to_dev(req), to_dev(q_pos), table, P,
                                     c.window, c.num_sinks, c.cap, block_view=False)
        rows, _, _ = stp.hot_lookup_swapin(host, hot, norm["slot"], to_dev(newest), dgi, lru,
                                           stride)
        kv = hot.view(torch.bfloat16).view(-1, 576)
        out, lse = stp.sparse_mla_decode(bf16_dev(c.q_bits[t]), kv, rows, norm["count"],
                                         576 ** -0.5, splits)
        stp.backup_rows(hot, host, to_dev(np.arange(c.batch, dtype=np.int32) * stride + H),
                        to_dev(newest))
        torch.cuda.synchronize()
        ref = oracle.normalize(c.topk[t], req, q_pos, c.window, c.num_sinks, c.block_table, P,
                               c.cap)
        o_ref, l_ref = oracle.attend_sparse(c.q_bits[t], pool_bits, ref["slot"], ref["count"],
                                            576 ** -0.5)
        assert_attention_close(out, lse, o_ref, l_ref, f"step {t}")


@pytest.mark.parametrize("splits", [1, 0])
def test_hot_decode_steps_fp8_rows(splits):
    """The same step over 656-byte fp8_ds_mla rows: the swap-in moves each row
    as 41 16-byte vectors, the fp8 decode reads the hot cache, the oracle
    dequantises the host pool rows by slot id."""
    import sparse_top_paged_amd as stp
    c = workloads.hot_steps_case(seed=3200, batch=4, ctx0=3000, steps=4, top_k=128, window=16,
                                 sinks=4, page_size=64, heads=32)
    H, stride, P = c.hot_size, c.region_stride, c.page_size
    host_np = workloads.fp8_rows(np.random.default_rng(3201), c.host_rows)
    host = torch.from_numpy(host_np.copy()).pin_memory()
    hot = torch.zeros((c.batch * stride, 656), dtype=torch.uint8, device=dev())
    dgi = torch.empty((c.batch, H), dtype=torch.int32, device=dev())
    lru = torch.empty((c.batch, H), dtype=torch.int16, device=dev())
    stp.hot_reset(dgi, lru)
    table = to_dev(c.block_table)
    req = np.arange(c.batch, dtype=np.int32)
    for t in range(c.steps):
        q_pos = c.q_pos(t)
        newest = np.asarray([c.block_table[r][q_pos[r] // P] * P + q_pos[r] % P
                             for r in range(c.batch)], np.int32)
        hot[torch.arange(c.batch, device=dev()) * stride + H] = to_dev(host_np[newest])
        norm = stp.normalize_indices(to_dev(c.topk[t]), to_dev(req), to_dev(q_pos), table, P,
                                     c.window, c.num_sinks, c.cap, block_view=False)
        rows, _, _ = stp.hot_lookup_swapin(host, hot, norm["slot"], to_dev(newest), dgi, lru,
                                           stride)
        out, lse = stp.sparse_mla_decode_fp8(bf16_dev(c.q_bits[t]), hot, rows, norm["count"],
                                             576 ** -0.5, splits)
        stp.backup_rows(hot, host, to_dev(np.arange(c.batch, dtype=np.int32) * stride + H),
                        to_dev(newest))
        torch.cuda.synchronize()
        ref = oracle.normalize(c.topk[t], req, q_pos, c.window, c.num_sinks, c.block_table, P,
                               c.cap)
        o_ref, l_ref = oracle.attend_sparse_fp8(c.q_bits[t], host_np, ref["slot"], ref["count"],
                                                576 ** -0.5)
        assert_attention_close(out, lse, o_ref, l_ref, f"fp8 step {t}")
        assert np.array_equal(host.numpy(), host_np)  # back-up rewrote the same bytes
