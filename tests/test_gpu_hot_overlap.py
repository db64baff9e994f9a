"""GPU parity of the hot-buffer decode step with the swap-in on a side stream.

"[HiCache] TMA-staged host<->device KV transfer kernel (sm_90+)", Motivation:
host-to-device loads run on a side stream while the forward pass runs;
"HiSparse" walkthrough, overview: the SwapIn interface.  The request rows
are split into chunks; chunk k+1's lookup / LRU / swap-in runs on a second
stream while chunk k's attention runs on the main stream, the two ordered by
HIP events (chunk k's decode waits for chunk k's swap-in; the next step's
first swap-in follows the back-up through the step's normalisation).  Each
request row's hot state is its own, so the chunked schedule must give, bit
for bit, the oracle's hot rows, miss masks, hit / miss counts, stored ids,
LRU order and hot-cache bytes, and attention within the bf16 bar.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_attention_close, bf16_dev, dev, to_dev

pytestmark = pytest.mark.gpu


def two_stream_step(stp, side, hot, host, norm, newest, dgi, lru, stride, q, counts, chunks,
                    rows, miss, stats, out, lse, scale, splits=0, host_ptr=None):
    """One step's lookup / swap-in (side stream) and attention (main stream),
    chunk by chunk over the request rows; `norm` was enqueued on the main
    stream.  Returns hot row ids relative to each chunk's region base."""
    main = torch.cuda.current_stream()
    B = rows.shape[0]
    bounds = np.linspace(0, B, chunks + 1).astype(int)
    ready = main.record_event()          # the normalisation (and the last back-up)
    side.wait_event(ready)
    for k in range(chunks):
        r0, r1 = int(bounds[k]), int(bounds[k + 1])
        with torch.cuda.stream(side):
            stp.hot_lookup_swapin(host, hot[r0 * stride:r1 * stride], norm["slot"][r0:r1],
                                  newest[r0:r1], dgi[r0:r1], lru[r0:r1], stride,
                                  hot_rows_out=rows[r0:r1], miss_mask=miss[r0:r1], stats=stats,
                                  host_pool_ptr=host_ptr)
            swapped = side.record_event()
        main.wait_event(swapped)
        kv = hot[r0 * stride:r1 * stride].view(torch.bfloat16).view(-1, 576)
        stp.sparse_mla_decode(q[r0:r1], kv, rows[r0:r1], counts[r0:r1], scale, splits,
                              out=out[r0:r1], lse=lse[r0:r1])
    return bounds


@pytest.mark.parametrize("chunks,row_bytes", [(2, 1152), (4, 1152), (3, 656)])
def test_two_stream_hot_decode(chunks, row_bytes):
    import sparse_top_paged_amd as stp
    c = workloads.hot_steps_case(seed=3200 + chunks, batch=8, ctx0=3000, steps=4, top_k=128,
                                 window=16, sinks=4, page_size=64, heads=32)
    B, H, stride, P = c.batch, c.hot_size, c.region_stride, c.page_size
    fp8 = row_bytes == 656
    if fp8:
        rows_np = workloads.fp8_rows(np.random.default_rng(5), c.host_rows)
        host_np = rows_np.copy()
    else:
        pool_bits = workloads.pool_bits(c.host_rows, c.pool_seed)
        host_np = pool_bits.view(np.uint8).reshape(c.host_rows, 1152).copy()
    host = torch.from_numpy(host_np.copy()).pin_memory()
    hot = torch.zeros((B * stride, row_bytes), dtype=torch.uint8, device=dev())
    hot_np = np.zeros((B * stride, row_bytes), np.uint8)
    dgi = torch.empty((B, H), dtype=torch.int32, device=dev())
    lru = torch.empty((B, H), dtype=torch.int16, device=dev())
    stp.hot_reset(dgi, lru)
    st = oracle.HotState(B, H)
    table = to_dev(c.block_table)
    req = np.arange(B, dtype=np.int32)
    side = torch.cuda.Stream()
    rows = torch.empty((B, c.cap), dtype=torch.int32, device=dev())
    miss = torch.empty((B, c.cap), dtype=torch.uint8, device=dev())
    out = torch.empty((B, c.heads, 512), dtype=torch.bfloat16, device=dev())
    lse = torch.empty((B, c.heads), dtype=torch.float32, device=dev())
    src = np.arange(B, dtype=np.int32) * stride + H
    for t in range(c.steps):
        q_pos = c.q_pos(t)
        newest = np.asarray([c.block_table[r][q_pos[r] // P] * P + q_pos[r] % P
                             for r in range(B)], np.int32)
        hot[torch.from_numpy(src.astype(np.int64)).to(dev())] = to_dev(host_np[newest])
        hot_np[src] = host_np[newest]
        norm = stp.normalize_indices(to_dev(c.topk[t]), to_dev(req), to_dev(q_pos), table, P,
                                     c.window, c.num_sinks, c.cap, block_view=False)
        stats = torch.zeros(2, dtype=torch.int64, device=dev())
        q = bf16_dev(c.q_bits[t])
        if fp8:
            # the fp8 rows: attention through the fp8 decode, chunk by chunk
            main = torch.cuda.current_stream()
            bounds = np.linspace(0, B, chunks + 1).astype(int)
            side.wait_event(main.record_event())
            for k in range(chunks):
                r0, r1 = int(bounds[k]), int(bounds[k + 1])
                with torch.cuda.stream(side):
                    stp.hot_lookup_swapin(host, hot[r0 * stride:r1 * stride],
                                          norm["slot"][r0:r1], to_dev(newest[r0:r1]),
                                          dgi[r0:r1], lru[r0:r1], stride,
                                          hot_rows_out=rows[r0:r1], miss_mask=miss[r0:r1],
                                          stats=stats)
                    swapped = side.record_event()
                main.wait_event(swapped)
                stp.sparse_mla_decode_fp8(q[r0:r1], hot[r0 * stride:r1 * stride], rows[r0:r1],
                                          norm["count"][r0:r1], 576 ** -0.5, out=out[r0:r1],
                                          lse=lse[r0:r1])
        else:
            bounds = two_stream_step(stp, side, hot, host, norm, to_dev(newest), dgi, lru, stride,
                                     q, norm["count"], chunks, rows, miss, stats, out, lse,
                                     576 ** -0.5)
        stp.backup_rows(hot, host, to_dev(src), to_dev(newest))
        torch.cuda.synchronize()

        ref = oracle.normalize(c.topk[t], req, q_pos, c.window, c.num_sinks, c.block_table, P,
                               c.cap)
        rows_ref, miss_ref, s_ref = oracle.hot_lookup_swapin(st, host_np, hot_np, ref["slot"],
                                                             newest, stride, B)
        got = rows.cpu().numpy().astype(np.int64)
        for k in range(chunks):  # chunk-relative hot rows -> absolute
            r0, r1 = int(bounds[k]), int(bounds[k + 1])
            got[r0:r1] = np.where(got[r0:r1] >= 0, got[r0:r1] + r0 * stride, -1)
        assert np.array_equal(got, rows_ref), f"step {t}: hot rows"
        assert np.array_equal(miss.cpu().numpy(), miss_ref), f"step {t}: miss mask"
        assert np.array_equal(stats.cpu().numpy(), s_ref), f"step {t}: hit / miss counts"
        assert np.array_equal(dgi.cpu().numpy(), st.dgi), f"step {t}: stored ids"
        assert np.array_equal(lru.cpu().numpy(), st.lru), f"step {t}: LRU order"
        assert np.array_equal(hot.cpu().numpy(), hot_np), f"step {t}: hot cache bytes"
        if fp8:
            o_ref, l_ref = oracle.attend_sparse_fp8(c.q_bits[t], host_np, ref["slot"],
                                                    ref["count"], 576 ** -0.5)
        else:
            o_ref, l_ref = oracle.attend_sparse(c.q_bits[t], pool_bits, ref["slot"],
                                                ref["count"], 576 ** -0.5)
        assert_attention_close(out, lse, o_ref, l_ref, f"step {t}")
        # the back-up reached host memory; the oracle's own back-up follows
        assert np.array_equal(host.numpy()[newest], hot_np[src]), f"step {t}: back-up rows"
        oracle.backup_rows(hot_np, host_np, src, newest)
