"""GPU parity of the hot-buffer decode at the HiSparse workload's full size.

64 requests, context 65536 + t at step t, 16 consecutive decode steps whose
top-k (2048) keeps 85% of the previous step's set, a 128-token window and 4
sinks, page size 64, a hot region of 2 * top_k = 4096 rows (+ the newest row)
per request, and the whole latent pool (65,600 pages = 4.2 M rows of 1152 B,
4.8 GB) in pinned host memory.  Per step: normalise -> lookup / LRU /
swap-in from the host pool -> sparse decode over the hot cache (the split
path) -> back-up of each request's new row.

Compared with the oracle, bit for bit, every step: hot rows, miss masks,
stored ids, LRU order, the hit / miss counts and every byte of the hot cache;
the back-up rows in host memory before the oracle writes them.  Attention is
compared against the fp64 oracle over the host pool rows (with the step's new
row for the newest position): every token on steps 0, 1 and 15, three
sampled tokens on the other steps.
"""

import time

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_attention_close, bf16_dev, dev, to_dev

pytestmark = pytest.mark.gpu

SAMPLED = (0, 37, 63)
ALL_TOKENS_STEPS = (0, 1, 15)  # the cold step, the first warm one and the last


def test_hot_buffer_decode_full_size():
    import sparse_top_paged_amd as stp
    t0 = time.time()
    c = workloads.hot_steps_case()  # seed 3000: B 64, ctx0 65536, 16 steps, top_k 2048, 128 heads
    B, H, stride, P = c.batch, c.hot_size, c.region_stride, c.page_size
    print(f"[hot full] case built in {time.time() - t0:.1f} s; host rows {c.host_rows}", flush=True)

    # the pool, generated on the device and moved to pinned host memory
    pool = workloads.pool_torch(c.host_rows, c.pool_seed, dev())
    host = torch.empty((c.host_rows, 1152), dtype=torch.uint8, pin_memory=True)
    host.copy_(pool.view(torch.uint8).view(c.host_rows, 1152))
    del pool
    torch.cuda.empty_cache()
    host_np = host.numpy()  # the oracle reads the same bytes (checked before each back-up)
    print(f"[hot full] pinned host pool ready at {time.time() - t0:.1f} s", flush=True)

    hot = torch.zeros((B * stride, 1152), dtype=torch.uint8, device=dev())
    hot_np = np.zeros((B * stride, 1152), np.uint8)
    dgi = torch.empty((B, H), dtype=torch.int32, device=dev())
    lru = torch.empty((B, H), dtype=torch.int16, device=dev())
    stp.hot_reset(dgi, lru)
    st = oracle.HotState(B, H)
    table = to_dev(c.block_table)
    req = np.arange(B, dtype=np.int32)
    rng = np.random.default_rng(7)
    kv = hot.view(torch.bfloat16).view(-1, 576)
    hits = misses = 0
    for t in range(c.steps):
        q_pos = c.q_pos(t)
        newest = np.asarray([c.block_table[r][q_pos[r] // P] * P + q_pos[r] % P
                             for r in range(B)], np.int32)
        # the step's new KV row: N(0, 1) values as bf16 (the row attention reads)
        new_rows = workloads.normal_bf16(rng, (B, 576)).view(np.uint8).reshape(B, 1152)
        hot_np[np.arange(B) * stride + H] = new_rows
        hot[torch.arange(B, device=dev()) * stride + H] = to_dev(new_rows)

        norm = stp.normalize_indices(to_dev(c.topk[t]), to_dev(req), to_dev(q_pos), table, P,
                                     c.window, c.num_sinks, c.cap, block_view=False)
        stats = torch.zeros(2, dtype=torch.int64, device=dev())
        rows, miss, _ = stp.hot_lookup_swapin(host, hot, norm["slot"], to_dev(newest), dgi, lru,
                                              stride, stats=stats)
        out, lse = stp.sparse_mla_decode(bf16_dev(c.q_bits[t]), kv, rows, norm["count"],
                                         576 ** -0.5, 0)
        src = np.arange(B, dtype=np.int32) * stride + H
        stp.backup_rows(hot, host, to_dev(src), to_dev(newest))
        torch.cuda.synchronize()

        ref = oracle.normalize(c.topk[t], req, q_pos, c.window, c.num_sinks, c.block_table, P,
                               c.cap)
        assert np.array_equal(norm["slot"].cpu().numpy(), ref["slot"]), f"step {t}: slots"
        rows_ref, miss_ref, s_ref = oracle.hot_lookup_swapin(st, host_np, hot_np, ref["slot"],
                                                             newest, stride, B)
        assert np.array_equal(rows.cpu().numpy(), rows_ref), f"step {t}: hot rows"
        assert np.array_equal(miss.cpu().numpy(), miss_ref), f"step {t}: miss mask"
        assert np.array_equal(stats.cpu().numpy(), s_ref), f"step {t}: hit / miss counts"
        assert np.array_equal(dgi.cpu().numpy(), st.dgi), f"step {t}: stored ids"
        assert np.array_equal(lru.cpu().numpy(), st.lru), f"step {t}: LRU order"
        assert np.array_equal(hot.cpu().numpy(), hot_np), f"step {t}: hot cache bytes"

        # attention on sampled tokens, over the host rows by slot id
        counts = ref["count"]
        for i in (range(B) if t in ALL_TOKENS_STEPS else SAMPLED):
            sl = ref["slot"][i, :counts[i]]
            bits = host_np[sl].copy()
            bits[sl == newest[i]] = new_rows[i]
            kv_i = bits.view(np.uint16).reshape(-1, 576)
            o_ref, l_ref = oracle.attend_sparse(c.q_bits[t][i:i + 1], kv_i,
                                                np.arange(len(sl), dtype=np.int32)[None, :],
                                                None, 576 ** -0.5)
            assert_attention_close(out[i:i + 1], lse[i:i + 1], o_ref, l_ref, f"step {t} token {i}")

        # the back-up reached host memory, then the oracle's own back-up
        assert np.array_equal(host_np[newest], hot_np[src]), f"step {t}: back-up rows"
        oracle.backup_rows(hot_np, host_np, src, newest)
        hits += int(s_ref[0])
        misses += int(s_ref[1])
        print(f"[hot full] step {t}: hits {s_ref[0]} misses {s_ref[1]} "
              f"({s_ref[0] / max(1, s_ref[0] + s_ref[1]):.3f}) at {time.time() - t0:.1f} s",
              flush=True)
    warm_rate = hits / max(1, hits + misses)
    print(f"[hot full] hit rate over all steps {warm_rate:.3f}", flush=True)
    assert misses > 0 and hits > 0
