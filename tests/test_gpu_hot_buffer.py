"""GPU parity: hot-buffer lookup / swap-in / reset / back-up against the oracle, bit-exact."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import dev, to_dev

pytestmark = pytest.mark.gpu


def pinned_bytes(arr):
    t = torch.from_numpy(np.ascontiguousarray(arr)).pin_memory()
    return t


def test_worked_example(golden):
    import sparse_top_paged_amd as stp
    g = golden("hisparse_swapin_example.txt")
    H, stride, row_bytes = g["hot_size"][0], 128, 1152
    rng = np.random.default_rng(0)
    host_np = rng.integers(0, 256, size=(2000, row_bytes), dtype=np.uint8)
    host = pinned_bytes(host_np)
    hot = torch.zeros((stride, row_bytes), dtype=torch.uint8, device=dev())
    dgi = to_dev(np.asarray([g["dgi_before"]], np.int32))
    lru = to_dev(np.asarray([g["lru_before"]], np.int16))
    ids = to_dev(np.asarray([g["global_ids"]], np.int32))
    newest = to_dev(np.asarray(g["newest"], np.int32))
    out, miss, stats = stp.hot_lookup_swapin(host, hot, ids, newest, dgi, lru, stride)
    torch.cuda.synchronize()
    assert out.cpu().tolist()[0] == g["out"]
    assert miss.cpu().tolist()[0] == g["miss_mask"]
    assert lru.cpu().tolist()[0] == g["lru_after"]
    assert dgi.cpu().tolist()[0] == g["dgi_after"]
    assert stats.cpu().tolist() == g["stats"]
    hot_np = hot.cpu().numpy()
    for src, slot in g["copies"]:
        assert np.array_equal(hot_np[slot], host_np[src])
    untouched = [s for s in range(stride) if s not in (3, 5)]
    assert np.all(hot_np[untouched] == 0)


def _run_steps(batch, steps, top_k, window, sinks, P, ctx0, num_real=None, row_bytes=1152,
               trim_host=0, hot_size=None):
    """Decode steps through normalise -> lookup/swap-in -> back-up on both sides."""
    import sparse_top_paged_amd as stp
    c = workloads.hot_steps_case(seed=3000 + batch, batch=batch, ctx0=ctx0, steps=steps,
                                 top_k=top_k, window=window, sinks=sinks, page_size=P, heads=1)
    num_real = batch if num_real is None else num_real
    H, stride = c.hot_size, c.region_stride
    if hot_size is not None:
        H, stride = hot_size, -(-(hot_size + 1) // 128) * 128
    rng = np.random.default_rng(1)
    host_rows = c.host_rows - trim_host
    host_np = rng.integers(0, 256, size=(host_rows, row_bytes), dtype=np.uint8)
    host = pinned_bytes(host_np)
    hot = torch.zeros((batch * stride, row_bytes), dtype=torch.uint8, device=dev())
    hot_np = np.zeros((batch * stride, row_bytes), np.uint8)
    dgi = torch.empty((batch, H), dtype=torch.int32, device=dev())
    lru = torch.empty((batch, H), dtype=torch.int16, device=dev())
    stp.hot_reset(dgi, lru)
    st = oracle.HotState(batch, H)
    table = to_dev(c.block_table)
    req = np.arange(batch, dtype=np.int32)
    stats = torch.zeros(2, dtype=torch.int64, device=dev())
    stats_ref = np.zeros(2, np.int64)
    for t in range(steps):
        q_pos = c.q_pos(t)
        newest_np = np.asarray([c.block_table[r][q_pos[r] // P] * P + q_pos[r] % P
                                for r in range(batch)], np.int32)
        # the newest token's row is produced by the step and written to its reserved row
        new_rows = rng.integers(0, 256, size=(batch, row_bytes), dtype=np.uint8)
        for r in range(batch):
            hot_np[r * stride + H] = new_rows[r]
        hot[torch.arange(batch, device=dev()) * stride + H] = to_dev(new_rows)

        norm = stp.normalize_indices(to_dev(c.topk[t]), to_dev(req), to_dev(q_pos), table, P,
                                     window, sinks, c.cap)
        out, miss, _ = stp.hot_lookup_swapin(host, hot, norm["slot"], to_dev(newest_np), dgi, lru,
                                             stride, num_real_rows=num_real, stats=stats)
        ref = oracle.normalize(c.topk[t], req, q_pos, window, sinks, c.block_table, P, c.cap)
        out_ref, miss_ref, s_ref = oracle.hot_lookup_swapin(st, host_np, hot_np, ref["slot"],
                                                            newest_np, stride, num_real)
        stats_ref += s_ref
        # back-up of the new rows (the host pool is the only full-size store)
        src = np.asarray([r * stride + H for r in range(num_real)], np.int32)
        dst = newest_np[:num_real]
        stp.backup_rows(hot, host, to_dev(src), to_dev(dst))
        oracle.backup_rows(hot_np, host_np, src, dst)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), out_ref), f"step {t}: hot rows"
        assert np.array_equal(miss.cpu().numpy(), miss_ref), f"step {t}: miss mask"
        assert np.array_equal(dgi.cpu().numpy(), st.dgi), f"step {t}: dgi"
        assert np.array_equal(lru.cpu().numpy(), st.lru), f"step {t}: lru"
        assert np.array_equal(hot.cpu().numpy(), hot_np), f"step {t}: hot cache bytes"
        assert np.array_equal(host.numpy(), host_np), f"step {t}: host pool bytes"
    assert np.array_equal(stats.cpu().numpy(), stats_ref)
    return stats_ref


def test_multistep_small():
    s = _run_steps(batch=4, steps=6, top_k=64, window=8, sinks=2, P=16, ctx0=2000)
    assert s[0] > 0 and s[1] > 0


def test_multistep_padded_rows():
    _run_steps(batch=5, steps=3, top_k=32, window=4, sinks=1, P=64, ctx0=700, num_real=3)


def test_multistep_full_width_rows():
    # 4 requests at the real top-k (2048) and hot size (4096), 1152-byte rows
    s = _run_steps(batch=4, steps=4, top_k=2048, window=128, sinks=4, P=64, ctx0=8192)
    assert s[0] > 0


def test_multistep_fp8_rows():
    # 656-byte fp8_ds_mla rows (41 16-byte vectors each) at the real top-k and
    # hot size: lookup, swap-in and back-up byte for byte against the oracle
    s = _run_steps(batch=4, steps=4, top_k=2048, window=128, sinks=4, P=64, ctx0=8192,
                   row_bytes=656)
    assert s[0] > 0


def test_multistep_unstaged_state():
    # hot_size 12288 at top-k 4096: the LRU order and stored ids no longer fit
    # in LDS beside the table and the staged candidates, so the lookup reads
    # them from global memory
    import sparse_top_paged_amd as stp
    H, cap = 12288, 4096 + 8 + 2
    assert stp.hot_lds_bytes(cap, H) > 0
    assert stp.hot_lds_bytes(cap, H) + 6 * H > 160 * 1024
    s = _run_steps(batch=2, steps=3, top_k=4096, window=8, sinks=2, P=64, ctx0=20000,
                   hot_size=H)
    assert s[0] > 0 and s[1] > 0


def test_out_of_range_lru_leaves_row_untouched():
    # an LRU order holding a slot outside the region is not state this kernel
    # left: that row's outputs are -1 and its state is not touched; the other
    # rows follow the oracle
    import sparse_top_paged_amd as stp
    rng = np.random.default_rng(9)
    R, H, stride, cap = 3, 64, 128, 20
    st = oracle.HotState(R, H)
    host_np = rng.integers(0, 256, size=(500, 16), dtype=np.uint8)
    host = pinned_bytes(host_np)
    hot_np = np.zeros((R * stride, 16), np.uint8)
    hot = torch.zeros((R * stride, 16), dtype=torch.uint8, device=dev())
    lru_bad = st.lru.copy()
    lru_bad[1, 5] = 999
    dgi = to_dev(st.dgi)
    lru = to_dev(lru_bad)
    ids = np.stack([rng.choice(400, size=cap, replace=False) for _ in range(R)]).astype(np.int32)
    newest = np.full(R, -1, np.int32)
    out, miss, stats = stp.hot_lookup_swapin(host, hot, to_dev(ids), to_dev(newest), dgi, lru,
                                             stride)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[1] == -1) and np.all(miss.cpu().numpy()[1] == 0)
    assert np.array_equal(lru.cpu().numpy()[1], lru_bad[1])
    assert np.all(dgi.cpu().numpy()[1] == -1)
    assert np.all(hot.cpu().numpy()[stride:2 * stride] == 0)
    rows = [0, 2]
    sub = oracle.HotState(2, H)
    out_ref, miss_ref, s_ref = oracle.hot_lookup_swapin(sub, host_np, hot_np[:2 * stride].copy(),
                                                        ids[rows], newest[rows], stride, 2)
    for k, r in enumerate(rows):
        assert np.array_equal(o[r] - (r - k) * stride * (o[r] >= 0), out_ref[k])
        assert np.array_equal(dgi.cpu().numpy()[r], sub.dgi[k])
    assert stats.cpu().tolist() == s_ref.tolist()


def test_missing_host_rows_revoke():
    # the last pages of the pool are not in host memory: their slots are zeroed and revoked
    _run_steps(batch=3, steps=3, top_k=48, window=4, sinks=2, P=16, ctx0=900, trim_host=600)


def test_reset_subset():
    # state after real lookups, then a subset reset (with out-of-range row
    # indices, which are skipped), compared with oracle.hot_reset bit for bit
    import sparse_top_paged_amd as stp
    rng = np.random.default_rng(4)
    R, H, stride, cap = 5, 64, 128, 40
    st = oracle.HotState(R, H)
    host_np = rng.integers(0, 256, size=(3000, 16), dtype=np.uint8)
    host = pinned_bytes(host_np)
    hot_np = np.zeros((R * stride, 16), np.uint8)
    hot = torch.zeros((R * stride, 16), dtype=torch.uint8, device=dev())
    dgi = to_dev(st.dgi)
    lru = to_dev(st.lru)
    for step in range(3):
        ids = np.full((R, cap), -1, np.int32)
        for r in range(R):
            ids[r, :30] = rng.choice(300, size=30, replace=False) + 100 * r
        newest = np.full(R, -1, np.int32)
        oracle.hot_lookup_swapin(st, host_np, hot_np, ids, newest, stride, R)
        stp.hot_lookup_swapin(host, hot, to_dev(ids), to_dev(newest), dgi, lru, stride)
    rows = np.asarray([1, 3, -2, 9], np.int32)
    oracle.hot_reset(st, rows=rows)
    stp.hot_reset(dgi, lru, rows=to_dev(rows))
    torch.cuda.synchronize()
    assert np.array_equal(dgi.cpu().numpy(), st.dgi)
    assert np.array_equal(lru.cpu().numpy(), st.lru)
    assert np.any(st.dgi[[0, 2, 4]] >= 0)  # the rows left out still hold their state
    oracle.hot_reset(st)
    stp.hot_reset(dgi, lru)
    torch.cuda.synchronize()
    assert np.array_equal(dgi.cpu().numpy(), st.dgi)
    assert np.array_equal(lru.cpu().numpy(), st.lru)


def test_backup_skips_out_of_range():
    import sparse_top_paged_amd as stp
    rng = np.random.default_rng(3)
    hot_np = rng.integers(0, 256, size=(10, 64), dtype=np.uint8)
    host = pinned_bytes(np.zeros((6, 64), np.uint8))
    host_np = np.zeros((6, 64), np.uint8)
    src = np.asarray([1, 9, -1, 4, 10], np.int32)
    dst = np.asarray([0, 5, 2, 6, 3], np.int32)
    stp.backup_rows(to_dev(hot_np), host, to_dev(src), to_dev(dst))
    oracle.backup_rows(hot_np, host_np, src, dst)
    torch.cuda.synchronize()
    assert np.array_equal(host.numpy(), host_np)
