"""GPU parity of the staged bulk KV transfer, byte for byte against the oracle.

Host pools in pinned host memory, device pools in HBM; several buffers per
call (layers' K and V); layer-first and page-first host views; whole page
runs, scattered rows and a ragged tail; row sizes 16, 256 (a GQA head row),
656 (an fp8 MLA row), 1152 (a bf16 MLA row) and 4096 bytes; positions outside
either pool; 1 to 8 workgroups; both directions.  Every byte of every
destination buffer is compared, so untouched rows must keep their values.
"""

import numpy as np
import pytest
import torch

import oracle
from helpers import dev, to_dev

pytestmark = pytest.mark.gpu


def _pinned(a):
    t = torch.empty(a.shape, dtype=torch.uint8, pin_memory=True)
    t.copy_(torch.from_numpy(a))
    return t


def _case(rng, rows_src, rows_dst, n, page, scattered_frac, bad_frac):
    """Source positions: runs of whole pages, then scattered rows; destination
    positions distinct; a fraction of positions out of range."""
    pages = rng.permutation(rows_src // page)[: max(1, int(n * (1 - scattered_frac)) // page)]
    runs = (pages[:, None] * page + np.arange(page)[None, :]).reshape(-1)
    rest = rng.choice(rows_src, size=max(0, n - len(runs)), replace=False)
    s = np.concatenate([runs, rest])[:n].astype(np.int32)
    d = rng.permutation(rows_dst)[:n].astype(np.int32)
    bad = rng.random(n) < bad_frac
    s[bad & (rng.random(n) < 0.5)] = -1
    d[bad & ~(s == -1)] = rows_dst + 3
    return s, d


@pytest.mark.parametrize("row_bytes", [16, 256, 656, 1152, 4096])
@pytest.mark.parametrize("blocks", [1, 3, 8])
def test_h2d_then_d2h(row_bytes, blocks):
    import sparse_top_paged_amd as stp
    rng = np.random.default_rng(row_bytes * 10 + blocks)
    L, hrows, drows, page = 3, 700, 520, 16
    n = 300 if row_bytes <= 1152 else 120
    host = [rng.integers(0, 256, (hrows, row_bytes), dtype=np.uint8) for _ in range(L)]
    devp = [rng.integers(0, 256, (drows, row_bytes), dtype=np.uint8) for _ in range(L)]
    s, d = _case(rng, hrows, drows, n, page, 0.3, 0.05)
    print(f"[transfer] rows {row_bytes} B, blocks {blocks}, n {n}", flush=True)
    h_t = [_pinned(h) for h in host]
    d_t = [to_dev(x) for x in devp]
    stp.kv_transfer(h_t, d_t, to_dev(s), to_dev(d), num_blocks=blocks)
    torch.cuda.synchronize()
    ref = oracle.kv_transfer([h.reshape(-1) for h in host], [x.reshape(-1) for x in devp],
                             row_bytes, row_bytes, row_bytes, s, d, hrows, drows)
    for b in range(L):
        assert np.array_equal(d_t[b].cpu().numpy().reshape(-1), ref[b]), f"H2D buffer {b}"
    # back into fresh host pools
    back_np = [rng.integers(0, 256, (hrows, row_bytes), dtype=np.uint8) for _ in range(L)]
    back = [_pinned(x) for x in back_np]
    stp.kv_transfer(d_t, back, to_dev(d), to_dev(s), num_blocks=blocks)
    torch.cuda.synchronize()
    ref2 = oracle.kv_transfer(ref, [x.reshape(-1) for x in back_np], row_bytes, row_bytes,
                              row_bytes, d, s, drows, hrows)
    for b in range(L):
        assert np.array_equal(back[b].numpy().reshape(-1), ref2[b]), f"D2H buffer {b}"


def test_page_first_host_view_and_long_list():
    """Host pool page-first ([rows][layers][row]): layer l's base is l * row
    bytes, stride layers * row bytes; 9000 positions cross the 4096-row
    chunks of a workgroup's range."""
    import sparse_top_paged_amd as stp
    rng = np.random.default_rng(11)
    L, hrows, drows, rb = 4, 12000, 9500, 64
    host = rng.integers(0, 256, (hrows, L, rb), dtype=np.uint8)
    s = rng.permutation(hrows)[:9000].astype(np.int32)
    d = rng.permutation(drows)[:9000].astype(np.int32)
    h_t = _pinned(host)
    d_np = [rng.integers(0, 256, (drows, rb), dtype=np.uint8) for _ in range(L)]
    d_t = [to_dev(x) for x in d_np]
    # per-layer views of the pinned page-first pool: offsets l * rb from its base
    flat = h_t.view(-1)
    views = [flat[l * rb:] for l in range(L)]
    stp.kv_transfer(views, d_t, to_dev(s), to_dev(d), row_bytes=rb, src_stride=L * rb,
                    src_rows=hrows, num_blocks=2)
    torch.cuda.synchronize()
    ref = oracle.kv_transfer([host.reshape(-1)[l * rb:] for l in range(L)],
                             [x.reshape(-1) for x in d_np], rb, L * rb, rb, s, d, hrows, drows)
    for b in range(L):
        assert np.array_equal(d_t[b].cpu().numpy().reshape(-1), ref[b]), f"buffer {b}"


def test_device_to_device_and_empty():
    import sparse_top_paged_amd as stp
    rng = np.random.default_rng(12)
    rb, rows = 1152, 2000
    a = rng.integers(0, 256, (rows, rb), dtype=np.uint8)
    b = rng.integers(0, 256, (rows, rb), dtype=np.uint8)
    s = rng.permutation(rows)[:1500].astype(np.int32)
    d = rng.permutation(rows)[:1500].astype(np.int32)
    a_t, b_t = to_dev(a), to_dev(b)
    stp.kv_transfer([a_t], [b_t], to_dev(s), to_dev(d), num_blocks=5)
    empty = torch.zeros(0, dtype=torch.int32, device=dev())
    stp.kv_transfer([a_t], [b_t], empty, empty)
    torch.cuda.synchronize()
    ref = oracle.kv_transfer([a.reshape(-1)], [b.reshape(-1)], rb, rb, rb, s, d, rows, rows)[0]
    assert np.array_equal(b_t.cpu().numpy().reshape(-1), ref)
