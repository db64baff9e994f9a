"""The row-gather diagnostic reads exactly the decode's rows: its per-workgroup
xor checksums equal the xor of the 32-bit words of the rows each workgroup's
range names (ragged ranges, replicas, invalid and out-of-range ids)."""

import numpy as np
import pytest
import torch

from helpers import dev, to_dev

pytestmark = pytest.mark.gpu


def expected(rows_u32, ids, counts, parts, replicas, blocks, T):
    cap = ids.shape[1]
    out = {}
    for bid in range(blocks):
        xk = bid >> 3
        per_token = parts * replicas
        t = (xk // per_token) * 8 + (bid & 7)
        part = (xk % per_token) // replicas
        if t >= T:
            continue
        n = min(max(int(counts[t]), 0), cap)
        chunk = -(-n // parts)
        lo = min(n, part * chunk)
        hi = min(n, lo + chunk)
        sel = [int(i) for i in ids[t, lo:hi] if 0 <= i < rows_u32.shape[0]]
        acc = np.uint32(0)
        if sel:
            acc = np.bitwise_xor.reduce(rows_u32[sel].ravel())
        out[bid] = np.uint32(acc)
    return out


@pytest.mark.parametrize("row_bytes", [1152, 256, 656, 4096])
@pytest.mark.parametrize("parts,replicas", [(1, 1), (3, 2), (8, 1), (4, 2)])
def test_row_gather_checksums(parts, replicas, row_bytes):
    # 1152 / 256 / 656-byte rows take the LDS ring (9 / 2 / 6 lines, the last
    # one partial for 656), 4096-byte rows the register pipeline
    from sparse_top_paged_amd import diag
    rng = np.random.default_rng(11 + parts * 10 + replicas + row_bytes)
    num_rows, T, cap = 700, 11, 90
    rows = rng.integers(0, 256, size=(num_rows, row_bytes), dtype=np.uint8)
    ids = rng.integers(-1, num_rows + 20, size=(T, cap)).astype(np.int32)
    counts = rng.integers(0, cap + 1, size=T).astype(np.int32)
    counts[0] = cap
    blocks = diag.row_gather_blocks(T, parts, replicas)
    sentinel = torch.full((blocks,), 0x5A5A5A5A, dtype=torch.int32, device=dev())
    diag.row_gather(to_dev(rows), to_dev(ids), to_dev(counts), parts, replicas, checksum=sentinel)
    got = sentinel.cpu().numpy().view(np.uint32)
    exp = expected(rows.view(np.uint32), ids, counts, parts, replicas, blocks, T)
    for bid in range(blocks):
        if bid in exp:
            assert got[bid] == exp[bid], f"block {bid}"
        else:
            assert got[bid] == 0x5A5A5A5A, f"block {bid} past the last token was written"


@pytest.mark.parametrize("n16,blocks", [(1, 1), (1000, 3), (4096 * 5 + 17, 4), (300000, 64)])
def test_stream_read_checksums(n16, blocks):
    # unit u is read by thread u mod (256 blocks): workgroup b folds the units
    # whose residue lies in [256 b, 256 b + 256)
    from sparse_top_paged_amd import diag
    rng = np.random.default_rng(n16 + blocks)
    words = rng.integers(0, 2 ** 32, size=(n16, 4), dtype=np.uint64).astype(np.uint32)
    src = to_dev(words.view(np.int32))
    got = diag.stream_read(src, blocks).cpu().numpy().view(np.uint32)
    unit_xor = np.bitwise_xor.reduce(words, axis=1)
    owner = (np.arange(n16) % (256 * blocks)) // 256
    for b in range(blocks):
        sel = unit_xor[owner == b]
        exp = np.bitwise_xor.reduce(sel) if len(sel) else np.uint32(0)
        assert got[b] == exp, f"block {b}"
