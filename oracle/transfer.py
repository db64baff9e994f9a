"""Staged bulk host <-> device KV transfer (oracle, plain definition).

TEST INFRASTRUCTURE ONLY -- see the package header.

What it states ("[HiCache] TMA-staged host<->device KV transfer kernel
(sm_90+)", Motivation and Modifications): a transfer moves whole KV rows
between a host pool and a device pool.  For every buffer b (a layer's K or
V) and list position i, the row at index src_idx[i] of the source buffer is
copied to index dst_idx[i] of the destination buffer; a buffer's row r starts
at byte r * stride (stride = row_bytes for a layer-first view, layers *
row_bytes for a page-first view with a per-layer base).  Positions whose
index lies outside the source or destination pool are skipped.  Bytes not
written keep their values.

The definition is a byte copy written out row by row; nothing is reordered
beyond the list order (duplicate destinations are left to the caller).

Pins (tests/test_oracle_transfer.py): a hand-worked three-row example of
16-byte rows; the identity list over a whole pool equals the pool itself; a
host-to-device transfer followed by its inverse restores the touched rows
and leaves every other byte alone; the page-first view of a layer equals the
layer-first pool it was built from; skipped positions write nothing.
"""

import numpy as np


def kv_transfer(src_bufs, dst_bufs, row_bytes, src_stride, dst_stride, src_idx, dst_idx,
                src_rows, dst_rows):
    """src_bufs / dst_bufs: lists of 1-D uint8 arrays (a buffer's bytes, from
    its base).  Returns the destination buffers after the transfer (copies)."""
    out = [np.array(d, dtype=np.uint8, copy=True) for d in dst_bufs]
    for b, src in enumerate(src_bufs):
        dst = out[b]
        for i in range(len(src_idx)):
            s, d = int(src_idx[i]), int(dst_idx[i])
            if not (0 <= s < src_rows and 0 <= d < dst_rows):
                continue
            dst[d * dst_stride:d * dst_stride + row_bytes] = \
                src[s * src_stride:s * src_stride + row_bytes]
    return out
