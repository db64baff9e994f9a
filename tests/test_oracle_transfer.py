"""Pins for the transfer oracle (CPU only).

A hand-worked example of three 16-byte rows; the identity list over a whole
pool reproduces the pool; a host-to-device transfer and its inverse restore
the touched rows and leave all other bytes alone; the page-first view of a
layer (rows strided by layers * row_bytes) holds the same rows as the
layer-first pool; positions outside either pool write nothing.
"""

import numpy as np

import oracle


def _rows(a, stride, row_bytes, r):
    return a[r * stride:r * stride + row_bytes]


def test_hand_worked_example():
    src = np.arange(4 * 16, dtype=np.uint8)            # rows 0..3: bytes 16r .. 16r + 15
    dst = np.full(5 * 16, 0xEE, dtype=np.uint8)
    # row 2 -> slot 0, row 0 -> slot 3, row 3 -> slot 4; (7 -> 1) and (1 -> 9) skipped
    out = oracle.kv_transfer([src], [dst], 16, 16, 16, [2, 0, 3, 7, 1], [0, 3, 4, 1, 9], 4, 5)[0]
    expect = np.full(80, 0xEE, dtype=np.uint8)
    expect[0:16] = np.arange(32, 48)
    expect[48:64] = np.arange(0, 16)
    expect[64:80] = np.arange(48, 64)
    assert np.array_equal(out, expect)
    assert np.array_equal(dst, np.full(80, 0xEE, dtype=np.uint8))  # input untouched


def test_identity_over_whole_pool():
    rng = np.random.default_rng(1)
    rows, rb = 37, 48
    src = rng.integers(0, 256, rows * rb, dtype=np.uint8)
    out = oracle.kv_transfer([src], [np.zeros_like(src)], rb, rb, rb, np.arange(rows),
                             np.arange(rows), rows, rows)[0]
    assert np.array_equal(out, src)


def test_round_trip_restores_and_leaves_the_rest():
    rng = np.random.default_rng(2)
    hrows, drows, rb, L = 50, 20, 32, 3
    host = [rng.integers(0, 256, hrows * rb, dtype=np.uint8) for _ in range(L)]
    dev = [rng.integers(0, 256, drows * rb, dtype=np.uint8) for _ in range(L)]
    s = np.asarray([5, 6, 7, 8, 40, 12, 3], np.int32)
    d = np.asarray([0, 1, 2, 3, 17, 9, 11], np.int32)
    dev2 = oracle.kv_transfer(host, dev, rb, rb, rb, s, d, hrows, drows)
    for b in range(L):
        for i in range(len(s)):
            assert np.array_equal(_rows(dev2[b], rb, rb, d[i]), _rows(host[b], rb, rb, s[i]))
        untouched = np.setdiff1d(np.arange(drows), d)
        for r in untouched:
            assert np.array_equal(_rows(dev2[b], rb, rb, r), _rows(dev[b], rb, rb, r))
    # back to a scratch host copy: the touched host rows come back unchanged
    scratch = [np.zeros_like(h) for h in host]
    back = oracle.kv_transfer(dev2, scratch, rb, rb, rb, d, s, drows, hrows)
    for b in range(L):
        for i in range(len(s)):
            assert np.array_equal(_rows(back[b], rb, rb, s[i]), _rows(host[b], rb, rb, s[i]))


def test_page_first_view_equals_layer_first():
    rng = np.random.default_rng(3)
    L, rows, rb = 4, 24, 32
    layer_first = [rng.integers(0, 256, rows * rb, dtype=np.uint8) for _ in range(L)]
    # page-first host pool: row r of layer l at (r * L + l) * rb
    page_first = np.stack([lf.reshape(rows, rb) for lf in layer_first], axis=1).reshape(-1)
    idx = np.asarray([3, 17, 4, 23, 0], np.int32)
    dst = [np.zeros(len(idx) * rb, np.uint8) for _ in range(L)]
    a = oracle.kv_transfer(layer_first, dst, rb, rb, rb, idx, np.arange(len(idx)), rows,
                           len(idx))
    b = oracle.kv_transfer([page_first[l * rb:] for l in range(L)], dst, rb, L * rb, rb, idx,
                           np.arange(len(idx)), rows, len(idx))
    for l in range(L):
        assert np.array_equal(a[l], b[l])
