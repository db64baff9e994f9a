"""GPU parity: stp_normalize_indices against the oracle, bit-exact."""

import numpy as np
import pytest

import oracle
import workloads
from helpers import to_dev

pytestmark = pytest.mark.gpu

KEYS = ["tok", "slot", "count", "dropped", "blk_indptr"]


def gpu_normalize(topk, req_id, q_pos, table, P, window, sinks, cap):
    import torch
    import sparse_top_paged_amd as stp
    res = stp.normalize_indices(to_dev(np.asarray(topk, np.int32)), to_dev(np.asarray(req_id, np.int32)),
                                to_dev(np.asarray(q_pos, np.int32)), to_dev(np.asarray(table, np.int32)),
                                P, window, sinks, cap)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


def check(topk, req_id, q_pos, table, P, window, sinks, cap):
    g = gpu_normalize(topk, req_id, q_pos, table, P, window, sinks, cap)
    o = oracle.normalize(np.asarray(topk), np.asarray(req_id), np.asarray(q_pos), window, sinks,
                         np.asarray(table), P, cap)
    for k in KEYS:
        assert np.array_equal(g[k], o[k]), k
    nnz = int(o["blk_indptr"][-1])
    assert np.array_equal(g["blk_logical"][:nnz], o["blk_logical"])
    assert np.array_equal(g["blk_page"][:nnz], o["blk_page"])
    assert np.array_equal(g["blk_mask"][:nnz].view(np.uint64), o["blk_mask"])
    return g


@pytest.mark.parametrize("name", ["index_example_page64.txt", "index_example_page16.txt"])
def test_worked_examples(golden, name):
    gd = golden(name)
    cands = gd["candidates"]
    g = check([cands], [0], [max(cands)], [gd["table"]], gd["page_size"][0], 0, 0, len(cands))
    n = g["count"][0]
    assert list(g["slot"][0, :n]) == gd["slots"]
    assert list(g["blk_logical"][:2]) == gd["indices"]
    assert list(g["blk_page"][:2]) == gd["pages"]


def test_tiny_case():
    c = workloads.tiny_case()
    g = check(c.topk, c.req_id, c.q_pos, c.block_table, c.page_size, c.window, c.num_sinks, c.cap)
    assert g["count"][0] <= 40 and g["dropped"][0] == 0


@pytest.mark.parametrize("seed", range(16))
def test_random_small(seed):
    P = [1, 4, 15, 16, 17, 32, 63, 64][seed % 8]
    c = workloads.random_small_case(seed, T=7, R=3, ctx=120 + 37 * seed, top_k=33 + seed,
                                    window=seed % 9, sinks=seed % 5, page_size=P)
    # padding rows: an out-of-range request and a negative position
    req = c.req_id.copy()
    req[1] = 5
    pos = c.q_pos.copy()
    pos[2] = -1
    check(c.topk, req, pos, c.block_table, P, c.window, c.num_sinks, c.cap + seed % 3)


@pytest.mark.parametrize("ctx", [15, 16, 17, 63, 64, 65])
def test_page_boundaries(ctx):
    rng = np.random.default_rng(ctx)
    P = 16
    table = rng.permutation(20)[: -(-ctx // P)][None, :]
    topk = rng.integers(-2, ctx + 3, size=(3, 10))
    check(topk, [0, 0, 0], [ctx - 1, ctx // 2, 0], table, P, 3, 2, 15)


def test_deepseek_shape_full():
    c = workloads.deepseek_case()
    check(c.topk, c.req_id, c.q_pos, c.block_table, c.page_size, c.window, c.num_sinks, c.cap)


@pytest.mark.parametrize("clustered", [False, True])
def test_long_context_full(clustered):
    c = workloads.locality_case(4002 if clustered else 4001, clustered)
    g = check(c.topk, c.req_id, c.q_pos, c.block_table, c.page_size, c.window, c.num_sinks, c.cap)
    assert np.all(g["count"] == 2048)


def test_empty_and_padding_only():
    g = gpu_normalize(np.zeros((0, 4), np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32),
                      np.zeros((1, 2), np.int32), 16, 0, 0, 4)
    assert g["count"].shape == (0,)
    check([[-1, -1]], [-1], [5], [[0, 1]], 16, 2, 2, 6)


def test_many_tokens_lookback():
    # more tokens than one 256-token look-back window of the block-view
    # offsets, with padding rows (zero blocks) spread through the batch
    c = workloads.random_small_case(77, T=600, R=5, ctx=900, top_k=60, window=7, sinks=3,
                                    page_size=16)
    req = c.req_id.copy()
    req[::37] = -1
    check(c.topk, req, c.q_pos, c.block_table, c.page_size, c.window, c.num_sinks, c.cap)


def test_long_topk_rows():
    # top_k beyond one round of per-thread loads (8 per thread x 256 threads)
    c = workloads.random_small_case(78, T=3, R=2, ctx=20000, top_k=5000, window=300, sinks=4,
                                    page_size=64)
    check(c.topk, c.req_id, c.q_pos, c.block_table, c.page_size, c.window, c.num_sinks, c.cap)


def test_table_in_global_memory():
    # page size 1: the page-table row (300,000 entries) does not fit in LDS
    # beside the bitmap, so it is read from global memory
    c = workloads.random_small_case(79, T=4, R=2, ctx=300000, top_k=500, window=100, sinks=2,
                                    page_size=1, unmapped_frac=0.01)
    check(c.topk, c.req_id, c.q_pos, c.block_table, c.page_size, c.window, c.num_sinks, c.cap)


@pytest.mark.parametrize("case", ["deepseek", "lookback", "global_table", "empty"])
def test_deferred_block_view_on_side_stream(case):
    # the normalisation split in two calls, the block view completed on a
    # second stream: the same arrays as the one-call normalisation
    import torch
    import sparse_top_paged_amd as stp
    if case == "deepseek":
        c = workloads.deepseek_case()
    elif case == "lookback":
        c = workloads.random_small_case(77, T=600, R=5, ctx=900, top_k=60, window=7, sinks=3,
                                        page_size=16)
    elif case == "global_table":
        c = workloads.random_small_case(79, T=4, R=2, ctx=300000, top_k=500, window=100,
                                        sinks=2, page_size=1, unmapped_frac=0.01)
    else:
        c = workloads.random_small_case(80, T=0, R=1, ctx=100, top_k=8, window=2, sinks=1,
                                        page_size=16)
    args = [to_dev(np.asarray(a, np.int32)) for a in (c.topk, c.req_id, c.q_pos, c.block_table)]
    want = stp.normalize_indices(*args, c.page_size, c.window, c.num_sinks, c.cap)
    torch.cuda.synchronize()
    want = {k: v.cpu().numpy() for k, v in want.items()}
    for _ in range(2):
        got = stp.normalize_indices(*args, c.page_size, c.window, c.num_sinks, c.cap,
                                    defer_block_view=True)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            stp.block_view_fill(got, args[1], args[2], args[3], c.page_size)
            # a repeated fill over the completed arrays changes nothing
            stp.block_view_fill(got, args[1], args[2], args[3], c.page_size)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy() for k, v in got.items()}
        for k in KEYS:
            assert np.array_equal(got[k], want[k]), k
        nnz = int(want["blk_indptr"][-1])
        for k in ("blk_logical", "blk_page", "blk_mask"):
            assert np.array_equal(got[k][:nnz], want[k][:nnz]), k
