"""GPU parity: stp_normalize_and_decode and its partial form, the
normalisation and the decode in one call.  Against the two calls it stands
for (stp_normalize_indices, then stp_sparse_mla_decode over its slot lists):
the normalisation outputs and the block view bit for bit, the attention
output and lse bit for bit; against the oracle: the normalisation exactly and
the attention at the bf16 bar.  Covered: the single launch (splits within the
LDS id list, bitmap and table row within two ring stages) at the
DeepSeek-shaped size and on small ragged batches with padding rows,
unmapped pages, invalid ids, slots past the pool, one and two head groups and
a single pass, a top-k list longer than the 2048 entries the output waves
hold in registers; the two-launch forms (a single pass over more ids than
the list holds, a bitmap past 72 KiB)."""

import numpy as np
import pytest

import oracle
import workloads
from helpers import assert_attention_close, bf16_bits_of, bf16_dev, dev, to_dev

pytestmark = pytest.mark.gpu

KEYS = ["tok", "slot", "count", "dropped", "blk_indptr"]


def _host(d):
    return {k: v.cpu().numpy() for k, v in d.items()}


def _same_norm(got, want, T):
    if T == 0:  # nothing is written for an empty batch
        return
    for k in KEYS:
        assert np.array_equal(got[k], want[k]), k
    nnz = int(want["blk_indptr"][-1]) if T else 0
    for k in ("blk_logical", "blk_page", "blk_mask"):
        assert np.array_equal(got[k][:nnz], want[k][:nnz]), k


def _run(c, q, kv, splits, oracle_tokens=()):
    import torch
    import sparse_top_paged_amd as stp
    T = c.topk.shape[0]
    args = [to_dev(np.asarray(a, np.int32)) for a in (c.topk, c.req_id, c.q_pos, c.block_table)]
    want = stp.normalize_indices(*args, c.page_size, c.window, c.num_sinks, c.cap)
    w_out, w_lse = stp.sparse_mla_decode(q, kv, want["slot"], want["count"], c.scale, splits)
    torch.cuda.synchronize()
    want_h = _host(want)
    w_out_b, w_lse_h = bf16_bits_of(w_out), w_lse.cpu().numpy()
    norm = None
    for rep in range(2):  # a second call over the first call's arrays
        out, lse, norm = stp.normalize_and_decode(*args, c.page_size, c.window, c.num_sinks, q,
                                                  kv, c.scale, splits, c.cap, norm=norm)
        torch.cuda.synchronize()
        got = _host(norm)
        _same_norm(got, want_h, T)
        assert np.array_equal(bf16_bits_of(out), w_out_b), f"out (call {rep})"
        assert np.array_equal(lse.cpu().numpy(), w_lse_h, equal_nan=True), f"lse (call {rep})"
    if T == 0:
        return
    o = oracle.normalize(c.topk, c.req_id, c.q_pos, c.window, c.num_sinks, c.block_table,
                         c.page_size, c.cap)
    for k in KEYS:
        assert np.array_equal(got[k], o[k]), k
    nnz = int(o["blk_indptr"][-1])
    assert np.array_equal(got["blk_logical"][:nnz], o["blk_logical"])
    assert np.array_equal(got["blk_page"][:nnz], o["blk_page"])
    assert np.array_equal(got["blk_mask"][:nnz].view(np.uint64), o["blk_mask"])
    import torch as _t
    q_bits = bf16_bits_of(q)
    for tk in oracle_tokens:  # rows gathered from the pool on the device
        n = int(o["count"][tk])
        slots = o["slot"][tk, :n].astype(np.int64)
        valid = slots < kv.shape[0]
        rows = bf16_bits_of(kv[_t.from_numpy(slots[valid]).to(kv.device)]) if valid.any() else \
            np.zeros((0, 576), np.uint16)
        ids = np.full((1, max(1, n)), -1, np.int32)
        ids[0, np.flatnonzero(valid)] = np.arange(int(valid.sum()), dtype=np.int32)
        o_ref, l_ref = oracle.attend_sparse(q_bits[tk:tk + 1], rows if len(rows) else
                                            np.zeros((1, 576), np.uint16), ids, None, c.scale)
        assert_attention_close(out[tk:tk + 1], lse[tk:tk + 1], o_ref, l_ref,
                               f"normalize_and_decode token {tk}")


def _small(seed, T, H, splits, kv_short=0, rows=None, **kw):
    c = workloads.random_small_case(seed, T=T, heads=H, **kw)
    rng = np.random.default_rng(seed + 7)
    q = bf16_dev(workloads.normal_bf16(rng, (T, H, 576)))
    if rows is None:
        rows = max(1, c.kv_rows - kv_short)  # a shorter pool: some slots fall past it
    kv = bf16_dev(workloads.normal_bf16(rng, (rows, 576)))
    return c, q, kv


def test_deepseek_shape():
    c = workloads.deepseek_case()
    kv = workloads.pool_torch(c.kv_rows, c.pool_seed, dev())
    q = bf16_dev(c.q_bits)
    print("[normalize_and_decode] deepseek T=32 H=128", flush=True)
    _run(c, q, kv, 0, oracle_tokens=(0, 13))


@pytest.mark.parametrize("seed,T,H,splits,kv_short,P", [
    (1, 7, 16, 2, 0, 16), (2, 9, 80, 3, 0, 64), (3, 5, 16, 1, 0, 32), (4, 12, 128, 4, 40, 16),
    (5, 3, 8, 2, 0, 1), (6, 10, 16, 0, 0, 63)])
def test_small_batches(seed, T, H, splits, kv_short, P):
    c, q, kv = _small(seed, T, H, splits, kv_short, R=3, ctx=400 + 50 * seed,
                      top_k=60 + 9 * seed, window=seed % 6, sinks=seed % 4, page_size=P)
    print(f"[normalize_and_decode] small seed={seed} T={T} H={H} splits={splits}", flush=True)
    _run(c, q, kv, splits, oracle_tokens=(0, T - 1))


def test_padding_rows():
    import sparse_top_paged_amd as stp  # noqa: F401
    c, q, kv = _small(11, 8, 16, 2, R=3, ctx=500, top_k=70, window=4, sinks=2, page_size=16)
    c.req_id[1] = -1      # padding: no request
    c.req_id[4] = 99      # padding: out of range
    c.q_pos[6] = -1       # padding: negative position
    _run(c, q, kv, 2, oracle_tokens=(0, 1, 6))


def test_single_pass_longer_than_the_id_list():
    # S = 1 over lists of up to 1500 ids: the normalisation takes its own launch
    c, q, kv = _small(12, 3, 16, 1, R=2, ctx=6000, top_k=1400, window=64, sinks=4, page_size=64)
    _run(c, q, kv, 1, oracle_tokens=(1,))


def test_bitmap_past_two_ring_stages():
    # page size 1 over 300,000 positions: bitmap and table row exceed 72 KiB
    c, q, kv = _small(13, 3, 16, 2, rows=200000, R=2, ctx=300000, top_k=400, window=50, sinks=2,
                      page_size=1, unmapped_frac=0.01)
    _run(c, q, kv, 2, oracle_tokens=(0,))


def test_bitmap_in_two_ring_stages():
    # 100,000 positions and 3200 top-k entries: bitmap, table row, D and the
    # word offsets take more than one ring stage (37,376 B) and at most two,
    # so tile 0 waits for the finished list instead of loading during it
    c, q, kv = _small(18, 3, 16, 4, R=2, ctx=100000, top_k=3200, window=64, sinks=4,
                      page_size=64, unmapped_frac=0.01)
    max_blocks = c.block_table.shape[1]
    nwords = (max_blocks * c.page_size + 63) // 64
    lds = nwords * 8 + max_blocks * 4 + 3200 * 4 + nwords * 4 + (nwords // 64 + 1) * 4
    assert 37376 < lds <= 2 * 37376
    _run(c, q, kv, 4, oracle_tokens=(0, 2))


def test_slots_past_int32():
    # pages at the top of the int32 slot range (page size 48): offsets whose
    # slot would pass 2^31 - 1 are dropped, whole pages and page tails
    c = workloads.int32_edge_case()
    rng = np.random.default_rng(19 + 7)
    q = bf16_dev(workloads.normal_bf16(rng, (c.T, 16, 576)))
    kv = bf16_dev(workloads.normal_bf16(rng, (c.kv_rows, 576)))
    for splits in (1, 3):
        print(f"[normalize_and_decode] int32 edge splits={splits}", flush=True)
        _run(c, q, kv, splits, oracle_tokens=(0, 1, 2))


def test_topk_longer_than_one_register_round():
    # 2600 top-k entries: past the 2048 the output waves hold in registers,
    # so D is staged in LDS for the dropped count
    c, q, kv = _small(16, 4, 16, 4, R=2, ctx=20000, top_k=2600, window=64, sinks=4,
                      page_size=64, unmapped_frac=0.02)
    _run(c, q, kv, 4, oracle_tokens=(0, 3))


def test_no_topk_entries():
    # top_k = 0: the window and the sinks alone
    c, q, kv = _small(17, 5, 16, 2, R=2, ctx=600, top_k=0, window=40, sinks=3, page_size=16)
    _run(c, q, kv, 2, oracle_tokens=(0, 4))


def test_empty_batch():
    c, q, kv = _small(14, 0, 16, 2, R=1, ctx=100, top_k=8, window=2, sinks=1, page_size=16)
    _run(c, q, kv, 2)


@pytest.mark.parametrize("splits", [2, 4])
def test_partial_then_merge_with_block_view(splits):
    import torch
    import sparse_top_paged_amd as stp
    c, q, kv = _small(15, 11, 80, splits, R=4, ctx=900, top_k=90, window=5, sinks=3,
                      page_size=16)
    T, H = c.topk.shape[0], 80
    args = [to_dev(np.asarray(a, np.int32)) for a in (c.topk, c.req_id, c.q_pos, c.block_table)]
    want = stp.normalize_indices(*args, c.page_size, c.window, c.num_sinks, c.cap)
    o1, m1, l1 = stp.sparse_mla_decode_partial_normalized(q, kv, want["slot"], want["count"],
                                                          c.scale, splits)
    w_out, w_lse = stp.splitkv_merge_normalized(o1, m1, l1)
    torch.cuda.synchronize()
    o2 = torch.empty_like(o1)
    m2 = torch.empty_like(m1)
    l2 = torch.empty_like(l1)
    norm = stp.normalize_and_decode_partial_normalized(*args, c.page_size, c.window, c.num_sinks,
                                                       q, kv, c.scale, splits, o2, m2, l2, c.cap)
    out, lse = stp.splitkv_merge_with_block_view(o2, m2, l2, norm, args[1], args[2], args[3],
                                                 c.page_size)
    torch.cuda.synchronize()
    _same_norm(_host(norm), _host(want), T)
    assert torch.equal(o2.view(torch.int16), o1.view(torch.int16))
    assert torch.equal(m2, m1) and torch.equal(l2, l1)
    assert np.array_equal(bf16_bits_of(out), bf16_bits_of(w_out))
    assert np.array_equal(lse.cpu().numpy(), w_lse.cpu().numpy(), equal_nan=True)
