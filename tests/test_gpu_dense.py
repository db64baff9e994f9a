"""GPU parity of the dense paged attention with grouped query heads.

Decode over block tables and prefix-extend over slot lists, against the
fp64 oracle element by element: small ragged batches (empty requests, one
token, lengths off the 64-key tile, unmapped pages, pages and slots outside
the pool, tokens past the end of the table, Lk < Lq, several query blocks)
for every supported group size, and the full-size workloads (decode: 128
requests of 1024..4096 tokens, 32 query / 8 KV heads; extend: 8 requests of
a 4096-token prefix + 512 new tokens) on sampled requests and heads.
"""

import time

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_fp16_attention_close, dev, to_dev

pytestmark = pytest.mark.gpu


def _pools(case):
    k, v = workloads.dense_pool(case.num_slots, case.hkv, case.pool_seed)
    return k, v, to_dev(k), to_dev(v)


@pytest.mark.parametrize("hq,hkv", [(8, 1), (32, 8), (8, 4), (4, 4), (6, 2), (16, 1)])
def test_decode_small_ragged(hq, hkv):
    import sparse_top_paged_amd as stp
    case = workloads.random_gqa_decode_case(hq * 10 + hkv, [0, 1, 15, 64, 65, 300, 1000, -3],
                                            hq=hq, hkv=hkv)
    k, v, kd, vd = _pools(case)
    print(f"[dense decode] {case.name} hq {hq} hkv {hkv}", flush=True)
    out, lse = stp.paged_gqa_decode(to_dev(case.q), kd, vd, to_dev(case.block_table),
                                    to_dev(case.ctx_lens), case.page_size, case.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.paged_gqa_decode(case.q, k, v, case.block_table, case.ctx_lens,
                                           case.page_size, case.scale)
    assert_fp16_attention_close(out, lse, o_ref, l_ref, case.name)


def test_decode_tokens_past_table():
    """A context longer than the table: the tokens past it take no part."""
    import sparse_top_paged_amd as stp
    case = workloads.random_gqa_decode_case(77, [200, 130, 64], hq=8, hkv=2, unmapped_frac=0.0)
    table = np.ascontiguousarray(case.block_table[:, :5])  # 80 tokens of table
    k, v, kd, vd = _pools(case)
    out, lse = stp.paged_gqa_decode(to_dev(case.q), kd, vd, to_dev(table), to_dev(case.ctx_lens),
                                    case.page_size, case.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.paged_gqa_decode(case.q, k, v, table, case.ctx_lens, case.page_size,
                                           case.scale)
    assert_fp16_attention_close(out, lse, o_ref, l_ref, "past table")


def test_decode_long_context_small_pages():
    """Page size 1 and 5000 tokens: the block table is read in several chunks."""
    import sparse_top_paged_amd as stp
    case = workloads.random_gqa_decode_case(91, [5000, 4097, 2048, 2049], hq=8, hkv=2, page_size=1,
                                            unmapped_frac=0.05)
    k, v, kd, vd = _pools(case)
    out, lse = stp.paged_gqa_decode(to_dev(case.q), kd, vd, to_dev(case.block_table),
                                    to_dev(case.ctx_lens), case.page_size, case.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.paged_gqa_decode(case.q, k, v, case.block_table, case.ctx_lens,
                                           case.page_size, case.scale)
    assert_fp16_attention_close(out, lse, o_ref, l_ref, case.name)


@pytest.mark.parametrize("num_splits", [1, 2, 7, 40])
def test_decode_partitions(num_splits):
    """Partitions of the token range (some empty for the shorter requests,
    some crossing a block-table chunk), merged; page size 1 and 5000 tokens."""
    import sparse_top_paged_amd as stp
    case = workloads.random_gqa_decode_case(93, [5000, 4097, 130, 0, 2049], hq=16, hkv=4,
                                            page_size=1, unmapped_frac=0.05)
    k, v, kd, vd = _pools(case)
    assert stp.paged_gqa_decode_splits(5, 4, case.block_table.shape[1], 1, num_splits) == num_splits
    out, lse = stp.paged_gqa_decode(to_dev(case.q), kd, vd, to_dev(case.block_table),
                                    to_dev(case.ctx_lens), case.page_size, case.scale,
                                    num_splits=num_splits)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.paged_gqa_decode(case.q, k, v, case.block_table, case.ctx_lens,
                                           case.page_size, case.scale)
    assert_fp16_attention_close(out, lse, o_ref, l_ref, f"{case.name} splits {num_splits}")


def test_decode_full_size_sampled():
    import sparse_top_paged_amd as stp
    t0 = time.time()
    case = workloads.gqa_decode_case()
    kd, vd = workloads.dense_pool_torch(case.num_slots, case.hkv, case.pool_seed, dev())
    S = stp.paged_gqa_decode_splits(len(case.ctx_lens), case.hkv, case.block_table.shape[1],
                                    case.page_size)
    out, lse = stp.paged_gqa_decode(to_dev(case.q), kd, vd, to_dev(case.block_table),
                                    to_dev(case.ctx_lens), case.page_size, case.scale)
    torch.cuda.synchronize()
    print(f"[dense decode full] {S} partitions, ran at {time.time() - t0:.1f} s", flush=True)
    assert torch.isfinite(out.float()).all()
    order = np.argsort(case.ctx_lens)
    sample = sorted({0, 57, 127, int(order[0]), int(order[-1])})
    for b in sample:
        n = int(case.ctx_lens[b])
        slots = oracle.decode_slots(case.block_table[b], n, case.page_size)
        sl = torch.from_numpy(slots).to(dev())
        k = kd[sl].cpu().numpy()  # this request's rows, as slots 0 .. n - 1
        v = vd[sl].cpu().numpy()
        tab = np.arange(-(-n // case.page_size), dtype=np.int32)[None, :]
        o_ref, l_ref = oracle.paged_gqa_decode(case.q[b:b + 1], k, v, tab,
                                               np.asarray([n], np.int32), case.page_size,
                                               case.scale)
        assert_fp16_attention_close(out[b:b + 1], lse[b:b + 1], o_ref, l_ref, f"request {b}")
    print(f"[dense decode full] checked {sample} at {time.time() - t0:.1f} s", flush=True)


EXTEND_SMALL = [
    # (Lq per request, Lk per request)
    ([0, 1, 70, 130, 200, 10, 5, 64], [0, 6, 170, 130, 264, 3, 0, 64]),
    ([129, 1, 63], [400, 1, 63]),
]


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (8, 4), (6, 2)])
@pytest.mark.parametrize("lens", range(len(EXTEND_SMALL)))
def test_extend_small_ragged(hq, hkv, lens):
    import sparse_top_paged_amd as stp
    lq, lk = EXTEND_SMALL[lens]
    case = workloads.random_extend_case(100 * hq + 10 * hkv + lens, lq, lk, hq=hq, hkv=hkv)
    k, v, kd, vd = _pools(case)
    print(f"[dense extend] {case.name} hq {hq} hkv {hkv}", flush=True)
    out, lse = stp.extend_attention(to_dev(case.q), kd, vd, to_dev(case.qo_indptr),
                                    to_dev(case.kv_indptr), to_dev(case.kv_indices),
                                    case.max_extend_len, case.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.extend_attention(case.q, k, v, case.qo_indptr, case.kv_indptr,
                                           case.kv_indices, case.scale)
    assert_fp16_attention_close(out, lse, o_ref, l_ref, case.name)


def test_extend_full_size_sampled():
    import sparse_top_paged_amd as stp
    t0 = time.time()
    case = workloads.extend_case()
    kd, vd = workloads.dense_pool_torch(case.num_slots, case.hkv, case.pool_seed, dev())
    out, lse = stp.extend_attention(to_dev(case.q), kd, vd, to_dev(case.qo_indptr),
                                    to_dev(case.kv_indptr), to_dev(case.kv_indices),
                                    case.max_extend_len, case.scale)
    torch.cuda.synchronize()
    print(f"[dense extend full] ran at {time.time() - t0:.1f} s", flush=True)
    k, v = kd.cpu().numpy(), vd.cpu().numpy()
    group = case.q.shape[1] // case.hkv
    for b in (0, 5):
        q0, q1 = int(case.qo_indptr[b]), int(case.qo_indptr[b + 1])
        k0, k1 = int(case.kv_indptr[b]), int(case.kv_indptr[b + 1])
        for g in (0, 3, 7):
            heads = list(range(g * group, (g + 1) * group))
            # this request and KV group alone: a one-request batch of Hkv 1
            qs = np.ascontiguousarray(case.q[q0:q1, heads])
            kvi = case.kv_indices[k0:k1]
            o_ref, l_ref = oracle.extend_attention(
                qs, k[:, g:g + 1], v[:, g:g + 1], np.asarray([0, q1 - q0]),
                np.asarray([0, k1 - k0]), kvi, case.scale)
            assert_fp16_attention_close(out[q0:q1, heads], lse[q0:q1, heads], o_ref, l_ref,
                                        f"request {b} kv head {g}")
    print(f"[dense extend full] checked at {time.time() - t0:.1f} s", flush=True)
