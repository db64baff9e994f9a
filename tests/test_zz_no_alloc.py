"""GPU parity of the no-alloc decode entry point (stp_sparse_mla_decode_noalloc),
called through the C ABI: bit for bit the output of stp_sparse_mla_decode with
a caller workspace (same kernels, same split count), and within the bf16 bar
of the fp64 oracle, on two calls in a row, the second with a smaller input
(the scratch keeps the first call's partials; nothing may leak into the
second)."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_attention_close, bf16_dev, dev, to_dev

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _noalloc(lib, q, kv, ids, counts, scale, splits):
    T, H, _ = q.shape
    out = torch.full((T, H, 512), float("nan"), dtype=torch.bfloat16, device=dev())
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device=dev())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.stp_sparse_mla_decode_noalloc(_ptr(q), _ptr(kv), kv.shape[0], _ptr(ids), _ptr(counts),
                                           ids.shape[1], T, H, float(scale), splits, _ptr(out),
                                           _ptr(lse), stream)
    assert rc == 0, lib.stp_last_error()
    return out, lse


@pytest.mark.parametrize("first,second", [((8, 128, 2180, 0), (3, 64, 500, 3)),
                                          ((6, 128, 700, 5), (2, 16, 40, 2))])
def test_noalloc_matches_workspace_entry_point(first, second):
    import sparse_top_paged_amd as stp
    from sparse_top_paged_amd._lib import lib
    rng = np.random.default_rng(sum(first) + sum(second))
    kv_rows = 20000
    kv_bits = workloads.normal_bf16(rng, (kv_rows, 576))
    kv = bf16_dev(kv_bits)
    for (T, H, cap, splits) in (first, second):
        assert stp.decode_splits(T, H, cap, splits) > 1  # the scratch is used
        q_bits = workloads.normal_bf16(rng, (T, H, 576))
        ids = rng.integers(-3, kv_rows + 3, size=(T, cap)).astype(np.int32)
        counts = np.asarray([cap - (7 * t) % max(1, cap) for t in range(T)], np.int32)
        q, ids_d, cnt_d = bf16_dev(q_bits), to_dev(ids), to_dev(counts)
        out, lse = _noalloc(lib, q, kv, ids_d, cnt_d, 576 ** -0.5, splits)
        ref_out, ref_lse = stp.sparse_mla_decode(q, kv, ids_d, cnt_d, 576 ** -0.5, splits)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), (T, H, cap)
        assert torch.equal(lse, ref_lse), (T, H, cap)
        o_ref, l_ref = oracle.attend_sparse(q_bits, kv_bits, ids, counts, 576 ** -0.5)
        assert_attention_close(out, lse, o_ref, l_ref, f"no-alloc T={T} H={H} cap={cap}")
