"""The C-ABI library loads and exports every symbol include/stp.h declares (CPU only).

No compute call is made: only host-side argument validation, which returns
before anything touches a GPU.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "stp.h")
LIB = os.path.join(ROOT, "sparse_top_paged_amd", "libstp.so")
DIAG_HEADER = os.path.join(ROOT, "include", "stp_diag.h")
DIAG_LIB = os.path.join(ROOT, "sparse_top_paged_amd", "libstp_diag.so")


def declared(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(stp_\w+)\s*\(", text)))


def test_header_declares_the_path():
    names = declared()
    for n in ["stp_normalize_indices", "stp_hot_lookup_swapin", "stp_backup_rows",
              "stp_sparse_mla_decode", "stp_splitkv_merge", "stp_hot_reset",
              "stp_sparse_mla_decode_partial", "stp_sparse_mla_decode_workspace"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    assert os.path.exists(LIB), "libstp.so not built"
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


def test_binding_declares_every_symbol():
    from sparse_top_paged_amd._lib import SIGNATURES
    assert sorted(SIGNATURES) == declared()


def test_measurement_kernels_live_in_their_own_library():
    """include/stp_diag.h's calls are exported by libstp_diag.so, declared by
    the binding's diagnostic table, and absent from libstp.so."""
    from sparse_top_paged_amd._lib import DIAG_SIGNATURES, STP_ERR_INVALID_ARG
    from sparse_top_paged_amd import diag
    names = declared(DIAG_HEADER)
    assert names == sorted(DIAG_SIGNATURES) and "stp_row_gather" in names
    assert not set(names) & set(declared())
    dl = ctypes.CDLL(DIAG_LIB)
    assert all(hasattr(dl, n) for n in names)
    main = ctypes.CDLL(LIB)
    assert not any(hasattr(main, n) for n in names)
    # row size must be a multiple of 16, ranges must fit its id list
    fake = ctypes.c_void_p(16)
    g = diag.dlib.stp_row_gather
    assert g(fake, 10, 1000, fake, None, 8, 1, 1, 1, fake, None) == STP_ERR_INVALID_ARG
    assert g(fake, 10, 1152, fake, None, 8200, 1, 2, 1, fake, None) == STP_ERR_INVALID_ARG
    assert g(fake, 10, 1152, fake, None, 8, 0, 1, 1, fake, None) == 0  # T = 0
    assert diag.row_gather_blocks(32, 4, 2) == 256
    assert diag.row_gather_blocks(33, 8, 1) == 320
    assert diag.dlib.stp_stream_read(fake, 20, 4, fake, None) == STP_ERR_INVALID_ARG


def test_host_side_validation():
    import sparse_top_paged_amd as stp
    from sparse_top_paged_amd._lib import STP_ERR_INVALID_ARG, STP_ERR_WORKSPACE, lib

    # page size outside [1, 64]
    assert lib.stp_normalize_indices(None, 0, None, None, 1, None, 0, 0, 65, 0, 0, 0, None, None,
                                     None, None, None, None, None, None, None) == STP_ERR_INVALID_ARG
    assert b"page_size" in lib.stp_last_error()
    # cap smaller than top_k + window + sinks
    assert lib.stp_normalize_indices(None, 8, None, None, 1, None, 0, 0, 16, 4, 4, 10, None, None,
                                     None, None, None, None, None, None, None) == STP_ERR_INVALID_ARG
    # the normalisation split in two: the same checks, before any launch
    assert lib.stp_normalize_indices_deferred(None, 0, None, None, 1, None, 0, 0, 65, 0, 0, 0,
                                              None, None, None, None, None, None, None, None,
                                              None) == STP_ERR_INVALID_ARG
    assert lib.stp_normalize_indices_deferred(None, 8, None, None, 1, None, 0, 0, 16, 4, 4, 10,
                                              None, None, None, None, None, None, None, None,
                                              None) == STP_ERR_INVALID_ARG
    fill = lib.stp_block_view_fill
    assert fill(None, None, None, None, -1, None, 0, 0, 16, 4, None, None, None, None, None) == STP_ERR_INVALID_ARG
    assert fill(None, None, None, None, 1, None, 0, 0, 0, 4, None, None, None, None, None) == STP_ERR_INVALID_ARG
    assert b"page_size" in lib.stp_last_error()
    assert fill(None, None, None, None, 1, None, 0, 0, 16, 4, None, None, None, None, None) == STP_ERR_INVALID_ARG
    assert b"null pointer" in lib.stp_last_error()
    assert fill(None, None, None, None, 0, None, 0, 0, 16, 4, None, None, None, None, None) == 0
    # the merge and the block view in one call: both sets of checks before any launch
    mbv = lib.stp_splitkv_merge_with_block_view
    fake = ctypes.c_void_p(16)
    assert mbv(fake, fake, fake, 2, 0, 4, 512, fake, None, fake, fake, fake, fake, fake, 1, 4, 16,
               8, fake, fake, fake, fake, None) == STP_ERR_INVALID_ARG
    assert mbv(fake, fake, fake, 2, 2, 4, 512, fake, None, fake, fake, fake, fake, fake, 1, 4, 65,
               8, fake, fake, fake, fake, None) == STP_ERR_INVALID_ARG
    assert b"page_size" in lib.stp_last_error()
    assert mbv(fake, fake, fake, 2, 2, 4, 512, fake, None, fake, fake, fake, fake, fake, 1, 4, 16,
               8, None, fake, fake, fake, None) == STP_ERR_INVALID_ARG
    assert b"null pointer" in lib.stp_last_error()
    assert mbv(None, fake, fake, 2, 2, 4, 512, fake, None, fake, fake, fake, fake, fake, 1, 4, 16,
               8, fake, fake, fake, fake, None) == STP_ERR_INVALID_ARG
    assert mbv(None, None, None, 0, 2, 4, 512, None, None, None, None, None, None, None, 0, 0, 16,
               8, None, None, None, None, None) == 0  # T = 0
    # normalisation and decode in one call: both sets of checks before any launch
    nd = lib.stp_normalize_and_decode
    ndp = lib.stp_normalize_and_decode_partial_normalized
    norm_ok = [fake, 8, fake, fake, 2, fake, 1, 4, 16, 2, 1, 11, fake, fake, fake, None, None]
    bad_page = list(norm_ok)
    bad_page[8] = 65
    assert nd(*bad_page, None, None, None, fake, fake, 100, 16, 0.04, 1, None, 0, fake, None,
              None) == STP_ERR_INVALID_ARG
    assert b"page_size" in lib.stp_last_error()
    small_cap = list(norm_ok)
    small_cap[11] = 10  # < top_k + window + sinks
    assert nd(*small_cap, None, None, None, fake, fake, 100, 16, 0.04, 1, None, 0, fake, None,
              None) == STP_ERR_INVALID_ARG
    assert nd(*norm_ok, None, None, None, fake, fake, 100, 16, float("nan"), 1, None, 0, fake,
              None, None) == STP_ERR_INVALID_ARG
    assert nd(*norm_ok, None, None, None, fake, fake, 100, 16, 0.04, 1, None, 0, None, None,
              None) == STP_ERR_INVALID_ARG  # null out
    with_view = list(norm_ok)
    with_view[16] = fake  # blk_indptr without the other arrays
    assert nd(*with_view, None, None, None, fake, fake, 100, 16, 0.04, 1, None, 0, fake, None,
              None) == STP_ERR_INVALID_ARG
    assert nd(*norm_ok, None, None, None, fake, fake, 100, 16, 0.04, 4, None, 0, fake, None,
              None) == STP_ERR_WORKSPACE  # a split path without its workspace
    assert ndp(*norm_ok, fake, fake, 100, 16, 0.04, 0, fake, fake, fake,
               None) == STP_ERR_INVALID_ARG  # num_splits must be >= 1
    assert ndp(*norm_ok, fake, fake, 100, 16, 0.04, 2, None, fake, fake,
               None) == STP_ERR_INVALID_ARG
    empty = list(norm_ok)
    empty[4] = 0  # T = 0: nothing to do
    assert nd(*empty, None, None, None, fake, fake, 100, 16, 0.04, 4, None, 0, None, None,
              None) == 0
    # 16-byte row rule of the hot buffer (656 passes, 1000 fails)
    assert lib.stp_hot_lookup_swapin(None, 0, None, 1000, None, 0, None, None, None, 16, 17, 0, 0,
                                     None, None, None, None) == STP_ERR_INVALID_ARG
    assert lib.stp_hot_lookup_swapin(None, 0, None, 656, None, 0, None, None, None, 16, 17, 0, 0,
                                     None, None, None, None) == 0  # zero rows: nothing to launch
    # cap > hot_size could need more evictable slots than exist
    assert lib.stp_hot_lookup_swapin(None, 0, None, 1152, None, 20, None, None, None, 16, 17, 0, 1,
                                     None, None, None, None) == STP_ERR_INVALID_ARG
    assert lib.stp_backup_rows(None, 0, None, 0, 24, None, None, 1, None) == STP_ERR_INVALID_ARG
    # split decode without workspace is rejected before any launch
    fake = ctypes.c_void_p(16)
    assert lib.stp_sparse_mla_decode(fake, fake, 100, fake, None, 2180, 32, 128, 0.04, 4, None, 0,
                                     fake, None, None) == STP_ERR_WORKSPACE
    assert lib.stp_sparse_mla_decode(fake, fake, 100, fake, None, 64, 1, 16, float("nan"), 1,
                                     None, 0, fake, None, None) == STP_ERR_INVALID_ARG
    # the no-alloc decode: its scratch holds 36 MiB; a split path that needs more is
    # rejected before anything is launched, bad arguments as the workspace form
    noal = lib.stp_sparse_mla_decode_noalloc
    assert lib.stp_sparse_mla_decode_noalloc_max_bytes() == 36 << 20
    assert lib.stp_sparse_mla_decode_workspace(64, 128, 16384, 16) > 36 << 20
    assert noal(fake, fake, 100, fake, None, 16384, 64, 128, 0.04, 16, fake, None,
                None) == STP_ERR_WORKSPACE
    assert b"scratch" in lib.stp_last_error()
    assert noal(fake, fake, 100, fake, None, 64, 1, 16, float("nan"), 1, fake, None,
                None) == STP_ERR_INVALID_ARG
    assert noal(fake, fake, 100, fake, None, 64, 1, 16, 0.04, -1, fake, None,
                None) == STP_ERR_INVALID_ARG
    assert noal(fake, fake, 100, fake, None, 64, 1, 16, 0.04, 1, None, None,
                None) == STP_ERR_INVALID_ARG
    assert noal(fake, fake, 100, fake, None, 64, 0, 16, 0.04, 1, None, None, None) == 0  # T = 0
    assert lib.stp_splitkv_merge(None, None, None, 1, 1, 1, 6, None, None, None) == STP_ERR_INVALID_ARG
    assert stp.decode_splits(32, 128, 2180) >= 1
    assert stp.decode_workspace_bytes(1, 16, 44) == 0          # tiny shape runs unsplit
    assert stp.hot_lds_bytes(2180, 4096) > 0
    assert stp.hot_lds_bytes(40000, 32767) == 0
    # dense paged attention: head_dim 128 only, whole groups of at most 16 (decode)
    # or 4 (extend) query heads per KV head, positive finite scale, page size >= 1
    dec = lib.stp_paged_gqa_decode
    assert dec(fake, fake, fake, 64, fake, 4, fake, 2, 32, 8, 64, 16, 0.1, 0, None, 0, fake, None, None) == STP_ERR_INVALID_ARG
    assert dec(fake, fake, fake, 64, fake, 4, fake, 2, 68, 4, 128, 16, 0.1, 0, None, 0, fake, None, None) == STP_ERR_INVALID_ARG
    assert dec(fake, fake, fake, 64, fake, 4, fake, 2, 30, 8, 128, 16, 0.1, 0, None, 0, fake, None, None) == STP_ERR_INVALID_ARG
    assert dec(fake, fake, fake, 64, fake, 4, fake, 2, 32, 8, 128, 0, 0.1, 0, None, 0, fake, None, None) == STP_ERR_INVALID_ARG
    assert dec(fake, fake, fake, 64, fake, 4, fake, 2, 32, 8, 128, 16, 0.0, 0, None, 0, fake, None, None) == STP_ERR_INVALID_ARG
    assert dec(fake, fake, fake, 64, fake, 4, fake, 0, 32, 8, 128, 16, 0.1, 0, None, 0, fake, None, None) == 0
    # more than one partition without workspace, negative split count
    assert dec(fake, fake, fake, 64, fake, 64, fake, 2, 32, 8, 128, 16, 0.1, 4, None, 0, fake, None, None) == STP_ERR_WORKSPACE
    assert dec(fake, fake, fake, 64, fake, 4, fake, 2, 32, 8, 128, 16, 0.1, -1, None, 0, fake, None, None) == STP_ERR_INVALID_ARG
    assert lib.stp_paged_gqa_decode_splits(128, 8, 256, 16, 0) >= 1
    assert lib.stp_paged_gqa_decode_splits(2, 8, 256, 16, 3) == 3
    assert lib.stp_paged_gqa_decode_splits(2, 8, 1, 16, 5) == 1     # one tile: one partition
    assert lib.stp_paged_gqa_decode_workspace(2, 32, 8, 256, 16, 1) == 0
    assert lib.stp_paged_gqa_decode_workspace(2, 32, 8, 256, 16, 4) == 2 * 4 * 32 * 130 * 4
    # staged transfer: row size a multiple of 16 in [16, 65536], strides >= row size,
    # 1..32 buffers, at least one workgroup; n = 0 launches nothing
    bufs = (ctypes.c_void_p * 1)(fake)
    tr = lib.stp_kv_transfer
    assert tr(bufs, bufs, 1, 1000, 1008, 10, 1008, 10, fake, fake, 4, 1, None) == STP_ERR_INVALID_ARG
    assert tr(bufs, bufs, 1, 1152, 1136, 10, 1152, 10, fake, fake, 4, 1, None) == STP_ERR_INVALID_ARG
    assert tr(bufs, bufs, 0, 1152, 1152, 10, 1152, 10, fake, fake, 4, 1, None) == STP_ERR_INVALID_ARG
    assert tr(bufs, bufs, 33, 1152, 1152, 10, 1152, 10, fake, fake, 4, 1, None) == STP_ERR_INVALID_ARG
    assert tr(bufs, bufs, 1, 1152, 1152, 10, 1152, 10, fake, fake, 4, 0, None) == STP_ERR_INVALID_ARG
    assert tr(bufs, bufs, 1, 1152, 1152, 10, 1152, 10, fake, fake, 0, 1, None) == 0
    ext = lib.stp_extend_attention
    assert ext(fake, fake, fake, 64, fake, fake, fake, 2, 32, 4, 128, 64, 0.1, fake, None, None) == STP_ERR_INVALID_ARG
    assert ext(fake, fake, fake, 64, fake, fake, fake, 2, 32, 8, 96, 64, 0.1, fake, None, None) == STP_ERR_INVALID_ARG
    assert ext(fake, fake, fake, 64, fake, fake, fake, 2, 32, 8, 128, -1, 0.1, fake, None, None) == STP_ERR_INVALID_ARG
    assert ext(fake, fake, fake, 64, fake, fake, fake, 2, 32, 8, 128, 0, 0.1, fake, None, None) == 0
    assert ext(fake, fake, fake, 64, fake, fake, fake, 0, 32, 8, 128, 64, 0.1, fake, None, None) == 0
    # plan / run: task size in [1, 1120], plan buffer and workspace sized for the tier
    assert lib.stp_decode_plan_bytes(3, 50, 16) == (36 + 4 * 3 * 4 + 32 * 4) * 4
    assert lib.stp_decode_plan_bytes(3, 0, 16) == 36 * 4
    assert lib.stp_decode_run_workspace(3, 16, 50, 16) == 12 * 16 * 1024 + 2 * 768
    assert lib.stp_decode_plan_rows_per_task(32, 128, 2180) % 32 == 0
    assert 32 <= lib.stp_decode_plan_rows_per_task(32, 128, 2180) <= 1120
    plan = lib.stp_decode_plan
    assert plan(fake, 3, 50, 0, fake, 1 << 20, None) == STP_ERR_INVALID_ARG
    assert plan(fake, 3, 50, 1121, fake, 1 << 20, None) == STP_ERR_INVALID_ARG
    assert plan(fake, -1, 50, 16, fake, 1 << 20, None) == STP_ERR_INVALID_ARG
    assert plan(fake, 3, 50, 16, fake, 847, None) == STP_ERR_WORKSPACE
    assert plan(fake, 3, 50, 16, None, 1 << 20, None) == STP_ERR_INVALID_ARG
    run = lib.stp_decode_run
    assert run(fake, fake, 10, fake, 50, 3, 16, 0.1, 16, fake, 847, fake, 1 << 20, fake, None, None) == STP_ERR_WORKSPACE
    assert run(fake, fake, 10, fake, 50, 3, 16, 0.1, 16, fake, 848, fake, 1000, fake, None, None) == STP_ERR_WORKSPACE
    assert run(fake, fake, 10, fake, 50, 3, 16, 0.1, 2000, fake, 1 << 20, fake, 1 << 20, fake, None, None) == STP_ERR_INVALID_ARG
    assert run(fake, fake, 10, fake, 50, 3, 16, 0.0, 16, fake, 1 << 20, fake, 1 << 20, fake, None, None) == STP_ERR_INVALID_ARG
    assert run(fake, fake, 10, fake, 50, 0, 16, 0.1, 16, fake, 0, None, 0, fake, None, None) == 0


def test_missing_library_fails_loudly(tmp_path):
    from sparse_top_paged_amd import _lib
    with pytest.raises(ImportError):
        _lib.load(str(tmp_path / "libstp.so"))
