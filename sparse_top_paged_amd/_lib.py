"""ctypes loader for libstp.so: declares every exported C-ABI function.

Fails loudly when the library has not been built: there is no fallback.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libstp.so")

STP_OK = 0
STP_ERR_INVALID_ARG = 1
STP_ERR_WORKSPACE = 2
STP_ERR_HIP = 3

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

# name -> (restype, argtypes), in the order of include/stp.h
SIGNATURES = {
    "stp_last_error": (ctypes.c_char_p, []),
    "stp_version": (ctypes.c_char_p, []),
    "stp_host_device_pointer": (ctypes.c_int, [_p, ctypes.POINTER(ctypes.c_void_p)]),
    "stp_normalize_indices": (ctypes.c_int, [
        _p, _i32, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32,
        _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "stp_normalize_indices_deferred": (ctypes.c_int, [
        _p, _i32, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32,
        _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "stp_block_view_fill": (ctypes.c_int, [
        _p, _p, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p]),
    "stp_hot_lookup_swapin": (ctypes.c_int, [
        _p, _i64, _p, _i64, _p, _i32, _p, _p, _p, _i32, _i32, _i32, _i32, _p, _p, _p, _p]),
    "stp_hot_lds_bytes": (_sz, [_i32, _i32]),
    "stp_hot_reset": (ctypes.c_int, [_p, _p, _i32, _i32, _p, _i32, _p]),
    "stp_backup_rows": (ctypes.c_int, [_p, _i64, _p, _i64, _i64, _p, _p, _i32, _p]),
    "stp_sparse_mla_decode": (ctypes.c_int, [
        _p, _p, _i64, _p, _p, _i32, _i32, _i32, _f32, _i32, _p, _sz, _p, _p, _p]),
    "stp_sparse_mla_decode_noalloc": (ctypes.c_int, [
        _p, _p, _i64, _p, _p, _i32, _i32, _i32, _f32, _i32, _p, _p, _p]),
    "stp_sparse_mla_decode_noalloc_max_bytes": (_sz, []),
    "stp_sparse_mla_decode_fp8": (ctypes.c_int, [
        _p, _p, _i64, _p, _p, _i32, _i32, _i32, _f32, _i32, _p, _sz, _p, _p, _p]),
    "stp_sparse_mla_decode_fp8_splits": (_i32, [_i32, _i32, _i32, _i32]),
    "stp_sparse_mla_decode_fp8_workspace": (_sz, [_i32, _i32, _i32, _i32]),
    "stp_decode_plan": (ctypes.c_int, [_p, _i32, _i32, _i32, _p, _sz, _p]),
    "stp_decode_run": (ctypes.c_int, [
        _p, _p, _i64, _p, _i32, _i32, _i32, _f32, _i32, _p, _sz, _p, _sz, _p, _p, _p]),
    "stp_decode_plan_bytes": (_sz, [_i32, _i32, _i32]),
    "stp_decode_run_workspace": (_sz, [_i32, _i32, _i32, _i32]),
    "stp_decode_plan_rows_per_task": (_i32, [_i32, _i32, _i32]),
    "stp_sparse_mla_decode_splits": (_i32, [_i32, _i32, _i32, _i32]),
    "stp_sparse_mla_decode_workspace": (_sz, [_i32, _i32, _i32, _i32]),
    "stp_sparse_mla_decode_partial": (ctypes.c_int, [
        _p, _p, _i64, _p, _p, _i32, _i32, _i32, _f32, _i32, _p, _p, _p, _p]),
    "stp_sparse_mla_decode_partial_normalized": (ctypes.c_int, [
        _p, _p, _i64, _p, _p, _i32, _i32, _i32, _f32, _i32, _p, _p, _p, _p]),
    "stp_splitkv_merge": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _i32, _p, _p, _p]),
    "stp_splitkv_merge_normalized": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _i32, _p, _p, _p]),
    "stp_normalize_and_decode": (ctypes.c_int, [
        _p, _i32, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32,
        _p, _p, _p, _p, _p, _p, _p, _p,
        _p, _p, _i64, _i32, _f32, _i32, _p, _sz, _p, _p, _p]),
    "stp_normalize_and_decode_partial_normalized": (ctypes.c_int, [
        _p, _i32, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _i32,
        _p, _p, _p, _p, _p,
        _p, _p, _i64, _i32, _f32, _i32, _p, _p, _p, _p]),
    "stp_splitkv_merge_with_block_view": (ctypes.c_int, [
        _p, _p, _p, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
        _p, _p, _p, _p, _p]),
    "stp_paged_gqa_decode": (ctypes.c_int, [
        _p, _p, _p, _i64, _p, _i32, _p, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _p, _sz,
        _p, _p, _p]),
    "stp_paged_gqa_decode_splits": (_i32, [_i32, _i32, _i32, _i32, _i32]),
    "stp_paged_gqa_decode_workspace": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "stp_kv_transfer": (ctypes.c_int, [
        _p, _p, _i32, _i64, _i64, _i64, _i64, _i64, _p, _p, _i32, _i32, _p]),
    "stp_extend_attention": (ctypes.c_int, [
        _p, _p, _p, _i64, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _f32, _p, _p, _p]),
}


# the measurement kernels of include/stp_diag.h (libstp_diag.so)
DIAG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libstp_diag.so")
DIAG_SIGNATURES = {
    "stp_row_gather": (ctypes.c_int, [_p, _i64, _i64, _p, _p, _i32, _i32, _i32, _i32, _p, _p]),
    "stp_row_gather_blocks": (_i32, [_i32, _i32, _i32]),
    "stp_stream_read": (ctypes.c_int, [_p, _i64, _i32, _p, _p]),
}


class StpError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"stp status {status}: {message}")
        self.status = status


def load(path=LIB_PATH, signatures=None):
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python sparse_top_paged_amd/build.py or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    for name, (res, args) in (SIGNATURES if signatures is None else signatures).items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = load()


def check(status):
    if status != STP_OK:
        raise StpError(status, lib.stp_last_error().decode(errors="replace"))
