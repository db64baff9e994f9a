"""Top-k sparse MLA decode over a paged KV cache, native on MI355X (gfx950).

Thin Python binding over libstp.so (include/stp.h): each function checks
tensor shapes, dtypes and devices, passes raw pointers and the current HIP
stream, and returns.  Every step of the path runs in the HIP kernels; torch
only provides device memory, pinned host memory and streams.
"""

import torch

from ._lib import STP_ERR_HIP, STP_ERR_INVALID_ARG, STP_ERR_WORKSPACE, STP_OK, StpError, check, lib

D_QK = 576
D_V = 512

__all__ = [
    "StpError", "version", "normalize_indices", "block_view_fill", "hot_lookup_swapin", "hot_reset", "backup_rows",
    "sparse_mla_decode", "sparse_mla_decode_partial", "sparse_mla_decode_partial_normalized",
    "splitkv_merge", "splitkv_merge_normalized", "decode_splits",
    "decode_workspace_bytes", "hot_lds_bytes", "host_device_pointer",
    "splitkv_merge_with_block_view", "normalize_and_decode",
    "normalize_and_decode_partial_normalized",
    "paged_gqa_decode", "paged_gqa_decode_splits", "paged_gqa_decode_workspace_bytes",
    "extend_attention", "kv_transfer", "sparse_mla_decode_fp8", "decode_fp8_splits",
    "decode_fp8_workspace_bytes", "decode_plan", "decode_run", "decode_plan_bytes",
    "decode_run_workspace_bytes", "decode_plan_rows_per_task", "plan_view", "plan_queues",
]


def version():
    return lib.stp_version().decode()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t, name, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _opt(t, name, dtype, device):
    return None if t is None else _dev(t, name, dtype, device)


def host_device_pointer(t):
    """Device-visible address of a pinned host tensor."""
    if t.is_cuda or not t.is_pinned():
        raise ValueError("expected a pinned host tensor (pin_memory=True)")
    import ctypes
    out = ctypes.c_void_p()
    check(lib.stp_host_device_pointer(ctypes.c_void_p(t.data_ptr()), ctypes.byref(out)))
    return out.value


def normalize_indices(topk, req_id, q_pos, block_table, page_size, window, num_sinks, cap=None,
                      block_view=True, out=None, defer_block_view=False):
    """Stage 1.  Returns a dict: tok, slot [T, cap], count, dropped [T] and,
    with block_view, blk_indptr [T+1], blk_logical, blk_page, blk_mask [T*cap]."""
    dev = topk.device
    T, top_k = topk.shape
    num_reqs, max_blocks = block_table.shape
    if cap is None:
        cap = top_k + window + num_sinks
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = {
            "tok": torch.empty((T, cap), **i32),
            "slot": torch.empty((T, cap), **i32),
            "count": torch.empty((T,), **i32),
            "dropped": torch.empty((T,), **i32),
        }
        if block_view:
            out["blk_indptr"] = torch.empty((T + 1,), **i32)
            out["blk_logical"] = torch.empty((max(1, T * cap),), **i32)
            out["blk_page"] = torch.empty((max(1, T * cap),), **i32)
            out["blk_mask"] = torch.empty((max(1, T * cap),), dtype=torch.int64, device=dev)
    bv = "blk_indptr" in out
    entry = lib.stp_normalize_indices_deferred if defer_block_view else lib.stp_normalize_indices
    check(entry(
        _dev(topk, "topk", torch.int32, dev), top_k,
        _dev(req_id, "req_id", torch.int32, dev), _dev(q_pos, "q_pos", torch.int32, dev), T,
        _dev(block_table, "block_table", torch.int32, dev), num_reqs, max_blocks, page_size,
        window, num_sinks, cap,
        _dev(out["tok"], "tok", torch.int32, dev), _dev(out["slot"], "slot", torch.int32, dev),
        _dev(out["count"], "count", torch.int32, dev),
        _opt(out.get("dropped"), "dropped", torch.int32, dev),
        _dev(out["blk_indptr"], "blk_indptr", torch.int32, dev) if bv else None,
        _dev(out["blk_logical"], "blk_logical", torch.int32, dev) if bv else None,
        _dev(out["blk_page"], "blk_page", torch.int32, dev) if bv else None,
        _dev(out["blk_mask"], "blk_mask", torch.int64, dev) if bv else None,
        _stream(dev)))
    return out


def block_view_fill(norm, req_id, q_pos, block_table, page_size):
    """Complete the block view of normalize_indices(..., defer_block_view=True)
    on the current stream (norm: the dict that call returned)."""
    dev = norm["tok"].device
    T, cap = norm["tok"].shape
    num_reqs, max_blocks = block_table.shape
    check(lib.stp_block_view_fill(
        _dev(norm["tok"], "tok", torch.int32, dev), _dev(norm["slot"], "slot", torch.int32, dev),
        _dev(req_id, "req_id", torch.int32, dev), _dev(q_pos, "q_pos", torch.int32, dev), T,
        _dev(block_table, "block_table", torch.int32, dev), num_reqs, max_blocks, page_size, cap,
        _dev(norm["blk_indptr"], "blk_indptr", torch.int32, dev),
        _dev(norm["blk_logical"], "blk_logical", torch.int32, dev),
        _dev(norm["blk_page"], "blk_page", torch.int32, dev),
        _dev(norm["blk_mask"], "blk_mask", torch.int64, dev), _stream(dev)))
    return norm


def hot_lds_bytes(cap, hot_size):
    return lib.stp_hot_lds_bytes(cap, hot_size)


def hot_lookup_swapin(host_pool, hot_cache, global_ids, newest_global, dgi, lru, region_stride,
                      num_real_rows=None, hot_rows_out=None, miss_mask=None, stats=None,
                      host_pool_ptr=None):
    """Stage 2 lookup, LRU update and swap-in.  host_pool: pinned uint8
    [host_rows, row_bytes]; hot_cache: device uint8 [rows*stride, row_bytes];
    dgi int32 / lru int16 [rows, hot_size] (updated in place).
    Returns (hot_rows_out, miss_mask, stats)."""
    dev = hot_cache.device
    num_rows, cap = global_ids.shape
    hot_size = dgi.shape[1]
    host_rows, row_bytes = host_pool.shape
    if host_pool.dtype != torch.uint8 or hot_cache.dtype != torch.uint8:
        raise TypeError("host_pool and hot_cache must be uint8 byte views")
    if hot_cache.shape[1] != row_bytes or hot_cache.shape[0] < num_rows * region_stride:
        raise ValueError("hot_cache must be [num_rows * region_stride, row_bytes]")
    if tuple(lru.shape) != tuple(dgi.shape) or dgi.shape[0] != num_rows:
        raise ValueError("dgi and lru must be [num_rows, hot_size]")
    if num_real_rows is None:
        num_real_rows = num_rows
    if hot_rows_out is None:
        hot_rows_out = torch.empty((num_rows, cap), dtype=torch.int32, device=dev)
    if miss_mask is None:
        miss_mask = torch.empty((num_rows, cap), dtype=torch.uint8, device=dev)
    if stats is None:
        stats = torch.zeros(2, dtype=torch.int64, device=dev)
    if host_pool_ptr is None:
        host_pool_ptr = host_device_pointer(host_pool)
    if not host_pool.is_contiguous():
        raise ValueError("host_pool must be contiguous")
    check(lib.stp_hot_lookup_swapin(
        host_pool_ptr, host_rows, _dev(hot_cache, "hot_cache", torch.uint8, dev), row_bytes,
        _dev(global_ids, "global_ids", torch.int32, dev), cap,
        _dev(newest_global, "newest_global", torch.int32, dev),
        _dev(dgi, "dgi", torch.int32, dev), _dev(lru, "lru", torch.int16, dev), hot_size,
        region_stride, num_real_rows, num_rows,
        _dev(hot_rows_out, "hot_rows_out", torch.int32, dev),
        _opt(miss_mask, "miss_mask", torch.uint8, dev), _opt(stats, "stats", torch.int64, dev),
        _stream(dev)))
    return hot_rows_out, miss_mask, stats


def hot_reset(dgi, lru, rows=None):
    """Drop the cached state of the given request rows (all when None)."""
    dev = dgi.device
    hot_size = dgi.shape[1]
    n = dgi.shape[0] if rows is None else rows.numel()
    if tuple(lru.shape) != tuple(dgi.shape):
        raise ValueError("dgi and lru must have the same shape")
    check(lib.stp_hot_reset(_dev(dgi, "dgi", torch.int32, dev), _dev(lru, "lru", torch.int16, dev),
                            hot_size, dgi.shape[0], _opt(rows, "rows", torch.int32, dev), n,
                            _stream(dev)))


def backup_rows(hot_cache, host_pool, src_rows, dst_ids, host_pool_ptr=None):
    """BackUp: host_pool[dst_ids[j]] <- hot_cache[src_rows[j]] (byte rows)."""
    dev = hot_cache.device
    if host_pool_ptr is None:
        host_pool_ptr = host_device_pointer(host_pool)
    check(lib.stp_backup_rows(
        _dev(hot_cache, "hot_cache", torch.uint8, dev), hot_cache.shape[0], host_pool_ptr,
        host_pool.shape[0], hot_cache.shape[1], _dev(src_rows, "src_rows", torch.int32, dev),
        _dev(dst_ids, "dst_ids", torch.int32, dev), src_rows.numel(), _stream(dev)))


def decode_splits(T, H, cap, num_splits=0):
    return lib.stp_sparse_mla_decode_splits(T, H, cap, num_splits)


def decode_workspace_bytes(T, H, cap, num_splits=0):
    return lib.stp_sparse_mla_decode_workspace(T, H, cap, num_splits)


def _decode_common(q, kv, row_ids, counts):
    dev = q.device
    T, H, d = q.shape
    if d != D_QK or kv.dim() != 2 or kv.shape[1] != D_QK:
        raise ValueError("q must be [T, H, 576] and kv [rows, 576]")
    if row_ids.dim() != 2 or row_ids.shape[0] != T:
        raise ValueError("row_ids must be [T, cap]")
    return dev, T, H, row_ids.shape[1]


def sparse_mla_decode(q, kv, row_ids, counts=None, scale=D_QK ** -0.5, num_splits=0,
                      workspace=None, out=None, lse=None):
    """Stage 3 (+ stage 4 when split).  q [T, H, 576] bf16, kv [rows, 576] bf16,
    row_ids [T, cap] int32, counts [T] int32.  Returns (out [T, H, 512] bf16,
    lse [T, H] float32)."""
    dev, T, H, cap = _decode_common(q, kv, row_ids, counts)
    if out is None:
        out = torch.empty((T, H, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    need = decode_workspace_bytes(T, H, cap, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_ptr = None if workspace is None else _dev(workspace, "workspace", torch.uint8, dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    check(lib.stp_sparse_mla_decode(
        _dev(q, "q", torch.bfloat16, dev), _dev(kv, "kv", torch.bfloat16, dev), kv.shape[0],
        _dev(row_ids, "row_ids", torch.int32, dev), _opt(counts, "counts", torch.int32, dev), cap,
        T, H, float(scale), num_splits, ws_ptr, ws_bytes,
        _dev(out, "out", torch.bfloat16, dev), _opt(lse, "lse", torch.float32, dev), _stream(dev)))
    return out, lse


def sparse_mla_decode_partial(q, kv, row_ids, counts=None, scale=D_QK ** -0.5, num_splits=1,
                              o_part=None, m_part=None, l_part=None):
    """Split partial states: o [T, S, H, 512] (unnormalised), m, l [T, S, H] float32."""
    dev, T, H, cap = _decode_common(q, kv, row_ids, counts)
    S = num_splits
    if o_part is None:
        o_part = torch.empty((T, S, H, D_V), dtype=torch.float32, device=dev)
    if m_part is None:
        m_part = torch.empty((T, S, H), dtype=torch.float32, device=dev)
    if l_part is None:
        l_part = torch.empty((T, S, H), dtype=torch.float32, device=dev)
    check(lib.stp_sparse_mla_decode_partial(
        _dev(q, "q", torch.bfloat16, dev), _dev(kv, "kv", torch.bfloat16, dev), kv.shape[0],
        _dev(row_ids, "row_ids", torch.int32, dev), _opt(counts, "counts", torch.int32, dev), cap,
        T, H, float(scale), S, _dev(o_part, "o_part", torch.float32, dev),
        _dev(m_part, "m_part", torch.float32, dev), _dev(l_part, "l_part", torch.float32, dev),
        _stream(dev)))
    return o_part, m_part, l_part



def _norm_out(T, cap, dev, block_view):
    i32 = dict(dtype=torch.int32, device=dev)
    out = {"tok": torch.empty((T, cap), **i32), "slot": torch.empty((T, cap), **i32),
           "count": torch.empty((T,), **i32), "dropped": torch.empty((T,), **i32)}
    if block_view:
        out["blk_indptr"] = torch.empty((T + 1,), **i32)
        out["blk_logical"] = torch.empty((max(1, T * cap),), **i32)
        out["blk_page"] = torch.empty((max(1, T * cap),), **i32)
        out["blk_mask"] = torch.empty((max(1, T * cap),), dtype=torch.int64, device=dev)
    return out


def _norm_args(topk, req_id, q_pos, block_table, page_size, window, num_sinks, cap, norm, dev):
    T, top_k = topk.shape
    num_reqs, max_blocks = block_table.shape
    return [_dev(topk, "topk", torch.int32, dev), top_k, _dev(req_id, "req_id", torch.int32, dev),
            _dev(q_pos, "q_pos", torch.int32, dev), T,
            _dev(block_table, "block_table", torch.int32, dev), num_reqs, max_blocks, page_size,
            window, num_sinks, cap, _dev(norm["tok"], "tok", torch.int32, dev),
            _dev(norm["slot"], "slot", torch.int32, dev),
            _dev(norm["count"], "count", torch.int32, dev),
            _opt(norm.get("dropped"), "dropped", torch.int32, dev),
            _opt(norm.get("blk_indptr"), "blk_indptr", torch.int32, dev)]


def normalize_and_decode(topk, req_id, q_pos, block_table, page_size, window, num_sinks, q, kv,
                         scale=D_QK ** -0.5, num_splits=0, cap=None, block_view=True, norm=None,
                         workspace=None, out=None, lse=None):
    """normalize_indices and sparse_mla_decode over its lists in one call.
    Returns (out [T, H, 512] bf16, lse [T, H] float32, norm) with norm the dict
    normalize_indices returns."""
    dev = q.device
    T, top_k = topk.shape
    H = q.shape[1]
    if q.dim() != 3 or q.shape[0] != T or q.shape[2] != D_QK:
        raise ValueError("q must be [T, H, 576] for the T rows of topk")
    if kv.dim() != 2 or kv.shape[1] != D_QK:
        raise ValueError("kv must be [rows, 576]")
    if cap is None:
        cap = top_k + window + num_sinks
    if norm is None:
        norm = _norm_out(T, cap, dev, block_view)
    bv = "blk_indptr" in norm
    if out is None:
        out = torch.empty((T, H, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    need = decode_workspace_bytes(T, H, cap, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_ptr = None if workspace is None else _dev(workspace, "workspace", torch.uint8, dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    args = _norm_args(topk, req_id, q_pos, block_table, page_size, window, num_sinks, cap, norm,
                      dev)
    check(lib.stp_normalize_and_decode(
        *args, _dev(norm["blk_logical"], "blk_logical", torch.int32, dev) if bv else None,
        _dev(norm["blk_page"], "blk_page", torch.int32, dev) if bv else None,
        _dev(norm["blk_mask"], "blk_mask", torch.int64, dev) if bv else None,
        _dev(q, "q", torch.bfloat16, dev), _dev(kv, "kv", torch.bfloat16, dev), kv.shape[0], H,
        float(scale), num_splits, ws_ptr, ws_bytes, _dev(out, "out", torch.bfloat16, dev),
        _opt(lse, "lse", torch.float32, dev), _stream(dev)))
    return out, lse, norm


def normalize_and_decode_partial_normalized(topk, req_id, q_pos, block_table, page_size, window,
                                            num_sinks, q, kv, scale, num_splits, o_norm, m_part,
                                            l_part, cap=None, norm=None, block_view=True):
    """normalize_indices(..., defer_block_view=True) and
    sparse_mla_decode_partial_normalized over its lists in one call; returns
    norm.  splitkv_merge_with_block_view completes both."""
    dev = q.device
    T, top_k = topk.shape
    H = q.shape[1]
    if q.dim() != 3 or q.shape[0] != T or q.shape[2] != D_QK:
        raise ValueError("q must be [T, H, 576] for the T rows of topk")
    if cap is None:
        cap = top_k + window + num_sinks
    if norm is None:
        norm = _norm_out(T, cap, dev, block_view)
    args = _norm_args(topk, req_id, q_pos, block_table, page_size, window, num_sinks, cap, norm,
                      dev)
    check(lib.stp_normalize_and_decode_partial_normalized(
        *args, _dev(q, "q", torch.bfloat16, dev), _dev(kv, "kv", torch.bfloat16, dev), kv.shape[0],
        H, float(scale), num_splits, _dev(o_norm, "o_norm", torch.bfloat16, dev),
        _dev(m_part, "m_part", torch.float32, dev), _dev(l_part, "l_part", torch.float32, dev),
        _stream(dev)))
    return norm

def splitkv_merge(o_part, m_part, l_part, out=None, lse=None):
    """Stage 4: merge split states o [T, S, H, dv], m/l [T, S, H]."""
    dev = o_part.device
    T, S, H, dv = o_part.shape
    if out is None:
        out = torch.empty((T, H, dv), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    check(lib.stp_splitkv_merge(
        _dev(o_part, "o_part", torch.float32, dev), _dev(m_part, "m_part", torch.float32, dev),
        _dev(l_part, "l_part", torch.float32, dev), T, S, H, dv,
        _dev(out, "out", torch.bfloat16, dev), _opt(lse, "lse", torch.float32, dev), _stream(dev)))
    return out, lse


def sparse_mla_decode_partial_normalized(q, kv, row_ids, counts=None, scale=D_QK ** -0.5,
                                         num_splits=1, o_norm=None, m_part=None, l_part=None):
    """Split partial states in normalised form: o_norm [T, S, H, 512] bf16
    (o / l), m, l [T, S, H] float32 -- the split path of sparse_mla_decode."""
    dev, T, H, cap = _decode_common(q, kv, row_ids, counts)
    S = num_splits
    if o_norm is None:
        o_norm = torch.empty((T, S, H, D_V), dtype=torch.bfloat16, device=dev)
    if m_part is None:
        m_part = torch.empty((T, S, H), dtype=torch.float32, device=dev)
    if l_part is None:
        l_part = torch.empty((T, S, H), dtype=torch.float32, device=dev)
    check(lib.stp_sparse_mla_decode_partial_normalized(
        _dev(q, "q", torch.bfloat16, dev), _dev(kv, "kv", torch.bfloat16, dev), kv.shape[0],
        _dev(row_ids, "row_ids", torch.int32, dev), _opt(counts, "counts", torch.int32, dev), cap,
        T, H, float(scale), S, _dev(o_norm, "o_norm", torch.bfloat16, dev),
        _dev(m_part, "m_part", torch.float32, dev), _dev(l_part, "l_part", torch.float32, dev),
        _stream(dev)))
    return o_norm, m_part, l_part


def splitkv_merge_normalized(o_norm, m_part, l_part, out=None, lse=None):
    """Stage 4 from normalised bf16 split outputs o_norm [T, S, H, dv]."""
    dev = o_norm.device
    T, S, H, dv = o_norm.shape
    if out is None:
        out = torch.empty((T, H, dv), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    check(lib.stp_splitkv_merge_normalized(
        _dev(o_norm, "o_norm", torch.bfloat16, dev), _dev(m_part, "m_part", torch.float32, dev),
        _dev(l_part, "l_part", torch.float32, dev), T, S, H, dv,
        _dev(out, "out", torch.bfloat16, dev), _opt(lse, "lse", torch.float32, dev), _stream(dev)))
    return out, lse



def splitkv_merge_with_block_view(o_norm, m_part, l_part, norm, req_id, q_pos, block_table,
                                  page_size, out=None, lse=None):
    """splitkv_merge_normalized and block_view_fill of the same tokens in one
    call (norm: the dict of normalize_indices(..., defer_block_view=True))."""
    dev = o_norm.device
    T, S, H, dv = o_norm.shape
    Tn, cap = norm["tok"].shape
    if Tn != T:
        raise ValueError("the merge and the normalisation must cover the same tokens")
    num_reqs, max_blocks = block_table.shape
    if out is None:
        out = torch.empty((T, H, dv), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    check(lib.stp_splitkv_merge_with_block_view(
        _dev(o_norm, "o_norm", torch.bfloat16, dev), _dev(m_part, "m_part", torch.float32, dev),
        _dev(l_part, "l_part", torch.float32, dev), T, S, H, dv,
        _dev(out, "out", torch.bfloat16, dev), _opt(lse, "lse", torch.float32, dev),
        _dev(norm["tok"], "tok", torch.int32, dev), _dev(norm["slot"], "slot", torch.int32, dev),
        _dev(req_id, "req_id", torch.int32, dev), _dev(q_pos, "q_pos", torch.int32, dev),
        _dev(block_table, "block_table", torch.int32, dev), num_reqs, max_blocks, page_size, cap,
        _dev(norm["blk_indptr"], "blk_indptr", torch.int32, dev),
        _dev(norm["blk_logical"], "blk_logical", torch.int32, dev),
        _dev(norm["blk_page"], "blk_page", torch.int32, dev),
        _dev(norm["blk_mask"], "blk_mask", torch.int64, dev), _stream(dev)))
    return out, lse

def _pool(k_pool, v_pool):
    if k_pool.dim() != 3 or k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool must both be [slots, Hkv, head_dim]")
    return k_pool.device, k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]


def paged_gqa_decode_splits(B, Hkv, max_blocks, page_size, num_splits=0):
    return lib.stp_paged_gqa_decode_splits(B, Hkv, max_blocks, page_size, num_splits)


def paged_gqa_decode_workspace_bytes(B, Hq, Hkv, max_blocks, page_size, num_splits=0):
    return lib.stp_paged_gqa_decode_workspace(B, Hq, Hkv, max_blocks, page_size, num_splits)


def paged_gqa_decode(q, k_pool, v_pool, block_table, ctx_lens, page_size, scale=None,
                     num_splits=0, workspace=None, out=None, lse=None):
    """Dense paged decode with grouped query heads.  q [B, Hq, 128] fp16,
    k_pool / v_pool [slots, Hkv, 128] fp16, block_table [B, max_blocks] int32,
    ctx_lens [B] int32.  Returns (out [B, Hq, 128] fp16, lse [B, Hq] float32)."""
    dev, slots, Hkv, D = _pool(k_pool, v_pool)
    B, Hq = q.shape[0], q.shape[1]
    if q.dim() != 3 or q.shape[2] != D:
        raise ValueError("q must be [B, Hq, head_dim]")
    if block_table.dim() != 2 or block_table.shape[0] != B or ctx_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_blocks] and ctx_lens [B]")
    scale = D ** -0.5 if scale is None else scale
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    need = paged_gqa_decode_workspace_bytes(B, Hq, Hkv, block_table.shape[1], page_size,
                                            num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_ptr = None if workspace is None else _dev(workspace, "workspace", torch.uint8, dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    check(lib.stp_paged_gqa_decode(
        _dev(q, "q", torch.float16, dev), _dev(k_pool, "k_pool", torch.float16, dev),
        _dev(v_pool, "v_pool", torch.float16, dev), slots,
        _dev(block_table, "block_table", torch.int32, dev), block_table.shape[1],
        _dev(ctx_lens, "ctx_lens", torch.int32, dev), B, Hq, Hkv, D, page_size, float(scale),
        num_splits, ws_ptr, ws_bytes,
        _dev(out, "out", torch.float16, dev), _opt(lse, "lse", torch.float32, dev), _stream(dev)))
    return out, lse


def extend_attention(q, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices, max_extend_len,
                     scale=None, out=None, lse=None):
    """Prefix-extend attention with the shifted causal mask.  q [N, Hq, 128]
    fp16 packed by qo_indptr [B + 1]; keys at kv_indices[kv_indptr[b] ..
    kv_indptr[b + 1]) of the pools.  max_extend_len >= every request's query
    count.  Returns (out [N, Hq, 128] fp16, lse [N, Hq] float32)."""
    dev, slots, Hkv, D = _pool(k_pool, v_pool)
    if q.dim() != 3 or q.shape[2] != D:
        raise ValueError("q must be [N, Hq, head_dim]")
    N, Hq = q.shape[0], q.shape[1]
    B = qo_indptr.shape[0] - 1
    if B < 0 or kv_indptr.shape[0] != B + 1:
        raise ValueError("qo_indptr and kv_indptr must both be [B + 1]")
    scale = D ** -0.5 if scale is None else scale
    if out is None:
        out = torch.empty((N, Hq, D), dtype=torch.float16, device=dev)
    if lse is None:
        lse = torch.empty((N, Hq), dtype=torch.float32, device=dev)
    kvi = kv_indices if kv_indices.numel() > 0 else torch.zeros(1, dtype=torch.int32, device=dev)
    check(lib.stp_extend_attention(
        _dev(q, "q", torch.float16, dev), _dev(k_pool, "k_pool", torch.float16, dev),
        _dev(v_pool, "v_pool", torch.float16, dev), slots,
        _dev(qo_indptr, "qo_indptr", torch.int32, dev), _dev(kv_indptr, "kv_indptr", torch.int32, dev),
        _dev(kvi, "kv_indices", torch.int32, dev), B, Hq, Hkv, D, int(max_extend_len),
        float(scale), _dev(out, "out", torch.float16, dev), _opt(lse, "lse", torch.float32, dev),
        _stream(dev)))
    return out, lse


def _visible_ptr(t):
    """Device-visible address of a device tensor or of a pinned host tensor
    (a view into pinned memory too: the allocation's base is mapped and the
    view's offset added)."""
    import ctypes
    if t.is_cuda:
        return t.data_ptr()
    if not t.is_pinned():
        raise ValueError("host buffers must be pinned (pin_memory=True)")
    base = t.untyped_storage().data_ptr()
    out = ctypes.c_void_p()
    check(lib.stp_host_device_pointer(ctypes.c_void_p(base), ctypes.byref(out)))
    return out.value + (t.data_ptr() - base)


def kv_transfer(src_bufs, dst_bufs, src_idx, dst_idx, row_bytes=None, src_stride=None,
                dst_stride=None, src_rows=None, dst_rows=None, num_blocks=4):
    """Staged bulk copy of rows: for every buffer pair and position i,
    dst[dst_idx[i]] <- src[src_idx[i]] (row_bytes each).  Buffers are device
    tensors or pinned host tensors, all of one side alike in shape; by default
    a buffer is [rows, row_bytes] bytes (strides = row_bytes, rows = its row
    count).  src_idx / dst_idx: device int32 [n]."""
    import ctypes
    if not src_bufs or len(src_bufs) != len(dst_bufs):
        raise ValueError("src_bufs and dst_bufs must be equally long, non-empty lists")
    dev = src_idx.device
    s0, d0 = src_bufs[0], dst_bufs[0]
    row_bytes = row_bytes or s0.shape[-1] * s0.element_size()
    src_stride = src_stride or row_bytes
    dst_stride = dst_stride or row_bytes
    if src_rows is None:
        src_rows = s0.numel() * s0.element_size() // src_stride
    if dst_rows is None:
        dst_rows = d0.numel() * d0.element_size() // dst_stride
    n = src_idx.numel()
    if dst_idx.numel() != n:
        raise ValueError("src_idx and dst_idx must have the same length")
    nb = len(src_bufs)
    sp = (ctypes.c_void_p * nb)(*[_visible_ptr(t) for t in src_bufs])
    dp = (ctypes.c_void_p * nb)(*[_visible_ptr(t) for t in dst_bufs])
    check(lib.stp_kv_transfer(sp, dp, nb, row_bytes, src_stride, src_rows, dst_stride, dst_rows,
                              _dev(src_idx, "src_idx", torch.int32, dev),
                              _dev(dst_idx, "dst_idx", torch.int32, dev), n, num_blocks,
                              _stream(dev)))


FP8_ROW_BYTES = 656


def decode_fp8_splits(T, H, cap, num_splits=0):
    return lib.stp_sparse_mla_decode_fp8_splits(T, H, cap, num_splits)


def decode_fp8_workspace_bytes(T, H, cap, num_splits=0):
    return lib.stp_sparse_mla_decode_fp8_workspace(T, H, cap, num_splits)


def sparse_mla_decode_fp8(q, kv, row_ids, counts=None, scale=D_QK ** -0.5, num_splits=0,
                          workspace=None, out=None, lse=None):
    """Stage 3 over fp8_ds_mla rows: q [T, H, 576] bf16, kv [rows, 656] uint8,
    row_ids [T, cap] int32, counts [T] int32.  Returns (out [T, H, 512] bf16,
    lse [T, H] float32)."""
    dev = q.device
    if q.dim() != 3 or q.shape[2] != D_QK:
        raise ValueError("q must be [T, H, 576]")
    if kv.dim() != 2 or kv.shape[1] != FP8_ROW_BYTES or kv.dtype != torch.uint8:
        raise ValueError("kv must be uint8 [rows, 656]")
    T, H = q.shape[0], q.shape[1]
    if row_ids.dim() != 2 or row_ids.shape[0] != T:
        raise ValueError("row_ids must be [T, cap]")
    cap = row_ids.shape[1]
    if out is None:
        out = torch.empty((T, H, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    need = decode_fp8_workspace_bytes(T, H, cap, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_ptr = None if workspace is None else _dev(workspace, "workspace", torch.uint8, dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    check(lib.stp_sparse_mla_decode_fp8(
        _dev(q, "q", torch.bfloat16, dev), _dev(kv, "kv", torch.uint8, dev), kv.shape[0],
        _dev(row_ids, "row_ids", torch.int32, dev), _opt(counts, "counts", torch.int32, dev), cap,
        T, H, float(scale), num_splits, ws_ptr, ws_bytes,
        _dev(out, "out", torch.bfloat16, dev), _opt(lse, "lse", torch.float32, dev), _stream(dev)))
    return out, lse


def decode_plan_rows_per_task(T, H, cap):
    return lib.stp_decode_plan_rows_per_task(T, H, cap)


def decode_plan_bytes(T, cap, rows_per_task):
    return lib.stp_decode_plan_bytes(T, cap, rows_per_task)


def decode_run_workspace_bytes(T, H, cap, rows_per_task):
    return lib.stp_decode_run_workspace(T, H, cap, rows_per_task)


def decode_plan(counts, T, cap, rows_per_task, plan=None, device=None):
    """Plan of a capacity tier (T rows, cap candidates, rows_per_task per
    task) from counts [T] int32 on the device (None: every row has cap).
    Returns the plan buffer (int32 device tensor), allocated when not given."""
    dev = counts.device if counts is not None else (device or torch.device("cuda"))
    need = decode_plan_bytes(T, cap, rows_per_task)
    if plan is None:
        plan = torch.empty((max(need, 4) // 4,), dtype=torch.int32, device=dev)
    check(lib.stp_decode_plan(_opt(counts, "counts", torch.int32, dev), T, cap, rows_per_task,
                              _dev(plan, "plan", torch.int32, dev), plan.numel() * 4,
                              _stream(dev)))
    return plan


def plan_view(plan, T):
    """(number of tasks, row_first [T + 1], tasks [n, 4]) views of a plan
    buffer, in the layout stp_decode_plan writes."""
    n = int(plan[0].item())
    off = (33 + T + 3) // 4 * 4
    return n, plan[32:33 + T], plan[off:off + 4 * n].view(n, 4)


def plan_queues(plan, T):
    """(qcount [8], segments [8, qcap, 4]) views of a plan buffer: the run's
    eight queues; queue x is segments[x, :qcount[x]], entries (row, start,
    length, slot)."""
    max_tasks, qcap = int(plan[3].item()), int(plan[20].item())
    off = (33 + T + 3) // 4 * 4 + 4 * max_tasks
    return plan[12:20], plan[off:off + 32 * qcap].view(8, qcap, 4)


def decode_run(q, kv, row_ids, plan, rows_per_task, scale=D_QK ** -0.5, workspace=None,
               out=None, lse=None):
    """Run over a plan: q [T, H, 576] bf16, kv [rows, 576] bf16, row_ids
    [T, cap] int32, plan from decode_plan with the same T, cap and
    rows_per_task.  Returns (out [T, H, 512] bf16, lse [T, H] float32)."""
    dev = q.device
    if q.dim() != 3 or q.shape[2] != D_QK:
        raise ValueError("q must be [T, H, 576]")
    if kv.dim() != 2 or kv.shape[1] != D_QK:
        raise ValueError("kv must be [rows, 576]")
    T, H = q.shape[0], q.shape[1]
    if row_ids.dim() != 2 or row_ids.shape[0] != T:
        raise ValueError("row_ids must be [T, cap]")
    cap = row_ids.shape[1]
    if out is None:
        out = torch.empty((T, H, D_V), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    need = decode_run_workspace_bytes(T, H, cap, rows_per_task)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_ptr = None if workspace is None else _dev(workspace, "workspace", torch.uint8, dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    check(lib.stp_decode_run(
        _dev(q, "q", torch.bfloat16, dev), _dev(kv, "kv", torch.bfloat16, dev), kv.shape[0],
        _dev(row_ids, "row_ids", torch.int32, dev), cap, T, H, float(scale), rows_per_task,
        _dev(plan, "plan", torch.int32, dev), plan.numel() * 4, ws_ptr, ws_bytes,
        _dev(out, "out", torch.bfloat16, dev), _opt(lse, "lse", torch.float32, dev), _stream(dev)))
    return out, lse
