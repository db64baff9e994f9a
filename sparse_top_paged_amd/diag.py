"""Measurement kernels beside the library (libstp_diag.so, include/stp_diag.h):
the decode's row gather with nothing else, and a plain sequential read --
the practical ceilings the decode's rates are set against.  Argument
marshalling only, as the main binding.
"""

import torch

from . import _lib
from ._lib import check
from . import _dev, _opt, _stream

dlib = _lib.load(_lib.DIAG_LIB_PATH, _lib.DIAG_SIGNATURES)

__all__ = ["row_gather", "row_gather_blocks", "stream_read"]


def row_gather_blocks(T, parts, replicas):
    """Workgroups (= checksum words) of row_gather."""
    return dlib.stp_row_gather_blocks(T, parts, replicas)


def row_gather(rows, row_ids, counts=None, parts=1, replicas=1, checksum=None):
    """Diagnostic: read the candidate rows exactly as the decode splits and
    places them, computing only an xor per workgroup.  rows: uint8
    [num_rows, row_bytes] (or any 2-D contiguous tensor, taken as bytes);
    row_ids [T, cap] int32.  Returns the uint32 checksums (as int32)."""
    dev = rows.device
    if rows.dim() != 2 or not rows.is_contiguous() or not rows.is_cuda:
        raise ValueError("rows must be a contiguous 2-D device tensor")
    T, cap = row_ids.shape
    row_bytes = rows.shape[1] * rows.element_size()
    nblk = dlib.stp_row_gather_blocks(T, parts, replicas)
    if checksum is None:
        checksum = torch.empty((max(1, nblk),), dtype=torch.int32, device=dev)
    check(dlib.stp_row_gather(
        rows.data_ptr(), rows.shape[0], row_bytes, _dev(row_ids, "row_ids", torch.int32, dev),
        _opt(counts, "counts", torch.int32, dev), cap, T, parts, replicas,
        _dev(checksum, "checksum", torch.int32, dev), _stream(dev)))
    return checksum


def stream_read(src, blocks=2048, checksum=None):
    """Diagnostic: a plain sequential read of a contiguous device tensor (its
    bytes, a multiple of 16) with `blocks` workgroups; returns the per-workgroup
    xor checksums (as int32)."""
    dev = src.device
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    if checksum is None:
        checksum = torch.empty((blocks,), dtype=torch.int32, device=dev)
    check(dlib.stp_stream_read(src.data_ptr(), src.numel() * src.element_size(), blocks,
                              _dev(checksum, "checksum", torch.int32, dev), _stream(dev)))
    return checksum
