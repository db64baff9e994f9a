"""Helpers shared by the GPU parity tests (marshalling and the tolerance rule)."""

import numpy as np
import torch

# bf16 attention output against the fp64 oracle: every element within 2e-2
# absolute, every (token, head) vector within 1e-2 of its largest reference
# magnitude, and lse within 1e-2.
ABS_TOL = 2e-2
REL_TOL = 1e-2
LSE_TOL = 1e-2


def dev():
    return torch.device("cuda:0")


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    return t if dtype is None else t.to(dtype)


def bf16_dev(bits):
    """uint16 bf16 bit patterns (numpy) -> device bf16 tensor."""
    return to_dev(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def bf16_bits_of(t):
    """device/host bf16 tensor -> numpy uint16 bits."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_attention_close(out, lse, out_ref, lse_ref, where=""):
    """Tolerance rule for bf16 attention outputs (out: torch bf16, refs fp64)."""
    o = to_f64(out)
    err = np.abs(o - out_ref)
    assert np.all(np.isfinite(o)), f"{where}: non-finite output"
    assert err.max(initial=0.0) <= ABS_TOL, f"{where}: max abs error {err.max()}"
    scale = np.abs(out_ref).max(axis=-1)
    row_err = err.max(axis=-1)
    live = scale > 0
    rel = np.where(live, row_err / np.where(live, scale, 1.0), row_err)
    assert rel.max(initial=0.0) <= REL_TOL, f"{where}: max rel error {rel.max()}"
    if lse is not None:
        l = lse.detach().cpu().numpy().astype(np.float64)
        both_inf = np.isneginf(l) & np.isneginf(lse_ref)
        assert np.array_equal(np.isneginf(l), np.isneginf(lse_ref)), f"{where}: empty rows differ"
        d = np.abs(np.where(both_inf, 0.0, l - np.where(both_inf, 0.0, lse_ref)))
        assert d.max(initial=0.0) <= LSE_TOL, f"{where}: max lse error {d.max()}"
    return err.max(initial=0.0), rel.max(initial=0.0)


# fp16 attention output against the fp64 oracle.  The output is rounded to
# fp16 once (half an ulp: <= 2^-11 |o|, about 1e-3 at |o| <= 2); the extend
# kernel also rounds the softmax weights to fp16 before the PV product
# (relative 2^-11 per weight, so |o~ - o| <= 2^-11 max |v| <= 2.5e-3 for
# N(0, 1) values below 5); scores and sums are fp32.  lse is computed from
# fp32 sums and maxima only.
FP16_ABS_TOL = 5e-3
FP16_LSE_TOL = 1e-3


def assert_fp16_attention_close(out, lse, out_ref, lse_ref, where=""):
    o = to_f64(out)
    assert np.all(np.isfinite(o)), f"{where}: non-finite output"
    err = np.abs(o - out_ref)
    assert err.max(initial=0.0) <= FP16_ABS_TOL, f"{where}: max abs error {err.max()}"
    if lse is not None:
        l = lse.detach().cpu().numpy().astype(np.float64) if hasattr(lse, "detach") else lse
        assert np.array_equal(np.isneginf(l), np.isneginf(lse_ref)), f"{where}: empty rows differ"
        fin = ~np.isneginf(lse_ref)
        d = np.abs(l[fin] - lse_ref[fin])
        assert d.max(initial=0.0) <= FP16_LSE_TOL, f"{where}: max lse error {d.max()}"
    return err.max(initial=0.0)
