"""Pins for the fp8_ds_mla row oracle (CPU only).

The E4M3 decoder against torch's float8_e4m3fn for all 256 codes and its
special values; the 512 + 16 + 128 = 656 byte layout of the HiSparse page; a
hand-built row dequantised by hand; the bf16 reconstruction of the latent
values on hand-worked roundings and against the exact product's error bound;
attention over fp8 rows whose values are exact in bf16 equals the pinned bf16
attention over the same values.
"""

import math

import numpy as np
import torch

import oracle
import workloads


def test_decoder_against_torch_float8():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_special_values():
    d = oracle.e4m3_to_f64
    assert d([0x38])[0] == 1.0
    assert d([0x7E])[0] == 448.0             # largest finite
    assert d([0x08])[0] == 2.0 ** -6          # smallest normal
    assert d([0x01])[0] == 2.0 ** -9          # smallest subnormal
    assert d([0x80])[0] == 0.0 and math.copysign(1, d([0x80])[0]) < 0
    assert np.isnan(d([0x7F])[0]) and np.isnan(d([0xFF])[0])
    assert d([0xC0])[0] == -2.0


def test_layout_and_hand_built_row():
    from oracle import fp8
    assert fp8.NOPE + (fp8.ROPE_OFF - fp8.SCALE_OFF) + fp8.ROPE * 2 == 656 == fp8.ROW_BYTES
    row = np.zeros(656, np.uint8)
    row[0], row[1], row[127] = 0x38, 0xC0, 0x08          # 1, -2, 2^-6 in group 0
    row[128], row[511] = 0x40, 0x7E                      # 2 in group 1, 448 in group 3
    row[512:528] = np.asarray([0.5, 3.0, 1.0, 0.25], "<f4").view(np.uint8)
    rope = np.zeros(64, "<u2")
    rope[0], rope[63] = 0x3F80, 0xC040                   # bf16 1.0 and -3.0
    row[528:] = rope.view(np.uint8)
    k = oracle.dequant_rows(row[None, :])[0]
    assert k.shape == (576,)
    assert k[0] == 0.5 and k[1] == -1.0 and k[127] == 0.5 * 2.0 ** -6
    assert k[128] == 6.0 and k[511] == 112.0
    assert k[512] == 1.0 and k[575] == -3.0
    assert np.count_nonzero(k) == 7


def test_attention_reduces_to_bf16_attention():
    """Power-of-two scales and E4M3 values are exact in bf16, so the fp8 rows'
    attention equals the bf16 oracle over rows holding the dequantised values."""
    rng = np.random.default_rng(4)
    rows = workloads.fp8_rows(rng, 40, pow2_scales=True)
    K = oracle.dequant_rows(rows)
    kv_bits = workloads.bf16_bits(K.astype(np.float32))
    assert np.array_equal(oracle.bf16_bits_to_f64(kv_bits), K)   # exact in bf16
    q = workloads.normal_bf16(rng, (2, 8, 576))
    ids = np.stack([rng.permutation(40)[:25], rng.permutation(40)[:25]]).astype(np.int32)
    counts = np.asarray([25, 17], np.int32)
    o8, l8 = oracle.attend_sparse_fp8(q, rows, ids, counts, 576 ** -0.5)
    ob, lb = oracle.attend_sparse(q, kv_bits, ids, counts, 576 ** -0.5)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


def test_reconstruction_rounds_to_nearest_even():
    """bf16(f32(code) * f32(scale)) on cases worked by hand: bf16 keeps 8
    significant bits, so 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 (even:
    1), 1 + 3 2^-8 halfway between 1 + 2^-7 and 1 + 2^-6 (even: 1 + 2^-6);
    0.37 = 1.0111101 0111... x 2^-2 rounds down to 1.0111101 x 2^-2; 448 x
    2^120 is past float32's range."""
    r = oracle.reconstruct
    one, c448, c_m2 = 0x38, 0x7E, 0xC0                   # 1.0, 448, -2
    assert r([one], [1.0 + 2.0 ** -8])[0] == 1.0
    assert r([one], [1.0 + 3 * 2.0 ** -8])[0] == 1.0 + 2.0 ** -6
    assert r([one], [1.0 + 5 * 2.0 ** -9])[0] == 1.0 + 2.0 ** -7   # above half: up
    assert r([one], [0.37])[0] == 0.369140625
    assert r([c_m2], [0.37])[0] == -0.73828125
    assert r([c448], [2.0 ** -20])[0] == 448.0 * 2.0 ** -20       # powers of two: exact
    assert np.isposinf(r([c448], [2.0 ** 120])[0])
    assert np.isnan(r([0x7F], [1.0])[0])
    k = oracle.dequant_rows(np.zeros((1, 656), np.uint8))[0]
    assert not np.any(k) and np.count_nonzero(np.signbit(k)) == 0


def test_reconstruction_error_bound():
    """|bf16(f32(x s)) - x s| <= 2^-8 |x s| (half a bf16 ulp, 2^-9 relative,
    after a float32 rounding of 2^-24): the reconstruction stays within the
    bound of the exact product over random codes and scales."""
    rng = np.random.default_rng(9)
    rows = workloads.fp8_rows(rng, 64)
    exact = oracle.dequant_rows(rows, exact=True)
    rec = oracle.dequant_rows(rows)
    ok = np.isfinite(exact)
    assert np.all(np.abs(rec[ok] - exact[ok]) <= 2.0 ** -8 * np.abs(exact[ok]))
    assert np.array_equal(rec[:, 512:], exact[:, 512:])           # RoPE values as stored
    assert np.count_nonzero(rec[ok] != exact[ok]) > 0              # arbitrary scales do round
