"""fp8_ds_mla latent rows (oracle, plain definition, fp64).

TEST INFRASTRUCTURE ONLY -- see the package header.

What it states ("HiSparse" walkthrough, the FlashMLASparseBackend cache
shape and the FP8_DS_MLA_ROW_BYTES constant with its comment; "5.1.1 · 从索引
到 Kernel" §7.2, dequantisation at tile load with the scale applied before
QK / AV): a 656-byte row holds 512 bytes of quantised latent (NoPE) values,
16 bytes of scales and 128 bytes of RoPE values.  Read here as:
  * bytes 0..511: 512 FP8 E4M3 codes (the OCP "fn" variant: bias 7, no
    infinities, S.1111.111 is NaN), latent value i reconstructed from code_i
    and scale_{i // 128};
  * bytes 512..527: the four scales, float32 little-endian, one per 128
    latent values;
  * bytes 528..655: the 64 RoPE values, bf16 little-endian.
The dequantised row is the 576-value key (latent then RoPE) and its first
512 values are the value vector, as for the bf16 rows of the same cache.
Attention over such rows is attend_sparse over the dequantised rows.

Reconstruction.  §7.2 has the scale applied as soon as the tile is loaded,
the reconstructed values then feeding QK and AV, and the correctness
baseline computing with the same reconstructed KV, so that the kernel's own
error is seen apart from the quantisation error.  The page fixes no type for
the reconstructed values; the reading taken is the type the products take
in the rest of the path, bf16: value = bf16(f32(e4m3(code)) * f32(scale)),
the product rounded to float32 and then to bf16, both to nearest, ties to
even.  dequant_rows(rows, exact=True) gives the exact fp64 product instead
(the quantisation error's reference).

Pins (tests/test_oracle_fp8.py): the decoder against torch's float8_e4m3fn
for all 256 codes, and its printed special values (1, 448, 2^-6, 2^-9, -0,
NaN); the byte layout 512 + 16 + 128 = 656 of the page; a hand-built row
dequantised by hand; the reconstruction's rounding on hand-worked cases
(ties to even both ways, 0.37, overflow to infinity) and its error bound
against the exact product; attention over fp8 rows whose dequantised values
are exact in bf16 equals the pinned bf16 attention over those values.
"""

import numpy as np

from .attention import attend_sparse, bf16_bits_to_f64

ROW_BYTES = 656
NOPE = 512
GROUP = 128
SCALE_OFF = 512
ROPE_OFF = 528
ROPE = 64


def e4m3_to_f64(codes):
    """OCP FP8 E4M3 (fn) codes -> float64, by the format's definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


def f32_to_bf16(x):
    """float32 values -> the nearest bf16 values (ties to even), as float64.
    NaN stays NaN; values past the largest bf16 round to infinity."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    upper = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    r = (upper.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.where(np.isnan(x), np.nan, r)


def reconstruct(codes, scales):
    """bf16(f32(e4m3(code)) * f32(scale)), broadcasting codes against scales."""
    with np.errstate(over="ignore"):  # a product past float32's range is infinite
        prod = e4m3_to_f64(codes).astype(np.float32) * np.asarray(scales, dtype=np.float32)
    return f32_to_bf16(prod)


def dequant_rows(rows, exact=False):
    """[n, 656] uint8 rows -> [n, 576] float64 keys (latent, then RoPE); the
    latent values reconstructed in bf16 (exact=True: the exact products)."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8).reshape(-1, ROW_BYTES)
    n = rows.shape[0]
    scales = rows[:, SCALE_OFF:ROPE_OFF].copy().view("<f4")  # [n, 4] float32
    codes = rows[:, :NOPE].reshape(n, NOPE // GROUP, GROUP)
    if exact:
        latent = e4m3_to_f64(codes) * scales.astype(np.float64)[:, :, None]
    else:
        latent = reconstruct(codes, scales[:, :, None])
    rope = bf16_bits_to_f64(rows[:, ROPE_OFF:].copy().view("<u2"))
    return np.concatenate([latent.reshape(n, NOPE), rope], axis=1)


class _Fp8Getter:
    def __init__(self, rows):
        self.pool = rows
        self.rows = rows.shape[0]

    def __call__(self, idx):
        return dequant_rows(self.pool[idx])


def attend_sparse_fp8(q_bits, rows656, row_ids, counts, scale):
    """attend_sparse over fp8_ds_mla rows: q [T, H, 576] bf16 bits, rows656
    [rows, 656] uint8 -> out [T, H, 512], lse [T, H] (fp64)."""
    return attend_sparse(q_bits, _Fp8Getter(np.asarray(rows656, dtype=np.uint8)), row_ids, counts,
                         scale)
