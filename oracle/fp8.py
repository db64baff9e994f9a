"""fp8_ds_mla latent rows (oracle, plain definition, fp64).

TEST INFRASTRUCTURE ONLY -- see the package header.

What it states ("HiSparse" walkthrough, the FlashMLASparseBackend cache
shape and the FP8_DS_MLA_ROW_BYTES constant with its comment; "5.1.1 · 从索引
到 Kernel" §7.2, dequantisation at tile load with the scale applied before
QK / AV): a 656-byte row holds 512 bytes of quantised latent (NoPE) values,
16 bytes of scales and 128 bytes of RoPE values.  Read here as:
  * bytes 0..511: 512 FP8 E4M3 codes (the OCP "fn" variant: bias 7, no
    infinities, S.1111.111 is NaN), latent value i = e4m3(code_i) *
    scale_{i // 128};
  * bytes 512..527: the four scales, float32 little-endian, one per 128
    latent values;
  * bytes 528..655: the 64 RoPE values, bf16 little-endian.
The dequantised row is the 576-value key (latent then RoPE) and its first
512 values are the value vector, as for the bf16 rows of the same cache.
Attention over such rows is attend_sparse over the dequantised rows.

Pins (tests/test_oracle_fp8.py): the decoder against torch's float8_e4m3fn
for all 256 codes, and its printed special values (1, 448, 2^-6, 2^-9, -0,
NaN); the byte layout 512 + 16 + 128 = 656 of the page; a hand-built row
dequantised by hand; attention over fp8 rows whose dequantised values are
exact in bf16 equals the pinned bf16 attention over those values.
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


def dequant_rows(rows):
    """[n, 656] uint8 rows -> [n, 576] float64 keys (latent, then RoPE)."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8).reshape(-1, ROW_BYTES)
    n = rows.shape[0]
    scales = rows[:, SCALE_OFF:ROPE_OFF].copy().view("<f4").astype(np.float64)  # [n, 4]
    latent = e4m3_to_f64(rows[:, :NOPE]).reshape(n, NOPE // GROUP, GROUP) * scales[:, :, None]
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
