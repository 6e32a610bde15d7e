"""FP8 (OCP e4m3) quantization of the FP8 forward's inputs, for the oracle side of its parity tests.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests, the smoke check and the benchmark's
CPU-baseline leg may use it.

The pages name FP8 attention without giving a recipe; the recipe of the FP8 forward is: the rotated
queries and keys and the values are scaled, per 64-token tile of each (batch, head), by the power of two
2^-e that puts the tile's largest |element| in [128, 256), then rounded to e4m3 (round to nearest,
ties to even, saturating at +-448).  `fp8_self_fwd_ref` is plain fp64 attention on the dequantized
inputs; the P -> e4m3 rounding inside the kernel is not part of the oracle (the tests' tolerance covers
it).  e4m3 values are built from the format's definition (sign, 4 exponent bits with bias 7, 3 mantissa
bits; exponent field 0 is subnormal, m * 2^-9; field 15 with mantissa 7 is NaN), and rounding picks the
nearest of them by search, not by arithmetic on the bits.  Pinned in tests/test_oracle_fp8.py.
"""

import numpy as np

from .reference import rope3d_ref, self_fwd_ref


def e4m3_positive_values() -> np.ndarray:
    """All finite non-negative e4m3 values in code order (code 0 .. 126), ascending."""
    vals = []
    for code in range(127):                      # 127 = 0x7F is NaN
        ef, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if ef == 0 else (1.0 + m / 8.0) * 2.0 ** (ef - 7))
    return np.array(vals)


_POS = e4m3_positive_values()


def e4m3_round(x) -> np.ndarray:
    """Round each finite value to the nearest e4m3 value, ties to the even code; saturate at +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), _POS[-1])
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, len(_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS) - 1)
    d_lo, d_hi = a - _POS[lo], _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    return np.sign(x) * _POS[idx]


def tile_exponent(maxabs: float) -> int:
    """e with maxabs * 2^-e in [128, 256); 0 for maxabs == 0."""
    if maxabs <= 0:
        return 0
    m, ex = np.frexp(maxabs)                     # maxabs = m * 2^ex, m in [0.5, 1)
    return int(ex) - 8


def quantize_tiles(x, tile: int = 64) -> np.ndarray:
    """Dequantized e4m3 copy of x [B, L, H, D] under the per-(b, h, 64-token tile) power-of-two recipe."""
    x = np.asarray(x, dtype=np.float64)
    B, L, H, D = x.shape
    out = np.empty_like(x)
    for b in range(B):
        for h in range(H):
            for t0 in range(0, L, tile):
                blk = x[b, t0:t0 + tile, h, :]
                e = tile_exponent(float(np.abs(blk).max()))
                out[b, t0:t0 + tile, h, :] = e4m3_round(blk * 2.0 ** -e) * 2.0 ** e
    return out


def fp8_self_fwd_ref(q, k, v, scale: float, grid=None, rope=None, rows=None):
    """Self-attention (fp64) on the e4m3-dequantized rotated queries, rotated keys and values."""
    qt = rope3d_ref(q, grid, rope) if rope is not None else np.asarray(q, dtype=np.float64)
    kt = rope3d_ref(k, grid, rope) if rope is not None else np.asarray(k, dtype=np.float64)
    return self_fwd_ref(quantize_tiles(qt), quantize_tiles(kt), quantize_tiles(v), scale, rows=rows)
