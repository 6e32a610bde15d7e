"""Pins of the oracle's e4m3 rounding and FP8 tile recipe (CPU).

Independent checks: the e4m3 format's known landmarks (max normal 448, min normal 2^-6, min subnormal
2^-9, the count of finite values), ties to even at known midpoints, saturation, idempotence on every
representable value, the tile exponent's range, and that inputs already representable after the
recipe's scaling pass through unchanged.
"""

import numpy as np

from oracle import fp8
from oracle import RopeSpec
import oracle


def test_e4m3_landmarks():
    v = fp8.e4m3_positive_values()
    assert len(v) == 127 and v[0] == 0.0
    assert v[-1] == 448.0                       # 0x7E: (1 + 6/8) * 2^8
    assert v[1] == 2.0 ** -9                    # smallest subnormal
    assert v[8] == 2.0 ** -6                    # smallest normal (code 0x08)
    assert v[7] == 7 * 2.0 ** -9                # largest subnormal
    assert np.all(np.diff(v) > 0)
    assert 1.0 in v and 1.125 in v and 0.875 in v


def test_e4m3_rounding_ties_and_saturation():
    r = fp8.e4m3_round
    assert r(1.0625) == 1.0                     # midway 1.0 (code even) / 1.125 -> even
    assert r(1.1875) == 1.25                    # midway 1.125 (odd) / 1.25 (even)
    assert r(-1.1875) == -1.25
    assert r(1.06) == 1.0 and r(1.07) == 1.125
    assert r(500.0) == 448.0 and r(-1e9) == -448.0
    assert r(2.0 ** -10) == 0.0                 # midway 0 / 2^-9 -> 0 (even)
    assert r(3 * 2.0 ** -11) == 2.0 ** -9
    assert r(0.0) == 0.0


def test_e4m3_round_is_idempotent_on_every_value():
    v = fp8.e4m3_positive_values()
    np.testing.assert_array_equal(fp8.e4m3_round(v), v)
    np.testing.assert_array_equal(fp8.e4m3_round(-v), -v)


def test_tile_exponent_range():
    rng = np.random.default_rng(3)
    for x in np.concatenate([rng.uniform(1e-6, 1e6, 200), [1.0, 128.0, 255.999, 256.0, 2.0 ** -30]]):
        e = fp8.tile_exponent(float(x))
        assert 128.0 <= x * 2.0 ** -e < 256.0
    assert fp8.tile_exponent(0.0) == 0


def test_recipe_is_identity_on_representable_tiles():
    """x = y * 2^3 with y on the e4m3 grid, |y| <= 240 and each tile's max |y| = 224: the recipe picks
    e = 3 for every tile and dequantizes x to itself."""
    rng = np.random.default_rng(4)
    v = fp8.e4m3_positive_values()
    v = v[v <= 240.0]
    y = rng.choice(np.concatenate([v, -v]), size=(1, 128, 2, 16))
    y[0, 0, :, 0] = 224.0                        # tile maxima (tiles: tokens 0..63 and 64..127)
    y[0, 64, :, 0] = -224.0
    y[0, 1:64, :, 0] = np.clip(y[0, 1:64, :, 0], -224.0, 224.0)
    y[0, 65:, :, 0] = np.clip(y[0, 65:, :, 0], -224.0, 224.0)
    y = np.clip(y, -224.0, 224.0)
    x = y * 2.0 ** 3
    assert fp8.tile_exponent(float(np.abs(x[0, :64, 0]).max())) == 3
    np.testing.assert_array_equal(fp8.quantize_tiles(x), x)


def test_fp8_reference_is_attention_on_dequantized_inputs():
    rng = np.random.default_rng(5)
    grid = (2, 2, 2)
    q, k, v = (rng.standard_normal((1, 8, 1, 16)) for _ in range(3))
    rope = RopeSpec(4, 6, 6, 10000.0)
    o, lse = fp8.fp8_self_fwd_ref(q, k, v, 0.3, grid, rope)
    qt = fp8.quantize_tiles(oracle.rope3d_ref(q, grid, rope))
    kt = fp8.quantize_tiles(oracle.rope3d_ref(k, grid, rope))
    o2, lse2 = oracle.self_fwd_ref(qt, kt, fp8.quantize_tiles(v), 0.3)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-15)
    # quantization moves the result, but only by e4m3-sized amounts
    o3, _ = oracle.self_fwd_ref(q, k, v, 0.3, grid, rope)
    assert 0 < np.abs(o - o3).max() < 0.25
