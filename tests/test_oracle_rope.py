"""Pins of the oracle's token grid and 3D rotary embedding (CPU only).

Each check is independent of the formula it pins: hand-evaluated grid shapes
from the pages' shape formula, nested-loop enumeration, the complex-number form
of rotary embedding, textbook cos/sin values, and invariants (norm, inverse,
relative position, axis isolation) that a dropped term, a wrong sign, a wrong
pairing or a wrong segment offset would break.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import RopeSpec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "token_grids.json")


def test_token_grid_golden():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        grid = oracle.latent_token_grid(c["frames"], c["height"], c["width"])
        assert list(grid) == c["grid"], c
        assert int(np.prod(grid)) == c["L"]
        assert c["latent"][0] == grid[0] and c["latent"][1] == 2 * grid[1] and c["latent"][2] == 2 * grid[2]


def test_token_grid_rejects_bad_shapes():
    for args in [(80, 480, 832), (81, 470, 832), (0, 16, 16), (81, 480, 840)]:
        with pytest.raises(ValueError):
            oracle.latent_token_grid(*args)


def test_positions_row_major_nested_loops():
    grid = (3, 4, 5)
    expect = []
    for f in range(grid[0]):
        for h in range(grid[1]):
            for w in range(grid[2]):
                expect.append((f, h, w))
    assert np.array_equal(oracle.positions(grid), np.array(expect))


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_rope_1d_complex_form():
    """Whole head dim on the time axis of an L x 1 x 1 grid is the classic 1-D rotary embedding:
    pair j is the complex number x[2j] + i x[2j+1] multiplied by exp(i n theta^(-2j/D))."""
    L, D, theta = 11, 16, 500.0
    x = _rand((2, L, 3, D), 1)
    y = oracle.rope3d_ref(x, (L, 1, 1), RopeSpec(D, 0, 0, theta))
    z = x[..., 0::2] + 1j * x[..., 1::2]
    n = np.arange(L)[None, :, None, None]
    j = np.arange(D // 2)[None, None, None, :]
    zr = z * np.exp(1j * n * theta ** (-2.0 * j / D))
    expect = np.empty_like(x)
    expect[..., 0::2] = zr.real
    expect[..., 1::2] = zr.imag
    np.testing.assert_allclose(y, expect, rtol=0, atol=1e-13)


def test_rope_textbook_values_per_segment():
    """Unit vector on the first element of each segment's first pair: frequency 1, so the pair
    becomes (cos p, sin p) with p the token's position on that segment's axis."""
    rope = RopeSpec(4, 6, 6, 10000.0)
    D = 16
    grid = (3, 4, 5)
    pos = oracle.positions(grid)
    n = 2 * 20 + 2 * 5 + 3          # token (f=2, h=2, w=3)
    assert tuple(pos[n]) == (2, 2, 3)
    textbook = {2: (-0.4161468365471424, 0.9092974268256817),
                3: (-0.9899924966004454, 0.1411200080598672)}
    for seg_start, p in [(0, 2), (4, 2), (10, 3)]:
        x = np.zeros((1, 60, 1, D))
        x[0, n, 0, seg_start] = 1.0
        y = oracle.rope3d_ref(x, grid, rope)[0, n, 0]
        c, s = textbook[p]
        expect = np.zeros(D)
        expect[seg_start] = c
        expect[seg_start + 1] = s
        np.testing.assert_allclose(y, expect, atol=1e-15)


def test_rope_last_pair_frequency():
    """Last pair of the height segment (j = d_h/2 - 1) turns by h * theta^(-(d_h-2)/d_h)."""
    rope = RopeSpec(4, 6, 6, 100.0)
    grid = (1, 5, 1)
    x = np.zeros((1, 5, 1, 16))
    x[0, :, 0, 4 + 4] = 1.0          # element 2j of pair j=2 of the height segment
    y = oracle.rope3d_ref(x, grid, rope)[0, :, 0]
    ang = np.arange(5) * 100.0 ** (-4.0 / 6.0)
    np.testing.assert_allclose(y[:, 8], np.cos(ang), atol=1e-15)
    np.testing.assert_allclose(y[:, 9], np.sin(ang), atol=1e-15)


def test_rope_preserves_pair_norms_and_inverts():
    grid = (3, 4, 5)
    x = _rand((2, 60, 3, 128), 2)
    y = oracle.rope3d_ref(x, grid, RopeSpec())
    np.testing.assert_allclose(y[..., 0::2] ** 2 + y[..., 1::2] ** 2,
                               x[..., 0::2] ** 2 + x[..., 1::2] ** 2, rtol=1e-12)
    back = oracle.rope3d_ref(y, grid, RopeSpec(), inverse=True)
    np.testing.assert_allclose(back, x, atol=1e-12)


def test_rope_relative_position():
    """<R(p) q, R(p') k> depends only on p' - p, per axis."""
    rope = RopeSpec()
    rng = np.random.default_rng(3)
    q = rng.standard_normal(128)
    k = rng.standard_normal(128)
    for _ in range(10):
        p = rng.integers(0, 50, size=(1, 3))
        pp = rng.integers(0, 50, size=(1, 3))
        c = rng.integers(-20, 80, size=(1, 3))
        a = oracle.rope_apply(q[None], oracle.rope_angles(p, rope, 128))[0]
        b = oracle.rope_apply(k[None], oracle.rope_angles(pp, rope, 128))[0]
        a2 = oracle.rope_apply(q[None], oracle.rope_angles(p + c, rope, 128))[0]
        b2 = oracle.rope_apply(k[None], oracle.rope_angles(pp + c, rope, 128))[0]
        assert abs(a @ b - a2 @ b2) < 1e-11


def test_rope_axis_isolation():
    rope = RopeSpec()
    segs = {0: slice(0, 48), 1: slice(48, 88), 2: slice(88, 128)}
    for axis, grid in [(0, (7, 1, 1)), (1, (1, 7, 1)), (2, (1, 1, 7))]:
        x = _rand((1, 7, 2, 128), 4 + axis)
        y = oracle.rope3d_ref(x, grid, rope)
        moved = np.zeros(128, dtype=bool)
        moved[segs[axis]] = True
        np.testing.assert_array_equal(y[..., ~moved], x[..., ~moved])
        assert np.abs(y[..., moved] - x[..., moved]).max() > 0.1


def test_rope_zero_angle_is_identity():
    x = _rand((5, 128), 9)
    np.testing.assert_array_equal(oracle.rope_apply(x, np.zeros((5, 64))), x)


def test_rope_brute_force_loops():
    """Scalar loops over tokens and pairs, positions from div/mod, against the vectorized oracle."""
    rope = RopeSpec(4, 6, 6, 10000.0)
    grid = (2, 2, 3)
    F, Hp, Wp = grid
    L, H, D = 12, 2, 16
    x = _rand((1, L, H, D), 5)
    y = oracle.rope3d_ref(x, grid, rope)
    widths = [4, 6, 6]
    for n in range(L):
        pos = (n // (Hp * Wp), (n // Wp) % Hp, n % Wp)
        for h in range(H):
            k = 0
            for a in range(3):
                for j in range(widths[a] // 2):
                    phi = pos[a] * math.pow(10000.0, -2.0 * j / widths[a])
                    x0, x1 = x[0, n, h, 2 * k], x[0, n, h, 2 * k + 1]
                    assert abs(y[0, n, h, 2 * k] - (x0 * math.cos(phi) - x1 * math.sin(phi))) < 1e-13
                    assert abs(y[0, n, h, 2 * k + 1] - (x0 * math.sin(phi) + x1 * math.cos(phi))) < 1e-13
                    k += 1


def test_rope_table_matches_angles():
    grid = (21, 45, 80)
    rope = RopeSpec()
    tab = oracle.rope_table_ref(grid, rope)
    assert [t.shape for t in tab] == [(21, 24, 2), (45, 20, 2), (80, 20, 2)]
    pos = oracle.positions(grid)
    ang = oracle.rope_angles(pos, rope, 128)
    for n in [0, 1, 79, 80, 3600 * 7 + 45 * 80 - 1, 75599]:
        f, h, w = pos[n]
        cos = np.concatenate([tab[0][f, :, 0], tab[1][h, :, 0], tab[2][w, :, 0]])
        sin = np.concatenate([tab[0][f, :, 1], tab[1][h, :, 1], tab[2][w, :, 1]])
        np.testing.assert_allclose(cos, np.cos(ang[n]), atol=1e-15)
        np.testing.assert_allclose(sin, np.sin(ang[n]), atol=1e-15)


def test_rope_split_validation():
    for bad in [RopeSpec(47, 41, 40), RopeSpec(48, 40, 38), RopeSpec(-2, 90, 40)]:
        with pytest.raises(ValueError):
            oracle.rope_axis_of_pair(bad, 128)
