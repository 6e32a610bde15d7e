"""Pins of the oracle's attention forward (self and cross) on the CPU.

Independent checks: scalar loops with math.fsum, closed forms (scale 0, a single
valid key, empty key set), invariants (softmax rows sum to 1, constant values),
and a library routine (fp64 CPU torch scaled_dot_product_attention, with a
boolean mask for cross-attention).
"""

import math

import numpy as np
import pytest

import oracle
from oracle import RopeSpec


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _brute_self(q, k, v, scale, grid, rope):
    """Scalar fsum loops: rotate with explicit cos/sin, then softmax attention row by row."""
    B, L, H, D = q.shape
    F, Hp, Wp = grid
    widths = [rope.d_f, rope.d_h, rope.d_w]

    def rot(x, n):
        pos = (n // (Hp * Wp), (n // Wp) % Hp, n % Wp)
        y = [0.0] * D
        kk = 0
        for a in range(3):
            for j in range(widths[a] // 2):
                phi = pos[a] * math.pow(rope.theta, -2.0 * j / widths[a])
                y[2 * kk] = x[2 * kk] * math.cos(phi) - x[2 * kk + 1] * math.sin(phi)
                y[2 * kk + 1] = x[2 * kk] * math.sin(phi) + x[2 * kk + 1] * math.cos(phi)
                kk += 1
        return y

    o = np.zeros_like(q)
    lse = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            qt = [rot(list(q[b, i, h]), i) for i in range(L)]
            kt = [rot(list(k[b, j, h]), j) for j in range(L)]
            for i in range(L):
                s = [scale * math.fsum(qt[i][d] * kt[j][d] for d in range(D)) for j in range(L)]
                m = max(s)
                z = math.fsum(math.exp(x - m) for x in s)
                lse[b, h, i] = m + math.log(z)
                for d in range(D):
                    o[b, i, h, d] = math.fsum(math.exp(s[j] - m) / z * v[b, j, h, d] for j in range(L))
    return o, lse


@pytest.mark.parametrize("D,rope,grid,H", [(16, RopeSpec(4, 6, 6, 10000.0), (2, 2, 3), 2),
                                           (128, RopeSpec(), (2, 2, 2), 1)])
def test_self_fwd_brute_force(D, rope, grid, H):
    L = int(np.prod(grid))
    q, k, v = (_rand((1, L, H, D), s) for s in (10, 11, 12))
    scale = 1 / math.sqrt(D)
    o, lse = oracle.self_fwd_ref(q, k, v, scale, grid, rope)
    ob, lb = _brute_self(q, k, v, scale, grid, rope)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(lse, lb, atol=1e-12)


def test_softmax_rows_sum_to_one_and_constant_values():
    L, H, D = 40, 2, 128
    q, k = _rand((1, L, H, D), 20, 3.0), _rand((1, L, H, D), 21)
    ones = np.ones((1, L, H, D))
    o, _ = oracle.self_fwd_ref(q, k, ones, 0.3, (5, 4, 2), RopeSpec())
    np.testing.assert_allclose(o, 1.0, atol=1e-13)
    const = np.broadcast_to(_rand((1, 1, H, D), 22), (1, L, H, D))
    o, _ = oracle.self_fwd_ref(q, k, const, 0.3, (5, 4, 2), RopeSpec())
    np.testing.assert_allclose(o, np.broadcast_to(const, o.shape), atol=1e-12)


def test_scale_zero_closed_form():
    L, H, D = 24, 2, 128
    q, k, v = (_rand((2, L, H, D), s) for s in (30, 31, 32))
    o, lse = oracle.self_fwd_ref(q, k, v, 0.0, (2, 3, 4), RopeSpec())
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), atol=1e-13)
    np.testing.assert_allclose(lse, math.log(L), atol=1e-14)
    lens = np.array([7, 24])
    o, lse = oracle.cross_fwd_ref(q, k, v, lens, 0.0)
    for b, n in enumerate(lens):
        np.testing.assert_allclose(o[b], np.broadcast_to(v[b, :n].mean(axis=0), o[b].shape), atol=1e-13)
        np.testing.assert_allclose(lse[b], math.log(n), atol=1e-14)


def test_cross_single_key_and_empty():
    B, Lq, Lk, H, D = 2, 9, 16, 3, 128
    q, k, v = _rand((B, Lq, H, D), 40), _rand((B, Lk, H, D), 41), _rand((B, Lk, H, D), 42)
    o, lse = oracle.cross_fwd_ref(q, k, v, np.array([1, 0]), 0.125)
    for h in range(H):
        np.testing.assert_allclose(o[0, :, h], np.broadcast_to(v[0, 0, h], (Lq, D)), atol=1e-14)
        np.testing.assert_allclose(lse[0, h], 0.125 * q[0, :, h] @ k[0, 0, h], atol=1e-13)
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))


def test_cross_full_length_equals_unmasked_and_clamps():
    B, Lq, Lk, H, D = 2, 7, 12, 2, 128
    q, k, v = _rand((B, Lq, H, D), 50), _rand((B, Lk, H, D), 51), _rand((B, Lk, H, D), 52)
    a = oracle.cross_fwd_ref(q, k, v, np.array([Lk, Lk]), 0.1)
    b = oracle.cross_fwd_ref(q, k, v, None, 0.1)
    c = oracle.cross_fwd_ref(q, k, v, np.array([Lk + 50, 10 ** 6]), 0.1)
    for x, y in [(a, b), (a, c)]:
        np.testing.assert_array_equal(x[0], y[0])
        np.testing.assert_array_equal(x[1], y[1])
    d = oracle.cross_fwd_ref(q, k, v, np.array([-3, 0]), 0.1)
    assert np.all(d[0] == 0)


def test_cross_masked_keys_never_matter():
    B, Lq, Lk, H, D = 2, 6, 20, 2, 128
    q, k, v = _rand((B, Lq, H, D), 60), _rand((B, Lk, H, D), 61), _rand((B, Lk, H, D), 62)
    lens = np.array([5, 13])
    o1, l1 = oracle.cross_fwd_ref(q, k, v, lens, 0.2)
    k2, v2 = k.copy(), v.copy()
    for b, n in enumerate(lens):
        k2[b, n:] = np.nan
        v2[b, n:] = np.inf
    o2, l2 = oracle.cross_fwd_ref(q, k2, v2, lens, 0.2)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_rows_subset_matches_full():
    grid = (3, 4, 5)
    q, k, v = (_rand((2, 60, 3, 128), s) for s in (70, 71, 72))
    o, lse = oracle.self_fwd_ref(q, k, v, 0.088, grid, RopeSpec())
    rows = np.stack([np.stack([np.array([0, 7, 59]) + h for h in range(3)]) for _ in range(2)]) % 60
    os_, ls_ = oracle.self_fwd_ref(q, k, v, 0.088, grid, RopeSpec(), rows=rows)
    for b in range(2):
        for h in range(3):
            np.testing.assert_allclose(os_[b, h], o[b, rows[b, h], h], atol=1e-13)
            np.testing.assert_allclose(ls_[b, h], lse[b, h, rows[b, h]], atol=1e-13)


def test_lse_against_scipy_logsumexp():
    from scipy.special import logsumexp
    q, k, v = (_rand((1, 30, 1, 128), s, 4.0) for s in (80, 81, 82))
    _, lse = oracle.self_fwd_ref(q, k, v, 0.5, None, None)
    s = 0.5 * q[0, :, 0] @ k[0, :, 0].T
    np.testing.assert_allclose(lse[0, 0], logsumexp(s, axis=1), atol=1e-12)


torch = pytest.importorskip("torch")


def test_self_fwd_matches_torch_sdpa_without_rope():
    B, L, H, D = 2, 33, 3, 128
    q, k, v = (_rand((B, L, H, D), s) for s in (90, 91, 92))
    o, _ = oracle.self_fwd_ref(q, k, v, 0.07, None, None)
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=0.07)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), atol=1e-13)


def test_self_fwd_with_rope_is_sdpa_of_rotated_inputs():
    grid = (3, 2, 5)
    B, L, H, D = 1, 30, 2, 128
    q, k, v = (_rand((B, L, H, D), s) for s in (93, 94, 95))
    o, _ = oracle.self_fwd_ref(q, k, v, 0.09, grid, RopeSpec())
    qt = oracle.rope3d_ref(q, grid, RopeSpec())
    kt = oracle.rope3d_ref(k, grid, RopeSpec())
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(t(qt), t(kt), t(v), scale=0.09)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), atol=1e-13)


def test_cross_fwd_matches_torch_sdpa_with_mask():
    B, Lq, Lk, H, D = 2, 17, 40, 2, 128
    q, k, v = _rand((B, Lq, H, D), 96), _rand((B, Lk, H, D), 97), _rand((B, Lk, H, D), 98)
    lens = np.array([23, 40])
    o, _ = oracle.cross_fwd_ref(q, k, v, lens, 0.1)
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
    mask = torch.arange(Lk)[None, None, None, :] < torch.from_numpy(lens)[:, None, None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask, scale=0.1)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), atol=1e-13)
