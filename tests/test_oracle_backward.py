"""Pins of the oracle's attention backward on the CPU.

Central finite differences of <dO, O> (RoPE on, so the rotary gradient is
covered), fp64 torch autograd through scaled_dot_product_attention (RoPE off;
boolean mask for cross-attention), the invariants sum_j dV_j = sum_i dO_i and
dQ = 0 for identical keys, and agreement of the sampled-row paths with the
full backward.
"""

import numpy as np
import pytest

import oracle
from oracle import RopeSpec


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _loss(q, k, v, do, scale, grid, rope):
    o, _ = oracle.self_fwd_ref(q, k, v, scale, grid, rope)
    return float(np.sum(do * o))


@pytest.mark.parametrize("rope,D,grid", [(RopeSpec(4, 6, 6, 10000.0), 16, (2, 2, 3)),
                                         (RopeSpec(48, 40, 40, 10000.0), 128, (2, 2, 2))])
def test_self_bwd_finite_differences(rope, D, grid):
    L = int(np.prod(grid))
    H = 2
    q, k, v, do = (_rand((1, L, H, D), s) for s in (1, 2, 3, 4))
    scale = 0.3
    dq, dk, dv = oracle.self_bwd_ref(q, k, v, do, scale, grid, rope)
    eps = 1e-6
    rng = np.random.default_rng(5)
    for name, x, g in [("q", q, dq), ("k", k, dk), ("v", v, dv)]:
        for _ in range(12):
            idx = tuple(rng.integers(0, n) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd = (_loss(args_p["q"], args_p["k"], args_p["v"], do, scale, grid, rope)
                  - _loss(args_m["q"], args_m["k"], args_m["v"], do, scale, grid, rope)) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(g[idx])), (name, idx, fd, g[idx])


def test_self_bwd_dv_sum_and_identical_keys():
    L, H, D = 30, 2, 128
    q, k, v, do = (_rand((1, L, H, D), s) for s in (6, 7, 8, 9))
    _, _, dv = oracle.self_bwd_ref(q, k, v, do, 0.2, (2, 3, 5), RopeSpec())
    np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), atol=1e-12)
    same_k = np.broadcast_to(k[:, :1], k.shape).copy()
    dq, _, _ = oracle.self_bwd_ref(q, same_k, v, do, 0.2, None, None)
    np.testing.assert_allclose(dq, 0.0, atol=1e-13)


def test_sampled_rows_match_full_backward():
    grid = (3, 4, 5)
    B, L, H, D = 1, 60, 2, 128
    q, k, v, do = (_rand((B, L, H, D), s) for s in (10, 11, 12, 13))
    dq, dk, dv = oracle.self_bwd_ref(q, k, v, do, 0.1, grid, RopeSpec())
    rows = np.array([[[0, 5, 33, 59], [1, 2, 3, 58]]])
    dq_r = oracle.self_bwd_dq_rows(q, k, v, do, 0.1, grid, RopeSpec(), rows)
    dk_r, dv_r = oracle.self_bwd_dkdv_rows(q, k, v, do, 0.1, grid, RopeSpec(), rows, block=16)
    for h in range(H):
        np.testing.assert_allclose(dq_r[0, h], dq[0, rows[0, h], h], atol=1e-13)
        np.testing.assert_allclose(dk_r[0, h], dk[0, rows[0, h], h], atol=1e-13)
        np.testing.assert_allclose(dv_r[0, h], dv[0, rows[0, h], h], atol=1e-13)
    dk_1, _ = oracle.self_bwd_dkdv_rows(q, k, v, do, 0.1, grid, RopeSpec(), rows, heads=[1])
    assert np.isnan(dk_1[0, 0]).all()
    np.testing.assert_allclose(dk_1[0, 1], dk[0, rows[0, 1], 1], atol=1e-13)


def test_cross_bwd_finite_differences_and_padding():
    B, Lq, Lk, H, D = 2, 5, 9, 1, 16
    q, do = _rand((B, Lq, H, D), 20), _rand((B, Lq, H, D), 21)
    k, v = _rand((B, Lk, H, D), 22), _rand((B, Lk, H, D), 23)
    lens = np.array([4, 9])
    dq, dk, dv = oracle.cross_bwd_ref(q, k, v, do, lens, 0.4)
    assert np.all(dk[0, 4:] == 0) and np.all(dv[0, 4:] == 0)

    def loss(q_, k_, v_):
        o, _ = oracle.cross_fwd_ref(q_, k_, v_, lens, 0.4)
        return float(np.sum(do * o))

    eps = 1e-6
    rng = np.random.default_rng(24)
    for name, x, g in [("q", q, dq), ("k", k, dk), ("v", v, dv)]:
        for _ in range(10):
            idx = tuple(rng.integers(0, n) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            a = {"q": q, "k": k, "v": v}
            bb = dict(a)
            a[name], bb[name] = xp, xm
            fd = (loss(a["q"], a["k"], a["v"]) - loss(bb["q"], bb["k"], bb["v"])) / (2 * eps)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(g[idx]))


torch = pytest.importorskip("torch")


def test_self_bwd_matches_torch_autograd_without_rope():
    B, L, H, D = 2, 21, 2, 128
    q, k, v, do = (_rand((B, L, H, D), s) for s in (30, 31, 32, 33))
    dq, dk, dv = oracle.self_bwd_ref(q, k, v, do, 0.11, None, None)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.11)
    out.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    for mine, t in [(dq, tq), (dk, tk), (dv, tv)]:
        np.testing.assert_allclose(mine, t.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12)


def test_cross_bwd_matches_torch_autograd_with_mask():
    B, Lq, Lk, H, D = 2, 13, 24, 2, 128
    q, do = _rand((B, Lq, H, D), 40), _rand((B, Lq, H, D), 41)
    k, v = _rand((B, Lk, H, D), 42), _rand((B, Lk, H, D), 43)
    lens = np.array([17, 24])
    dq, dk, dv = oracle.cross_bwd_ref(q, k, v, do, lens, 0.09)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).requires_grad_() for x in (q, k, v))
    mask = torch.arange(Lk)[None, None, None, :] < torch.from_numpy(lens)[:, None, None, None]
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.09)
    out.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    for mine, t in [(dq, tq), (dk, tk), (dv, tv)]:
        np.testing.assert_allclose(mine, t.grad.permute(0, 2, 1, 3).numpy(), atol=1e-12)
