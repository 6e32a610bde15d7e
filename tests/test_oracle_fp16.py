"""Pins of the oracle's fp16 score-operand recipe (oracle/fp16_scores.py), CPU only.

Independent checks: numpy's binary16 rounding against code points built from the format's definition
(sign, 5 exponent bits with bias 15, 10 fraction bits; field 0 subnormal, f * 2^-24), its landmarks and
ties to even; the tile exponent's range; the recipe's per-tile independence and error bound; that bf16
operands without rotation pass through exactly (so the attention at rounded operands is the exact
oracle there); that the LSE moves by no more than the proven score bound; that a planted coarser
rounding (bf16 instead of fp16) moves it several times more; and finite differences of the backward at
the rounded operands.
"""

import math

import numpy as np

import oracle
import synth
from oracle import RopeSpec, fp16_scores as f16

ROPE = RopeSpec()
SCALE = 1.0 / math.sqrt(128)


def binary16_positive_values() -> np.ndarray:
    vals = []
    for code in range(0x7C00):                  # 0x7C00 = +inf; every lower code is finite
        ef, m = code >> 10, code & 0x3FF
        vals.append(m * 2.0 ** -24 if ef == 0 else (1.0 + m / 1024.0) * 2.0 ** (ef - 15))
    return np.array(vals)


_POS = binary16_positive_values()


def _round_by_search(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, len(_POS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS) - 1)
    d_lo, d_hi = a - _POS[lo], _POS[hi] - a
    idx = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    return np.sign(x) * _POS[idx]


def test_binary16_landmarks():
    assert len(_POS) == 31744 and _POS[-1] == 65504.0
    assert _POS[1] == 2.0 ** -24 and _POS[0x400] == 2.0 ** -14
    r = f16.fp16_round
    assert r(65504.0) == 65504.0 and r(2.0 ** -14) == 2.0 ** -14 and r(2.0 ** -24) == 2.0 ** -24
    assert r(1.0 + 2.0 ** -11) == 1.0                        # midpoint, even code below
    assert r(1.0 + 3 * 2.0 ** -11) == 1.0 + 2.0 ** -9        # midpoint, even code above
    assert r(-(1.0 + 3 * 2.0 ** -11)) == -(1.0 + 2.0 ** -9)
    assert r(2049.0) == 2048.0 and r(2051.0) == 2052.0       # spacing 2 in [2048, 4096)


def test_binary16_rounding_matches_definition():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(200_000) * np.exp2(rng.uniform(-20, 15, 200_000))
    x = x[np.abs(x) < 65504]
    mids = 0.5 * (_POS[1:] + _POS[:-1])                      # every tie between neighbours
    for v in (x, mids, -mids[::7]):
        np.testing.assert_array_equal(f16.fp16_round(v), _round_by_search(v))


def test_tile_exponent_range():
    rng = np.random.default_rng(6)
    for m in np.exp2(rng.uniform(-60, 60, 1000)):
        e = f16.tile_exponent15(m)
        assert 2.0 ** 14 <= m * 2.0 ** -e < 2.0 ** 15
    assert f16.tile_exponent15(2.0 ** 14) == 0 and f16.tile_exponent15(2.0 ** 15) == 1
    assert f16.tile_exponent15(1.0) == -14 and f16.tile_exponent15(0.0) == 0


def test_round_tiles_recipe():
    x = synth.bf16_bits_to_f64(synth.random_bf16(41, (2, 200, 3, 128), scale=3.0))
    x = oracle.rope3d_ref(x, (2, 10, 10), ROPE)              # rotated values: not bf16, not fp16
    r = f16.round_tiles(x)
    assert not np.array_equal(r, x)
    # relative error at most half an fp16 ulp, 2^-11 (every element is far inside the normal range)
    assert np.all(np.abs(r - x) <= 2.0 ** -11 * np.abs(x))
    np.testing.assert_array_equal(f16.round_tiles(r), r)     # idempotent
    # tiles are independent: scaling one 64-token tile by a power of two scales only its rounding
    y = x.copy()
    y[1, 64:128, 2] *= 2.0 ** 9
    ry = f16.round_tiles(y)
    np.testing.assert_array_equal(ry[1, 64:128, 2], r[1, 64:128, 2] * 2.0 ** 9)
    mask = np.ones(x.shape, bool)
    mask[1, 64:128, 2] = False
    np.testing.assert_array_equal(ry[mask], r[mask])
    # a tile holding one huge element rounds the small ones on the huge one's scale
    z = x.copy()
    z[0, 0, 0, 0] = 2.0 ** 20
    rz = f16.round_tiles(z)
    e = f16.tile_exponent15(2.0 ** 20)
    np.testing.assert_array_equal(rz[0, :64, 0], f16.fp16_round(z[0, :64, 0] * 2.0 ** -e) * 2.0 ** e)


def test_bf16_operands_pass_through_without_rotation():
    qb, kb, vb = (synth.bf16_bits_to_f64(synth.random_bf16(50 + i, (1, 150, 2, 128), scale=4.0)) for i in range(3))
    qr, kr = f16.rounded_operands(qb, kb, None, None)
    np.testing.assert_array_equal(qr, qb)
    np.testing.assert_array_equal(kr, kb)
    o1, l1 = f16.self_fwd_fp16_ref(qb, kb, vb, SCALE, None, None)
    o2, l2 = oracle.self_fwd_ref(qb, kb, vb, SCALE)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    do = synth.bf16_bits_to_f64(synth.random_bf16(60, (1, 150, 2, 128)))
    for a, b in zip(f16.self_bwd_fp16_ref(qb, kb, vb, do, SCALE, None, None),
                    oracle.self_bwd_ref(qb, kb, vb, do, SCALE)):
        np.testing.assert_array_equal(a, b)


def _peaked(seed, grid, qmul, H=2):
    L = int(np.prod(grid))
    q = synth.bf16_bits_to_f64(synth.random_bf16(seed, (1, L, H, 128), scale=qmul))
    k, v, do = (synth.bf16_bits_to_f64(synth.random_bf16(seed + i, (1, L, H, 128))) for i in (1, 2, 3))
    return q, k, v, do


def test_lse_moves_within_the_score_bound():
    grid = (5, 8, 8)
    for qmul in (1.0, 4.0, 8.0):
        q, k, v, _ = _peaked(70, grid, qmul)
        _, l_exact = oracle.self_fwd_ref(q, k, v, SCALE, grid, ROPE)
        _, l_r = f16.self_fwd_fp16_ref(q, k, v, SCALE, grid, ROPE)
        bound = f16.score_rounding_bound(q, k, SCALE, grid, ROPE)
        d = np.abs(l_r - l_exact)
        assert np.all(d <= bound), qmul
        assert d.max() > 0                                   # the rounding is really applied
        print(f"  q x{qmul}: max |dLSE| {d.max():.2e}, bound {bound.max():.2e}")


def test_fp16_rounding_is_finer_than_bf16():
    """A planted mistake: bf16 tiles (8-bit significand) instead of fp16 (11-bit). The worst-case bound above
    is loose, so this pins the format by the size of the effect: three more significand bits move the
    LSE several times less, over the same peaked inputs."""
    grid = (5, 8, 8)
    q, k, v, _ = _peaked(80, grid, 8.0)
    qt, kt = oracle.rope3d_ref(q, grid, ROPE), oracle.rope3d_ref(k, grid, ROPE)
    bf16 = lambda x: synth.bf16_bits_to_f64(synth.fp32_to_bf16_bits(x.astype(np.float32)))
    _, l_bad = oracle.self_fwd_ref(bf16(qt), bf16(kt), v, SCALE)
    _, l_exact = oracle.self_fwd_ref(q, k, v, SCALE, grid, ROPE)
    _, l_r = f16.self_fwd_fp16_ref(q, k, v, SCALE, grid, ROPE)
    e16, e_bf = np.abs(l_r - l_exact), np.abs(l_bad - l_exact)
    print(f"  LSE error: fp16 tiles max {e16.max():.2e} rms {np.sqrt((e16 ** 2).mean()):.2e}; "
          f"bf16 max {e_bf.max():.2e} rms {np.sqrt((e_bf ** 2).mean()):.2e}")
    assert np.sqrt((e16 ** 2).mean()) * 4 < np.sqrt((e_bf ** 2).mean())


def test_fp16_backward_is_the_gradient_at_rounded_operands():
    """Central finite differences of <dO, O(q~, k~, v)> in the rounded rotated operands, for one element
    of each, against the backward (before the inverse rotation, which tests/test_oracle_backward.py pins)."""
    grid = (2, 3, 4)
    q, k, v, do = _peaked(90, grid, 4.0, H=1)
    dq, dk, dv = f16.self_bwd_fp16_ref(q, k, v, do, SCALE, grid, ROPE)
    qt, kt = f16.rounded_operands(q, k, grid, ROPE)
    L = q.shape[1]
    pos = oracle.positions(grid)
    dqt = oracle.rope_apply(dq[0, :, 0], oracle.rope_angles(pos, ROPE, 128))   # back to the rotated frame
    dkt = oracle.rope_apply(dk[0, :, 0], oracle.rope_angles(pos, ROPE, 128))

    def f(qq, kk):
        o, _ = oracle.attention_rows_ref(qq, kk, v[0, :, 0], SCALE)
        return float((o * do[0, :, 0]).sum())

    h = 1e-6
    for (i, d) in ((3, 5), (L - 1, 100)):
        e = np.zeros_like(qt[0, :, 0])
        e[i, d] = h
        num_q = (f(qt[0, :, 0] + e, kt[0, :, 0]) - f(qt[0, :, 0] - e, kt[0, :, 0])) / (2 * h)
        num_k = (f(qt[0, :, 0], kt[0, :, 0] + e) - f(qt[0, :, 0], kt[0, :, 0] - e)) / (2 * h)
        assert abs(num_q - dqt[i, d]) < 1e-6 * max(1.0, abs(num_q))
        assert abs(num_k - dkt[i, d]) < 1e-6 * max(1.0, abs(num_k))


def _fp32_rotation(x, grid):
    """A rotation computed in fp32 (fp32 table, one fused multiply-add per output), rounded per step as an
    fp32 machine would: a test-side stand-in for any fp32 implementation of the rotation."""
    pos = oracle.positions(grid)
    ang = oracle.rope_angles(pos, ROPE, 128)
    c = np.cos(ang).astype(np.float32).astype(np.float64)[:, None, :]
    s = np.sin(ang).astype(np.float32).astype(np.float64)[:, None, :]
    x0, x1 = x[0, :, :, 0::2], x[0, :, :, 1::2]
    f32 = lambda a: a.astype(np.float32).astype(np.float64)
    y = np.empty_like(x)
    y[0, :, :, 0::2] = f32(x0 * c - f32(x1 * s))
    y[0, :, :, 1::2] = f32(x0 * s + f32(x1 * c))
    return y


def test_ambiguous_elements_cover_fp32_rotation_flips():
    """Every element whose fp16 tile rounding differs between an fp32 and the exact rotation is marked
    ambiguous, and the marked set is small (the allowance stays tight)."""
    grid = (5, 8, 8)
    flips = marked = total = 0
    for seed, qmul in ((5328, 8.0), (5324, 4.0), (77, 1.0)):
        q = synth.bf16_bits_to_f64(synth.random_bf16(seed, (1, 320, 2, 128), scale=qmul))
        r32 = f16.round_tiles(_fp32_rotation(q, grid))
        r64 = f16.round_tiles(oracle.rope3d_ref(q, grid, ROPE))
        mask, ulp = f16.ambiguous_elements(q, grid, ROPE)
        diff = r32 != r64
        assert np.all(mask[diff]), "an fp32-rotation rounding flip was not marked ambiguous"
        assert np.all(np.abs(r32 - r64)[diff] <= ulp[diff] * (1 + 1e-12))   # one ulp apart
        flips += int(diff.sum())
        marked += int(mask.sum())
        total += mask.size
    assert flips > 0                      # the inputs do produce flips (the check has teeth)
    assert marked < 1e-2 * total, (marked, total)
    print(f"  flips {flips}, marked {marked} of {total}")


def test_tie_allowance_covers_fp32_rotation_flips():
    """Attention at the fp16 roundings of an fp32 rotation stays within the tie allowance of the module's
    own rounding, row by row, for peaked inputs."""
    grid = (5, 8, 8)
    q, k, v, _ = _peaked(5328, grid, 8.0)
    _, l_ref = f16.self_fwd_fp16_ref(q, k, v, SCALE, grid, ROPE)
    _, l_32 = oracle.self_fwd_ref(f16.round_tiles(_fp32_rotation(q, grid)),
                                  f16.round_tiles(_fp32_rotation(k, grid)), v, SCALE)
    allow = f16.score_tie_allowance(q, k, SCALE, grid, ROPE)
    d = np.abs(l_32 - l_ref)
    assert np.all(d <= allow + 1e-12)
    assert d.max() > 1e-4                 # flips do move some rows
    print(f"  max |dLSE| {d.max():.2e}; allowance there {allow.flat[np.argmax(d)]:.2e}, max {allow.max():.2e}")


def test_backward_with_a_given_output():
    """Delta from a handed-in output: with the function's own output it is the default; with another
    output only Delta (hence dS, dQ, dK) moves, dV not at all, by exactly the change of Delta."""
    grid = (2, 3, 4)
    q, k, v, do = _peaked(95, grid, 4.0, H=1)
    qt, kt = f16.rounded_operands(q, k, grid, ROPE)
    o, _ = oracle.self_fwd_ref(qt, kt, v, SCALE)
    for a, b in zip(f16.self_bwd_fp16_ref(q, k, v, do, SCALE, grid, ROPE, o=o),
                    f16.self_bwd_fp16_ref(q, k, v, do, SCALE, grid, ROPE)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    o2 = o + 0.01 * synth.bf16_bits_to_f64(synth.random_bf16(96, o.shape))
    dq1, dk1, dv1 = f16.self_bwd_fp16_ref(q, k, v, do, SCALE, grid, ROPE)
    dq2, dk2, dv2 = f16.self_bwd_fp16_ref(q, k, v, do, SCALE, grid, ROPE, o=o2)
    np.testing.assert_array_equal(dv1, dv2)
    # dq~_i changes by -scale * dDelta_i * sum_j P_ij k~_j
    s = SCALE * (qt[0, :, 0] @ kt[0, :, 0].T)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    d_delta = (do[0, :, 0] * (o2 - o)[0, :, 0]).sum(axis=1)
    pos = oracle.positions(grid)
    ddq_rot = oracle.rope_apply((dq2 - dq1)[0, :, 0], oracle.rope_angles(pos, ROPE, 128))
    np.testing.assert_allclose(ddq_rot, -SCALE * d_delta[:, None] * (p @ kt[0, :, 0]), rtol=1e-9, atol=1e-12)
