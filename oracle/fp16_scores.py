"""fp16 score operands of the RoPE path, for the oracle side of its parity tests.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests, the smoke check and the benchmark's
CPU-baseline leg may use it.

A rotated query or key (3D RoPE over time, height and width: Wan2.1 reading notes, "2. Model Design",
DiT block paragraph) is not a bf16 number, and the pages fix no precision for the score product. The
library's reading: with RoPE the score product takes fp16 operands. Every 64-token tile of one
(batch, head) of the rotated queries, and of the rotated keys, is multiplied by the power of two 2^-e that
puts the tile's largest |element| in [2^14, 2^15), rounded to fp16 (IEEE binary16, round to nearest, ties
to even), and the power of two is undone exactly afterwards. The scores, the softmax and everything after
them are the plain definitions of `oracle.reference`, evaluated at these rounded operands.

This module supplies the rounding and the attention at rounded operands, so that a test can separate
what the documented operand rounding moves (the distance between `self_fwd_fp16_ref` and the exact
`self_fwd_ref`) from any other difference.

The rounding of a value is unique except next to a rounding tie: the library rotates in fp32, whose
result may lie on the other side of a tie than the exact rotation this module rounds, and then rounds
to the neighbouring fp16 value (about one element in 10^4 for random inputs). `ambiguous_elements`
marks every element where that can happen, from the exact values alone, and `score_tie_allowance`
bounds how far such alternative roundings can move a row's LSE and output. Rounding is numpy's float64 -> float16 conversion (a library
primitive); tests/test_oracle_fp16.py pins it against binary16 code points built from the format's
definition and pins the tile recipe, the attention at rounded operands and the rounding bound.
"""

import numpy as np

from .reference import _head_bwd, _rotated, rope3d_ref, self_fwd_ref

TILE = 64


def fp16_round(x) -> np.ndarray:
    """Nearest IEEE binary16 value of each element (ties to even), as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def tile_exponent15(maxabs: float) -> int:
    """e with maxabs * 2^-e in [2^14, 2^15); 0 for maxabs == 0."""
    if not maxabs > 0:
        return 0
    _, ex = np.frexp(maxabs)                    # maxabs = m * 2^ex, m in [0.5, 1)
    return int(ex) - 15


def round_tiles(x, tile: int = TILE) -> np.ndarray:
    """x [B, L, H, D] (already rotated) with every (b, h, 64-token tile) rounded under the recipe."""
    x = np.asarray(x, dtype=np.float64)
    B, L, H, D = x.shape
    out = np.empty_like(x)
    for b in range(B):
        for h in range(H):
            for t0 in range(0, L, tile):
                blk = x[b, t0:t0 + tile, h, :]
                e = tile_exponent15(float(np.abs(blk).max()))
                out[b, t0:t0 + tile, h, :] = fp16_round(blk * 2.0 ** -e) * 2.0 ** e
    return out


def _rot(x, grid, rope):
    return np.asarray(x, dtype=np.float64) if rope is None else rope3d_ref(x, grid, rope)


def rounded_operands(q, k, grid, rope):
    """The rotated queries and keys as the score product sees them (fp16 tiles, exponents undone).
    rope=None: no rotation (then bf16 inputs pass through exactly: binary16 holds every bf16 value
    within 2^28 of its tile's maximum)."""
    return round_tiles(_rot(q, grid, rope)), round_tiles(_rot(k, grid, rope))


def self_fwd_fp16_ref(q, k, v, scale: float, grid, rope, rows=None):
    """Self-attention (fp64) with the scores formed from the fp16-rounded rotated q and k.

    Same outputs and `rows` convention as `self_fwd_ref`."""
    qt, kt = rounded_operands(q, k, grid, rope)
    return self_fwd_ref(qt, kt, v, scale, rows=rows)


def self_bwd_fp16_ref(q, k, v, dout, scale: float, grid, rope, o=None):
    """dQ, dK, dV (w.r.t. the unrotated q and k) of attention evaluated at the fp16-rounded rotated
    operands: the plain backward of `oracle.reference` with q~, k~ replaced by their rounded tiles,
    the gradients rotated back by minus the angle.  o (optional, [B, L, H, D]): the forward output
    handed to the backward, from which Delta_i = <dO_i, o_i> is formed (default: this function's own)."""
    qt, kt = rounded_operands(q, k, grid, rope)
    B, L, H, D = q.shape
    idx = np.arange(L)
    dq = np.empty((B, L, H, D))
    dk = np.empty((B, L, H, D))
    dv = np.empty((B, L, H, D))
    for b in range(B):
        for h in range(H):
            dqt, dkt, dvh = _head_bwd(qt[b, :, h, :], kt[b, :, h, :], np.asarray(v[b, :, h, :], dtype=np.float64),
                                      np.asarray(dout[b, :, h, :], dtype=np.float64), scale,
                                      None if o is None else o[b, :, h, :])
            dq[b, :, h, :] = _rotated(dqt, idx, grid, rope, inverse=True)
            dk[b, :, h, :] = _rotated(dkt, idx, grid, rope, inverse=True)
            dv[b, :, h, :] = dvh
    return dq, dk, dv


FP32_ROTATION_ERR = 2.0 ** -22   # |fp32 rotation - exact| <= this * (|x_2j| + |x_2j+1|) of the input pair


def _pair_magnitude(x):
    """|x_2j| + |x_2j+1| for each element's rotation pair, [B, L, H, D]."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    s = a[..., 0::2] + a[..., 1::2]
    return np.repeat(s, 2, axis=-1)


def ambiguous_elements(x, grid, rope, tile: int = TILE):
    """(mask, ulp) for x [B, L, H, D] (unrotated): mask marks the elements whose fp16 tile rounding may
    differ from this module's when the rotation is computed in fp32 (the exact rotated value lies within
    the fp32 rotation's error bound of a rounding tie, or the tile's exponent itself is in doubt, in which
    case the whole tile is marked); ulp is the fp16 spacing at each rounded element, in unscaled units."""
    xr = _rot(x, grid, rope)
    err = FP32_ROTATION_ERR * _pair_magnitude(x) if rope is not None else np.zeros_like(xr)
    B, L, H, D = xr.shape
    mask = np.zeros(xr.shape, bool)
    ulp = np.zeros(xr.shape)
    for b in range(B):
        for h in range(H):
            for t0 in range(0, L, tile):
                blk = xr[b, t0:t0 + tile, h, :]
                eb = err[b, t0:t0 + tile, h, :]
                mx = float(np.abs(blk).max())
                e = tile_exponent15(mx)
                z = np.abs(blk) * 2.0 ** -e
                u = np.exp2(np.floor(np.log2(np.maximum(z, 2.0 ** -14))) - 10)   # fp16 spacing at z
                frac = z / u - np.floor(z / u)
                near = np.abs(frac - 0.5) * u <= eb * 2.0 ** -e
                me = float(eb.max())
                if tile_exponent15(mx + me) != e or tile_exponent15(max(mx - me, 0.0)) != e:
                    near[:] = True
                mask[b, t0:t0 + tile, h, :] = near
                ulp[b, t0:t0 + tile, h, :] = u * 2.0 ** e
    return mask, ulp


def score_tie_allowance(q, k, scale: float, grid, rope) -> np.ndarray:
    """Per query row ([B, H, L]) a bound A_i on how far alternative roundings of ambiguous elements can
    move the row's LSE.  Each ambiguous element may land one fp16 ulp away, so score s_ij moves by at most
    D_ij = scale * (sum_{d amb in q_i} ulp_id |k~_jd| + sum_{d amb in k_j} |q~_id| ulp_jd).  Since
    LSE(s + delta) - LSE(s) = ln sum_j P_ij exp(delta_ij), |dLSE_i| <= A_i = ln sum_j P_ij exp(D_ij) (P at
    the rounded operands), and the softmax weights move by at most sum_j |dP_ij| <= exp(2 A_i) - 1, so
    |dO_i| <= (exp(2 A_i) - 1) max_j |v_j| elementwise."""
    qm, qu = ambiguous_elements(q, grid, rope)
    km, ku = ambiguous_elements(k, grid, rope)
    qr, kr = rounded_operands(q, k, grid, rope)
    B, L, H, D = qr.shape
    out = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            qh, kh = qr[b, :, h, :], kr[b, :, h, :]
            dmax = float(scale) * ((qm[b, :, h, :] * qu[b, :, h, :]) @ np.abs(kh).T
                                   + np.abs(qh) @ (km[b, :, h, :] * ku[b, :, h, :]).T)     # [L, Lk]
            s = float(scale) * (qh @ kh.T)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            out[b, h] = np.log((p * np.exp(dmax)).sum(axis=1))
    return out


def score_rounding_bound(q, k, scale: float, grid, rope) -> np.ndarray:
    """Per query row (shape [B, H, L]) a bound on how far the rounding can move any of the row's scores.

    Each rounded element differs from the exact one by at most 2^-11 of its magnitude: binary16 has an
    11-bit significand, and after the tile scaling every element is in its normal range unless it lies
    more than 2^28 below the tile's maximum (the bound assumes no such element, as for any input the
    tests draw). Hence
    |s~_ij - s_ij| <= scale * sum_d (|q_d| |dk_d| + |k_d| |dq_d| + |dq_d| |dk_d|)
                   <= scale * (2^-10 + 2^-22) * sum_d |q_d| |k_d|.
    LSE is 1-Lipschitz in the largest score change, so the bound applies to each row's LSE too."""
    qr = np.abs(_rot(q, grid, rope))
    kr = np.abs(_rot(k, grid, rope))
    B, L, H, D = q.shape
    out = np.empty((B, H, L))
    for b in range(B):
        for h in range(H):
            out[b, h] = (qr[b, :, h, :] @ kr[b, :, h, :].T).max(axis=1)
    return float(scale) * (2.0 ** -10 + 2.0 ** -22) * out
