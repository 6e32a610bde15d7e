"""Plain fp64 definitions of the attention hot path (test infrastructure only).

Sources, cited by page and section:
  [notes]  "Wan -- Open and Advanced Large-Scale Video Generative Models (Wan2.1)",
           gojay.top reading notes: "2. Model Design" (Wan-VAE and DiT backbone
           paragraphs, DiT block paragraph), the code-notes config table
           ("1.3B vs 14B"), "3. Training", the symbol table.
  [lit619] "Wan Team, Alibaba (2025) -- ARXIV-2503.20314", anthology note,
           "Key takeaways" (Backbone; Attention dominates).
  [ctol]   "Wan: Alibaba's Open-Source Powerhouse for AI Video Generation",
           "Engineering the Core".

What the pages fix: self-attention is full (every latent-patch token attends
to every other, no causal mask) [lit619 Backbone; ctol Engineering the Core];
positions enter through a 3D rotary embedding over time, height and width
[notes, DiT block paragraph]; the latent grid of a 1+T frame video is
[1+T/4, H/8, W/8] and the (1,2,2) patch divides the spatial axes by two more
[notes, 2. Model Design]; video tokens cross-attend to at most 512 text tokens
[notes, config table and symbol table].

Readings where the pages are silent (each is a parameter or a documented
convention of the library interface, not a claim about Wan's checkpoint):
  * tokens are enumerated row-major over (f, h, w);
  * the head dim splits into time/height/width segments (d_f, d_h, d_w), each
    rotated as an independent 1-D rotary embedding of its own axis position,
    frequency theta^(-2j/d_axis) for pair j of the segment;
  * pairs are adjacent elements (2j, 2j+1) rotated as the complex number
    x[2j] + i x[2j+1] multiplied by exp(i * angle);
  * positions are 0-based integer grid indices;
  * softmax scale is a parameter (the workloads use 1/sqrt(D));
  * the log-sum-exp is the natural log of the row's exp-sum;
  * an empty key set gives O = 0 and LSE = -inf;
  * gradients are taken with respect to the unrotated q and k.
"""

from __future__ import annotations

import math
from typing import NamedTuple

import numpy as np


class RopeSpec(NamedTuple):
    """Head-dim split between the time, height and width axes, and the rotary base."""
    d_f: int = 48
    d_h: int = 40
    d_w: int = 40
    theta: float = 10000.0


# ----------------------------------------------------------------------------
# Token grid and positions
# ----------------------------------------------------------------------------

def latent_token_grid(frames: int, height: int, width: int) -> tuple:
    """Token grid (F, Hp, Wp) of a clip of `frames` RGB frames at height x width pixels.

    The VAE maps 1+T frames to a latent grid [1+T/4, H/8, W/8] (the first frame
    is compressed spatially only) and the DiT patchifies it with a (1,2,2)
    patch, so L = (1+T/4) * H/16 * W/16 tokens [notes, 2. Model Design].
    """
    if frames < 1 or (frames - 1) % 4 != 0:
        raise ValueError("frame count must be 1 + a multiple of 4")
    if height % 16 != 0 or width % 16 != 0:
        raise ValueError("height and width must be multiples of 16")
    t = frames - 1
    latent = (1 + t // 4, height // 8, width // 8)
    patch = (1, 2, 2)
    return tuple(n // p for n, p in zip(latent, patch))


def positions(grid) -> np.ndarray:
    """Integer (f, h, w) position of every token, tokens in row-major grid order. Shape [L, 3]."""
    F, Hp, Wp = (int(x) for x in grid)
    return np.indices((F, Hp, Wp)).reshape(3, -1).T.astype(np.int64)


# ----------------------------------------------------------------------------
# 3D rotary position embedding
# ----------------------------------------------------------------------------

def rope_axis_of_pair(rope: RopeSpec, D: int):
    """For each of the D/2 pairs: (axis index 0/1/2, index j of the pair within its axis segment)."""
    widths = (rope.d_f, rope.d_h, rope.d_w)
    if sum(widths) != D or any(w < 0 or w % 2 for w in widths):
        raise ValueError("rotary split must be three even widths summing to the head dim")
    axis = np.empty(D // 2, dtype=np.int64)
    j = np.empty(D // 2, dtype=np.int64)
    start = 0
    for a, w in enumerate(widths):
        n = w // 2
        axis[start:start + n] = a
        j[start:start + n] = np.arange(n)
        start += n
    return axis, j


def rope_frequencies(rope: RopeSpec, D: int):
    """Per pair: axis and angular frequency theta^(-2j/d_axis)."""
    axis, j = rope_axis_of_pair(rope, D)
    widths = np.array([rope.d_f, rope.d_h, rope.d_w], dtype=np.float64)
    omega = np.power(float(rope.theta), -2.0 * j / widths[axis])
    return axis, omega


def rope_angles(pos: np.ndarray, rope: RopeSpec, D: int) -> np.ndarray:
    """Rotation angle of every (token, pair): position on the pair's axis times its frequency. [N, D/2]."""
    axis, omega = rope_frequencies(rope, D)
    return pos[:, axis].astype(np.float64) * omega[None, :]


def rope_table_ref(grid, rope: RopeSpec):
    """cos/sin of p * theta^(-2j/d_a) for every axis a, position p < grid[a] and pair j < d_a/2.

    Returns a list of three arrays, one per axis, each [grid[a], d_a/2, 2] holding (cos, sin).
    """
    out = []
    for size, width in zip(grid, (rope.d_f, rope.d_h, rope.d_w)):
        j = np.arange(width // 2, dtype=np.float64)
        omega = np.power(float(rope.theta), -2.0 * j / width) if width else j
        ang = np.arange(size, dtype=np.float64)[:, None] * omega[None, :]
        out.append(np.stack([np.cos(ang), np.sin(ang)], axis=-1))
    return out


def rope_apply(x: np.ndarray, angles: np.ndarray, inverse: bool = False) -> np.ndarray:
    """Rotate each adjacent pair (x[2j], x[2j+1]) of the last axis by its angle (or by minus it).

    x: [..., N, D] with angles [N, D/2] broadcast over the leading axes.
    """
    c = np.cos(angles)
    s = np.sin(angles)
    if inverse:
        s = -s
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    y = np.empty(np.broadcast_shapes(x.shape), dtype=np.float64)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


def rope3d_ref(x: np.ndarray, grid, rope: RopeSpec, inverse: bool = False) -> np.ndarray:
    """3D RoPE of a [B, L, H, D] tensor whose L tokens enumerate `grid` row-major."""
    B, L, H, D = x.shape
    ang = rope_angles(positions(grid), rope, D)            # [L, D/2]
    if ang.shape[0] != L:
        raise ValueError("grid does not match the token count")
    xt = np.transpose(np.asarray(x, dtype=np.float64), (0, 2, 1, 3))   # [B, H, L, D]
    return np.transpose(rope_apply(xt, ang, inverse), (0, 2, 1, 3))


# ----------------------------------------------------------------------------
# Attention forward
# ----------------------------------------------------------------------------

def attention_rows_ref(qt: np.ndarray, kt: np.ndarray, v: np.ndarray, scale: float):
    """Softmax attention of query rows qt [R, D] over keys kt [N, D] with values v [N, D].

    s_ij = scale * <qt_i, kt_j>;  LSE_i = ln sum_j exp(s_ij);  P_ij = exp(s_ij - LSE_i);
    O_i = sum_j P_ij v_j.  N = 0 gives O = 0, LSE = -inf.
    """
    R, D = qt.shape
    if kt.shape[0] == 0:
        return np.zeros((R, v.shape[1])), np.full(R, -np.inf)
    s = float(scale) * (qt @ kt.T)
    m = s.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    p = np.exp(s - lse[:, None])
    return p @ v, lse


def _rotated(x_rows: np.ndarray, token_idx: np.ndarray, grid, rope, inverse=False):
    if rope is None:
        return np.asarray(x_rows, dtype=np.float64)
    pos = positions(grid)[token_idx]
    return rope_apply(np.asarray(x_rows, dtype=np.float64), rope_angles(pos, rope, x_rows.shape[-1]), inverse)


def self_fwd_ref(q, k, v, scale: float, grid=None, rope: RopeSpec | None = None, rows=None):
    """Full (non-causal) self-attention with optional 3D RoPE on q and k.

    q, k, v: [B, L, H, D] float arrays.  rope=None means no rotation.
    rows=None: returns O [B, L, H, D] and LSE [B, H, L].
    rows=[B, H, R] int array: returns O [B, H, R, D] and LSE [B, H, R] for those query rows only.
    """
    B, L, H, D = q.shape
    if rope is not None and int(np.prod(grid)) != L:
        raise ValueError("grid does not match the token count")
    all_idx = np.arange(L)
    if rows is None:
        o = np.empty((B, L, H, D))
        lse = np.empty((B, H, L))
    else:
        o = np.empty((B, H, rows.shape[2], D))
        lse = np.empty((B, H, rows.shape[2]))
    for b in range(B):
        for h in range(H):
            kt = _rotated(k[b, :, h, :], all_idx, grid, rope)
            vv = np.asarray(v[b, :, h, :], dtype=np.float64)
            idx = all_idx if rows is None else rows[b, h]
            qt = _rotated(q[b, idx, h, :], idx, grid, rope)
            ob, lb = attention_rows_ref(qt, kt, vv, scale)
            if rows is None:
                o[b, :, h, :] = ob
                lse[b, h] = lb
            else:
                o[b, h] = ob
                lse[b, h] = lb
    return o, lse


def cross_fwd_ref(q, k, v, k_lens, scale: float, rows=None):
    """Cross-attention of video queries over text keys with a valid-prefix length per batch item.

    q: [B, Lq, H, D]; k, v: [B, Lk, H, D]; k_lens: [B] ints (None: all Lk keys valid),
    clamped to [0, Lk]; keys j >= k_len[b] are excluded.  No rotary embedding.
    rows as in self_fwd_ref.
    """
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    lens = np.full(B, Lk) if k_lens is None else np.clip(np.asarray(k_lens, dtype=np.int64), 0, Lk)
    if rows is None:
        o = np.empty((B, Lq, H, D))
        lse = np.empty((B, H, Lq))
    else:
        o = np.empty((B, H, rows.shape[2], D))
        lse = np.empty((B, H, rows.shape[2]))
    for b in range(B):
        n = int(lens[b])
        for h in range(H):
            kk = np.asarray(k[b, :n, h, :], dtype=np.float64)
            vv = np.asarray(v[b, :n, h, :], dtype=np.float64)
            idx = np.arange(Lq) if rows is None else rows[b, h]
            qq = np.asarray(q[b, idx, h, :], dtype=np.float64)
            ob, lb = attention_rows_ref(qq, kk, vv, scale)
            if rows is None:
                o[b, :, h, :] = ob
                lse[b, h] = lb
            else:
                o[b, h] = ob
                lse[b, h] = lb
    return o, lse


# ----------------------------------------------------------------------------
# Attention backward (standard calculus of the forward above)
# ----------------------------------------------------------------------------

def self_fwd_varlen_ref(q, k, v, seq_lens, scale: float, grid=None, rope: RopeSpec | None = None):
    """Self-attention of each batch item over its first seq_lens[b] tokens only.

    q, k, v: [B, L, H, D]; seq_lens: [B] ints, clamped to [0, L].  Positions
    for RoPE are those of the padded grid (row-major, f*h*w == L), so a
    prefix of whole frames keeps the positions it has in a sequence of its
    own.  Returns O [B, L, H, D] and LSE [B, H, L] with NaN in the rows past
    an item's length (those rows are not defined by the operation).
    Joint image + video batches and the seq_len argument: Wan2.1 reading
    notes, 3. Training and the code notes (WanModel forward, sampler).
    Pinned in tests/test_oracle_shards.py (item = separate self-attention
    call; full lengths = self_fwd_ref).
    """
    B, L, H, D = q.shape
    o = np.full((B, L, H, D), np.nan)
    lse = np.full((B, H, L), np.nan)
    for b in range(B):
        n = int(min(max(int(seq_lens[b]), 0), L))
        if n == 0:
            continue
        idx = np.arange(n)
        for h in range(H):
            kt = _rotated(k[b, :n, h, :], idx, grid, rope)
            qt = _rotated(q[b, :n, h, :], idx, grid, rope)
            ob, lb = attention_rows_ref(qt, kt, np.asarray(v[b, :n, h, :], dtype=np.float64), scale)
            o[b, :n, h, :] = ob
            lse[b, h, :n] = lb
    return o, lse


def partial_fwd_ref(q, k, v, scale: float, q_offset: int, k_offset: int, grid=None, rope: RopeSpec | None = None,
                    rows=None):
    """Attention of a query shard over a key/value shard of one longer sequence.

    q: [B, Lq, H, D] holds global tokens q_offset .. q_offset+Lq-1, k and v
    [B, Lk, H, D] tokens k_offset .. k_offset+Lk-1 of the sequence whose
    token grid is `grid`; RoPE uses the global positions.  Returns the
    shard-local O [B, Lq, H, D] and LSE [B, H, Lq] (or, with rows [B, H, R]
    of local query indices, O [B, H, R, D] and LSE [B, H, R]).  The per-hop
    step of Ring attention (anthology note, Key takeaways: Ring outside,
    Ulysses inside).  Pinned in tests/test_oracle_shards.py.
    """
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    if rope is not None and (q_offset + Lq > int(np.prod(grid)) or k_offset + Lk > int(np.prod(grid))):
        raise ValueError("shard past the end of the grid")
    qidx_all = q_offset + np.arange(Lq)
    kidx = k_offset + np.arange(Lk)
    if rows is None:
        o = np.empty((B, Lq, H, D))
        lse = np.empty((B, H, Lq))
    else:
        o = np.empty((B, H, rows.shape[2], D))
        lse = np.empty((B, H, rows.shape[2]))
    for b in range(B):
        for h in range(H):
            kt = _rotated(k[b, :, h, :], kidx, grid, rope)
            loc = np.arange(Lq) if rows is None else rows[b, h]
            qt = _rotated(q[b, loc, h, :], qidx_all[loc], grid, rope)
            ob, lb = attention_rows_ref(qt, kt, np.asarray(v[b, :, h, :], dtype=np.float64), scale)
            if rows is None:
                o[b, :, h, :] = ob
                lse[b, h] = lb
            else:
                o[b, h] = ob
                lse[b, h] = lb
    return o, lse


def lse_merge_ref(o_parts, lse_parts):
    """Merge partial results over disjoint key sets: LSE = ln sum_r exp(LSE_r),
    O = sum_r exp(LSE_r - LSE) O_r.  o_parts: list of [B, L, H, D] arrays,
    lse_parts: list of [B, H, L].  Rows where every LSE_r is -inf get O = 0 and
    LSE = -inf.  Pinned in tests/test_oracle_shards.py (merging the shards of
    a key split reproduces the unsplit attention)."""
    lse_st = np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts])      # [R, B, H, L]
    m = lse_st.max(axis=0)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):          # log(0) only where every part is empty
        tot = np.log(np.exp(lse_st - safe_m).sum(axis=0)) + safe_m
    tot = np.where(np.isfinite(m), tot, -np.inf)
    w = np.where(np.isfinite(m), np.exp(lse_st - np.where(np.isfinite(tot), tot, 0.0)), 0.0)   # [R, B, H, L]
    o = np.zeros(np.asarray(o_parts[0]).shape)
    for r, op in enumerate(o_parts):
        o += np.asarray(op, dtype=np.float64) * np.transpose(w[r], (0, 2, 1))[..., None]
    return o, tot


def _head_bwd(qt, kt, v, dout, scale, o_given=None):
    """Gradients of sum(dout * O) w.r.t. the rotated qt, kt and v of one head (full L x N).

    o_given: the forward output the caller hands to the backward (as the library's backward takes
    o); Delta is then formed from it instead of from this function's own O."""
    if kt.shape[0] == 0:
        return np.zeros_like(qt), np.zeros_like(kt), np.zeros_like(v)
    s = scale * (qt @ kt.T)
    m = s.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    p = np.exp(s - lse[:, None])
    o = p @ v if o_given is None else np.asarray(o_given, dtype=np.float64)
    delta = (dout * o).sum(axis=1)                      # Delta_i = <dO_i, O_i>
    dv = p.T @ dout                                     # dV_j = sum_i P_ij dO_i
    dp = dout @ v.T                                     # dP_ij = <dO_i, v_j>
    ds = p * (dp - delta[:, None])                      # dS_ij = P_ij (dP_ij - Delta_i)
    dqt = scale * (ds @ kt)
    dkt = scale * (ds.T @ qt)
    return dqt, dkt, dv


def self_bwd_ref(q, k, v, dout, scale: float, grid=None, rope: RopeSpec | None = None):
    """dQ, dK, dV of self-attention with 3D RoPE, w.r.t. the unrotated q and k. All [B, L, H, D]."""
    B, L, H, D = q.shape
    idx = np.arange(L)
    dq = np.empty((B, L, H, D))
    dk = np.empty((B, L, H, D))
    dv = np.empty((B, L, H, D))
    for b in range(B):
        for h in range(H):
            qt = _rotated(q[b, :, h, :], idx, grid, rope)
            kt = _rotated(k[b, :, h, :], idx, grid, rope)
            dqt, dkt, dvh = _head_bwd(qt, kt, np.asarray(v[b, :, h, :], dtype=np.float64),
                                      np.asarray(dout[b, :, h, :], dtype=np.float64), scale)
            # q~ = R q, so dL/dq = R^T dL/dq~: rotate the gradient back by minus the angle.
            dq[b, :, h, :] = _rotated(dqt, idx, grid, rope, inverse=True)
            dk[b, :, h, :] = _rotated(dkt, idx, grid, rope, inverse=True)
            dv[b, :, h, :] = dvh
    return dq, dk, dv


def cross_bwd_ref(q, k, v, dout, k_lens, scale: float):
    """dQ [B, Lq, H, D], dK and dV [B, Lk, H, D] of masked cross-attention; padded keys get zero gradient."""
    B, Lq, H, D = q.shape
    Lk = k.shape[1]
    lens = np.full(B, Lk) if k_lens is None else np.clip(np.asarray(k_lens, dtype=np.int64), 0, Lk)
    dq = np.zeros((B, Lq, H, D))
    dk = np.zeros((B, Lk, H, D))
    dv = np.zeros((B, Lk, H, D))
    for b in range(B):
        n = int(lens[b])
        for h in range(H):
            dqh, dkh, dvh = _head_bwd(np.asarray(q[b, :, h, :], dtype=np.float64),
                                      np.asarray(k[b, :n, h, :], dtype=np.float64),
                                      np.asarray(v[b, :n, h, :], dtype=np.float64),
                                      np.asarray(dout[b, :, h, :], dtype=np.float64), scale)
            dq[b, :, h, :] = dqh
            dk[b, :n, h, :] = dkh
            dv[b, :n, h, :] = dvh
    return dq, dk, dv


def self_bwd_dq_rows(q, k, v, dout, scale: float, grid, rope, rows):
    """dQ for selected query rows only (each row's gradient needs only its own softmax row).

    rows: [B, H, R].  Returns dQ [B, H, R, D] w.r.t. the unrotated q.
    """
    B, L, H, D = q.shape
    all_idx = np.arange(L)
    out = np.empty((B, H, rows.shape[2], D))
    for b in range(B):
        for h in range(H):
            idx = rows[b, h]
            kt = _rotated(k[b, :, h, :], all_idx, grid, rope)
            vv = np.asarray(v[b, :, h, :], dtype=np.float64)
            qt = _rotated(q[b, idx, h, :], idx, grid, rope)
            do = np.asarray(dout[b, idx, h, :], dtype=np.float64)
            s = scale * (qt @ kt.T)
            m = s.max(axis=1, keepdims=True)
            lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
            p = np.exp(s - lse[:, None])
            o = p @ vv
            delta = (do * o).sum(axis=1)
            ds = p * (do @ vv.T - delta[:, None])
            out[b, h] = _rotated(scale * (ds @ kt), idx, grid, rope, inverse=True)
    return out


def self_bwd_dkdv_rows(q, k, v, dout, scale: float, grid, rope, key_rows, heads=None, block: int = 512):
    """dK and dV for selected key rows, w.r.t. the unrotated k.

    key_rows: [B, H, R] (only the heads listed in `heads`, default all, are computed).
    Every query row contributes, so each row's full softmax statistics are formed
    first; query rows are taken `block` at a time so an L x L matrix is never held.
    Returns (dK, dV), each [B, H, R, D]; heads not computed are NaN.
    """
    B, L, H, D = q.shape
    heads = range(H) if heads is None else heads
    all_idx = np.arange(L)
    dk_out = np.full((B, H, key_rows.shape[2], D), np.nan)
    dv_out = np.full((B, H, key_rows.shape[2], D), np.nan)
    for b in range(B):
        for h in heads:
            J = key_rows[b, h]
            kt = _rotated(k[b, :, h, :], all_idx, grid, rope)
            vv = np.asarray(v[b, :, h, :], dtype=np.float64)
            dkt = np.zeros((len(J), D))
            dvj = np.zeros((len(J), D))
            for start in range(0, L, block):
                idx = all_idx[start:start + block]
                qt = _rotated(q[b, idx, h, :], idx, grid, rope)
                do = np.asarray(dout[b, idx, h, :], dtype=np.float64)
                s = scale * (qt @ kt.T)
                m = s.max(axis=1, keepdims=True)
                # P_ij = exp(s_ij - m_i) / sum_j exp(s_ij - m_i): the softmax by its definition, with
                # one exponential per score (the L x L scores dominate this function's time)
                p = np.exp(np.subtract(s, m, out=s), out=s)
                p /= p.sum(axis=1, keepdims=True)
                delta = (do * (p @ vv)).sum(axis=1)
                pj = p[:, J]
                dsj = pj * (do @ vv[J].T - delta[:, None])
                dvj += pj.T @ do
                dkt += scale * (dsj.T @ qt)
            dk_out[b, h] = _rotated(dkt, J, grid, rope, inverse=True)
            dv_out[b, h] = dvj
    return dk_out, dv_out


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
