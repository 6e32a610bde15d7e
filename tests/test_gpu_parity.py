"""GPU parity: the HIP path (through the C-ABI binding) against the fp64 oracle.

Inputs are the seeded synthetic workloads of `synth` (the same host arrays feed
both sides).  Bar (bf16 I/O, fp32 statistics): max-abs <= 2e-2 and relative
L2 <= 5e-3 on O, dQ, dK, dV; |LSE error| <= 1e-3.  Large workloads are checked
on 64 seeded rows per (batch, head).
"""

import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_to_f64, check_close, check_lse, f32_to_np, to_dev
from oracle import RopeSpec
from oracle import fp16_scores

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import spatio_temporal_attention_amd as wa  # noqa: E402

ROPE = RopeSpec()
SCALE = 1.0 / math.sqrt(128)


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    wa.lib()   # the compiled library must be present: no fallback exists


def _f64(bits):
    return synth.bf16_bits_to_f64(bits)


def _table(grid):
    return wa.rope_table(grid, ROPE)


# ---------------------------------------------------------------------------
# RoPE table and standalone rotation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("grid", [(5, 8, 8), (21, 30, 52), (21, 45, 80), (64, 64, 64), (1, 1, 1)])
def test_rope_table_matches_oracle(grid):
    got = _table(grid).cpu().numpy().astype(np.float64)
    ref = np.concatenate([t.reshape(-1) for t in oracle.rope_table_ref(grid, ROPE)])
    assert got.shape == ref.shape
    err = np.abs(got - ref).max()
    print(f"  table {grid}: max_abs={err:.3e}")
    assert err <= 6e-8     # fp32 rounding of |cos|, |sin| <= 1


@pytest.mark.parametrize("inverse", [False, True])
def test_rope3d_matches_oracle(inverse):
    grid = (5, 8, 8)
    bits = synth.random_bf16(101, (2, 320, 3, 128), scale=2.0)
    x = to_dev(bits)
    y = wa.rope3d(x, grid, _table(grid), ROPE, inverse=inverse)
    torch.cuda.synchronize()
    got = bf16_to_f64(y)
    ref = oracle.rope3d_ref(_f64(bits), grid, ROPE, inverse=inverse)
    # one bf16 rounding (half an ulp, 2^-9 relative) of an fp32 result: the bar is relative per
    # element (inputs have sigma 2, so an absolute bar would only measure the bf16 ulp of large values)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5)
    check_close("rope3d", got, ref, max_abs=np.inf)
    # in place gives the same bits
    wa.rope3d(x, grid, _table(grid), ROPE, inverse=inverse, out=x)
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_rope3d_round_trip():
    grid = (3, 4, 5)
    bits = synth.random_bf16(102, (1, 60, 4, 128))
    x = to_dev(bits)
    t = _table(grid)
    back = wa.rope3d(wa.rope3d(x, grid, t, ROPE), grid, t, ROPE, inverse=True)
    torch.cuda.synchronize()
    x64 = _f64(bits)
    # two roundings of at most 2^-9 of the rotated pair's norm each; rotation preserves that norm
    # and spreads the error over both elements of the pair
    pair = np.sqrt(x64[..., 0::2] ** 2 + x64[..., 1::2] ** 2).repeat(2, axis=-1)
    assert np.all(np.abs(bf16_to_f64(back) - x64) <= 2.0 ** -7 * pair + 1e-5)


# ---------------------------------------------------------------------------
# Self-attention forward
# ---------------------------------------------------------------------------

def _run_self_fwd(qb, kb, vb, grid, rope_on, scale=SCALE):
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    table = _table(grid) if rope_on else None
    o, lse = wa.self_fwd(q, k, v, grid=grid, table=table, rope=ROPE, scale=scale)
    torch.cuda.synchronize()
    return bf16_to_f64(o), f32_to_np(lse)


def test_self_fwd_tiny_workload():
    w = synth.WORKLOADS[1]
    inp = synth.make_inputs(1)
    o, lse = _run_self_fwd(inp["q"], inp["k"], inp["v"], w.grid, True)
    ro, rl = oracle.self_fwd_ref(_f64(inp["q"]), _f64(inp["k"]), _f64(inp["v"]), SCALE, w.grid, ROPE)
    check_close("O", o, ro)
    check_lse("LSE", lse, rl)


# Peaked cases here run without RoPE: q and k are then exact bf16 and enter the products unrounded,
# so the bar applies as stated.  The peaked cases with RoPE follow below (test_self_fwd_peaked_rope).
@pytest.mark.parametrize("B,grid,H,rope_on,qmul", [
    (2, (2, 10, 10), 3, True, 1.0),     # L = 200: ragged against 64-key tiles and 128-row tiles
    (1, (1, 1, 1), 2, True, 1.0),       # a single token
    (1, (3, 5, 7), 2, False, 1.0),      # L = 105, no rotary
    (1, (4, 8, 8), 2, False, 8.0),      # peaked softmax: exercises the running-max rescale
    (3, (1, 9, 15), 1, False, 3.0),     # B > 1, L = 135, peaked
    (2, (3, 7, 9), 2, True, 1.0),       # B > 1, L = 189 with RoPE
    (1, (2, 13, 20), 2, True, 1.0),     # L = 520: three 256-row workgroups (the last with 8 rows), 9 key tiles
    (1, (2, 16, 16), 1, True, 1.0),     # L = 512: two full workgroups, an even number of full key tiles
])
def test_self_fwd_small(B, grid, H, rope_on, qmul):
    L = int(np.prod(grid))
    seed = 1000 + L + B
    qb = synth.random_bf16(seed, (B, L, H, 128), scale=qmul)
    kb = synth.random_bf16(seed + 1, (B, L, H, 128))
    vb = synth.random_bf16(seed + 2, (B, L, H, 128))
    o, lse = _run_self_fwd(qb, kb, vb, grid, rope_on)
    ro, rl = oracle.self_fwd_ref(_f64(qb), _f64(kb), _f64(vb), SCALE, grid, ROPE if rope_on else None)
    check_close("O", o, ro)
    check_lse("LSE", lse, rl)


# Peaked cases with RoPE.  The rotated q and k enter the score product as fp16 tiles (a power of two per
# 64-token tile, then binary16 rounding), and with q scaled up that rounding alone moves scores by up to
# ~1e-2 (oracle.fp16_scores; tests/test_oracle_fp16.py measures 7e-3 in LSE at q x 8 on 320 tokens): more
# than the 1e-3 LSE bar, whatever the kernel does.  So the GPU is held to the stated bar against the oracle
# evaluated at the rounded operands (which takes the kernel's documented operand rounding and nothing
# else), and against the exact oracle to the stated bar plus the distance between the two oracles.  The
# kernel rotates in fp32, so an element whose exact value sits next to an fp16 rounding tie may round to
# the neighbouring value (about one element in 10^4); the oracle marks every such element and bounds what
# the alternative rounding can move (score_tie_allowance, A_i per row), which is added per row: LSE by at
# most A_i, O by at most (exp(2 A_i) - 1) max|v|.
# Scores of std 8*1.44 in log2 units exceed the running max by more than the 2^16 partial-sum limit on
# later key tiles, so the lazy-rescale branch (per-tile factor 2^e_t, m moved, O and l rescaled) runs
# after the first tile; q x 4 mostly stays on the fast path.
@pytest.mark.parametrize("grid,H,qmul", [
    ((5, 8, 8), 2, 4.0),       # 320 tokens, 5 key tiles
    ((5, 8, 8), 2, 8.0),
    ((3, 7, 9), 2, 8.0),       # L = 189: ragged, masked last key tile
    ((2, 32, 32), 1, 4.0),     # 2,048 tokens, 32 key tiles
    ((2, 32, 32), 2, 8.0),
])
def test_self_fwd_peaked_rope(grid, H, qmul):
    L = int(np.prod(grid))
    seed = 5000 + L + int(qmul)
    qb = synth.random_bf16(seed, (1, L, H, 128), scale=qmul)
    kb = synth.random_bf16(seed + 1, (1, L, H, 128))
    vb = synth.random_bf16(seed + 2, (1, L, H, 128))
    o, lse = _run_self_fwd(qb, kb, vb, grid, True)
    q, k, v = _f64(qb), _f64(kb), _f64(vb)
    eo, el = fp16_scores.self_fwd_fp16_ref(q, k, v, SCALE, grid, ROPE)
    ro, rl = oracle.self_fwd_ref(q, k, v, SCALE, grid, ROPE)
    allow = fp16_scores.score_tie_allowance(q, k, SCALE, grid, ROPE)                 # [B, H, L]
    o_allow = np.broadcast_to(np.expm1(2.0 * allow).transpose(0, 2, 1)[..., None] * np.abs(v).max(), o.shape)
    print(f"  oracle at rounded operands vs exact: O {np.abs(eo - ro).max():.2e}, LSE {np.abs(el - rl).max():.2e}; "
          f"rows with a tie allowance {int((allow > 0).sum())} of {allow.size}, max {allow.max():.2e}")
    # a peaked softmax makes O close to single value rows (|O| up to ~4.5, not O(1)): the O bar adds the
    # bf16 output quantum (check_close out_quantum)
    check_close("O vs oracle at rounded operands", o, eo, extra_abs=o_allow, out_quantum=True)
    check_lse("LSE vs oracle at rounded operands", lse, el, extra=allow)
    check_close("O vs exact oracle (+ rounding distance)", o, ro, out_quantum=True,
                extra_abs=np.abs(eo - ro) + o_allow, extra_rel=float(np.linalg.norm(eo - ro) / np.linalg.norm(ro)))
    check_lse("LSE vs exact oracle (+ rounding distance)", lse, rl, extra=np.abs(el - rl) + allow)


def test_self_fwd_scale_zero_closed_form():
    grid = (5, 8, 8)
    qb, kb, vb = (synth.random_bf16(s, (1, 320, 2, 128)) for s in (201, 202, 203))
    o, lse = _run_self_fwd(qb, kb, vb, grid, True, scale=0.0)
    mean_v = _f64(vb).mean(axis=1, keepdims=True)
    check_close("O", o, np.broadcast_to(mean_v, o.shape))
    check_lse("LSE", lse, np.full(lse.shape, math.log(320)))


def _sampled_self_fwd_check(index):
    w = synth.WORKLOADS[index]
    inp = synth.make_inputs(index, with_dout=False)
    print(f"  workload {index} ({w.name}): generated", flush=True)
    o, lse = _run_self_fwd(inp["q"], inp["k"], inp["v"], w.grid, True)
    print(f"  workload {index}: GPU done", flush=True)
    rows = inp["rows"]
    got_o, ref_o, got_l, ref_l = [], [], [], []
    for b in range(w.B):
        for h in range(w.H):
            sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
            ro, rl = oracle.self_fwd_ref(_f64(inp["q"][sl]), _f64(inp["k"][sl]), _f64(inp["v"][sl]), SCALE,
                                         w.grid, ROPE, rows=rows[b:b + 1, h:h + 1])
            got_o.append(o[b, rows[b, h], h])
            ref_o.append(ro[0, 0])
            got_l.append(lse[b, h, rows[b, h]])
            ref_l.append(rl[0, 0])
    check_close("O (sampled)", np.stack(got_o), np.stack(ref_o))
    check_lse("LSE (sampled)", np.stack(got_l), np.stack(ref_l))


def test_self_fwd_480p_sampled():
    _sampled_self_fwd_check(2)


def test_self_fwd_720p_sampled():
    _sampled_self_fwd_check(4)


def test_self_fwd_long_sampled():
    """Grid 64x64x64 = 262144 tokens, 40 heads: 64 seeded rows per head."""
    _sampled_self_fwd_check(5)


# ---------------------------------------------------------------------------
# Cross-attention forward
# ---------------------------------------------------------------------------

def _run_cross(qb, kb, vb, lens, scale=SCALE):
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    kl = None if lens is None else torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    o, lse = wa.cross_fwd(q, k, v, kl, scale=scale)
    torch.cuda.synchronize()
    return bf16_to_f64(o), f32_to_np(lse)


def test_cross_workload_sampled():
    w = synth.WORKLOADS[3]
    inp = synth.make_inputs(3)
    o, lse = _run_cross(inp["q"], inp["k"], inp["v"], inp["k_lens"])
    rows = inp["rows"]
    ro, rl = oracle.cross_fwd_ref(_f64(inp["q"]), _f64(inp["k"]), _f64(inp["v"]), inp["k_lens"], SCALE, rows=rows)
    got_o = np.stack([[o[b, rows[b, h], h] for h in range(w.H)] for b in range(w.B)])
    got_l = np.stack([[lse[b, h, rows[b, h]] for h in range(w.H)] for b in range(w.B)])
    check_close("O (sampled)", got_o, ro)
    check_lse("LSE (sampled)", got_l, rl)


def test_cross_masking_edge_cases():
    B, Lq, Lk, H = 4, 150, 100, 2
    qb = synth.random_bf16(301, (B, Lq, H, 128))
    kb = synth.random_bf16(302, (B, Lk, H, 128))
    vb = synth.random_bf16(303, (B, Lk, H, 128))
    lens = np.array([1, 100, 37, 64], dtype=np.int32)
    # padded keys hold NaN: they must never reach an output
    kb_nan, vb_nan = kb.copy(), vb.copy()
    for b, n in enumerate(lens):
        kb_nan[b, n:] = 0x7FC0
        vb_nan[b, n:] = 0x7FC0
    o, lse = _run_cross(qb, kb_nan, vb_nan, lens)
    ro, rl = oracle.cross_fwd_ref(_f64(qb), _f64(kb), _f64(vb), lens, SCALE)
    check_close("O", o, ro)
    check_lse("LSE", lse, rl)
    # k_len = 1: O is exactly v_0 up to bf16 output rounding
    np.testing.assert_allclose(o[0], np.broadcast_to(_f64(vb)[0, :1], o[0].shape), atol=2e-2)


def test_cross_all_valid_and_empty():
    B, Lq, Lk, H = 2, 70, 512, 3
    qb = synth.random_bf16(311, (B, Lq, H, 128))
    kb = synth.random_bf16(312, (B, Lk, H, 128))
    vb = synth.random_bf16(313, (B, Lk, H, 128))
    o, lse = _run_cross(qb, kb, vb, None)
    ro, rl = oracle.cross_fwd_ref(_f64(qb), _f64(kb), _f64(vb), None, SCALE)
    check_close("O (no mask)", o, ro)
    check_lse("LSE (no mask)", lse, rl)
    o2, lse2 = _run_cross(qb, kb, vb, [Lk, 0])
    check_close("O (k_len = Lk)", o2[0], ro[0])
    assert np.all(o2[1] == 0.0) and np.all(np.isneginf(lse2[1]))


def test_cross_many_items_and_heads():
    """One launch over 4 items x 3 heads x 125 query tiles of 128 rows (15,950 rows: the last tile holds 78;
    the short-key path of 4-wave workgroups): items with 77 valid keys (a masked last key tile), one (a single
    partial key tile), none, and all 200, NaN in the padded keys and values."""
    B, Lq, Lk, H = 4, 15_950, 200, 3
    qb = synth.random_bf16(331, (B, Lq, H, 128))
    kb = synth.random_bf16(332, (B, Lk, H, 128))
    vb = synth.random_bf16(333, (B, Lk, H, 128))
    lens = np.array([77, 1, 0, 200], dtype=np.int32)
    kb_nan, vb_nan = kb.copy(), vb.copy()
    for b, n in enumerate(lens):
        kb_nan[b, n:] = 0x7FC0
        vb_nan[b, n:] = 0x7FC0
    o, lse = _run_cross(qb, kb_nan, vb_nan, lens)
    ro, rl = oracle.cross_fwd_ref(_f64(qb), _f64(kb), _f64(vb), lens, SCALE)
    for b in (0, 1, 3):
        check_close(f"O (item {b}, k_len {lens[b]})", o[b], ro[b])
        check_lse(f"LSE (item {b})", lse[b], rl[b])
    assert np.all(o[2] == 0.0) and np.all(np.isneginf(lse[2]))


def test_cross_720p_text_sampled():
    """The measured text cross-attention: 75,600 video tokens over 512 text tokens (336 valid), 40 heads,
    64 seeded rows per head."""
    Lq, Lk, H, n = 75600, 512, 40, 336
    qb = synth.random_bf16(7100, (1, Lq, H, 128))
    kb = synth.random_bf16(7101, (1, Lk, H, 128))
    vb = synth.random_bf16(7102, (1, Lk, H, 128))
    o, lse = _run_cross(qb, kb, vb, [n])
    rows = np.stack([[synth.sample_rows(7110 + h, Lq, 64) for h in range(H)]])
    ro, rl = oracle.cross_fwd_ref(_f64(qb), _f64(kb), _f64(vb), [n], SCALE, rows=rows)
    got_o = np.stack([[o[0, rows[0, h], h] for h in range(H)]])
    got_l = np.stack([[lse[0, h, rows[0, h]] for h in range(H)]])
    check_close("O (sampled)", got_o, ro)
    check_lse("LSE (sampled)", got_l, rl)


def test_cross_scale_zero():
    B, Lq, Lk, H = 2, 33, 40, 1
    qb, kb, vb = (synth.random_bf16(s, (B, L, H, 128)) for s, L in ((321, Lq), (322, Lk), (323, Lk)))
    lens = [7, 40]
    o, lse = _run_cross(qb, kb, vb, lens, scale=0.0)
    for b, n in enumerate(lens):
        check_close("O", o[b], np.broadcast_to(_f64(vb)[b, :n].mean(axis=0), o[b].shape))
        check_lse("LSE", lse[b], np.full(lse[b].shape, math.log(n)))


# ---------------------------------------------------------------------------
# Self-attention backward
# ---------------------------------------------------------------------------

def _run_self_bwd(qb, kb, vb, dob, grid, rope_on, scale=SCALE):
    q, k, v, do = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(dob)
    table = _table(grid) if rope_on else None
    o, lse = wa.self_fwd(q, k, v, grid=grid, table=table, rope=ROPE, scale=scale)
    dq, dk, dv = wa.self_bwd(q, k, v, o, lse, do, grid=grid, table=table, rope=ROPE, scale=scale)
    torch.cuda.synchronize()
    return bf16_to_f64(dq), bf16_to_f64(dk), bf16_to_f64(dv)


def test_self_bwd_tiny_workload():
    w = synth.WORKLOADS[1]
    inp = synth.make_inputs(1)
    dq, dk, dv = _run_self_bwd(inp["q"], inp["k"], inp["v"], inp["dout"], w.grid, True)
    rq, rk, rv = oracle.self_bwd_ref(_f64(inp["q"]), _f64(inp["k"]), _f64(inp["v"]), _f64(inp["dout"]), SCALE,
                                     w.grid, ROPE)
    check_close("dQ", dq, rq)
    check_close("dK", dk, rk)
    check_close("dV", dv, rv)


@pytest.mark.parametrize("B,grid,H,rope_on,qmul", [
    (2, (2, 10, 10), 2, True, 1.0),
    (1, (3, 5, 7), 1, False, 1.0),
    (1, (4, 8, 8), 2, False, 4.0),      # peaked (exact operands, see the forward cases)
    (2, (3, 7, 9), 1, True, 1.0),
    (1, (2, 32, 32), 1, True, 1.0),     # L = 2048, one key block: the dK/dV passes split the query range 4 ways
])
def test_self_bwd_small(B, grid, H, rope_on, qmul):
    L = int(np.prod(grid))
    seed = 2000 + L + B
    qb = synth.random_bf16(seed, (B, L, H, 128), scale=qmul)
    kb, vb, dob = (synth.random_bf16(seed + i, (B, L, H, 128)) for i in (1, 2, 3))
    dq, dk, dv = _run_self_bwd(qb, kb, vb, dob, grid, rope_on)
    rq, rk, rv = oracle.self_bwd_ref(_f64(qb), _f64(kb), _f64(vb), _f64(dob), SCALE, grid,
                                     ROPE if rope_on else None)
    unit = qmul == 1.0
    check_close("dQ", dq, rq, unit_scale=unit)
    check_close("dK", dk, rk, unit_scale=unit)
    check_close("dV", dv, rv, unit_scale=unit)


@pytest.mark.parametrize("grid,H,qmul", [
    ((5, 8, 8), 2, 4.0),
    ((5, 8, 8), 1, 8.0),
    ((3, 7, 9), 1, 8.0),       # ragged: masked last key tile in dK/dV and dQ
    ((2, 32, 32), 1, 8.0),     # 2,048 tokens: one key block, the dK/dV passes split the query range
])
def test_self_bwd_peaked_rope(grid, H, qmul):
    """The backward with RoPE on peaked inputs (see test_self_fwd_peaked_rope), given its inputs: o (bf16)
    and lse (fp32) are the oracle's, at the fp16-rounded operands, so both sides form Delta = <dO, o> from
    the same bf16 o.  (With a peaked softmax |O| ~ |v| is not averaged down, and o's bf16 rounding alone
    moves Delta by ~1e-2, which dS = P (dP - Delta) passes on where P ~ 1; the backward takes o as given.)
    The recomputed scores use the forward's fp16 tiles, so the gradients are held to the bar against the
    backward of the oracle at the rounded operands with that o, and against the exact oracle to the bar
    plus the distance between the two.  q is scaled up, so dK is too: the absolute bar is relative to the
    peak (check_close unit_scale)."""
    L = int(np.prod(grid))
    seed = 6000 + L + int(qmul)
    qb = synth.random_bf16(seed, (1, L, H, 128), scale=qmul)
    kb, vb, dob = (synth.random_bf16(seed + i, (1, L, H, 128)) for i in (1, 2, 3))
    q, k, v, do = _f64(qb), _f64(kb), _f64(vb), _f64(dob)
    eo, el = fp16_scores.self_fwd_fp16_ref(q, k, v, SCALE, grid, ROPE)
    ob = synth.fp32_to_bf16_bits(eo.astype(np.float32))
    o_dev = to_dev(ob)
    lse_dev = torch.from_numpy(el.astype(np.float32)).cuda()
    table = _table(grid)
    dq_d, dk_d, dv_d = wa.self_bwd(to_dev(qb), to_dev(kb), to_dev(vb), o_dev, lse_dev, to_dev(dob), grid=grid,
                                   table=table, rope=ROPE, scale=SCALE)
    torch.cuda.synchronize()
    dq, dk, dv = bf16_to_f64(dq_d), bf16_to_f64(dk_d), bf16_to_f64(dv_d)
    emu = fp16_scores.self_bwd_fp16_ref(q, k, v, do, SCALE, grid, ROPE, o=_f64(ob))
    ref = oracle.self_bwd_ref(q, k, v, do, SCALE, grid, ROPE)
    for name, g, e, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), emu, ref):
        print(f"  {name}: oracle at rounded operands (given o) vs exact: max {np.abs(e - r).max():.2e}, "
              f"rel {np.linalg.norm(e - r) / np.linalg.norm(r):.2e}")
        check_close(f"{name} vs oracle at rounded operands", g, e, unit_scale=False)
        check_close(f"{name} vs exact oracle (+ rounding distance)", g, r, unit_scale=False,
                    extra_abs=np.abs(e - r), extra_rel=float(np.linalg.norm(e - r) / np.linalg.norm(r)))


def test_self_bwd_single_token():
    """L = 1: P = 1, so dS = 0 and the exact dQ, dK are zero (relative L2 is undefined there);
    dV = dO exactly up to the output rounding."""
    grid = (1, 1, 1)
    qb, kb, vb, dob = (synth.random_bf16(2100 + i, (2, 1, 3, 128)) for i in range(4))
    dq, dk, dv = _run_self_bwd(qb, kb, vb, dob, grid, True)
    assert np.abs(dq).max() <= 2e-2 and np.abs(dk).max() <= 2e-2
    check_close("dV", dv, _f64(dob))


@pytest.fixture(scope="module")
def bwd_720p():
    """The 720p workload's inputs and GPU gradients, shared by the tests below."""
    w = synth.WORKLOADS[4]
    inp = synth.make_inputs(4)
    print("  720p: generated", flush=True)
    dq, dk, dv = _run_self_bwd(inp["q"], inp["k"], inp["v"], inp["dout"], w.grid, True)
    print("  720p: GPU done", flush=True)
    return w, inp, dq, dk, dv


def test_self_bwd_720p_sampled(bwd_720p):
    w, inp, dq, dk, dv = bwd_720p
    rows = inp["rows"]
    got, ref = [], []
    for h in range(w.H):
        sl = (slice(0, 1), slice(None), slice(h, h + 1))
        r = oracle.self_bwd_dq_rows(_f64(inp["q"][sl]), _f64(inp["k"][sl]), _f64(inp["v"][sl]),
                                    _f64(inp["dout"][sl]), SCALE, w.grid, ROPE, rows[:, h:h + 1])
        got.append(dq[0, rows[0, h], h])
        ref.append(r[0, 0])
    check_close("dQ (sampled, all heads)", np.stack(got), np.stack(ref))


DKDV_HEADS_720P = [int(h) for h in synth.sample_rows(404, 40, 4)]   # four seeded heads of the 40


@pytest.mark.parametrize("pair", [0, 1])
def test_self_bwd_720p_dkdv_heads(bwd_720p, pair):
    """dK/dV on the 64 seeded key rows of four seeded heads (two per test).  Each key's gradient needs
    every query row's LSE and Delta, so the oracle runs a blocked fp64 forward of the whole head (about
    2.9e12 flop); the two heads of a test run in two threads (numpy releases the GIL in its ufuncs and
    BLAS calls)."""
    from concurrent.futures import ThreadPoolExecutor
    w, inp, dq, dk, dv = bwd_720p
    rows = inp["rows"]
    heads = DKDV_HEADS_720P[2 * pair:2 * pair + 2]

    def one(h):
        sl = (slice(0, 1), slice(None), slice(h, h + 1))
        return oracle.self_bwd_dkdv_rows(_f64(inp["q"][sl]), _f64(inp["k"][sl]), _f64(inp["v"][sl]),
                                         _f64(inp["dout"][sl]), SCALE, w.grid, ROPE, rows[:, h:h + 1], block=1024)

    with ThreadPoolExecutor(len(heads)) as ex:
        res = list(ex.map(one, heads))
    for h, (rk, rv) in zip(heads, res):
        check_close(f"dK (sampled key rows, head {h})", dk[0, rows[0, h], h], rk[0, 0])
        check_close(f"dV (sampled key rows, head {h})", dv[0, rows[0, h], h], rv[0, 0])


def test_self_bwd_720p_tail_split_keys(bwd_720p):
    """dK and dV of head 39 at 720p, mostly on keys of its last 64 blocks of 256 (keys 59,392 .. 75,599): 40 heads
    give 11,840 key blocks, 46 rounds of 256 and 64 left over, which the dK/dV passes run as 4 query ranges each
    (head 39's dQ rows were sampled with every head above, its last 64 query blocks being the dQ pass's tail)."""
    w, inp, dq, dk, dv = bwd_720p
    blocks_per_head = (w.L + 255) // 256
    n = w.H * blocks_per_head
    tail = n % 256
    assert (blocks_per_head, n, tail) == (296, 11840, 64)
    first_tail_key = (blocks_per_head - tail) * 256
    assert first_tail_key == 59392
    h = 39
    keys = np.unique(np.concatenate([first_tail_key + synth.sample_rows(405, w.L - first_tail_key, 24),
                                     synth.sample_rows(406, first_tail_key, 8), [first_tail_key, w.L - 1]]))
    sl = (slice(0, 1), slice(None), slice(h, h + 1))
    rk, rv = oracle.self_bwd_dkdv_rows(_f64(inp["q"][sl]), _f64(inp["k"][sl]), _f64(inp["v"][sl]),
                                       _f64(inp["dout"][sl]), SCALE, w.grid, ROPE, keys[None, None, :], block=1024)
    check_close("dK (head 39, tail-split keys)", dk[0, keys, h], rk[0, 0])
    check_close("dV (head 39, tail-split keys)", dv[0, keys, h], rv[0, 0])
