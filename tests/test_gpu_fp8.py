"""GPU parity of the FP8 (e4m3) self-attention forward against the fp64 oracle evaluated on the
e4m3-dequantized inputs (oracle.fp8).  Tolerance, derived from the one rounding the oracle leaves
out, P -> e4m3 before P.V (relative error up to 2^-4 per element, ~3.6% rms): O max-abs 6e-2 and
relative L2 4e-2 (a CPU emulation of that rounding gives 1.1e-2 / 2.4e-2 at 320 tokens and
3.5e-2 / 6.5e-3 on peaked rows); LSE 1e-3 as in the bf16 path (its sums use fp32 P)."""

import math

import numpy as np
import pytest

import synth
from gpu_util import bf16_to_f64, check_close, check_lse, f32_to_np, to_dev
from oracle import RopeSpec
from oracle import fp8 as ofp8

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import spatio_temporal_attention_amd as wa  # noqa: E402

ROPE = RopeSpec()
SCALE = 1.0 / math.sqrt(128)
O_MAX_ABS, O_REL_L2 = 6e-2, 4e-2


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    wa.lib()


def _run(qb, kb, vb, grid, rope_on, scale=SCALE):
    table = wa.rope_table(grid, ROPE) if rope_on else None
    o, lse = wa.self_fwd_fp8(to_dev(qb), to_dev(kb), to_dev(vb), grid=grid, table=table, rope=ROPE, scale=scale)
    torch.cuda.synchronize()
    return bf16_to_f64(o), f32_to_np(lse)


def test_fp8_tiny_workload():
    w = synth.WORKLOADS[1]
    inp = synth.make_inputs(1)
    go, gl = _run(inp["q"], inp["k"], inp["v"], w.grid, True)
    f = synth.bf16_bits_to_f64
    ro, rl = ofp8.fp8_self_fwd_ref(f(inp["q"]), f(inp["k"]), f(inp["v"]), SCALE, w.grid, ROPE)
    check_close("O", go, ro, max_abs=O_MAX_ABS, rel_l2=O_REL_L2)
    check_lse("LSE", gl, rl)


@pytest.mark.parametrize("B,L,H,rope_on,qmul", [(2, 135, 3, False, 1.0), (1, 200, 2, True, 1.0),
                                                 (1, 189, 2, False, 4.0)])
def test_fp8_small(B, L, H, rope_on, qmul):
    grid = {135: (1, 1, 135), 200: (2, 10, 10), 189: (1, 1, 189)}[L]
    qb = synth.random_bf16(900, (B, L, H, 128), scale=qmul)
    kb = synth.random_bf16(901, (B, L, H, 128))
    vb = synth.random_bf16(902, (B, L, H, 128))
    go, gl = _run(qb, kb, vb, grid, rope_on)
    f = synth.bf16_bits_to_f64
    ro, rl = ofp8.fp8_self_fwd_ref(f(qb), f(kb), f(vb), SCALE, grid if rope_on else None, ROPE if rope_on else None)
    check_close("O", go, ro, max_abs=O_MAX_ABS, rel_l2=O_REL_L2, unit_scale=qmul == 1.0)
    check_lse("LSE", gl, rl)


def test_fp8_720p_sampled_heads():
    """The 720p workload: 64 seeded rows on 4 of the 40 heads (the oracle quantizes those heads' whole
    K and V)."""
    w = synth.WORKLOADS[4]
    inp = synth.make_inputs(4)
    go, gl = _run(inp["q"], inp["k"], inp["v"], w.grid, True)
    heads = [0, 13, 26, 39]
    f = synth.bf16_bits_to_f64
    rows = inp["rows"][:, heads]
    ro, rl = ofp8.fp8_self_fwd_ref(f(inp["q"][:, :, heads]), f(inp["k"][:, :, heads]), f(inp["v"][:, :, heads]),
                                   SCALE, w.grid, ROPE, rows=rows)
    got_o = np.stack([[go[0, rows[0, j], h] for j, h in enumerate(heads)]])
    got_l = np.stack([[gl[0, h, rows[0, j]] for j, h in enumerate(heads)]])
    check_close("O", got_o, ro, max_abs=O_MAX_ABS, rel_l2=O_REL_L2)
    check_lse("LSE", got_l, rl)
