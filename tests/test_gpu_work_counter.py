"""GPU parity of the forward launches whose workgroups take their query tiles
from a work counter, at item counts around the spare workgroups.

A launch of n items runs n + ceil(n / 8) workgroups; each takes the counter's
next value and those past the last item leave at once.  These shapes put n at
1, 7, 8, 9 and 17 (one 256-row query tile per head) and at 8 with a ragged
second tile per head, so the first, the last and the spare workgroups all
occur; they also run the partial (ring-hop) forward at 7 items and the
cross-attention forward over 640 text tokens (the 8-wave path, counted).  Every
output row is compared with the fp64 oracle at the other parity tests' bar
(max-abs 2e-2, rel-L2 5e-3 on O; |LSE error| 1e-3)."""

import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_to_f64, check_close, check_lse, f32_to_np, to_dev
from oracle import RopeSpec

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import spatio_temporal_attention_amd as wa  # noqa: E402

ROPE = RopeSpec()
SCALE = 1.0 / math.sqrt(128)


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    wa.lib()


def _inputs(seed, shape):
    return [synth.random_bf16(seed + i, shape) for i in range(3)]


@pytest.mark.parametrize("grid,H", [
    ((1, 16, 16), 1),     # 1 item: one workgroup and one spare
    ((1, 16, 16), 7),     # 7 items, 8 workgroups
    ((1, 16, 16), 8),     # 8 items, 9 workgroups
    ((1, 16, 16), 9),     # 9 items, 11 workgroups
    ((1, 16, 16), 17),    # 17 items, 20 workgroups
    ((3, 10, 10), 4),     # L = 300: 2 tiles per head (the second 44 rows), 8 items
])
def test_counted_forward_matches_oracle(grid, H):
    L = grid[0] * grid[1] * grid[2]
    qb, kb, vb = _inputs(700 + H, (1, L, H, 128))
    table = wa.rope_table(grid, ROPE)
    o, lse = wa.self_fwd(to_dev(qb), to_dev(kb), to_dev(vb), grid=grid, table=table, rope=ROPE, scale=SCALE)
    torch.cuda.synchronize()
    ro, rl = oracle.self_fwd_ref(synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb),
                                 synth.bf16_bits_to_f64(vb), SCALE, grid, ROPE)
    check_close("O", bf16_to_f64(o), ro)
    check_lse("LSE", f32_to_np(lse), rl)


def test_counted_partial_forward_matches_oracle():
    """The ring-hop forward: 256 query tokens x 7 heads (7 items) against 300 keys, at offsets."""
    grid, H = (3, 10, 10), 7
    full = _inputs(760, (1, 300, H, 128))
    q_off, k_off = 44, 0
    q, k, v = full[0][:, q_off:q_off + 256], full[1], full[2]
    table = wa.rope_table(grid, ROPE)
    o, lse = wa.partial_fwd(to_dev(q), to_dev(k), to_dev(v), q_off, k_off, grid=grid, table=table, rope=ROPE,
                            scale=SCALE)
    torch.cuda.synchronize()
    ro, rl = oracle.partial_fwd_ref(synth.bf16_bits_to_f64(q), synth.bf16_bits_to_f64(k),
                                    synth.bf16_bits_to_f64(v), SCALE, q_off, k_off, grid, ROPE)
    check_close("O", bf16_to_f64(o), ro)
    check_lse("LSE", f32_to_np(lse), rl)


def test_counted_cross_forward_long_text():
    """Cross-attention over 640 text tokens (10 key tiles: the 8-wave path, which takes its query tiles from the
    counter), 2 items x 3 heads x 2 query tiles (300 rows: the second holds 44), valid lengths 640 and 333."""
    B, Lq, Lk, H = 2, 300, 640, 3
    qb = synth.random_bf16(781, (B, Lq, H, 128))
    kb = synth.random_bf16(782, (B, Lk, H, 128))
    vb = synth.random_bf16(783, (B, Lk, H, 128))
    lens = np.array([640, 333], dtype=np.int32)
    o, lse = wa.cross_fwd(to_dev(qb), to_dev(kb), to_dev(vb), torch.from_numpy(lens).cuda(), scale=SCALE)
    torch.cuda.synchronize()
    ro, rl = oracle.cross_fwd_ref(synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb),
                                  synth.bf16_bits_to_f64(vb), lens, SCALE)
    check_close("O", bf16_to_f64(o), ro)
    check_lse("LSE", f32_to_np(lse), rl)
