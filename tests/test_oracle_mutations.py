"""The oracle's pins have teeth: plant a plausible mistake in the oracle (on the CPU,
by patching one of its functions) and check that at least one pin then fails."""

import numpy as np
import pytest

import oracle.reference as ref
import test_oracle_attention as fwd_pins
import test_oracle_backward as bwd_pins
import test_oracle_rope as rope_pins
import test_oracle_shards as shard_pins


def _rope_apply_wrong_sign(x, angles, inverse=False):
    return _ORIG_APPLY(x, angles, not inverse)


def _rope_apply_rotate_half(x, angles, inverse=False):
    c, s = np.cos(angles), np.sin(angles)
    if inverse:
        s = -s
    h = x.shape[-1] // 2
    y = np.empty(np.broadcast_shapes(x.shape), dtype=np.float64)
    y[..., :h] = x[..., :h] * c - x[..., h:] * s
    y[..., h:] = x[..., :h] * s + x[..., h:] * c
    return y


def _freq_full_dim(rope, D):
    axis, j = ref.rope_axis_of_pair(rope, D)
    return axis, np.power(float(rope.theta), -2.0 * j / D)


def _positions_swapped(grid):
    p = _ORIG_POS(grid)
    return p[:, ::-1].copy()


def _head_bwd_no_delta(qt, kt, v, dout, scale):
    s = scale * (qt @ kt.T)
    lse = np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1)
    p = np.exp(s - lse[:, None])
    ds = p * (dout @ v.T)
    return scale * ds @ kt, scale * ds.T @ qt, p.T @ dout


def _rotated_no_inverse(x_rows, token_idx, grid, rope, inverse=False):
    return _ORIG_ROTATED(x_rows, token_idx, grid, rope, False)


def _attention_no_scale(qt, kt, v, scale):
    return _ORIG_ATTN(qt, kt, v, 1.0 if scale != 0 else 0.0)


def _partial_local_positions(q, k, v, scale, q_offset, k_offset, grid=None, rope=None, rows=None):
    return _ORIG_PARTIAL(q, k, v, scale, 0, 0, grid, rope, rows)


def _merge_unnormalized(o_parts, lse_parts):
    lse_st = np.stack(lse_parts)
    m = lse_st.max(axis=0)
    o = sum(np.asarray(op) * np.transpose(np.exp(l - m), (0, 2, 1))[..., None] for op, l in zip(o_parts, lse_parts))
    return o, m + np.log(np.exp(lse_st - m).sum(axis=0))


_ORIG_PARTIAL = ref.partial_fwd_ref
_ORIG_APPLY = ref.rope_apply
_ORIG_POS = ref.positions
_ORIG_ROTATED = ref._rotated
_ORIG_ATTN = ref.attention_rows_ref

MUTATIONS = [
    ("rotation sign", "rope_apply", _rope_apply_wrong_sign,
     [rope_pins.test_rope_1d_complex_form, rope_pins.test_rope_textbook_values_per_segment]),
    ("rotate-half pairing", "rope_apply", _rope_apply_rotate_half,
     [rope_pins.test_rope_1d_complex_form]),
    ("frequency over full head dim", "rope_frequencies", _freq_full_dim,
     [rope_pins.test_rope_last_pair_frequency]),
    ("axis order", "positions", _positions_swapped,
     [rope_pins.test_rope_textbook_values_per_segment]),
    ("dropped Delta term", "_head_bwd", _head_bwd_no_delta,
     [lambda: bwd_pins.test_self_bwd_finite_differences(ref.RopeSpec(4, 6, 6, 10000.0), 16, (2, 2, 3))]),
    ("missing inverse rotation of the gradient", "_rotated", _rotated_no_inverse,
     [lambda: bwd_pins.test_self_bwd_finite_differences(ref.RopeSpec(4, 6, 6, 10000.0), 16, (2, 2, 3))]),
    ("dropped softmax scale", "attention_rows_ref", _attention_no_scale,
     [fwd_pins.test_self_fwd_matches_torch_sdpa_without_rope]),
    ("shard positions taken as local indices", "partial_fwd_ref", _partial_local_positions,
     [shard_pins.test_query_shard_rows_match_brute_force, shard_pins.test_merge_of_key_shards_is_full_attention]),
    ("merge weights not normalized by the total LSE", "lse_merge_ref", _merge_unnormalized,
     [shard_pins.test_merge_of_key_shards_is_full_attention, shard_pins.test_merge_closed_forms]),
]


@pytest.mark.parametrize("name,attr,bad,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, attr, bad, pins):
    for pin in pins:
        pin()                      # passes on the real oracle
    monkeypatch.setattr(ref, attr, bad)
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake: {name}"
