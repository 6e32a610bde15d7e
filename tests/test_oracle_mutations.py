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


# ---------------------------------------------------------------------------
# Mistakes in the other oracle functions (masking, variable lengths, the row
# samplers of the backward, the FP8 and fp16 rounding recipes).  The planted
# function replaces the real one wherever the pins look it up: in its module
# and, for the names the oracle package re-exports, in the package.
# ---------------------------------------------------------------------------

import oracle                                                     # noqa: E402
from oracle import fp8 as fp8_mod, fp16_scores as f16_mod         # noqa: E402
import test_oracle_fp8 as fp8_pins                                # noqa: E402
import test_oracle_fp16 as f16_pins                               # noqa: E402

_ORIG_CROSS = ref.cross_fwd_ref
_ORIG_CROSS_BWD = ref.cross_bwd_ref
_ORIG_SELF = ref.self_fwd_ref
_ORIG_DKDV_ROWS = ref.self_bwd_dkdv_rows
_ORIG_DQ_ROWS = ref.self_bwd_dq_rows
_ORIG_E4M3 = fp8_mod.e4m3_round
_ORIG_TEXP8 = fp8_mod.tile_exponent
_ORIG_TEXP15 = f16_mod.tile_exponent15
_F16_POS = np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)   # finite non-negative binary16


def _cross_one_padded_key(q, k, v, k_lens, scale, rows=None):
    """Keys j <= k_len[b] taken as valid (an off-by-one in the mask)."""
    return _ORIG_CROSS(q, k, v, None if k_lens is None else np.asarray(k_lens) + 1, scale, rows)


def _varlen_keys_over_padding(q, k, v, seq_lens, scale, grid=None, rope=None):
    """Each item's valid queries attend to all L keys, padding included."""
    o, lse = _ORIG_SELF(q, k, v, scale, grid, rope)
    for b, n in enumerate(seq_lens):
        o[b, int(n):] = np.nan
        lse[b, :, int(n):] = np.nan
    return o, lse


def _cross_bwd_softmax_over_padding(q, k, v, dout, k_lens, scale):
    """Gradients of the unmasked attention, with the padded keys' dK and dV then set to zero."""
    dq, dk, dv = _ORIG_CROSS_BWD(q, k, v, dout, None, scale)
    if k_lens is not None:
        for b, n in enumerate(np.clip(np.asarray(k_lens), 0, k.shape[1])):
            dk[b, int(n):] = 0.0
            dv[b, int(n):] = 0.0
    return dq, dk, dv


def _rotate_rows_forward(x, J, grid, rope, D):
    return ref.rope_apply(x, ref.rope_angles(ref.positions(grid)[J], rope, D))


def _dkdv_rows_in_rotated_frame(q, k, v, dout, scale, grid, rope, key_rows, heads=None, block=512):
    """dK of the sampled keys left as the gradient w.r.t. the rotated keys."""
    dk, dv = _ORIG_DKDV_ROWS(q, k, v, dout, scale, grid, rope, key_rows, heads, block)
    for b in range(dk.shape[0]):
        for h in (range(dk.shape[1]) if heads is None else heads):
            dk[b, h] = _rotate_rows_forward(dk[b, h], key_rows[b, h], grid, rope, q.shape[-1])
    return dk, dv


def _dq_rows_in_rotated_frame(q, k, v, dout, scale, grid, rope, rows):
    """dQ of the sampled queries left as the gradient w.r.t. the rotated queries."""
    dq = _ORIG_DQ_ROWS(q, k, v, dout, scale, grid, rope, rows)
    for b in range(dq.shape[0]):
        for h in range(dq.shape[1]):
            dq[b, h] = _rotate_rows_forward(dq[b, h], rows[b, h], grid, rope, q.shape[-1])
    return dq


def _e4m3_ties_away(x):
    """e4m3 rounding with ties away from zero instead of to the even code."""
    x = np.asarray(x, dtype=np.float64)
    pos = fp8_mod._POS
    a = np.minimum(np.abs(x), pos[-1])
    hi = np.clip(np.searchsorted(pos, a, side="left"), 0, len(pos) - 1)
    lo = np.clip(hi - 1, 0, len(pos) - 1)
    idx = np.where(pos[hi] - a <= a - pos[lo], hi, lo)
    return np.sign(x) * pos[idx]


def _fp16_truncate(x):
    """binary16 rounding toward zero instead of to nearest."""
    x = np.asarray(x, dtype=np.float64)
    idx = np.clip(np.searchsorted(_F16_POS, np.abs(x), side="right") - 1, 0, len(_F16_POS) - 1)
    return np.sign(x) * _F16_POS[idx]


MUTATIONS_ELSEWHERE = [
    ("cross-attention mask admits one padded key", [(ref, "cross_fwd_ref"), (oracle, "cross_fwd_ref")],
     _cross_one_padded_key,
     [fwd_pins.test_cross_single_key_and_empty, fwd_pins.test_cross_fwd_matches_torch_sdpa_with_mask]),
    ("variable-length keys run over the padding", [(ref, "self_fwd_varlen_ref"), (oracle, "self_fwd_varlen_ref")],
     _varlen_keys_over_padding,
     [shard_pins.test_varlen_items_equal_separate_sequences]),
    ("cross-attention backward softmax over padded keys", [(ref, "cross_bwd_ref"), (oracle, "cross_bwd_ref")],
     _cross_bwd_softmax_over_padding,
     [bwd_pins.test_cross_bwd_finite_differences_and_padding, bwd_pins.test_cross_bwd_matches_torch_autograd_with_mask]),
    ("sampled dK rows not rotated back", [(ref, "self_bwd_dkdv_rows"), (oracle, "self_bwd_dkdv_rows")],
     _dkdv_rows_in_rotated_frame,
     [bwd_pins.test_sampled_rows_match_full_backward]),
    ("sampled dQ rows not rotated back", [(ref, "self_bwd_dq_rows"), (oracle, "self_bwd_dq_rows")],
     _dq_rows_in_rotated_frame,
     [bwd_pins.test_sampled_rows_match_full_backward]),
    ("e4m3 ties away from zero", [(fp8_mod, "e4m3_round")], _e4m3_ties_away,
     [fp8_pins.test_e4m3_rounding_ties_and_saturation]),
    ("FP8 tile exponent one too small (tile max in [256, 512))", [(fp8_mod, "tile_exponent")],
     lambda m: _ORIG_TEXP8(m) - 1 if m > 0 else 0,
     [fp8_pins.test_tile_exponent_range, fp8_pins.test_recipe_is_identity_on_representable_tiles]),
    ("binary16 rounding toward zero", [(f16_mod, "fp16_round")], _fp16_truncate,
     [f16_pins.test_binary16_landmarks, f16_pins.test_binary16_rounding_matches_definition]),
    ("fp16 tile exponent one too small (tile max in [2^15, 2^16))", [(f16_mod, "tile_exponent15")],
     lambda m: _ORIG_TEXP15(m) - 1 if m > 0 else 0,
     [f16_pins.test_tile_exponent_range, f16_pins.test_round_tiles_recipe]),
]


@pytest.mark.parametrize("name,targets,bad,pins", MUTATIONS_ELSEWHERE, ids=[m[0] for m in MUTATIONS_ELSEWHERE])
def test_planted_mistake_elsewhere_is_caught(monkeypatch, name, targets, bad, pins):
    for pin in pins:
        pin()                      # passes on the real oracle
    for module, attr in targets:
        monkeypatch.setattr(module, attr, bad)
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake: {name}"
