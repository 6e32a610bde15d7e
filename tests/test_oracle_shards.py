"""Pins of the oracle's shard, merge and variable-length functions on the CPU.

Independent checks: the scalar fsum brute force of the full self-attention
(test_oracle_attention._brute_self, explicit cos/sin rotation of every token
at its global position), the algebra of key sharding (merging the partial
results of a key split reproduces the unsplit attention), closed forms of the
merge, and separate per-item calls for variable lengths.
"""

import math

import numpy as np
import pytest

import oracle.reference as ref
from oracle import RopeSpec
from test_oracle_attention import _brute_self, _rand

ROPE = RopeSpec(4, 6, 6, 10000.0)
D = 16
GRID = (3, 2, 3)           # L = 18
L = 18
SCALE = 0.3


def _qkv(B=1, H=2, seed=40):
    return tuple(_rand((B, L, H, D), seed + i) for i in range(3))


def test_partial_with_whole_shards_is_self_attention():
    q, k, v = _qkv()
    o, lse = ref.partial_fwd_ref(q, k, v, SCALE, 0, 0, GRID, ROPE)
    o2, lse2 = ref.self_fwd_ref(q, k, v, SCALE, GRID, ROPE)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-14)


def test_query_shard_rows_match_brute_force():
    q, k, v = _qkv(seed=50)
    ob, lb = _brute_self(q, k, v, SCALE, GRID, ROPE)
    qo, lq = 5, 7
    o, lse = ref.partial_fwd_ref(q[:, qo:qo + lq], k, v, SCALE, qo, 0, GRID, ROPE)
    np.testing.assert_allclose(o, ob[:, qo:qo + lq], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lb[:, :, qo:qo + lq], rtol=0, atol=1e-12)


def test_merge_of_key_shards_is_full_attention():
    """Ring attention's algebra: partial results over a key split, merged, equal the unsplit
    attention (brute force) for a query shard in the middle of the sequence."""
    q, k, v = _qkv(seed=60)
    ob, lb = _brute_self(q, k, v, SCALE, GRID, ROPE)
    qo, lq = 4, 9
    cuts = [0, 5, 11, 18]
    parts = [ref.partial_fwd_ref(q[:, qo:qo + lq], k[:, a:b], v[:, a:b], SCALE, qo, a, GRID, ROPE)
             for a, b in zip(cuts[:-1], cuts[1:])]
    o, lse = ref.lse_merge_ref([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(o, ob[:, qo:qo + lq], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lb[:, :, qo:qo + lq], rtol=0, atol=1e-12)


def test_merge_closed_forms():
    rng = np.random.default_rng(70)
    o1 = rng.standard_normal((1, 5, 2, D))
    l1 = rng.standard_normal((1, 2, 5))
    o, lse = ref.lse_merge_ref([o1], [l1])                 # one part: identity
    np.testing.assert_allclose(o, o1, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, l1, rtol=0, atol=1e-15)
    o, lse = ref.lse_merge_ref([o1, o1], [l1, l1])         # two equal parts: same O, LSE + ln 2
    np.testing.assert_allclose(o, o1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, l1 + math.log(2.0), rtol=0, atol=1e-14)
    o2 = rng.standard_normal((1, 5, 2, D))
    empty = np.full((1, 2, 5), -np.inf)
    o, lse = ref.lse_merge_ref([o1, o2], [l1, empty])      # an empty shard has weight 0
    np.testing.assert_allclose(o, o1, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, l1, rtol=0, atol=1e-15)
    o, lse = ref.lse_merge_ref([o1, o2], [empty, empty])   # nothing valid: O = 0, LSE = -inf
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_varlen_items_equal_separate_sequences():
    """Item b with n_b = whole frames of the padded grid equals a separate sequence of its own
    (grid (n_b / (h w), h, w)), by brute force; NaN padding never leaks into valid rows."""
    B, H = 3, 1
    q, k, v = (_rand((B, L, H, D), s) for s in (80, 81, 82))
    lens = np.array([18, 12, 6])
    for b, n in enumerate(lens):
        q[b, n:] = np.nan
        k[b, n:] = np.nan
        v[b, n:] = np.nan
    o, lse = ref.self_fwd_varlen_ref(q, k, v, lens, SCALE, GRID, ROPE)
    for b, n in enumerate(lens):
        own_grid = (n // 6, 2, 3)
        ob, lb = _brute_self(q[b:b + 1, :n], k[b:b + 1, :n], v[b:b + 1, :n], SCALE, own_grid, ROPE)
        np.testing.assert_allclose(o[b:b + 1, :n], ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b:b + 1, :, :n], lb, rtol=0, atol=1e-12)
        assert np.all(np.isnan(o[b, n:])) and np.all(np.isnan(lse[b, :, n:]))


def test_varlen_full_and_zero_lengths():
    q, k, v = _qkv(B=2, seed=90)
    o, lse = ref.self_fwd_varlen_ref(q, k, v, np.array([L, 0]), SCALE, GRID, ROPE)
    o2, lse2 = ref.self_fwd_ref(q[:1], k[:1], v[:1], SCALE, GRID, ROPE)
    np.testing.assert_allclose(o[:1], o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[:1], lse2, rtol=0, atol=1e-14)
    assert np.all(np.isnan(o[1])) and np.all(np.isnan(lse[1]))
