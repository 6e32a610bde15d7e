"""GPU parity of the tail splits against the fp64 oracle.

The forward and the backward's dQ pass run 256-row query blocks, the dK/dV
passes 256-key blocks, 256 at a time; when a large problem's block count n is
not a multiple of 256, the last n % 256 blocks run as several key (or query)
ranges each, whose fp32 partials are combined after (the forward merges softmax
partials exactly; the backward sums its partials in range order).  The
fixed-length forward runs its pieces as the last workgroups of its main launch
and, from eight rounds on, splits one more round too.  These shapes
put the split on known heads (logical block = (head * B + item) *
blocks_per_head + block, batch item innermost) and check those heads in full;
same bar as the other parity tests (max-abs 2e-2, rel-L2 5e-3 on O, dQ, dK, dV;
|LSE error| 1e-3)."""

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
GRID = (2, 32, 32)        # L = 2048: 8 query tiles of 256 rows, 32 key tiles of 64 per head


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    wa.lib()


def _split_rule(B, L, H):
    """(main tiles, tail tiles, key ranges) of the documented split rule."""
    n = B * H * ((L + 255) // 256)
    if n < 1024 or n % 256 == 0:
        return n, 0, 1
    tail = n % 256
    S = min(8, 256 // tail)
    return (n, 0, 1) if S < 2 else (n - tail, tail, S)


def test_tail_split_heads_match_oracle():
    B, H = 1, 130
    L = int(np.prod(GRID))
    n_main, tail, S = _split_rule(B, L, H)
    assert (n_main, tail, S) == (1024, 16, 8)     # heads 128 and 129 run split, 8 key ranges of 4 tiles
    q, k, v = (synth.random_bf16(9100 + i, (B, L, H, 128)) for i in range(3))
    o, lse = wa.self_fwd(to_dev(q), to_dev(k), to_dev(v), grid=GRID, table=wa.rope_table(GRID, ROPE), rope=ROPE,
                         scale=SCALE)
    torch.cuda.synchronize()
    go, gl = bf16_to_f64(o), f32_to_np(lse)
    heads = [128, 129, 0]                          # the two split heads, and one of the main launch
    f = synth.bf16_bits_to_f64
    ro, rl = oracle.self_fwd_ref(f(q[:, :, heads]), f(k[:, :, heads]), f(v[:, :, heads]), SCALE, GRID, ROPE)
    for j, h in enumerate(heads):
        print(f"  head {h}:")
        check_close("O", go[:, :, h], ro[:, :, j])
        check_lse("LSE", gl[:, h], rl[:, j])


def _fwd_split_rule(B, L, H):
    """The self-attention forward's own split: from eight rounds on, the last n % 256 tiles and one more round
    run as 4 key ranges each, as the last workgroups of the same launch."""
    n = B * H * ((L + 255) // 256)
    if n < 2048:
        return _split_rule(B, L, H)
    tail = n % 256 + 256
    return n - tail, tail, 4


def test_forward_split_extra_round_heads_match_oracle():
    B, H = 1, 272                                  # 2,176 query tiles: 8.5 rounds
    L = int(np.prod(GRID))
    n_main, tail, S = _fwd_split_rule(B, L, H)
    assert (n_main, tail, S) == (1792, 384, 4)     # heads 224..271 run as 4 key ranges of 8 tiles each
    q, k, v = (synth.random_bf16(9150 + i, (B, L, H, 128)) for i in range(3))
    o, lse = wa.self_fwd(to_dev(q), to_dev(k), to_dev(v), grid=GRID, table=wa.rope_table(GRID, ROPE), rope=ROPE,
                         scale=SCALE)
    torch.cuda.synchronize()
    go, gl = bf16_to_f64(o), f32_to_np(lse)
    heads = [223, 224, 250, 271]                   # the last whole-tile head, then split heads
    f = synth.bf16_bits_to_f64
    ro, rl = oracle.self_fwd_ref(f(q[:, :, heads]), f(k[:, :, heads]), f(v[:, :, heads]), SCALE, GRID, ROPE)
    for j, h in enumerate(heads):
        print(f"  head {h}:")
        check_close("O", go[:, :, h], ro[:, :, j])
        check_lse("LSE", gl[:, h], rl[:, j])


def test_tail_split_varlen_masked_ranges_and_rows():
    """Two items (lengths 2048 and 1500, so 32 and 24 key tiles, the last one partial) with 65 heads: the
    tail is head 64 of both items, split 8 ways; rows past an item's length stay unwritten."""
    B, H = 2, 65
    L = int(np.prod(GRID))
    n_main, tail, S = _split_rule(B, L, H)
    assert (n_main, tail, S) == (1024, 16, 8)
    lens = np.array([2048, 1500], dtype=np.int32)
    q, k, v = (synth.random_bf16(9200 + i, (B, L, H, 128)) for i in range(3))
    nan_bits = np.uint16(0x7FC0)
    for b, n in enumerate(lens):                   # padding holds NaN: must never be read
        q[b, n:] = nan_bits
        k[b, n:] = nan_bits
        v[b, n:] = nan_bits
    o = torch.full((B, L, H, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, L), 5.0, dtype=torch.float32, device="cuda")
    wa.self_fwd_varlen(to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(lens).cuda(), grid=GRID,
                       table=wa.rope_table(GRID, ROPE), rope=ROPE, scale=SCALE, out=o, lse=lse)
    torch.cuda.synchronize()
    go, gl = bf16_to_f64(o), f32_to_np(lse)
    heads = [64, 3]                                # the split head, and one of the main launch
    f = synth.bf16_bits_to_f64
    ro, rl = oracle.self_fwd_varlen_ref(f(q[:, :, heads]), f(k[:, :, heads]), f(v[:, :, heads]), lens, SCALE, GRID,
                                        ROPE)
    for j, h in enumerate(heads):
        for b, n in enumerate(lens):
            print(f"  head {h}, item {b} (len {n}):")
            check_close("O", go[b, :n, h], ro[b, :n, j])
            check_lse("LSE", gl[b, h, :n], rl[b, j, :n])
            assert np.all(go[b, n:, h] == 7.0), "rows past the length were written"
            assert np.all(gl[b, h, n:] == 5.0), "LSE past the length was written"


def test_dq_tail_split_heads_match_oracle():
    """Self-attention backward with 130 heads at L = 2048: the dQ blocks of heads 128 and 129 run as 8 key
    ranges of 4 key tiles, their dK/dV blocks as 8 query ranges of 4 query tiles; their gradients (and one
    head of the main launch) against the oracle, and all gradients bit-identical over two calls."""
    B, H = 1, 130
    L = int(np.prod(GRID))
    assert _split_rule(B, L, H) == (1024, 16, 8)
    q, k, v, do = (synth.random_bf16(9300 + i, (B, L, H, 128)) for i in range(4))
    table = wa.rope_table(GRID, ROPE)
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = wa.self_fwd(qd, kd, vd, grid=GRID, table=table, rope=ROPE, scale=SCALE)
    dq, dk, dv = wa.self_bwd(qd, kd, vd, o, lse, dod, grid=GRID, table=table, rope=ROPE, scale=SCALE)
    again = [torch.full_like(dq, 3.0) for _ in range(3)]
    wa.self_bwd(qd, kd, vd, o, lse, dod, grid=GRID, table=table, rope=ROPE, scale=SCALE, dq=again[0], dk=again[1],
                dv=again[2])
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), (dq, dk, dv), again):
        assert torch.equal(a.view(torch.int16).cpu(), b.view(torch.int16).cpu()), f"{name} differs between two calls"
    gq, gk, gv = bf16_to_f64(dq), bf16_to_f64(dk), bf16_to_f64(dv)
    heads = [128, 129, 0]
    f = synth.bf16_bits_to_f64
    rq, rk, rv = oracle.self_bwd_ref(f(q[:, :, heads]), f(k[:, :, heads]), f(v[:, :, heads]), f(do[:, :, heads]),
                                     SCALE, GRID, ROPE)
    for j, h in enumerate(heads):
        print(f"  head {h}:")
        check_close("dQ", gq[:, :, h], rq[:, :, j])
        check_close("dK", gk[:, :, h], rk[:, :, j])
        check_close("dV", gv[:, :, h], rv[:, :, j])


def test_dq_tail_split_cross_with_empty_key_ranges():
    """Cross-attention backward, 2 items x 65 heads x 2048 queries over 512 text tokens, lengths 512 and 100:
    head 64's dQ blocks run as 8 key ranges; item 1 has 2 key tiles, so 6 of its ranges hold no key and
    contribute zero partials."""
    B, Lq, Lk, H = 2, 2048, 512, 65
    assert _split_rule(B, Lq, H) == (1024, 16, 8)
    q, do = (synth.random_bf16(9400 + i, (B, Lq, H, 128)) for i in range(2))
    k, v = (synth.random_bf16(9410 + i, (B, Lk, H, 128)) for i in range(2))
    lens = np.array([512, 100], dtype=np.int32)
    nan_bits = np.uint16(0x7FC0)
    for b, n in enumerate(lens):                   # padded keys hold NaN: never read
        k[b, n:] = nan_bits
        v[b, n:] = nan_bits
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    kl = torch.from_numpy(lens).cuda()
    o, lse = wa.cross_fwd(qd, kd, vd, kl, scale=SCALE)
    dq, dk, dv = wa.cross_bwd(qd, kd, vd, kl, o, lse, dod, scale=SCALE)
    torch.cuda.synchronize()
    gq, gk, gv = bf16_to_f64(dq), bf16_to_f64(dk), bf16_to_f64(dv)
    heads = [64, 5]                                # the split head, and one of the main launch
    f = synth.bf16_bits_to_f64
    rq, rk, rv = oracle.cross_bwd_ref(f(q[:, :, heads]), f(k[:, :, heads]), f(v[:, :, heads]), f(do[:, :, heads]),
                                      lens, SCALE)
    for j, h in enumerate(heads):
        for b, n in enumerate(lens):
            print(f"  head {h}, item {b} (k_len {n}):")
            check_close("dQ", gq[b, :, h], rq[b, :, j])
            check_close("dK", gk[b, :n, h], rk[b, :n, j])
            check_close("dV", gv[b, :n, h], rv[b, :n, j])


def test_kv_tail_split_cross_with_empty_query_ranges():
    """Cross-attention backward, 2 items x 65 heads x 300 queries over 2048 keys, lengths 2048 and 1500:
    1,040 key blocks of 256 with no query split, so head 64's key blocks run as 8 query ranges over 5 query
    tiles (3 of them empty, zero partials); item 1's keys past 1500 are masked and get zero gradients."""
    B, Lq, Lk, H = 2, 300, 2048, 65
    assert _split_rule(B, Lk, H) == (1024, 16, 8)
    q, do = (synth.random_bf16(9500 + i, (B, Lq, H, 128)) for i in range(2))
    k, v = (synth.random_bf16(9510 + i, (B, Lk, H, 128)) for i in range(2))
    lens = np.array([2048, 1500], dtype=np.int32)
    nan_bits = np.uint16(0x7FC0)
    for b, n in enumerate(lens):                   # padded keys hold NaN: never read
        k[b, n:] = nan_bits
        v[b, n:] = nan_bits
    qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    kl = torch.from_numpy(lens).cuda()
    o, lse = wa.cross_fwd(qd, kd, vd, kl, scale=SCALE)
    dq, dk, dv = wa.cross_bwd(qd, kd, vd, kl, o, lse, dod, scale=SCALE)
    torch.cuda.synchronize()
    gq, gk, gv = bf16_to_f64(dq), bf16_to_f64(dk), bf16_to_f64(dv)
    heads = [64, 7]                                # the split head, and one of the main launch
    f = synth.bf16_bits_to_f64
    rq, rk, rv = oracle.cross_bwd_ref(f(q[:, :, heads]), f(k[:, :, heads]), f(v[:, :, heads]), f(do[:, :, heads]),
                                      lens, SCALE)
    for j, h in enumerate(heads):
        for b, n in enumerate(lens):
            print(f"  head {h}, item {b} (k_len {n}):")
            check_close("dQ", gq[b, :, h], rq[b, :, j])
            check_close("dK", gk[b, :n, h], rk[b, :n, j])
            check_close("dV", gv[b, :n, h], rv[b, :n, j])
            assert np.all(gk[b, n:, h] == 0) and np.all(gv[b, n:, h] == 0), "padded keys got a gradient"
