"""GPU parity of the variable-length forward, the sharded (Ring-hop) partial
forward and the exact LSE merge, against the fp64 oracle; same bar as the
other parity tests (max-abs 2e-2, rel-L2 5e-3 on O; |LSE error| 1e-3)."""

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
GRID = (5, 8, 8)          # 320 tokens, 64 per frame


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    wa.lib()


def _inputs(seed, shape):
    return [synth.random_bf16(seed + i, shape) for i in range(3)]


@pytest.mark.parametrize("rope_on", [True, False])
def test_varlen_matches_oracle_and_leaves_padding(rope_on):
    B, L, H = 4, 320, 2
    lens = np.array([320, 128, 64, 201], dtype=np.int32)   # whole frames, one frame, a ragged prefix
    qb, kb, vb = _inputs(500, (B, L, H, 128))
    nan_bits = np.uint16(0x7FC0)
    for b, n in enumerate(lens):                               # padding holds NaN: must never be read
        qb[b, n:] = nan_bits
        kb[b, n:] = nan_bits
        vb[b, n:] = nan_bits
    table = wa.rope_table(GRID, ROPE) if rope_on else None
    o = torch.full((B, L, H, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, L), 5.0, dtype=torch.float32, device="cuda")
    wa.self_fwd_varlen(to_dev(qb), to_dev(kb), to_dev(vb), torch.from_numpy(lens).cuda(), grid=GRID, table=table,
                       rope=ROPE, scale=SCALE, out=o, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.self_fwd_varlen_ref(synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb),
                                        synth.bf16_bits_to_f64(vb), lens, SCALE, GRID, ROPE if rope_on else None)
    go, gl = bf16_to_f64(o), f32_to_np(lse)
    for b, n in enumerate(lens):
        print(f"  item {b} (len {n}):")
        check_close("O", go[b, :n], ro[b, :n])
        check_lse("LSE", gl[b, :, :n], rl[b, :, :n])
        assert np.all(go[b, n:] == 7.0), "rows past the length were written"
        assert np.all(gl[b, :, n:] == 5.0), "LSE past the length was written"


def test_varlen_with_empty_items():
    """Items of length 0 (no key tile, no row) next to a full one: nothing of theirs is written."""
    B, L, H = 3, 320, 2
    lens = np.array([0, 320, 0], dtype=np.int32)
    qb, kb, vb = _inputs(700, (B, L, H, 128))
    table = wa.rope_table(GRID, ROPE)
    o = torch.full((B, L, H, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, L), 5.0, dtype=torch.float32, device="cuda")
    wa.self_fwd_varlen(to_dev(qb), to_dev(kb), to_dev(vb), torch.from_numpy(lens).cuda(), grid=GRID, table=table,
                       rope=ROPE, scale=SCALE, out=o, lse=lse)
    torch.cuda.synchronize()
    ro, rl = oracle.self_fwd_varlen_ref(synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb),
                                        synth.bf16_bits_to_f64(vb), lens, SCALE, GRID, ROPE)
    go, gl = bf16_to_f64(o), f32_to_np(lse)
    check_close("O", go[1], ro[1])
    check_lse("LSE", gl[1], rl[1])
    for b in (0, 2):
        assert np.all(go[b] == 7.0) and np.all(gl[b] == 5.0), f"item {b} (length 0) was written"


@pytest.mark.parametrize("q_off,lq,k_off,lk", [(96, 120, 200, 120), (0, 64, 0, 320), (250, 70, 3, 61)])
def test_partial_fwd_matches_oracle(q_off, lq, k_off, lk):
    H = 2
    full = _inputs(520, (1, 320, H, 128))
    q, k, v = full[0][:, q_off:q_off + lq], full[1][:, k_off:k_off + lk], full[2][:, k_off:k_off + lk]
    table = wa.rope_table(GRID, ROPE)
    o, lse = wa.partial_fwd(to_dev(q), to_dev(k), to_dev(v), q_off, k_off, grid=GRID, table=table, rope=ROPE,
                            scale=SCALE)
    torch.cuda.synchronize()
    ro, rl = oracle.partial_fwd_ref(synth.bf16_bits_to_f64(q), synth.bf16_bits_to_f64(k),
                                    synth.bf16_bits_to_f64(v), SCALE, q_off, k_off, GRID, ROPE)
    check_close("O", bf16_to_f64(o), ro)
    check_lse("LSE", f32_to_np(lse), rl)


def test_ring_shards_merge_to_full_attention():
    """A query shard against 3 key shards (ragged), merged on the GPU, equals the unsharded
    oracle attention; and the merge equals the oracle's merge of the same GPU partials."""
    H = 3
    qb, kb, vb = _inputs(540, (1, 320, H, 128))
    q_off, lq = 64, 160
    cuts = [0, 100, 229, 320]
    table = wa.rope_table(GRID, ROPE)
    qd = to_dev(qb[:, q_off:q_off + lq])
    parts = [wa.partial_fwd(qd, to_dev(kb[:, a:b]), to_dev(vb[:, a:b]), q_off, a, grid=GRID, table=table,
                            rope=ROPE, scale=SCALE) for a, b in zip(cuts[:-1], cuts[1:])]
    o, lse = wa.lse_merge([p[0] for p in parts], [p[1] for p in parts])
    torch.cuda.synchronize()
    rows = np.tile(np.arange(q_off, q_off + lq), (1, H, 1))
    ro, rl = oracle.self_fwd_ref(synth.bf16_bits_to_f64(qb), synth.bf16_bits_to_f64(kb), synth.bf16_bits_to_f64(vb),
                                 SCALE, GRID, ROPE, rows=rows)
    go = bf16_to_f64(o)                                        # [1, lq, H, 128]
    check_close("O vs unsharded", np.transpose(go, (0, 2, 1, 3)), ro)
    check_lse("LSE vs unsharded", f32_to_np(lse), rl)
    mo, ml = oracle.lse_merge_ref([bf16_to_f64(p[0]) for p in parts], [f32_to_np(p[1]) for p in parts])
    check_close("O vs merge of the same partials", go, mo, max_abs=2 ** -7, rel_l2=2 ** -8)
    check_lse("LSE vs merge of the same partials", f32_to_np(lse), ml, tol=1e-5)


def test_merge_empty_parts_and_aliasing():
    rng = np.random.default_rng(7)
    B, L, H = 2, 70, 2
    o1 = torch.from_numpy(rng.standard_normal((B, L, H, 128))).to(torch.bfloat16).cuda()
    o2 = torch.from_numpy(rng.standard_normal((B, L, H, 128))).to(torch.bfloat16).cuda()
    l1 = torch.from_numpy(rng.standard_normal((B, H, L)).astype(np.float32)).cuda()
    l2 = torch.full((B, H, L), -math.inf, device="cuda")
    l2[1] = torch.from_numpy(rng.standard_normal((H, L)).astype(np.float32)).cuda()
    l1[1, 0] = -math.inf                                       # rows of item 1, head 0: only part 2 counts
    l2[1, 0, :5] = -math.inf                                   # ... and 5 of them have no keys at all
    ref_o, ref_l = oracle.lse_merge_ref([bf16_to_f64(o1), bf16_to_f64(o2)], [f32_to_np(l1), f32_to_np(l2)])
    out, lse = wa.lse_merge([o1, o2], [l1, l2], out=o1)        # in place over part 0
    torch.cuda.synchronize()
    check_close("O", bf16_to_f64(out), ref_o, max_abs=2 ** -7, rel_l2=2 ** -8, unit_scale=False)
    check_lse("LSE", f32_to_np(lse), ref_l, tol=1e-5)
    assert np.all(bf16_to_f64(out)[1, :5, 0] == 0) and np.all(f32_to_np(lse)[1, 0, :5] == -np.inf)
