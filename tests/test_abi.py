"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host with the documented
status codes (validation runs before anything is enqueued, so these calls
never reach the GPU)."""

import ctypes
import os
import re

import pytest

import spatio_temporal_attention_amd as wa
from spatio_temporal_attention_amd import Grid, Rope

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wanattn.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS = 0, 1, 2, 3, 4, 5
P = 0x10000          # a 16-byte-aligned stand-in address; never dereferenced by validation
ODD = 0x10008        # 8-byte aligned only
GRID = Grid(5, 8, 8)
ROPE = Rope(48, 40, 40, 10000.0)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(wa.LIB_PATH):
        from spatio_temporal_attention_amd import build
        build.build()
    return wa.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wanattn_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 20, names
    for n in names:
        assert hasattr(lib, n), f"{n} missing from libwanattn.so"
        assert n in wa._SIGNATURES, f"{n} has no binding"


def test_strerror(lib):
    for code in range(7):
        s = lib.wanattn_strerror(code).decode()
        assert s.startswith("wanattn:")
    assert "unknown" in lib.wanattn_strerror(99).decode()


def test_rope_table_bytes(lib):
    assert lib.wanattn_rope_table_bytes(Grid(21, 45, 80), ROPE) == 8 * (21 * 24 + 45 * 20 + 80 * 20)
    assert lib.wanattn_rope_table_bytes(Grid(64, 64, 64), ROPE) == 8 * 64 * 64
    assert lib.wanattn_rope_table_bytes(Grid(0, 45, 80), ROPE) == 0
    assert lib.wanattn_rope_table_bytes(GRID, Rope(47, 41, 40, 1e4)) == 0
    assert lib.wanattn_rope_table_bytes(GRID, Rope(48, 40, 40, -1.0)) == 0


def test_workspace_sizes(lib):
    B, L, H, D = 1, 75600, 40, 128
    n = B * L * H * D
    tiled = B * H * ((L + 63) // 64) * 64 * D           # elements of K or V in 64-key tiles, zero-padded
    assert tiled > n
    n_tiles = B * H * ((L + 63) // 64)
    # 11,840 query tiles of 256 rows = 46 rounds of 256 + 64: the last 64 and one more round (320 tiles) run
    # as 4 key ranges each, whose fp32 partials (rows of 132 floats) follow the tiles and the main launch's
    # work counter (256 bytes), each on a 256-byte boundary
    part = (64 + 256) * 4 * 256 * 132 * 4
    up = lambda x: (x + 255) // 256 * 256
    assert lib.wanattn_self_fwd_workspace_bytes(B, L, H, D, 0) == up(2 * tiled * 2) + 256 + part
    assert lib.wanattn_self_fwd_workspace_bytes(B, L, H, D, 1) == up(2 * tiled * 2 + 4 * n_tiles) + 256 + part
    # K and V^T tiles (+ exponents), then the counter
    assert lib.wanattn_partial_fwd_workspace_bytes(B, L, H, D, 0) == up(2 * tiled * 2) + 256
    assert lib.wanattn_partial_fwd_workspace_bytes(B, L, H, D, 1) == up(2 * tiled * 2 + 4 * n_tiles) + 256
    assert lib.wanattn_self_fwd_workspace_bytes(1, 1, 1, D, 0) == 2 * 64 * D * 2 + 256
    # a multiple of 256 tiles (32 heads: 9,472 = 37 x 256) still splits its last round; no split below four
    # rounds
    small = B * 32 * ((L + 63) // 64) * 64 * D
    assert lib.wanattn_self_fwd_workspace_bytes(B, L, 32, D, 0) == up(2 * small * 2) + 256 * 4 * 256 * 132 * 4 + 256
    assert lib.wanattn_self_fwd_workspace_bytes(1, 2048, 127, D, 0) == 2 * 127 * 2048 * D * 2 + 256   # 1,016 tiles
    # 1,040 tiles: the last 16 split 8 ways
    assert lib.wanattn_self_fwd_workspace_bytes(1, 2048, 130, D, 0) == 2 * 130 * 2048 * D * 2 + 16 * 8 * 256 * 132 * 4 + 256
    stats = B * H * ((L + 63) // 64) * 1024   # LSE log2 e, -Delta and the exponent, 1 KB per query tile
    exps = (4 * n_tiles + 255) // 256 * 256 + 4 * n_tiles
    # row statistics, 7 tile arrays (Q fp16, (Rq)^T, dO, dO^T, K fp16, (Rk)^T, V), Q and K tile exponents, then the
    # tail splits (the forward's rule over blocks of 256 keys or queries): the dK/dV passes' fp32 partials
    # of dK~ and dV (64 key blocks x 4 query ranges each), then the dQ pass's (64 query blocks x 4 key ranges)
    kv_part, dq_part = 2 * 64 * 4 * 256 * D * 4, 64 * 4 * 256 * D * 4
    assert lib.wanattn_self_bwd_workspace_bytes(B, L, H, D, 1) == up(stats + 7 * tiled * 2 + exps) + kv_part + dq_part
    assert lib.wanattn_self_bwd_workspace_bytes(B, L, H, D, 0) == up(stats + 7 * tiled * 2 + exps) + kv_part + dq_part
    # no tail split: the layout ends with the key tile exponents (32 heads: 37 rounds of 256 blocks)
    t32 = B * 32 * ((L + 63) // 64)
    d32 = t32 * 1024
    assert lib.wanattn_self_bwd_workspace_bytes(B, L, 32, D, 1) == (
        d32 + 7 * small * 2 + (4 * t32 + 255) // 256 * 256 + 4 * t32)
    assert lib.wanattn_self_fwd_workspace_bytes(B, L, H, 64, 1) == 0


def _q_split(B, Lq, Lk, H):
    """Query-range split of the dK/dV passes: none while the key blocks of 256 give >= 256 workgroups; else at
    least two rounds of 256 workgroups, at most 32 ranges of >= 8 query tiles, the fullest last round."""
    blocks = (Lk + 255) // 256 * H * B
    if blocks >= 256:
        return 1
    lo, hi = -(-512 // blocks), max(1, min(32, ((Lq + 63) // 64) // 8))
    if lo >= hi:
        return hi
    fill = lambda s: blocks * s / (256 * -(-(blocks * s) // 256))
    return max(range(lo, hi + 1), key=lambda s: (fill(s), -s))


def test_cross_bwd_workspace_with_query_split(lib):
    B, Lq, Lk, H, D = 1, 75600, 512, 40, 128          # 720p video tokens over 512 text tokens
    assert _q_split(B, Lq, Lk, H) == 16               # 80 key blocks x 16 ranges: 5 full rounds
    assert _q_split(1, 75600, 75600, 40) == 1          # the self-attention backward is not split
    a256 = lambda x: (x + 255) // 256 * 256
    qt, kt = B * H * ((Lq + 63) // 64), B * H * ((Lk + 63) // 64)
    # row statistics (1 KB per query tile), 4 query-side and 3 key-side tile arrays, the two exponent arrays
    base = 1024 * qt + 4 * a256(qt * 64 * D * 2) + 3 * a256(kt * 64 * D * 2) + a256(4 * qt) + 4 * kt
    # then the dK/dV partials of the 16 query ranges (no dK/dV tail split with a query split), then the dQ
    # tail split's (64 query blocks x 4 key ranges)
    assert lib.wanattn_cross_bwd_workspace_bytes(B, Lq, Lk, H, D) == (
        a256(a256(base) + 2 * 16 * B * H * Lk * D * 4) + 64 * 4 * 256 * D * 4)
    # no split: the layout ends with the key tile exponents
    qt, kt = 2 * 2 * 2, 2 * 2 * 8                      # 64-token tiles over B x H
    assert lib.wanattn_cross_bwd_workspace_bytes(2, 100, 512, 2, D) == (
        1024 * qt + 4 * a256(qt * 64 * D * 2) + 3 * a256(kt * 64 * D * 2) + a256(4 * qt) + 4 * kt)


def _fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, L=320, H=2, D=128, g=GRID, r=ROPE, table=P, scale=0.088,
         ws=P, ws_bytes=1 << 30):
    return lib.wanattn_self_fwd(q, k, v, o, lse, B, L, H, D, g, r, table, scale, ws, ws_bytes, None)


def test_self_fwd_validation(lib):
    assert _fwd(lib, q=None) == NULL
    assert _fwd(lib, o=None) == NULL
    assert _fwd(lib, L=0) == SHAPE
    assert _fwd(lib, B=-1) == SHAPE
    assert _fwd(lib, D=64) == UNSUP
    assert _fwd(lib, L=321) == SHAPE                          # f*h*w != L
    assert _fwd(lib, r=Rope(48, 40, 38, 1e4)) == UNSUP         # split does not sum to D
    assert _fwd(lib, r=Rope(47, 41, 40, 1e4)) == UNSUP         # odd width
    assert _fwd(lib, r=Rope(48, 40, 40, 0.0)) == UNSUP         # theta <= 0
    assert _fwd(lib, scale=float("nan")) == UNSUP
    assert _fwd(lib, scale=float("inf")) == UNSUP
    assert _fwd(lib, q=ODD) == ALIGN
    assert _fwd(lib, lse=P + 2) == ALIGN
    assert _fwd(lib, table=ODD) == ALIGN
    assert _fwd(lib, ws=None) == WS
    assert _fwd(lib, ws_bytes=320 * 2 * 128 * 2 - 1) == WS
    assert _fwd(lib, table=None, ws=None) == WS
    need0 = lib.wanattn_self_fwd_workspace_bytes(1, 320, 2, 128, 0)
    assert _fwd(lib, ws_bytes=lib.wanattn_self_fwd_workspace_bytes(1, 320, 2, 128, 1) - 1) == WS
    assert _fwd(lib, table=None, ws_bytes=need0 - 1) == WS
    assert _fwd(lib, table=None, ws=ODD, ws_bytes=need0, q=None) == NULL
    assert _fwd(lib, L=1 << 30, g=Grid(1 << 10, 1 << 10, 1 << 10), H=1 << 14) == SHAPE   # too large


def test_self_bwd_validation(lib):
    def bwd(**kw):
        a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, L=320, H=2, D=128, g=GRID, r=ROPE,
                 table=P, scale=0.088, ws=P, ws_bytes=1 << 30)
        a.update(kw)
        return lib.wanattn_self_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                                    a["B"], a["L"], a["H"], a["D"], a["g"], a["r"], a["table"], a["scale"],
                                    a["ws"], a["ws_bytes"], None)
    assert bwd(lse=None) == NULL
    assert bwd(dv=None) == NULL
    assert bwd(D=256) == UNSUP
    assert bwd(g=Grid(5, 8, 7)) == SHAPE
    assert bwd(dk=ODD) == ALIGN
    assert bwd(ws=None) == WS
    need = lib.wanattn_self_bwd_workspace_bytes(1, 320, 2, 128, 1)
    assert bwd(ws_bytes=need - 1) == WS
    assert bwd(table=None, ws_bytes=lib.wanattn_self_bwd_workspace_bytes(1, 320, 2, 128, 0) - 1) == WS


def test_cross_and_rope_validation(lib):
    def cross(**kw):
        a = dict(q=P, k=P, v=P, kl=P, o=P, lse=P, B=2, Lq=100, Lk=512, H=2, D=128, scale=0.088, ws=P,
                 ws_bytes=1 << 30)
        a.update(kw)
        return lib.wanattn_cross_fwd(a["q"], a["k"], a["v"], a["kl"], a["o"], a["lse"], a["B"], a["Lq"], a["Lk"],
                                     a["H"], a["D"], a["scale"], a["ws"], a["ws_bytes"], None)
    assert cross(v=None) == NULL
    assert cross(Lk=0) == SHAPE
    assert cross(Lq=-5) == SHAPE
    assert cross(D=127) == UNSUP
    assert cross(kl=P + 1) == ALIGN
    assert cross(scale=float("nan")) == UNSUP
    need = lib.wanattn_cross_fwd_workspace_bytes(2, 512, 2, 128)
    assert need == 2 * (2 * 2 * 8 * 64 * 128 * 2) + 256                 # K and V^T tiles, 8 per (b, h); 256 bytes
    assert lib.wanattn_cross_fwd_workspace_bytes(1, 336, 40, 128) == 2 * 40 * 6 * 64 * 128 * 2 + 256
    assert cross(ws=None) == WS
    assert cross(ws_bytes=need - 1) == WS
    assert cross(ws=ODD) == ALIGN

    def rope(**kw):
        a = dict(x=P, y=P, B=1, L=320, H=2, D=128, g=GRID, r=ROPE, table=P, inv=0)
        a.update(kw)
        return lib.wanattn_rope3d(a["x"], a["y"], a["B"], a["L"], a["H"], a["D"], a["g"], a["r"], a["table"],
                                  a["inv"], None)
    assert rope(table=None) == NULL
    assert rope(L=300) == SHAPE
    assert rope(y=ODD) == ALIGN
    assert rope(r=Rope(48, 40, 40, float("inf"))) == UNSUP
    assert lib.wanattn_rope_table_init(None, GRID, ROPE, None) == NULL
    assert lib.wanattn_rope_table_init(P, Grid(0, 1, 1), ROPE, None) == SHAPE
    assert lib.wanattn_rope_table_init(ODD, GRID, ROPE, None) == ALIGN


def test_binding_token_grid_matches_golden():
    import json
    cases = json.load(open(os.path.join(ROOT, "tests", "golden", "token_grids.json")))["cases"]
    for c in cases:
        assert list(wa.token_grid(c["frames"], c["height"], c["width"])) == c["grid"]
    with pytest.raises(ValueError):
        wa.token_grid(80, 480, 832)


def test_varlen_partial_merge_validation(lib):
    """Every call below has at least one invalid argument, so nothing is launched."""
    import ctypes
    lens_ok = P
    def varlen(**kw):
        a = dict(q=P, k=P, v=P, o=P, lse=P, lens=lens_ok, B=1, L=320, H=2, D=128, g=GRID, r=ROPE, table=P,
                 scale=0.088, ws=P, ws_bytes=1 << 30)
        a.update(kw)
        return lib.wanattn_self_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["lens"], a["B"], a["L"], a["H"],
                                           a["D"], a["g"], a["r"], a["table"], a["scale"], a["ws"], a["ws_bytes"], None)
    assert varlen(lens=None) == NULL
    assert varlen(lens=P + 2) == ALIGN
    assert varlen(L=321) == SHAPE
    assert varlen(ws=None) == WS

    def partial(**kw):
        a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Lq=100, Lk=64, H=2, D=128, g=GRID, r=ROPE, table=P, qo=0, ko=0,
                 scale=0.088, ws=P, ws_bytes=1 << 30)
        a.update(kw)
        return lib.wanattn_partial_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Lq"], a["Lk"], a["H"],
                                       a["D"], a["g"], a["r"], a["table"], a["qo"], a["ko"], a["scale"], a["ws"],
                                       a["ws_bytes"], None)
    assert partial(qo=-1) == SHAPE
    assert partial(qo=221) == SHAPE                  # 221 + 100 > 320 grid tokens
    assert partial(ko=257) == SHAPE
    assert partial(Lk=0) == SHAPE
    assert partial(table=ODD) == ALIGN
    assert partial(ws_bytes=lib.wanattn_partial_fwd_workspace_bytes(1, 64, 2, 128, 1) - 1) == WS
    assert partial(v=None) == NULL
    # the same layout: tiles and counter (no split at this size)
    assert lib.wanattn_partial_fwd_workspace_bytes(1, 64, 2, 128, 1) == lib.wanattn_self_fwd_workspace_bytes(
        1, 64, 2, 128, 1)

    def merge(R=2, parts=None, lparts=None, o=P, lse=P, B=1, L=70, H=2):
        arr = ctypes.c_void_p * max(R, 1)
        op = arr(*(parts if parts is not None else [P] * max(R, 1)))
        lp = arr(*(lparts if lparts is not None else [P] * max(R, 1)))
        return lib.wanattn_lse_merge(op, lp, R, o, lse, B, L, H, 128, None)
    assert merge(R=0) == SHAPE
    assert merge(R=17) == SHAPE
    assert merge(parts=[P, None]) == NULL
    assert merge(lparts=[P, P + 2]) == ALIGN
    assert merge(parts=[P, ODD]) == ALIGN
    assert merge(o=None) == NULL
    assert merge(L=0) == SHAPE


def test_cross_bwd_validation(lib):
    """Every call below has at least one invalid argument, so nothing is launched."""
    def cb(**kw):
        a = dict(q=P, k=P, v=P, kl=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=2, Lq=100, Lk=512, H=2, D=128,
                 scale=0.088, ws=P, ws_bytes=1 << 30)
        a.update(kw)
        return lib.wanattn_cross_bwd(a["q"], a["k"], a["v"], a["kl"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                                     a["dv"], a["B"], a["Lq"], a["Lk"], a["H"], a["D"], a["scale"], a["ws"],
                                     a["ws_bytes"], None)
    assert cb(lse=None) == NULL
    assert cb(dk=None) == NULL
    assert cb(Lk=0) == SHAPE
    assert cb(D=64) == UNSUP
    assert cb(kl=P + 2) == ALIGN
    assert cb(dv=ODD) == ALIGN
    assert cb(ws=None) == WS
    need = lib.wanattn_cross_bwd_workspace_bytes(2, 100, 512, 2, 128)
    assert cb(ws_bytes=need - 1) == WS
    # Delta [B, H, Lq] + 4 query-side and 3 key-side tile arrays + the two exponent arrays
    qt, kt = 2 * 2 * 2, 2 * 2 * 8
    assert need == 1024 * qt + 4 * qt * 16384 + 3 * kt * 16384 + 256 + kt * 4


def test_fp8_validation(lib):
    """Every call below has at least one invalid argument, so nothing is launched."""
    def f8(**kw):
        a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, L=320, H=2, D=128, g=GRID, r=ROPE, table=P, scale=0.088, ws=P,
                 ws_bytes=1 << 30)
        a.update(kw)
        return lib.wanattn_self_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["L"], a["H"], a["D"],
                                        a["g"], a["r"], a["table"], a["scale"], a["ws"], a["ws_bytes"], None)
    need = lib.wanattn_self_fwd_fp8_workspace_bytes(1, 320, 2, 128)
    # K and V^T e4m3 tiles, then the two exponent arrays, then the work counter (256 bytes)
    assert need == 2 * 10 * 8192 + 256 + 256 + 256
    assert f8(ws_bytes=need - 1) == WS
    assert f8(ws=None) == WS
    assert f8(q=None) == NULL
    assert f8(L=321) == SHAPE
    assert f8(D=64) == UNSUP
    assert f8(scale=float("inf")) == UNSUP



def test_mfma_peak_argument_checks(lib):
    """The measurement aid validates on the host (no GPU is touched on these paths)."""
    assert lib.wanattn_measure_mfma_peak(None, 512, 10, None) == 1          # NULL sink
    fake = ctypes.c_void_p(0x1000)                                          # never dereferenced: rejected first
    assert lib.wanattn_measure_mfma_peak(fake, 0, 10, None) == 2
    assert lib.wanattn_measure_mfma_peak(fake, 512, 0, None) == 2
    assert lib.wanattn_measure_mfma_peak(fake, (1 << 20) + 1, 10, None) == 2
    assert lib.wanattn_measure_mfma_peak(ctypes.c_void_p(0x1002), 512, 10, None) == 4   # misaligned
