"""The library's host-side argument checks, built without HIP (CPU only).

spatio_temporal_attention_amd/csrc/validate.cpp is plain C++: it is compiled here with g++ together with
tests/host/validate_harness.cpp (C-linkage forwards) into a throwaway shared library, and every rule of
include/wanattn.h's error contract is driven through it: sizes and the grid (WANATTN_ERR_SHAPE), head dim,
rotary split, base and scale (_UNSUPPORTED), NULL pointers (_NULL), alignment (_ALIGN) and workspace size
(_WORKSPACE), plus the tail-split and query-split rules the workspace sizes follow.  The checks never
dereference a pointer, so fake addresses stand in for buffers.
"""

import ctypes
import math
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, UNSUP, ALIGN, WS = 0, 1, 2, 3, 4, 5


class Grid(ctypes.Structure):
    _fields_ = [("f", ctypes.c_int32), ("h", ctypes.c_int32), ("w", ctypes.c_int32)]


class Rope(ctypes.Structure):
    _fields_ = [("d_f", ctypes.c_int32), ("d_h", ctypes.c_int32), ("d_w", ctypes.c_int32), ("theta", ctypes.c_float)]


R = Rope(48, 40, 40, 1e4)
G = Grid(21, 45, 80)
L720, H720 = 75600, 40

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGS = {
    "h_check_dims": (_i, [_i, _i, _i, _i]),
    "h_check_grid_rope": (_i, [Grid, Rope, _i, _i]),
    "h_check_scale": (_i, [_f]),
    "h_rope_table_entries": (ctypes.c_longlong, [Grid, Rope]),
    "h_fwd_tail_split": (None, [_i, _i, _i, ctypes.POINTER(_i)]),
    "h_fwd_split": (None, [_i, _i, _i, ctypes.POINTER(_i)]),
    "h_bwd_q_split": (_i, [_i, _i, _i, _i]),
    "h_self_fwd_ws_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "h_fwd_tiles_ws_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "h_self_bwd_ws_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "h_cross_bwd_ws_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "h_validate_rope3d": (_i, [_vp, _vp, _i, _i, _i, _i, Grid, Rope, _vp]),
    "h_validate_self_fwd": (_i, [_vp] * 5 + [_i] * 4 + [Grid, Rope, _vp, _f, _vp, _sz]),
    "h_validate_self_fwd_varlen": (_i, [_vp] * 6 + [_i] * 4 + [Grid, Rope, _vp, _f, _vp, _sz]),
    "h_validate_partial_fwd": (_i, [_vp] * 5 + [_i] * 5 + [Grid, Rope, _vp, _i, _i, _f, _vp, _sz]),
    "h_validate_lse_merge": (_i, [ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i, _vp, _vp, _i, _i, _i, _i]),
    "h_validate_self_bwd": (_i, [_vp] * 9 + [_i] * 4 + [Grid, Rope, _vp, _f, _vp, _sz]),
    "h_validate_cross_bwd": (_i, [_vp] * 10 + [_i] * 5 + [_f, _vp, _sz]),
    "h_validate_cross_fwd": (_i, [_vp] * 6 + [_i] * 5 + [_f, _vp, _sz]),
}


@pytest.fixture(scope="module")
def h(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("validate_host") / "libvalidate_host.so")
    cmd = [gxx, "-std=c++17", "-O1", "-Wall", "-Werror", "-shared", "-fPIC",
           os.path.join(ROOT, "tests", "host", "validate_harness.cpp"),
           os.path.join(ROOT, "spatio_temporal_attention_amd", "csrc", "validate.cpp"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    lib = ctypes.CDLL(out)
    for name, (res, args) in SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def buf(i, misalign=0):
    """A fake, never dereferenced device address: 16-byte aligned unless misalign != 0."""
    return ctypes.c_void_p(0x10000000 + 0x100000 * i + misalign)


def test_built_without_hip(h):
    # the harness library links against no HIP runtime
    deps = subprocess.run(["ldd", h._name], capture_output=True, text=True).stdout
    assert "amdhip" not in deps and "hsa" not in deps


def test_dims(h):
    assert h.h_check_dims(1, L720, H720, 128) == OK
    for B, L, H in ((0, 1, 1), (1, 0, 1), (1, 1, 0), (-1, 5, 5)):
        assert h.h_check_dims(B, L, H, 128) == SHAPE
    assert h.h_check_dims(1, 64, 1, 64) == UNSUP                    # head dim must be 128
    assert h.h_check_dims(1, 1 << 30, 16, 128) == SHAPE             # 2^41 elements > 2^40
    assert h.h_check_dims(1, 1 << 30, 8, 128) == OK                 # 2^40 exactly


def test_grid_rope_and_scale(h):
    assert h.h_check_grid_rope(G, R, L720, 128) == OK
    assert h.h_check_grid_rope(G, R, L720 - 1, 128) == SHAPE        # f*h*w != L
    assert h.h_check_grid_rope(Grid(0, 45, 80), R, 0, 128) == SHAPE
    for bad in (Rope(47, 41, 40, 1e4), Rope(48, 40, 42, 1e4), Rope(-2, 90, 40, 1e4), Rope(48, 40, 40, 0.0),
                Rope(48, 40, 40, -1.0), Rope(48, 40, 40, math.inf), Rope(48, 40, 40, math.nan)):
        assert h.h_check_grid_rope(G, bad, L720, 128) == UNSUP, (bad.d_f, bad.d_h, bad.d_w, bad.theta)
    assert h.h_check_grid_rope(Grid(5, 1, 1), Rope(128, 0, 0, 1e4), 5, 128) == OK   # zero-width segments
    assert h.h_check_scale(0.0) == OK and h.h_check_scale(-3.0) == OK
    assert h.h_check_scale(math.nan) == UNSUP and h.h_check_scale(math.inf) == UNSUP
    assert h.h_rope_table_entries(G, R) == 21 * 24 + 45 * 20 + 80 * 20
    assert h.h_rope_table_entries(Grid(64, 64, 64), R) == 64 * 64
    assert h.h_rope_table_entries(G, Rope(47, 41, 40, 1e4)) == -1


def test_split_rules(h):
    out = (_i * 4)()
    h.h_fwd_tail_split(1, L720, H720, out)
    assert list(out) == [11840, 11776, 64, 4]                       # 46 rounds + 64: 4 key ranges each
    h.h_fwd_tail_split(1, 2048, 127, out)
    assert list(out) == [1016, 1016, 0, 1]                          # under four rounds: no split
    h.h_fwd_tail_split(1, 2048, 128, out)
    assert list(out) == [1024, 1024, 0, 1]                          # a whole number of rounds
    h.h_fwd_tail_split(1, 256 * 200, 6, out)
    assert list(out) == [1200, 1200, 0, 1]                          # tail 176: S = 1 < 2, no split
    h.h_fwd_tail_split(1, 2048, 130, out)
    assert list(out) == [1040, 1024, 16, 8]                         # S capped at 8
    # the forward's own split: from eight rounds on, one more round of tiles as 4 key ranges each
    h.h_fwd_split(1, L720, H720, out)
    assert list(out) == [11840, 11520, 320, 4]
    h.h_fwd_split(1, L720, 32, out)
    assert list(out) == [9472, 9216, 256, 4]                        # a whole number of rounds: the last one
    h.h_fwd_split(1, 2048, 255, out)
    assert list(out) == [2040, 2040, 0, 1]                          # under eight rounds: fwd_tail_split's rule
    h.h_fwd_split(1, 2048, 130, out)
    assert list(out) == [1040, 1024, 16, 8]
    h.h_fwd_split(1, 2048, 256, out)
    assert list(out) == [2048, 1792, 256, 4]                        # eight rounds exactly
    assert h.h_bwd_q_split(1, L720, L720, H720) == 1                # 11,840 key blocks fill the chip
    assert h.h_bwd_q_split(1, L720, 512, H720) == 16                # 80 key blocks: 1,280 workgroups, 5 full rounds
    assert h.h_bwd_q_split(2, 32760, 512, 12) == 16                 # 48 key blocks: 768 workgroups, 3 full rounds
    assert h.h_bwd_q_split(1, 512, 512, 1) == 1                     # each split needs >= 8 query tiles


def test_workspace_sizes(h):
    up = lambda x: (x + 255) // 256 * 256
    tiles = 40 * ((L720 + 63) // 64)
    tile_bytes = tiles * 64 * 128 * 2
    part = (64 + 256) * 4 * 256 * 132 * 4   # the forward's split: the last 64 tiles and one more round
    # the tiles (+ exponents), the work counter (256 bytes), then the split's partials
    assert h.h_self_fwd_ws_bytes(1, L720, H720, 128, 1) == up(up(2 * tile_bytes) + 4 * tiles) + 256 + part
    assert h.h_self_fwd_ws_bytes(1, L720, H720, 128, 0) == up(2 * tile_bytes) + 256 + part
    assert h.h_fwd_tiles_ws_bytes(1, L720, H720, 128, 1) == up(up(2 * tile_bytes) + 4 * tiles) + 256
    assert h.h_self_fwd_ws_bytes(1, L720, H720, 64, 1) == 0         # invalid shapes size to 0
    assert h.h_self_bwd_ws_bytes(1, L720, H720, 128, 1) == h.h_cross_bwd_ws_bytes(1, L720, L720, H720, 128)
    assert h.h_cross_bwd_ws_bytes(1, L720, 512, H720, 128) > h.h_cross_bwd_ws_bytes(1, 256, 512, H720, 128)


def _self_fwd_args(**over):
    a = dict(q=buf(1), k=buf(2), v=buf(3), o=buf(4), lse=buf(5), B=1, L=320, H=2, D=128, g=Grid(5, 8, 8), r=R,
             table=buf(6), scale=0.088, ws=buf(7), ws_bytes=1 << 30)
    a.update(over)
    return list(a.values())


def test_validate_self_fwd(h):
    f = h.h_validate_self_fwd
    assert f(*_self_fwd_args()) == OK
    for i, name in enumerate(("q", "k", "v", "o")):
        assert f(*_self_fwd_args(**{name: None})) == NULL
        assert f(*_self_fwd_args(**{name: buf(1 + i, 8)})) == ALIGN          # bf16 buffers: 16 bytes
    assert f(*_self_fwd_args(lse=None)) == OK                                 # lse is optional
    assert f(*_self_fwd_args(lse=buf(5, 4))) == OK                            # fp32: 4 bytes
    assert f(*_self_fwd_args(lse=buf(5, 2))) == ALIGN
    assert f(*_self_fwd_args(table=buf(6, 8))) == ALIGN
    assert f(*_self_fwd_args(g=Grid(5, 8, 9))) == SHAPE                       # grid checked with a table
    assert f(*_self_fwd_args(g=Grid(5, 8, 9), table=None)) == OK              # and ignored without one
    assert f(*_self_fwd_args(r=Rope(48, 40, 41, 1e4))) == UNSUP
    assert f(*_self_fwd_args(scale=math.nan)) == UNSUP
    assert f(*_self_fwd_args(D=96)) == UNSUP
    assert f(*_self_fwd_args(L=0)) == SHAPE
    need = h.h_self_fwd_ws_bytes(1, 320, 2, 128, 1)
    assert f(*_self_fwd_args(ws_bytes=need)) == OK
    assert f(*_self_fwd_args(ws_bytes=need - 1)) == WS
    assert f(*_self_fwd_args(ws=None)) == WS
    assert f(*_self_fwd_args(ws=buf(7, 8))) == ALIGN
    # the varlen call adds its lengths array
    args = _self_fwd_args()
    assert h.h_validate_self_fwd_varlen(*args[:5], buf(8), *args[5:]) == OK
    assert h.h_validate_self_fwd_varlen(*args[:5], None, *args[5:]) == NULL
    assert h.h_validate_self_fwd_varlen(*args[:5], buf(8, 2), *args[5:]) == ALIGN


def test_validate_rope3d(h):
    f = h.h_validate_rope3d
    assert f(buf(1), buf(2), 1, 320, 2, 128, Grid(5, 8, 8), R, buf(3)) == OK
    assert f(buf(1), buf(1), 1, 320, 2, 128, Grid(5, 8, 8), R, buf(3)) == OK      # in place
    assert f(buf(1), buf(2), 1, 320, 2, 128, Grid(5, 8, 8), R, None) == NULL       # a table is required
    assert f(buf(1), buf(2), 1, 321, 2, 128, Grid(5, 8, 8), R, buf(3)) == SHAPE
    assert f(buf(1, 8), buf(2), 1, 320, 2, 128, Grid(5, 8, 8), R, buf(3)) == ALIGN


def test_validate_partial_and_merge(h):
    f = h.h_validate_partial_fwd
    g = Grid(64, 64, 64)
    ws = h.h_fwd_tiles_ws_bytes(1, 4096, 2, 128, 1)
    base = [buf(1), buf(2), buf(3), buf(4), buf(5), 1, 4096, 4096, 2, 128, g, R, buf(6)]
    assert f(*base, 0, 4096, 0.088, buf(7), ws) == OK
    assert f(*base, -1, 0, 0.088, buf(7), ws) == SHAPE
    assert f(*base, 0, 262144 - 4095, 0.088, buf(7), ws) == SHAPE                  # key shard past the grid
    assert f(*base, 262144 - 4096, 0, 0.088, buf(7), ws) == OK
    assert f(*base, 0, 0, 0.088, buf(7), ws - 1) == WS
    o_parts = (_vp * 2)(buf(10).value, buf(11).value)
    l_parts = (_vp * 2)(buf(12).value, buf(13).value)
    m = h.h_validate_lse_merge
    assert m(o_parts, l_parts, 2, buf(14), buf(15), 1, 100, 2, 128) == OK
    assert m(o_parts, l_parts, 0, buf(14), buf(15), 1, 100, 2, 128) == SHAPE
    assert m(o_parts, l_parts, 17, buf(14), buf(15), 1, 100, 2, 128) == SHAPE
    bad = (_vp * 2)(buf(10).value, None)
    assert m(o_parts, bad, 2, buf(14), buf(15), 1, 100, 2, 128) == NULL
    mis = (_vp * 2)(buf(10).value, buf(11, 8).value)
    assert m(mis, l_parts, 2, buf(14), buf(15), 1, 100, 2, 128) == ALIGN


def test_validate_backward_and_cross(h):
    f = h.h_validate_self_bwd
    ws = h.h_self_bwd_ws_bytes(1, 320, 2, 128, 1)
    ptrs = [buf(i) for i in range(1, 10)]
    tail = [1, 320, 2, 128, Grid(5, 8, 8), R, buf(11), 0.088]
    assert f(*ptrs, *tail, buf(12), ws) == OK
    for i in range(9):
        p = list(ptrs)
        p[i] = None
        assert f(*p, *tail, buf(12), ws) == NULL                                   # lse is required here
    assert f(*ptrs, *tail, buf(12), ws - 1) == WS
    c = h.h_validate_cross_bwd
    cws = h.h_cross_bwd_ws_bytes(2, 1000, 512, 3, 128)
    cptr = [buf(1), buf(2), buf(3), buf(4), buf(5), buf(6), buf(7), buf(8), buf(9), buf(10)]
    assert c(*cptr, 2, 1000, 512, 3, 128, 0.088, buf(11), cws) == OK
    cptr_nolens = list(cptr)
    cptr_nolens[3] = None                                                          # k_lens optional
    assert c(*cptr_nolens, 2, 1000, 512, 3, 128, 0.088, buf(11), cws) == OK
    cptr_mis = list(cptr)
    cptr_mis[3] = buf(4, 2)
    assert c(*cptr_mis, 2, 1000, 512, 3, 128, 0.088, buf(11), cws) == ALIGN
    assert c(*cptr, 2, 1000, 0, 3, 128, 0.088, buf(11), cws) == SHAPE
    assert c(*cptr, 2, 1000, 512, 3, 128, 0.088, buf(11), cws - 1) == WS
    x = h.h_validate_cross_fwd
    xws = h.h_fwd_tiles_ws_bytes(2, 512, 12, 128, 0)
    w = (buf(7), xws)
    assert x(buf(1), buf(2), buf(3), buf(4), buf(5), buf(6), 2, 32760, 512, 12, 128, 0.088, *w) == OK
    assert x(buf(1), buf(2), buf(3), None, buf(5), None, 2, 32760, 512, 12, 128, 0.088, *w) == OK
    assert x(buf(1), buf(2), buf(3), buf(4), buf(5), buf(6), 2, 32760, 0, 12, 128, 0.088, *w) == SHAPE
    assert x(buf(1), None, buf(3), buf(4), buf(5), buf(6), 2, 32760, 512, 12, 128, 0.088, *w) == NULL
    assert x(buf(1), buf(2), buf(3), buf(4, 1), buf(5), buf(6), 2, 32760, 512, 12, 128, 0.088, *w) == ALIGN
    assert x(buf(1), buf(2), buf(3), buf(4), buf(5), buf(6), 2, 32760, 512, 12, 128, math.inf, *w) == UNSUP
    assert x(buf(1), buf(2), buf(3), buf(4), buf(5), buf(6), 2, 32760, 512, 12, 128, 0.088, None, xws) == WS
    assert x(buf(1), buf(2), buf(3), buf(4), buf(5), buf(6), 2, 32760, 512, 12, 128, 0.088, buf(7), xws - 1) == WS
    assert x(buf(1), buf(2), buf(3), buf(4), buf(5), buf(6), 2, 32760, 512, 12, 128, 0.088, buf(7, 8), xws) == ALIGN
