"""wanattn: spatio-temporal attention with 3D RoPE for Wan-style video DiTs on MI355X.

A thin ctypes binding over libwanattn.so (see include/wanattn.h).  It only
marshals arguments: shapes and dtypes are checked, device pointers and the
current HIP stream are passed through, and every step of the computation runs
in the library's HIP kernels.  PyTorch supplies device memory and streams.

If the compiled library is missing, every call raises RuntimeError; there is
no fallback implementation.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import NamedTuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwanattn.so")
HEAD_DIM = 128

STATUS = {
    0: "WANATTN_OK",
    1: "WANATTN_ERR_NULL",
    2: "WANATTN_ERR_SHAPE",
    3: "WANATTN_ERR_UNSUPPORTED",
    4: "WANATTN_ERR_ALIGN",
    5: "WANATTN_ERR_WORKSPACE",
    6: "WANATTN_ERR_HIP",
}


class Grid(ctypes.Structure):
    """Post-patchify token grid (frames, rows, columns)."""
    _fields_ = [("f", ctypes.c_int32), ("h", ctypes.c_int32), ("w", ctypes.c_int32)]


class Rope(ctypes.Structure):
    """Head-dim split (time, height, width) and rotary base."""
    _fields_ = [("d_f", ctypes.c_int32), ("d_h", ctypes.c_int32), ("d_w", ctypes.c_int32),
                ("theta", ctypes.c_float)]


class RopeConfig(NamedTuple):
    d_f: int = 48
    d_h: int = 40
    d_w: int = 40
    theta: float = 10000.0


DEFAULT_ROPE = RopeConfig()

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

_SIGNATURES = {
    "wanattn_strerror": (ctypes.c_char_p, [_i]),
    "wanattn_rope_table_bytes": (_sz, [Grid, Rope]),
    "wanattn_rope_table_init": (_i, [_vp, Grid, Rope, _vp]),
    "wanattn_rope3d": (_i, [_vp, _vp, _i, _i, _i, _i, Grid, Rope, _vp, _i, _vp]),
    "wanattn_self_fwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "wanattn_self_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, Grid, Rope, _vp, _f, _vp, _sz, _vp]),
    "wanattn_self_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "wanattn_self_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, Grid, Rope, _vp, _f,
                              _vp, _sz, _vp]),
    "wanattn_cross_fwd_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "wanattn_cross_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp]),
    "wanattn_self_fwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, Grid, Rope, _vp, _f, _vp, _sz,
                                     _vp]),
    "wanattn_partial_fwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "wanattn_partial_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, Grid, Rope, _vp, _i, _i, _f, _vp, _sz,
                                 _vp]),
    "wanattn_lse_merge": (_i, [ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i, _vp, _vp, _i, _i, _i, _i, _vp]),
    "wanattn_self_fwd_fp8_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "wanattn_self_fwd_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, Grid, Rope, _vp, _f, _vp, _sz, _vp]),
    "wanattn_cross_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "wanattn_cross_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _sz,
                               _vp]),
    "wanattn_measure_mfma_peak": (_i, [_vp, _i, _i, _vp]),
    "wanattn_self_fwd_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, Grid, Rope, _vp, _f, _vp]),
}

_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded libwanattn (raises RuntimeError if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m spatio_temporal_attention_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


class WanattnError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {lib().wanattn_strerror(status).decode()}")


def _check(rc: int):
    if rc != 0:
        raise WanattnError(rc)


def token_grid(frames: int, height: int, width: int) -> tuple:
    """Post-patchify token grid of a clip: latent [1+T/4, H/8, W/8] for 1+T frames, then a (1,2,2) patch."""
    if frames < 1 or (frames - 1) % 4 or height % 16 or width % 16:
        raise ValueError("need 1 + 4k frames and a height and width divisible by 16")
    return (1 + (frames - 1) // 4, height // 16, width // 16)


def _grid(grid) -> Grid:
    return Grid(*(int(x) for x in grid))


def _rope(rope) -> Rope:
    r = DEFAULT_ROPE if rope is None else rope
    return Rope(int(r[0]), int(r[1]), int(r[2]), float(r[3]))


# ---------------------------------------------------------------------------
# torch-facing wrappers (torch is imported lazily so the module loads without it)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(device) -> ctypes.c_void_p:
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, dtype, name, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def rope_table_bytes(grid, rope=None) -> int:
    return int(lib().wanattn_rope_table_bytes(_grid(grid), _rope(rope)))


def rope_table(grid, rope=None, device="cuda"):
    """fp32 (cos, sin) table for `grid` (layout documented in include/wanattn.h)."""
    torch = _torch()
    n = rope_table_bytes(grid, rope)
    if n == 0:
        raise ValueError("invalid grid or rotary split")
    table = torch.empty(n // 4, dtype=torch.float32, device=device)
    _check(lib().wanattn_rope_table_init(_ptr(table), _grid(grid), _rope(rope), _stream(table.device)))
    return table


def rope3d(x, grid, table, rope=None, inverse=False, out=None):
    """3D RoPE of a [B, L, H, 128] bf16 tensor (out may be x for in place)."""
    torch = _torch()
    _need(x, torch.bfloat16, "x")
    B, L, H, D = x.shape
    y = torch.empty_like(x) if out is None else out
    _need(y, torch.bfloat16, "out", x.shape)
    _need(table, torch.float32, "table")
    _check(lib().wanattn_rope3d(_ptr(x), _ptr(y), B, L, H, D, _grid(grid), _rope(rope), _ptr(table),
                                1 if inverse else 0, _stream(x.device)))
    return y


def self_fwd_workspace_bytes(B, L, H, D=HEAD_DIM, with_rope=True) -> int:
    return int(lib().wanattn_self_fwd_workspace_bytes(B, L, H, D, 1 if with_rope else 0))


def self_bwd_workspace_bytes(B, L, H, D=HEAD_DIM, with_rope=True) -> int:
    return int(lib().wanattn_self_bwd_workspace_bytes(B, L, H, D, 1 if with_rope else 0))


def _workspace(nbytes, device, given):
    torch = _torch()
    if nbytes == 0:
        return None
    if given is not None:
        return given
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def self_fwd(q, k, v, grid=None, table=None, rope=None, scale=None, out=None, lse=None, workspace=None,
             want_lse=True):
    """Full self-attention forward with optional 3D RoPE.  Returns (o, lse)."""
    torch = _torch()
    _need(q, torch.bfloat16, "q")
    B, L, H, D = q.shape
    _need(k, torch.bfloat16, "k", q.shape)
    _need(v, torch.bfloat16, "v", q.shape)
    if table is not None:
        _need(table, torch.float32, "table")
    o = torch.empty_like(q) if out is None else out
    _need(o, torch.bfloat16, "out", q.shape)
    if lse is None and want_lse:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, torch.float32, "lse", (B, H, L))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    nbytes = self_fwd_workspace_bytes(B, L, H, D, table is not None)
    ws = _workspace(nbytes, q.device, workspace)
    g = _grid(grid if grid is not None else (1, 1, L))
    _check(lib().wanattn_self_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, L, H, D, g, _rope(rope),
                                  _ptr(table), scale, _ptr(ws), nbytes if ws is None else ws.numel(),
                                  _stream(q.device)))
    return o, lse


def self_fwd_noalloc(q, k, v, out, lse=None, grid=None, table=None, rope=None, scale=None):
    """wanattn_self_fwd without a workspace (the library's static scratch instead): the caller passes the
    output `out` and optionally `lse`; nothing is allocated here or in the call.  Returns (out, lse)."""
    torch = _torch()
    _need(q, torch.bfloat16, "q")
    B, L, H, D = q.shape
    _need(k, torch.bfloat16, "k", q.shape)
    _need(v, torch.bfloat16, "v", q.shape)
    _need(out, torch.bfloat16, "out", q.shape)
    if lse is not None:
        _need(lse, torch.float32, "lse", (B, H, L))
    if table is not None:
        _need(table, torch.float32, "table")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    g = _grid(grid if grid is not None else (1, 1, L))
    _check(lib().wanattn_self_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, L, H, D, g,
                                          _rope(rope), _ptr(table), scale, _stream(q.device)))
    return out, lse


def self_bwd(q, k, v, o, lse, dout, grid=None, table=None, rope=None, scale=None, workspace=None,
             dq=None, dk=None, dv=None):
    """Self-attention backward.  Returns (dq, dk, dv) w.r.t. the unrotated q and k."""
    torch = _torch()
    _need(q, torch.bfloat16, "q")
    B, L, H, D = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _need(t, torch.bfloat16, name, q.shape)
    _need(lse, torch.float32, "lse", (B, H, L))
    if table is not None:
        _need(table, torch.float32, "table")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _need(t, torch.bfloat16, name, q.shape)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    nbytes = self_bwd_workspace_bytes(B, L, H, D, table is not None)
    ws = _workspace(nbytes, q.device, workspace)
    g = _grid(grid if grid is not None else (1, 1, L))
    _check(lib().wanattn_self_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                                  _ptr(dv), B, L, H, D, g, _rope(rope), _ptr(table), scale, _ptr(ws),
                                  ws.numel(), _stream(q.device)))
    return dq, dk, dv


def cross_fwd_workspace_bytes(B, Lk, H, D=HEAD_DIM) -> int:
    return int(lib().wanattn_cross_fwd_workspace_bytes(B, Lk, H, D))


def cross_fwd(q, k, v, k_lens=None, scale=None, out=None, lse=None, want_lse=True, workspace=None):
    """Cross-attention forward over key-padded text tokens.  Returns (o, lse)."""
    torch = _torch()
    _need(q, torch.bfloat16, "q")
    B, Lq, H, D = q.shape
    _need(k, torch.bfloat16, "k")
    Lk = k.shape[1]
    _need(k, torch.bfloat16, "k", (B, Lk, H, D))
    _need(v, torch.bfloat16, "v", (B, Lk, H, D))
    if k_lens is not None:
        _need(k_lens, torch.int32, "k_lens", (B,))
    o = torch.empty_like(q) if out is None else out
    _need(o, torch.bfloat16, "out", q.shape)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, torch.float32, "lse", (B, H, Lq))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    nbytes = cross_fwd_workspace_bytes(B, Lk, H, D)
    ws = _workspace(nbytes, q.device, workspace)
    _check(lib().wanattn_cross_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(k_lens), _ptr(o), _ptr(lse), B, Lq, Lk, H, D,
                                   scale, _ptr(ws), nbytes if ws is None else ws.numel(), _stream(q.device)))
    return o, lse


def self_fwd_varlen(q, k, v, seq_lens, grid=None, table=None, rope=None, scale=None, out=None, lse=None,
                    workspace=None, want_lse=True):
    """Self-attention forward where item b uses only its first seq_lens[b] tokens.  Returns (o, lse);
    rows past an item's length are left as they were in `out` / `lse`."""
    torch = _torch()
    _need(q, torch.bfloat16, "q")
    B, L, H, D = q.shape
    _need(k, torch.bfloat16, "k", q.shape)
    _need(v, torch.bfloat16, "v", q.shape)
    _need(seq_lens, torch.int32, "seq_lens", (B,))
    if table is not None:
        _need(table, torch.float32, "table")
    o = torch.zeros_like(q) if out is None else out
    _need(o, torch.bfloat16, "out", q.shape)
    if lse is None and want_lse:
        lse = torch.zeros((B, H, L), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, torch.float32, "lse", (B, H, L))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    nbytes = self_fwd_workspace_bytes(B, L, H, D, table is not None)
    ws = _workspace(nbytes, q.device, workspace)
    g = _grid(grid if grid is not None else (1, 1, L))
    _check(lib().wanattn_self_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(seq_lens), B, L, H, D,
                                         g, _rope(rope), _ptr(table), scale, _ptr(ws),
                                         nbytes if ws is None else ws.numel(), _stream(q.device)))
    return o, lse


def partial_fwd_workspace_bytes(B, Lk, H, D=HEAD_DIM, with_rope=True) -> int:
    return int(lib().wanattn_partial_fwd_workspace_bytes(B, Lk, H, D, 1 if with_rope else 0))


def partial_fwd(q, k, v, q_offset, k_offset, grid=None, table=None, rope=None, scale=None, out=None, lse=None,
                workspace=None):
    """Attention of a query shard (global tokens q_offset ...) over a key/value shard (k_offset ...) of one
    sequence on token grid `grid`.  Returns (o, lse), the partial result for wanattn_lse_merge."""
    torch = _torch()
    _need(q, torch.bfloat16, "q")
    B, Lq, H, D = q.shape
    _need(k, torch.bfloat16, "k")
    Lk = k.shape[1]
    _need(k, torch.bfloat16, "k", (B, Lk, H, D))
    _need(v, torch.bfloat16, "v", (B, Lk, H, D))
    if table is not None:
        _need(table, torch.float32, "table")
    o = torch.empty_like(q) if out is None else out
    _need(o, torch.bfloat16, "out", q.shape)
    lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(lse, torch.float32, "lse", (B, H, Lq))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    nbytes = partial_fwd_workspace_bytes(B, Lk, H, D, table is not None)
    ws = _workspace(nbytes, q.device, workspace)
    g = _grid(grid if grid is not None else (1, 1, max(q_offset + Lq, k_offset + Lk)))
    _check(lib().wanattn_partial_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Lq, Lk, H, D, g, _rope(rope),
                                     _ptr(table), int(q_offset), int(k_offset), scale, _ptr(ws),
                                     nbytes if ws is None else ws.numel(), _stream(q.device)))
    return o, lse


def lse_merge(o_parts, lse_parts, out=None, lse=None, want_lse=True):
    """Exact merge of partial (O_r, LSE_r) over disjoint key sets.  Returns (o, lse)."""
    torch = _torch()
    R = len(o_parts)
    if R != len(lse_parts) or not 1 <= R <= 16:
        raise ValueError("need 1..16 matching partial outputs and LSEs")
    B, L, H, D = o_parts[0].shape
    for t in o_parts:
        _need(t, torch.bfloat16, "o_parts[r]", (B, L, H, D))
    for t in lse_parts:
        _need(t, torch.float32, "lse_parts[r]", (B, H, L))
    o = torch.empty_like(o_parts[0]) if out is None else out
    _need(o, torch.bfloat16, "out", (B, L, H, D))
    if lse is None and want_lse:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=o.device)
    if lse is not None:
        _need(lse, torch.float32, "lse", (B, H, L))
    optrs = (_vp * R)(*[t.data_ptr() for t in o_parts])
    lptrs = (_vp * R)(*[t.data_ptr() for t in lse_parts])
    _check(lib().wanattn_lse_merge(optrs, lptrs, R, _ptr(o), _ptr(lse), B, L, H, D, _stream(o.device)))
    return o, lse


def cross_bwd_workspace_bytes(B, Lq, Lk, H, D=HEAD_DIM) -> int:
    return int(lib().wanattn_cross_bwd_workspace_bytes(B, Lq, Lk, H, D))


def cross_bwd(q, k, v, k_lens, o, lse, dout, scale=None, workspace=None, dq=None, dk=None, dv=None):
    """Cross-attention backward (key padding by k_lens).  Returns (dq, dk, dv)."""
    torch = _torch()
    _need(q, torch.bfloat16, "q")
    B, Lq, H, D = q.shape
    _need(k, torch.bfloat16, "k")
    Lk = k.shape[1]
    _need(k, torch.bfloat16, "k", (B, Lk, H, D))
    _need(v, torch.bfloat16, "v", (B, Lk, H, D))
    if k_lens is not None:
        _need(k_lens, torch.int32, "k_lens", (B,))
    _need(o, torch.bfloat16, "o", q.shape)
    _need(dout, torch.bfloat16, "dout", q.shape)
    _need(lse, torch.float32, "lse", (B, H, Lq))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, torch.bfloat16, "dq", q.shape)
    _need(dk, torch.bfloat16, "dk", k.shape)
    _need(dv, torch.bfloat16, "dv", v.shape)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    nbytes = cross_bwd_workspace_bytes(B, Lq, Lk, H, D)
    ws = _workspace(nbytes, q.device, workspace)
    _check(lib().wanattn_cross_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(k_lens), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                   _ptr(dk), _ptr(dv), B, Lq, Lk, H, D, scale, _ptr(ws),
                                   nbytes if ws is None else ws.numel(), _stream(q.device)))
    return dq, dk, dv


def self_fwd_fp8_workspace_bytes(B, L, H, D=HEAD_DIM) -> int:
    return int(lib().wanattn_self_fwd_fp8_workspace_bytes(B, L, H, D))


def self_fwd_fp8(q, k, v, grid=None, table=None, rope=None, scale=None, out=None, lse=None, workspace=None,
                 want_lse=True):
    """FP8 (e4m3) self-attention forward with optional 3D RoPE.  Returns (o, lse)."""
    torch = _torch()
    _need(q, torch.bfloat16, "q")
    B, L, H, D = q.shape
    _need(k, torch.bfloat16, "k", q.shape)
    _need(v, torch.bfloat16, "v", q.shape)
    if table is not None:
        _need(table, torch.float32, "table")
    o = torch.empty_like(q) if out is None else out
    _need(o, torch.bfloat16, "out", q.shape)
    if lse is None and want_lse:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, torch.float32, "lse", (B, H, L))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    nbytes = self_fwd_fp8_workspace_bytes(B, L, H, D)
    ws = _workspace(nbytes, q.device, workspace)
    g = _grid(grid if grid is not None else (1, 1, L))
    _check(lib().wanattn_self_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, L, H, D, g, _rope(rope),
                                      _ptr(table), scale, _ptr(ws), nbytes if ws is None else ws.numel(),
                                      _stream(q.device)))
    return o, lse



MFMA_PEAK_WAVES_PER_WG = 4
MFMA_PEAK_FLOP_PER_WAVE_ITER = 4 * 2 * 32 * 32 * 16   # four 32x32x16 MFMAs per wave and iteration


def measure_mfma_peak(workgroups: int, iters: int, sink=None):
    """Enqueue the library's bf16 MFMA loop (a measurement aid) on the current stream and return its
    algorithmic flop count; time it with events on that stream."""
    torch = _torch()
    sink = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda") if sink is None else sink
    _need(sink, torch.float32, "sink", (workgroups * 256,))
    _check(lib().wanattn_measure_mfma_peak(_ptr(sink), int(workgroups), int(iters), _stream(sink.device)))
    return float(workgroups) * MFMA_PEAK_WAVES_PER_WG * iters * MFMA_PEAK_FLOP_PER_WAVE_ITER
