"""Seeded synthetic inputs for the Wan-shaped attention workloads.

This module draws random tensors and nothing else: it holds none of the
attention or rotary arithmetic, so both the fp64 CPU oracle and the HIP path
can be fed from it without sharing any of the method's code.

Workloads (shapes follow the Wan2.1 reading notes, "2. Model Design": a video of
1+T frames becomes a latent grid [1+T/4, H/8, W/8], and the (1,2,2) patch turns
that into (1+T/4) * H/16 * W/16 tokens; head dim 128 follows from the config
table, 1536/12 = 5120/40; text context is 512 umT5 tokens):

  1 tiny   grid 5x8x8      L=320     B=1 H=2   self-attention, forward (+ backward in tests)
  2 480p   grid 21x30x52   L=32760   B=1 H=12  self-attention forward
  3 cross  Lq=32760 Lk=512           B=2 H=12  text cross-attention, valid lengths U[20,512]
  4 720p   grid 21x45x80   L=75600   B=1 H=40  self-attention forward + backward
  5 long   grid 64x64x64   L=262144  B=1 H=40  self-attention forward

Every value is standard normal, drawn in fp32 and rounded to bf16 with
round-to-nearest-even.  Workload c seeds numpy's SeedSequence(20250 + c) and
spawns independent streams for q, k, v, dO, valid lengths and row samples.
bf16 tensors travel as uint16 bit patterns (numpy has no bf16 dtype).
"""

from __future__ import annotations

import dataclasses

import numpy as np

SEED_BASE = 20250
STREAMS = ("q", "k", "v", "dout", "k_lens", "rows")


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    kind: str            # "self" or "cross"
    B: int
    H: int
    D: int
    grid: tuple | None   # (F, Hp, Wp) for self-attention
    Lq: int
    Lk: int
    backward: bool
    k_len_range: tuple | None = None   # inclusive range for cross-attention valid lengths

    @property
    def L(self) -> int:
        return self.Lq


def _self(index, name, grid, B, H, backward=False):
    L = grid[0] * grid[1] * grid[2]
    return Workload(index, name, "self", B, H, 128, tuple(grid), L, L, backward)


WORKLOADS = {
    1: _self(1, "tiny", (5, 8, 8), 1, 2, backward=True),
    2: _self(2, "480p", (21, 30, 52), 1, 12),
    3: Workload(3, "cross", "cross", 2, 12, 128, None, 32760, 512, False, (20, 512)),
    4: _self(4, "720p", (21, 45, 80), 1, 40, backward=True),
    5: _self(5, "long", (64, 64, 64), 1, 40),
}


def streams(index: int):
    """Independent numpy Generators for workload `index`, keyed by STREAMS."""
    children = np.random.SeedSequence(SEED_BASE + index).spawn(len(STREAMS))
    return {name: np.random.Generator(np.random.PCG64(s)) for name, s in zip(STREAMS, children)}


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp64."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def normal_bf16(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    """N(0,1) fp32 draws rounded to bf16, returned as uint16 bits; drawn in chunks to bound memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for start in range(0, n, chunk):
        stop = min(n, start + chunk)
        out[start:stop] = fp32_to_bf16_bits(rng.standard_normal(stop - start, dtype=np.float32))
    return out.reshape(shape)


def make_inputs(index: int, with_dout: bool | None = None, rows_per_head: int = 64):
    """All inputs of workload `index` as a dict of numpy arrays.

    q/k/v/(dout) are uint16 bf16 bits in [B, L, H, D] layout; `k_lens` is int32 [B]
    (cross-attention only); `rows` is int64 [B, H, r] of distinct sorted row indices
    used by sampled checks (r = min(rows_per_head, Lq)).
    """
    w = WORKLOADS[index]
    g = streams(index)
    out = {
        "q": normal_bf16(g["q"], (w.B, w.Lq, w.H, w.D)),
        "k": normal_bf16(g["k"], (w.B, w.Lk, w.H, w.D)),
        "v": normal_bf16(g["v"], (w.B, w.Lk, w.H, w.D)),
    }
    if with_dout is None:
        with_dout = w.backward
    if with_dout:
        out["dout"] = normal_bf16(g["dout"], (w.B, w.Lq, w.H, w.D))
    if w.kind == "cross":
        lo, hi = w.k_len_range
        out["k_lens"] = g["k_lens"].integers(lo, hi + 1, size=w.B, dtype=np.int64).astype(np.int32)
    r = min(rows_per_head, w.Lq)
    rows = np.empty((w.B, w.H, r), dtype=np.int64)
    for b in range(w.B):
        for h in range(w.H):
            rows[b, h] = np.sort(g["rows"].choice(w.Lq, size=r, replace=False))
    out["rows"] = rows
    return out


def workload_k_lens(index: int) -> np.ndarray:
    """The valid text lengths of cross-attention workload `index` alone (the same draw as make_inputs)."""
    w = WORKLOADS[index]
    lo, hi = w.k_len_range
    return streams(index)["k_lens"].integers(lo, hi + 1, size=w.B, dtype=np.int64).astype(np.int32)


def random_bf16(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    """Small ad-hoc bf16 tensors for edge-case tests: N(0, scale^2) rounded to bf16 bits."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32) * np.float32(scale)
    return fp32_to_bf16_bits(x).reshape(shape)


def sample_rows(seed: int, n: int, r: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return np.sort(rng.choice(n, size=min(r, n), replace=False))


def make_text_context(index: int, B: int, H: int, Lk: int = 512, D: int = 128, k_len_range=(20, 512)):
    """Text-token keys/values [B, Lk, H, D] (bf16 bits) and valid lengths [B] drawn like workload 3,
    from workload `index`'s seed (streams spawned after the standard ones)."""
    children = np.random.SeedSequence(SEED_BASE + index).spawn(len(STREAMS) + 3)[len(STREAMS):]
    gk, gv, gl = (np.random.Generator(np.random.PCG64(s)) for s in children)
    lo, hi = k_len_range
    return {
        "k": normal_bf16(gk, (B, Lk, H, D)),
        "v": normal_bf16(gv, (B, Lk, H, D)),
        "k_lens": gl.integers(lo, hi + 1, size=B, dtype=np.int64).astype(np.int32),
    }
