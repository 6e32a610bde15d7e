"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over one batch of the Wan-14B-shaped
720p workload (grid 21x45x80 = 75600 tokens, B=1, 40 heads of 128, bf16):
  1. self-attention forward with 3D RoPE  (keys pre-rotated, queries rotated on load; O, LSE)
  2. text cross-attention forward         (75600 video tokens x 512 text tokens, valid length ~U[20,512])
  3. self-attention backward              (dQ, dK, dV incl. the RoPE gradient)
Inputs are synthetic (seeded N(0,1) in bf16) and resident in HBM before timing.

The reported metric is the self-attention forward's throughput: algorithmic
4*B*H*L^2*D flop divided by the forward's median duration over the timed
steps, measured with HIP events on the stream the library launches on.

After the timed steps, each of the five workloads' forward calls is timed on
its own shape (HIP events, median over repeats): the 320-token tiny case, the
480p 1.3B forward (32,760 tokens, 12 heads), the 480p text cross-attention
(B=2, 12 heads, 512 text tokens with the workload's seeded valid lengths), the
720p forward (the headline) and the 262,144-token forward (40 heads); each with
TFLOP/s against the published bf16 dense peak and against the MFMA rate a
plain MFMA loop reaches in the same run.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_fwd_720p_hbm_traffic.json")
# Query rows per head the oracle computes for the CPU baseline (about 10-17 s of fp64 work on 16 host threads).
CPU_SAMPLE_ROWS = 256
FWD_SOURCES = ("attn_fwd_pp.hip", "common.h", "kernels.h", "validate.h", "validate.cpp")


def measured_traffic():
    """HBM bytes per forward launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE passes,
    or None when the kernel sources have changed since they were taken."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_PROFILE))
    except (OSError, ValueError):
        return None
    csrc = os.path.join(ROOT, "spatio_temporal_attention_amd", "csrc")
    src = b"".join(open(os.path.join(csrc, n), "rb").read() for n in FWD_SOURCES)
    if hashlib.sha256(src).hexdigest() != rec.get("kernel_source_sha256"):
        return None
    return rec["traffic_bytes"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fwd-only", action="store_true", help="time only the forward (profiling runs)")
    ap.add_argument("--no-extras", action="store_true", help="skip the varlen / ring-shard / merge measurements")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload forward timings and the MFMA loop (profiling runs of the step)")
    ap.add_argument("--configs-only", action="store_true",
                    help="only the per-workload forward timings and the MFMA loop (profiling runs of those)")
    ap.add_argument("--cross-only", action="store_true",
                    help="only the text cross-attention forward and backward at the 720p text shape (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain device copy of known size (for scaling HBM counters)")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads():
    try:
        import threadpoolctl
        info = [d for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
        return [{"library": d.get("internal_api"), "threads": d.get("num_threads")} for d in info]
    except Exception:   # threadpoolctl missing or unable to inspect: report nothing rather than guess
        return []


def cpu_baseline(inp, w, rope, scale):
    """The fp64 oracle on a bounded sample: CPU_SAMPLE_ROWS seeded query rows of every head."""
    import numpy as np
    import oracle
    import synth
    rows = inp["rows"]
    t0 = time.perf_counter()
    for h in range(w.H):
        sl = (slice(0, 1), slice(None), slice(h, h + 1))
        oracle.self_fwd_ref(synth.bf16_bits_to_f64(inp["q"][sl]), synth.bf16_bits_to_f64(inp["k"][sl]),
                            synth.bf16_bits_to_f64(inp["v"][sl]), scale, w.grid, rope, rows=rows[:, h:h + 1])
    dt = time.perf_counter() - t0
    n_rows = rows.shape[1] * rows.shape[2]
    flop = 4.0 * n_rows * w.L * w.D
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    blas = _blas_threads()
    threads = max([b["threads"] for b in blas if b["threads"]] or [int(os.environ.get("OMP_NUM_THREADS", cores))])
    full_flop = 4.0 * w.B * w.H * w.L * w.L * w.D
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": min(cores, threads), "kind": "oracle",
            "sample": f"self-attention forward (fp64 NumPy, 3D RoPE) of {rows.shape[2]} seeded query rows "
                      f"x {w.H} heads against all {w.L} keys of the 720p workload; {dt:.2f} s",
            "seconds": dt, "flop": flop, "cpu_model": _cpu_model(), "affinity_cores": cores, "blas": blas,
            "extrapolated_full_forward_s": round(dt * full_flop / flop, 1),
            "extrapolated_note": "EXTRAPOLATED, not measured: the sample's rate applied to the whole 720p forward "
                                 "(all 75,600 query rows x 40 heads)"}


def _time(fn, reps=3):
    """Mean ms of `fn` over `reps` calls after one warm call (HIP events on the current stream)."""
    import torch
    fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        fn()
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) / reps


def _median_ms(fn, reps, warm=3):
    """Median ms of `fn` over `reps` calls, each bracketed by its own HIP events on the current stream
    (the stream the library launches on), after `warm` untimed calls."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    n = len(t)
    return 0.5 * (t[(n - 1) // 2] + t[n // 2])


def measure_mfma_peak(wa):
    """TFLOP/s of the library's plain bf16 MFMA loop on every SIMD (two waves per SIMD), median of 5."""
    import torch
    wgs, iters = 512, 100000
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    flop = wa.measure_mfma_peak(wgs, iters, sink)
    ms = _median_ms(lambda: wa.measure_mfma_peak(wgs, iters, sink), reps=5, warm=1)
    return {"tflops": round(flop / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 3),
            "kernel": "v_mfma_f32_32x32x16_bf16 back to back, 4 accumulators per wave, 512 workgroups x 4 waves, "
                      "register operands with varied values"}


def _rate(flop, ms, peak_meas):
    tf = flop / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "tflops": round(tf, 1), "pct_bf16_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2),
            "pct_measured_mfma_peak": round(100.0 * tf / peak_meas, 2) if peak_meas else None}


def bench_configs(wa, torch, synth, dev, rope, peak_meas, c4_ms):
    """Each workload's forward on its own shape (median over repeats), the 720p one from the timed steps."""
    out = {}
    g = torch.Generator(device=dev).manual_seed(20250)

    def rand(shape):
        return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)

    for idx, reps in ((1, 100), (2, 20), (5, 5)):
        w = synth.WORKLOADS[idx]
        q, k, v = (rand((w.B, w.L, w.H, w.D)) for _ in range(3))
        table = wa.rope_table(w.grid, rope, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.L), dtype=torch.float32, device=dev)
        ws = torch.empty(wa.self_fwd_workspace_bytes(w.B, w.L, w.H, w.D, True), dtype=torch.uint8, device=dev)
        ms = _median_ms(lambda: wa.self_fwd(q, k, v, grid=w.grid, table=table, rope=rope, out=o, lse=lse,
                                            workspace=ws), reps=reps, warm=2 if idx == 5 else 3)
        flop = 4.0 * w.B * w.H * w.L * w.L * w.D
        out[f"C{idx}"] = dict(workload=f"{w.name}: self-attention forward, grid {'x'.join(map(str, w.grid))} "
                                       f"(L={w.L}), B={w.B}, H={w.H}, D=128, 3D RoPE", reps=reps,
                              **_rate(flop, ms, peak_meas))
        del q, k, v, o, lse, ws
        torch.cuda.empty_cache()
    # text cross-attention: B=2, 12 heads, 32,760 video tokens over 512 text tokens, seeded valid lengths
    w = synth.WORKLOADS[3]
    lens = synth.workload_k_lens(3)
    q = rand((w.B, w.Lq, w.H, w.D))
    k, v = rand((w.B, w.Lk, w.H, w.D)), rand((w.B, w.Lk, w.H, w.D))
    kl = torch.from_numpy(lens).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Lq), dtype=torch.float32, device=dev)
    xws = torch.empty(wa.cross_fwd_workspace_bytes(w.B, w.Lk, w.H, w.D), dtype=torch.uint8, device=dev)
    ms = _median_ms(lambda: wa.cross_fwd(q, k, v, kl, out=o, lse=lse, workspace=xws), reps=100)
    sk = float(lens.astype("int64").sum())
    flop = 4.0 * w.H * w.D * w.Lq * sk
    nbytes = 2.0 * (w.B * w.Lq * w.H * w.D * 2) + sk * w.H * w.D * 4 + w.B * w.H * w.Lq * 4
    r = _rate(flop, ms, peak_meas)
    r.update(gbs=round(nbytes / (ms * 1e-3) / 1e9, 1), pct_hbm_peak=round(100.0 * nbytes / (ms * 1e-3) / 1e9
                                                                          / PEAK_HBM_GBS, 2),
             algorithmic_bytes=nbytes, bound_ms=round(max(flop / (PEAK_BF16_TFLOPS * 1e12),
                                                          nbytes / (PEAK_HBM_GBS * 1e9)) * 1e3, 4))
    r["pct_of_bound"] = round(100.0 * r["bound_ms"] / ms, 1)
    out["C3"] = dict(workload=f"cross: text cross-attention forward, Lq={w.Lq}, Lk={w.Lk}, B={w.B}, H={w.H}, "
                              f"valid lengths {lens.tolist()}", reps=100, **r)
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    w = synth.WORKLOADS[4]
    if c4_ms is not None:
        out["C4"] = dict(workload=f"720p: self-attention forward, grid 21x45x80 (L={w.L}), B=1, H=40, D=128, "
                                  f"3D RoPE (the headline; median over the timed steps)",
                         **_rate(4.0 * w.H * w.L * w.L * w.D, c4_ms, peak_meas))
    return {k: out[k] for k in ("C1", "C2", "C3", "C4", "C5") if k in out}


def bench_rope3d(wa, torch, dev, rope):
    """The standalone 3D RoPE call on the 720p query tensor [1, 75600, 40, 128], out of place: HBM-bound
    (every element read once and written once, plus the angle table)."""
    grid, L, H = (21, 45, 80), 75600, 40
    g = torch.Generator(device=dev).manual_seed(31)
    x = torch.randn((1, L, H, 128), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    y = torch.empty_like(x)
    table = wa.rope_table(grid, rope, device=dev)
    ms = _median_ms(lambda: wa.rope3d(x, grid, table, rope=rope, out=y), reps=50)
    nbytes = 2.0 * x.numel() * 2 + table.numel() * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    del x, y
    return {"workload": "wanattn_rope3d on q [1, 75600, 40, 128] bf16 (720p grid 21x45x80), out of place",
            "ms": round(ms, 4), "algorithmic_bytes": nbytes, "gbs": round(gbs, 1),
            "pct_hbm_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2)}


def bench_cross(wa, torch, dev, g, with_fwd=False):
    """Text cross-attention at the step's shape: 75,600 video tokens over 512 text tokens (336 valid), 40 heads;
    the backward (and with_fwd: the forward) timed on its own."""
    out = {}
    L, H, Lt = 75600, 40, 512
    q, do = (torch.randn((1, L, H, 128), generator=g, device=dev).to(torch.bfloat16) for _ in range(2))
    tk, tv = (torch.randn((1, Lt, H, 128), generator=g, device=dev).to(torch.bfloat16) for _ in range(2))
    kl = torch.tensor([336], dtype=torch.int32, device=dev)
    o, lse = torch.empty_like(q), torch.empty((1, H, L), dtype=torch.float32, device=dev)
    wsf = torch.empty(wa.cross_fwd_workspace_bytes(1, Lt, H), dtype=torch.uint8, device=dev)
    ms = _time(lambda: wa.cross_fwd(q, tk, tv, kl, out=o, lse=lse, workspace=wsf), reps=20)
    if with_fwd:
        out["cross_fwd"] = {"workload": "720p video tokens (75,600) over 512 text tokens (336 valid), 40 heads",
                            "ms": round(ms, 4), "tflops": round(4.0 * H * L * 336 * 128 / (ms * 1e-3) / 1e12, 1)}
    ws = torch.empty(wa.cross_bwd_workspace_bytes(1, L, Lt, H), dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(tk), torch.empty_like(tv)
    ms = _time(lambda: wa.cross_bwd(q, tk, tv, kl, o, lse, do, workspace=ws, dq=dq, dk=dk, dv=dv))
    flop = 8.0 * H * L * 336 * 128
    out["cross_bwd"] = {"workload": "720p video tokens (75,600) over 512 text tokens (336 valid), 40 heads",
                        "ms": round(ms, 3), "tflops": round(flop / (ms * 1e-3) / 1e12, 1)}
    return out


def bench_next_rows(wa, torch, synth, dev, rope):
    """The rows beyond the step, each on its own realistic shape (timed after the step, not in it):
    - one Ring hop of Ulysses-8 x Ring-2 context parallelism at 256K tokens (grid 64x64x64): a
      131,072-token query shard x a 131,072-token key/value shard, 5 heads, global RoPE positions,
      then the exact merge of the two hops' partial results;
    - the text cross-attention backward at the step's shape;
    - the FP8 (e4m3) forward on the headline workload;
    - a joint video + image batch: a 720p clip (75,600 tokens) and one image frame (3,600 tokens)
      padded to 75,600, 40 heads, variable-length self-attention."""
    out = {}
    grid = (64, 64, 64)
    Lh, H = 131072, 5
    g = torch.Generator(device=dev).manual_seed(7)
    q, k, v = (torch.randn((1, Lh, H, 128), generator=g, device=dev).to(torch.bfloat16) for _ in range(3))
    table = wa.rope_table(grid, rope, device=dev)
    ws = torch.empty(wa.partial_fwd_workspace_bytes(1, Lh, H), dtype=torch.uint8, device=dev)
    o1, l1 = torch.empty_like(q), torch.empty((1, H, Lh), dtype=torch.float32, device=dev)
    o2, l2 = torch.empty_like(q), torch.empty((1, H, Lh), dtype=torch.float32, device=dev)
    ms = _time(lambda: wa.partial_fwd(q, k, v, Lh, 0, grid=grid, table=table, rope=rope, out=o1, lse=l1,
                                      workspace=ws))
    wa.partial_fwd(q, k, v, Lh, Lh, grid=grid, table=table, rope=rope, out=o2, lse=l2, workspace=ws)
    flop = 4.0 * H * Lh * Lh * 128
    out["partial_fwd"] = {"workload": "ring hop at 256K tokens: q tokens [131072, 262144) x k/v tokens [0, 131072), "
                                      "5 heads, grid 64x64x64, RoPE at global positions",
                          "ms": round(ms, 3), "tflops": round(flop / (ms * 1e-3) / 1e12, 1)}
    om, lm = torch.empty_like(q), torch.empty((1, H, Lh), dtype=torch.float32, device=dev)
    ms = _time(lambda: wa.lse_merge([o1, o2], [l1, l2], out=om, lse=lm), reps=10)
    nbytes = 3.0 * q.numel() * 2 + 3.0 * l1.numel() * 4
    out["lse_merge"] = {"workload": "2 partials [1, 131072, 5, 128] bf16 + LSE", "ms": round(ms, 4),
                        "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    del q, k, v, o1, o2, om, ws
    out["cross_bwd"] = bench_cross(wa, torch, dev, g)["cross_bwd"]
    # FP8 (e4m3) forward on the headline workload: 720p, 40 heads, 3D RoPE
    L, H = 75600, 40
    q, k, v = (torch.randn((1, L, H, 128), generator=g, device=dev).to(torch.bfloat16) for _ in range(3))
    table = wa.rope_table((21, 45, 80), rope, device=dev)
    ws = torch.empty(wa.self_fwd_fp8_workspace_bytes(1, L, H), dtype=torch.uint8, device=dev)
    o, lse = torch.empty_like(q), torch.empty((1, H, L), dtype=torch.float32, device=dev)
    ms = _time(lambda: wa.self_fwd_fp8(q, k, v, grid=(21, 45, 80), table=table, rope=rope, out=o, lse=lse,
                                       workspace=ws), reps=2)
    flop = 4.0 * H * L * L * 128
    out["fp8_fwd"] = {"workload": "720p self-attention (75,600 tokens, 40 heads, 3D RoPE), e4m3 operands",
                      "ms": round(ms, 3), "tflops": round(flop / (ms * 1e-3) / 1e12, 1),
                      "pct_fp8_peak": round(100.0 * flop / (ms * 1e-3) / 5.0e15, 2)}
    del q, k, v, o, ws
    L, H = 75600, 40
    q, k, v = (torch.randn((2, L, H, 128), generator=g, device=dev).to(torch.bfloat16) for _ in range(3))
    lens = torch.tensor([L, 3600], dtype=torch.int32, device=dev)
    table = wa.rope_table((21, 45, 80), rope, device=dev)
    ws = torch.empty(wa.self_fwd_workspace_bytes(2, L, H), dtype=torch.uint8, device=dev)
    o, lse = torch.empty_like(q), torch.empty((2, H, L), dtype=torch.float32, device=dev)
    ms = _time(lambda: wa.self_fwd_varlen(q, k, v, lens, grid=(21, 45, 80), table=table, rope=rope, out=o, lse=lse,
                                          workspace=ws), reps=2)
    flop = 4.0 * H * 128 * (L * L + 3600 * 3600)
    out["varlen_fwd"] = {"workload": "720p clip (75,600 tokens) + 1-frame image (3,600) padded to 75,600, 40 heads",
                         "ms": round(ms, 3), "tflops": round(flop / (ms * 1e-3) / 1e12, 1)}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(heads would split across GPUs by an all-to-all, key blocks by ring passes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import spatio_temporal_attention_amd as wa
    import synth

    if not os.path.exists(wa.LIB_PATH):
        from spatio_temporal_attention_amd import build
        build.build()
    wa.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}))
        return

    rope = wa.RopeConfig(48, 40, 40, 10000.0)
    if args.cross_only:
        print(json.dumps(bench_cross(wa, torch, dev, torch.Generator(device=dev).manual_seed(7), with_fwd=True)),
              flush=True)
        return
    if args.configs_only:
        peak = measure_mfma_peak(wa)
        print(json.dumps({"mfma_peak_measured": peak,
                          "configs": bench_configs(wa, torch, synth, dev, rope, peak["tflops"], None),
                          "rope3d": bench_rope3d(wa, torch, dev, rope)}), flush=True)
        return
    w = synth.WORKLOADS[4]
    B, L, H, D = w.B, w.L, w.H, w.D
    scale = 1.0 / math.sqrt(D)
    t0 = time.perf_counter()
    inp = synth.make_inputs(4, rows_per_head=CPU_SAMPLE_ROWS)
    ctx = synth.make_text_context(4, B, H)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = (dev_bf16(inp[n]) for n in ("q", "k", "v", "dout"))
    tk, tv = dev_bf16(ctx["k"]), dev_bf16(ctx["v"])
    k_lens = torch.from_numpy(ctx["k_lens"]).to(dev)
    table = wa.rope_table(w.grid, rope, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=dev)
    xo = torch.empty_like(q)
    xlse = torch.empty((B, H, L), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws_f = torch.empty(wa.self_fwd_workspace_bytes(B, L, H, D, True), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(wa.self_bwd_workspace_bytes(B, L, H, D, True), dtype=torch.uint8, device=dev)
    ws_x = torch.empty(wa.cross_fwd_workspace_bytes(B, tk.shape[1], H, D), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        wa.self_fwd(q, k, v, grid=w.grid, table=table, rope=rope, scale=scale, out=o, lse=lse, workspace=ws_f)
        if ev is not None:
            ev[1].record()
        if args.fwd_only:
            return
        wa.cross_fwd(q, tk, tv, k_lens, scale=scale, out=xo, lse=xlse, workspace=ws_x)
        if ev is not None:
            ev[2].record()
        wa.self_bwd(q, k, v, o, lse, do, grid=w.grid, table=table, rope=rope, scale=scale, workspace=ws_b,
                    dq=dq, dk=dk, dv=dv)
        if ev is not None:
            ev[3].record()

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    fwd_ms = [e[0].elapsed_time(e[1]) for e in events]
    if not args.fwd_only:
        cross_ms = [e[1].elapsed_time(e[2]) for e in events]
        bwd_ms = [e[2].elapsed_time(e[3]) for e in events]
    log(f"timed {args.steps} steps in {elapsed:.2f} s; forward ms: {[round(x, 2) for x in fwd_ms]}")

    def median(x):
        t = sorted(x)
        return 0.5 * (t[(len(t) - 1) // 2] + t[len(t) // 2])

    fwd_flop = 4.0 * B * H * L * L * D
    fwd_mean = sum(fwd_ms) / len(fwd_ms)
    fwd_med = median(fwd_ms)
    fwd_tflops = fwd_flop / (fwd_med * 1e-3) / 1e12
    extra = {}
    if not args.fwd_only:
        kl = ctx["k_lens"].astype(np.int64)
        cross_flop = 4.0 * H * D * L * float(kl.sum())
        cross_bytes = 2.0 * (B * L * H * D * 2) + float(kl.sum()) * H * D * 4 + B * H * L * 4
        bwd_flop = 8.0 * B * H * L * L * D
        cross_mean = median(cross_ms)
        bwd_mean = median(bwd_ms)
        extra = {
            "fwd_ms": round(fwd_med, 3),
            "fwd_ms_mean": round(fwd_mean, 3),
            "fwd_ms_min_max": [round(min(fwd_ms), 3), round(max(fwd_ms), 3)],
            "bwd_ms": round(bwd_mean, 3),
            "bwd_tflops": round(bwd_flop / (bwd_mean * 1e-3) / 1e12, 1),
            "cross_ms": round(cross_mean, 4),
            "cross_tflops": round(cross_flop / (cross_mean * 1e-3) / 1e12, 2),
            "cross_gbs": round(cross_bytes / (cross_mean * 1e-3) / 1e9, 1),
            "cross_k_lens": [int(x) for x in kl],
        }
    ms_per_step = elapsed * 1e3 / args.steps

    result = {
        "metric": "self-attn fwd TFLOP/s + % bf16 MFMA peak, L=75600 H=40 D=128 (14B 720p)",
        "value": round(fwd_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16/fp16",
        "data": "synthetic (seeded N(0,1) bf16; no dataset or weights involved)",
        "compute": "bf16 in/out; with RoPE the QK^T MFMAs take fp16 (rotated q/k rescaled by powers of two), "
                   "PV and the backward's gradient products bf16; fp32 accumulation and softmax",
        "config": {"workload": "wan14b-720p self-attn fwd+bwd + text cross-attn",
                   "grid": list(w.grid), "B": B, "L": L, "H": H, "D": D, "rope_split": [48, 40, 40],
                   "rope_theta": 10000.0, "text_tokens": 512, "parallelism": "none (1 GPU)",
                   "step": "self_fwd + cross_fwd + self_bwd" if not args.fwd_only else "self_fwd"},
        "pct_bf16_peak": round(100.0 * fwd_tflops / PEAK_BF16_TFLOPS, 2),
        "timing": "HIP events on the library's stream around each forward call; value uses the median over "
                  "the timed steps",
        "roofline": {"bound": "mfma", "achieved": round(fwd_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(), "traffic_unit": "bytes per launch",
                     "kernel": "attn_fwd_pp_kernel (+ the K/V tile prep pass, the work-counter reset and the merge of the split tiles, inside the same timed call)",
                     "flop_per_launch": fwd_flop},
    }
    result.update(extra)
    if not args.fwd_only and not args.no_extras:
        result["next_rows"] = bench_next_rows(wa, torch, synth, dev, rope)
        log("next rows done")
    if not args.fwd_only and not args.no_configs:
        del q, k, v, do, o, xo, dq, dk, dv, ws_f, ws_b, ws_x
        torch.cuda.empty_cache()
        peak = measure_mfma_peak(wa)
        result["mfma_peak_measured"] = peak
        result["pct_measured_mfma_peak"] = round(100.0 * fwd_tflops / peak["tflops"], 2)
        log(f"MFMA loop: {peak['tflops']} TFLOP/s")
        result["configs"] = bench_configs(wa, torch, synth, dev, rope, peak["tflops"], fwd_med)
        result["rope3d"] = bench_rope3d(wa, torch, dev, rope)
        log("per-config forward timings and the standalone RoPE done")
    if not args.no_cpu_baseline:
        log("running the CPU oracle baseline ...")
        result["cpu_baseline"] = cpu_baseline(inp, w, rope, scale)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
