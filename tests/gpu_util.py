"""Helpers shared by the GPU parity tests: device transfer of bf16 bit patterns
and the parity bar (max-abs 2e-2 and relative L2 5e-3 on O/dQ/dK/dV, 1e-3
absolute on LSE)."""

import numpy as np

import synth

TOL_MAX_ABS = 2e-2
TOL_REL_L2 = 5e-3
TOL_LSE = 1e-3


def to_dev(bits, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bf16_to_f64(t):
    """Device bf16 tensor -> fp64 numpy (exact)."""
    import torch
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return synth.bf16_bits_to_f64(bits)


def f32_to_np(t):
    return t.detach().cpu().numpy().astype(np.float64)


def bf16_half_ulp(x):
    """Half a bf16 ulp at |x| (2^(floor(log2|x|) - 8)): the largest error of rounding x to bf16."""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 8)


def check_close(name, got, ref, max_abs=TOL_MAX_ABS, rel_l2=TOL_REL_L2, unit_scale=True, out_quantum=False,
                extra_abs=None, extra_rel=0.0):
    """The parity bar: max |got - ref| <= max_abs and ||got - ref|| / ||ref|| <= rel_l2.

    unit_scale=False: the inputs were scaled away from unit variance (peaked softmax cases).  bf16
    errors are relative (each rounding is at most 2^-9 of the value), and the absolute bar is stated
    for tensors whose entries are O(1); for scaled inputs it is applied relative to the reference's
    peak magnitude, max_abs * max(1, max|ref|).  The relative-L2 bar is scale-free and unchanged.

    out_quantum=True: outputs that are sums over many rows (a key's dK or dV sums over every query)
    are not O(1) even for unit-variance inputs.  Their bf16 output rounding alone can be half an ulp
    at |ref|, 2^-6 = 1.6e-2 for |ref| in [4, 8), before any arithmetic error.  The bar then holds
    per element as max_abs + bf16_half_ulp(ref): the stated bar for the computation plus the
    output's rounding quantum.  The relative-L2 bar is unchanged.

    extra_abs (array like ref) / extra_rel: a documented, separately measured difference added to the
    bar, e.g. what the fp16 rounding of the rotated score operands moves (oracle.fp16_scores)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    bar = np.full(ref.shape, float(max_abs))
    if not unit_scale:
        bar *= max(1.0, float(np.abs(ref).max())) if ref.size else 1.0
    if out_quantum:
        bar = bar + bf16_half_ulp(ref)
    if extra_abs is not None:
        bar = bar + np.asarray(extra_abs, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    worst = float((err / bar).max()) if err.size else 0.0
    rl = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    print(f"  {name}: max_abs={mx:.3e} (worst err/bar {worst:.2f}) rel_l2={rl:.3e}", flush=True)
    assert np.all(err <= bar), f"{name}: max abs error {mx:.3e}, {worst:.2f} x its bar"
    assert rl <= rel_l2 + extra_rel, f"{name}: relative L2 error {rl:.3e} > {rel_l2 + extra_rel:.3e}"
    return mx, rl


def check_lse(name, got, ref, tol=TOL_LSE, extra=None):
    """|got - ref| <= tol (+ extra, an array like ref: a documented, separately measured difference)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)), f"{name}: -inf pattern differs"
    assert np.array_equal(got[~fin], ref[~fin]), f"{name}: non-finite values differ"
    bar = np.full(ref.shape, float(tol))
    if extra is not None:
        bar = bar + np.asarray(extra, dtype=np.float64)
    err = np.abs(got[fin] - ref[fin])
    mx = float(err.max()) if fin.any() else 0.0
    worst = float((err / bar[fin]).max()) if fin.any() else 0.0
    print(f"  {name}: max_abs={mx:.3e} (worst err/bar {worst:.2f})", flush=True)
    assert np.all(err <= bar[fin]), f"{name}: LSE error {mx:.3e}, {worst:.2f} x its bar"
    return mx
