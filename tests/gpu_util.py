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


def check_close(name, got, ref, max_abs=TOL_MAX_ABS, rel_l2=TOL_REL_L2, unit_scale=True):
    """unit_scale=False: inputs were scaled away from unit variance.  bf16 errors are
    relative (each rounding is at most 2^-9 of the value), and the absolute bar is stated
    for tensors whose entries are O(1); for scaled inputs it is applied relative to the
    reference's peak magnitude, max_abs * max(1, max|ref|).  The relative-L2 bar is
    scale-free and applies unchanged."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not unit_scale:
        max_abs = max_abs * max(1.0, float(np.abs(ref).max()))
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    rl = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    print(f"  {name}: max_abs={mx:.3e} rel_l2={rl:.3e}", flush=True)
    assert mx <= max_abs, f"{name}: max abs error {mx:.3e} > {max_abs}"
    assert rl <= rel_l2, f"{name}: relative L2 error {rl:.3e} > {rel_l2}"
    return mx, rl


def check_lse(name, got, ref, tol=TOL_LSE):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)), f"{name}: -inf pattern differs"
    assert np.array_equal(got[~fin], ref[~fin]), f"{name}: non-finite values differ"
    err = float(np.abs(got[fin] - ref[fin]).max()) if fin.any() else 0.0
    print(f"  {name}: max_abs={err:.3e}", flush=True)
    assert err <= tol, f"{name}: LSE error {err:.3e} > {tol}"
    return err
