"""fp64 CPU oracle for Wan-style spatio-temporal attention with 3D RoPE.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or run anything in this package; the
product path (the HIP library and its Python binding) never does, and it fails
loudly when its compiled library is missing instead of falling back here.

The oracle is the plain definition of what the hot path computes, written in
NumPy float64 with no blocking, fusion or reordering beyond what the
definition states (the one exception, `self_bwd_dkdv_rows`, processes query
rows in blocks only so that an L x L matrix is never held; the sum it forms is
the same).  It shares no code with the HIP path.

Parity status: every function here is pinned by CPU tests against brute force,
closed forms, invariants, finite differences or a library routine (see the
tests named in each docstring).  The exact Wan RoPE convention (axis split,
pairing, base) is not printed on the pages, so parity with a trained Wan
checkpoint's rotary embedding is unpinned; the convention used here is fixed
by the library's interface instead.
"""

from .reference import (  # noqa: F401
    RopeSpec,
    latent_token_grid,
    positions,
    rope_axis_of_pair,
    rope_frequencies,
    rope_angles,
    rope_table_ref,
    rope_apply,
    rope3d_ref,
    attention_rows_ref,
    self_fwd_ref,
    self_fwd_varlen_ref,
    partial_fwd_ref,
    lse_merge_ref,
    cross_fwd_ref,
    self_bwd_ref,
    cross_bwd_ref,
    self_bwd_dq_rows,
    self_bwd_dkdv_rows,
)
