"""The allocation-free self-attention forward (wanattn_self_fwd_noalloc) against wanattn_self_fwd.

Both run the same kernels, the first on the library's static per-GPU scratch, the second on a caller
workspace, so their outputs must agree bit for bit.  Two calls in a row on one GPU, the second smaller
than the first (the scratch keeps the first call's contents), then a call without RoPE; and a problem
larger than the scratch must be refused on the host with the output left untouched.
"""

import numpy as np
import pytest

import synth
from gpu_util import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import spatio_temporal_attention_amd as wa  # noqa: E402

ROPE = wa.RopeConfig(48, 40, 40, 10000.0)


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    wa.lib()


def _pair(grid, H, rope_on, seed):
    L = int(np.prod(grid))
    q, k, v = (to_dev(synth.random_bf16(seed + i, (1, L, H, 128))) for i in range(3))
    table = wa.rope_table(grid, ROPE) if rope_on else None
    o_ref, l_ref = wa.self_fwd(q, k, v, grid=grid, table=table, rope=ROPE)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, H, L), float("nan"), dtype=torch.float32, device=q.device)
    wa.self_fwd_noalloc(q, k, v, o, lse, grid=grid, table=table, rope=ROPE)
    torch.cuda.synchronize()
    print(f"  grid {grid}, H {H}, rope {rope_on}: workspace {wa.self_fwd_workspace_bytes(1, L, H, 128, rope_on)} B",
          flush=True)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "O differs from wanattn_self_fwd"
    assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32)), "LSE differs from wanattn_self_fwd"


def test_noalloc_matches_workspace_forward_twice():
    # 2,048 tokens x 130 heads: 1,040 query tiles, the last 16 run as 8 key ranges each, so the
    # scratch holds the K/V tiles (~136 MB) and the tail split's partials (~17 MB)
    _pair((2, 32, 32), 130, True, 9100)
    # then a smaller problem on the same scratch (it still holds the first call's tiles)
    _pair((5, 8, 8), 2, True, 9200)
    # and one without RoPE (bf16 key tiles, no exponents)
    _pair((3, 7, 9), 3, False, 9300)


def test_noalloc_refuses_problems_beyond_its_scratch():
    L, H = 75600, 40                       # the 720p workload needs ~1.6 GB of workspace
    assert wa.self_fwd_workspace_bytes(1, L, H, 128, True) > 256 << 20
    q = torch.zeros((1, L, H, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 3.0)
    table = wa.rope_table((21, 45, 80), ROPE)
    with pytest.raises(wa.WanattnError) as e:
        wa.self_fwd_noalloc(q, q, q, o, None, grid=(21, 45, 80), table=table, rope=ROPE)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()), "a refused call wrote its output"
