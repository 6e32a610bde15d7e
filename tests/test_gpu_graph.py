"""The forwards captured in a HIP graph and replayed.

The forward launches take their query tiles from a work counter in the
workspace (or in the allocation-free variant's static scratch), zeroed by a
kernel of the same call, so a captured call must give on every replay what it
gives when run eagerly.  Each case runs the call eagerly, captures it, and
replays it three times with eager work of the program in between (the outputs
overwritten, a synchronization), checking every replay bit for bit against the
eager result: which workgroup takes which tile does not change any tile's
arithmetic, and the split tiles' merge has a fixed order.  The eager results
themselves are checked against the oracle by the parity tests."""

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import spatio_temporal_attention_amd as wa  # noqa: E402

GRID = (2, 32, 32)        # L = 2048: 8 query tiles of 256 rows per head


@pytest.fixture(scope="module", autouse=True)
def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    wa.lib()


def _inputs(B, H, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    L = GRID[0] * GRID[1] * GRID[2]
    return [torch.randn((B, L, H, 128), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3)]


def _replays(call, outs, reset):
    """Eager result of `call` (which writes `outs`), then three graph replays, each compared with it."""
    reset()
    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                   # warm-up on the capture's side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for _ in range(3):
        reset()                                  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got, want)


def test_graph_self_fwd_with_split():
    """130 heads: 1,040 query tiles, the last 16 as 8 key ranges each (partials and merge in the graph)."""
    B, H = 1, 130
    q, k, v = _inputs(B, H, 11)
    L = q.shape[1]
    rope = wa.RopeConfig(48, 40, 40, 10000.0)
    table = wa.rope_table(GRID, rope, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    ws = torch.empty(wa.self_fwd_workspace_bytes(B, L, H, 128, True), dtype=torch.uint8, device="cuda")
    _replays(lambda: wa.self_fwd(q, k, v, grid=GRID, table=table, rope=rope, out=o, lse=lse, workspace=ws),
             [o, lse], lambda: (o.fill_(float("nan")), lse.fill_(float("nan"))))


def test_graph_self_fwd_noalloc():
    """The allocation-free entry point: its counter and tiles live in the library's static scratch."""
    B, H = 1, 130
    q, k, v = _inputs(B, H, 12)
    L = q.shape[1]
    rope = wa.RopeConfig(48, 40, 40, 10000.0)
    table = wa.rope_table(GRID, rope, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    _replays(lambda: wa.self_fwd_noalloc(q, k, v, o, lse, grid=GRID, table=table, rope=rope),
             [o, lse], lambda: (o.fill_(float("nan")), lse.fill_(float("nan"))))


def test_graph_self_fwd_varlen():
    """Two items of 2,048 and 1,000 tokens: rows past an item's length are left as they were."""
    B, H = 2, 8
    q, k, v = _inputs(B, H, 13)
    L = q.shape[1]
    lens = torch.tensor([L, 1000], dtype=torch.int32, device="cuda")
    rope = wa.RopeConfig(48, 40, 40, 10000.0)
    table = wa.rope_table(GRID, rope, device="cuda")
    o = torch.zeros_like(q)
    lse = torch.zeros((B, H, L), dtype=torch.float32, device="cuda")
    ws = torch.empty(wa.self_fwd_workspace_bytes(B, L, H, 128, True), dtype=torch.uint8, device="cuda")
    _replays(lambda: wa.self_fwd_varlen(q, k, v, lens, grid=GRID, table=table, rope=rope, out=o, lse=lse,
                                        workspace=ws),
             [o, lse], lambda: (o.zero_(), lse.zero_()))


def test_graph_self_fwd_fp8():
    B, H = 1, 8
    q, k, v = _inputs(B, H, 14)
    L = q.shape[1]
    rope = wa.RopeConfig(48, 40, 40, 10000.0)
    table = wa.rope_table(GRID, rope, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    ws = torch.empty(wa.self_fwd_fp8_workspace_bytes(B, L, H), dtype=torch.uint8, device="cuda")
    _replays(lambda: wa.self_fwd_fp8(q, k, v, grid=GRID, table=table, rope=rope, out=o, lse=lse, workspace=ws),
             [o, lse], lambda: (o.fill_(float("nan")), lse.fill_(float("nan"))))
