"""The forward pass captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

mita_forward enqueues kernels only (the workspace is cleared by a fill
kernel, not a memset node), so a caller can capture it once and replay it
to remove the launch cost on small, launch-bound shapes.  Each replay is
checked bitwise against the eager result (the forward is deterministic),
with the program's own eager work and synchronisations between replays.
"""
import numpy as np
import pytest
import torch

from efficient_long_sequence_amd import mita, synth
from tests import gpu_harness as gh_

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("shape", [
    # (B, H, grid_h, grid_w, land_h, land_w, k, s): DeiT-S-shaped and ADE-shaped batches, an s = 2 long one
    (64, 6, 14, 14, 5, 5, 25, 1),
    (8, 6, 32, 32, 7, 7, 49, 1),
    (1, 2, 1, 16384, 1, 64, 64, 2),
])
def test_graph_replays_match_eager(shape):
    B, H, gh, gw, lh, lw, k, s = shape
    N, d = gh * gw, 64
    gh_.say(f"[gpu] graph B={B} H={H} N={N} m={lh * lw} k={k} s={s}")
    Q, K, V = synth.make(B, H, N, d, "clustered", 16, "bf16", 11)
    q, kk, v = (gh_.to_device(x, "bf16") for x in (Q, K, V))
    pool = (gh, gw, lh, lw)
    ws = torch.empty(mita.workspace_bytes(q.dtype, B, H, N, d, pool, k, s), dtype=torch.uint8, device="cuda")
    ref = mita.forward(q, kk, v, pool, k, s, workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    # warm up on a side stream, as graph capture requires
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mita.forward(q, kk, v, pool, k, s, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mita.forward(q, kk, v, pool, k, s, workspace=ws, out=out)
    other_ws = torch.empty_like(ws)
    for rep in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}"
        # eager work in between, on the same inputs and another workspace
        e = mita.forward(q, kk, v, pool, k, s, workspace=other_ws)
        torch.cuda.synchronize()
        assert torch.equal(e, ref)
    del g
