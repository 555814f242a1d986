"""mita_forward_noalloc -- the entry point that allocates nothing (its scratch
is the library's static device array) -- against mita_forward on the same
inputs: two calls in a row, the second smaller than the first, each bitwise
equal to mita_forward's output (same kernels, same plan; mita_forward is
itself checked against the oracle by the parity tests)."""
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


# (B, H, N, pool, d, k, s, kind, clusters): an ADE20K-shaped batch with two
# routing slots, then a smaller DeiT-S-shaped one
CALLS = [
    (8, 6, 1024, (32, 32, 7, 7), 64, 49, 2, "clustered", 16),
    (2, 3, 196, (14, 14, 5, 5), 64, 25, 1, "clustered", 16),
]


def test_noalloc_matches_forward_on_two_calls():
    sizes = []
    for i, (B, H, N, pool, d, k, s, kind, nc) in enumerate(CALLS):
        Q, K, V = synth.make(B, H, N, d, kind, nc, "bf16", seed=40 + i)
        q, kk, v = (gh_.to_device(x, "bf16") for x in (Q, K, V))
        need = mita.workspace_bytes(q.dtype, B, H, N, d, pool, k, s)
        assert 0 < need <= mita.NOALLOC_SCRATCH_BYTES
        sizes.append(need)
        gh_.say(f"[gpu] noalloc call {i}: B={B} H={H} N={N} k={k} s={s}, scratch {need / 2**20:.1f} MiB")
        ref = mita.forward(q, kk, v, pool, k, s)
        out = torch.empty_like(q)
        got = mita.forward_noalloc(q, kk, v, pool, k, s, out=out)
        torch.cuda.synchronize()
        assert got is out
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got, ref), f"call {i}: noalloc output differs from mita_forward"
    assert sizes[1] < sizes[0]


def test_noalloc_rejects_a_call_beyond_its_scratch():
    B, H, N, d, m, k = 1, 2, 65536, 64, 128, 128
    pool = (1, N, 1, m)
    assert mita.workspace_bytes(torch.bfloat16, B, H, N, d, pool, k, 1) > mita.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mita.MitaError) as exc:
        mita.forward_noalloc(q, q, q, pool, k, 1)
    assert exc.value.code == 5
