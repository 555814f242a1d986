"""The Python binding's checks on device tensors: buffers that do not match
the call's sizes are rejected before any launch (the C ABI takes plain
pointers and cannot see them)."""
import pytest
import torch

from efficient_long_sequence_amd import mita, synth
from tests import gpu_harness as gh_

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _qkv(N=512, d=64):
    Q, K, V = synth.make(1, 2, N, d, "clustered", 8, "bf16", 4)
    return tuple(gh_.to_device(x, "bf16") for x in (Q, K, V))


def test_mismatched_output_buffer_is_rejected():
    gh_.say("[gpu] binding: output buffer check")
    q, k, v = _qkv()
    pool = (1, 512, 1, 16)
    with pytest.raises(mita.MitaError):
        mita.forward(q, k, v, pool, 32, 1, out=torch.empty(1, 2, 256, 64, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(mita.MitaError):
        mita.forward(q, k, v, pool, 32, 1, out=torch.empty(1, 2, 512, 64, dtype=torch.float32, device="cuda"))


def test_saved_tensors_of_another_call_are_rejected():
    gh_.say("[gpu] binding: saved tensor check")
    q, k, v = _qkv()
    pool = (1, 512, 1, 16)
    O, sv = mita.forward_train(q, k, v, pool, 32, 1)
    dO = torch.ones_like(O)
    # k differs from the forward's: topk has the wrong shape
    with pytest.raises(mita.MitaError):
        mita.backward(q, k, v, O, dO, pool, 48, 1, sv)
    # the same call goes through
    dq, dk, dv = mita.backward(q, k, v, O, dO, pool, 32, 1, sv)
    torch.cuda.synchronize()
    assert torch.isfinite(dq.float()).all() and torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()
