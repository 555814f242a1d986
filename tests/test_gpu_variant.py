"""GPU parity of the "official" shared-logit variant (q . q~ / d) through the C ABI.

The MiTA tutorial (chapter 8, third check) notes that the authors' code scales
the shared logits by 1/d while routed logits keep 1/sqrt(d).  The same HIP
kernels run with the shared scale switched; the oracle evaluates the joint
softmax with that scale on the GPU's own (validated) experts and routes.
Cases cover both attention paths (LDS-resident and streaming, the latter with
a landmark count that is not a multiple of the 32-entry step), s = 1 and 2,
d = 32 and 64, bf16 and fp32.
"""
import zlib

import numpy as np
import pytest
import torch

from efficient_long_sequence_amd import mita, synth
from efficient_long_sequence_amd.configs import WORKLOADS
from tests import gpu_harness as gh_

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = {
    # label: (B, H, grid_h, grid_w, d, land_h, land_w, k, s, kind, clusters, dtype)
    "ade_2d": (2, 2, 32, 32, 64, 7, 7, 49, 1, "clustered", 16, "bf16"),
    "long_s2": (1, 2, 1, 16384, 64, 1, 64, 64, 2, "runs", 64, "bf16"),
    "streaming_m600": (1, 1, 1, 12000, 64, 1, 600, 24, 2, "runs", 32, "bf16"),
    "d32_s1": (1, 2, 1, 777, 32, 1, 13, 50, 1, "clustered", 8, "bf16"),
    "f32_d64_s2": (2, 1, 12, 20, 64, 4, 5, 20, 2, "iid", 0, "f32"),
}


@pytest.mark.parametrize("label", list(CASES))
def test_official_variant_parity(label):
    B, H, gh, gw, d, lh, lw, k, s, kind, nc, dtype = CASES[label]
    Q, K, V = synth.make(B, H, gh * gw, d, kind, nc, dtype, zlib.crc32(label.encode()) % 1000)
    gh_.run_and_check(Q, K, V, (gh, gw, lh, lw), k, s, dtype, label=label, variant="official")


def test_official_variant_long_1m_sampled():
    """The benchmark's N = 1M shape, sampled rows and queries."""
    w = WORKLOADS["long_n1m"]
    Q, K, V = synth.make_from_workload(w)
    queries = np.sort(np.random.default_rng(2).choice(w.N, size=2048, replace=False))
    rows = np.sort(np.random.default_rng(3).choice(w.m, size=32, replace=False))
    gh_.run_and_check(Q, K, V, (w.grid_h, w.grid_w, w.land_h, w.land_w), w.k, w.s, w.dtype, heads=[(0, 1)],
                      queries=queries, rows=rows, label="long_n1m", variant="official")


def test_official_variant_closed_form():
    """k = N, s = 1: dense attention over keys [Q~ / sqrt(d); K] and values
    [V~; V] (torch, fp32 on the CPU) from the GPU's own Q~ and V~."""
    B, H, N, d = 1, 1, 256, 64
    Q, K, V = synth.make(B, H, N, d, "iid", 0, "bf16", 41)
    q, kk, v = (gh_.to_device(x, "bf16") for x in (Q, K, V))
    O, dbg = mita.forward(q, kk, v, (1, N, 1, 4), N, 1, debug=True, variant="official")
    torch.cuda.synchronize()
    Qt = dbg.qtilde[0, 0].float().cpu()
    Vt = dbg.vtilde[0, 0].cpu()
    keys = torch.cat([Qt / d ** 0.5, torch.tensor(K[0, 0])])
    vals = torch.cat([Vt, torch.tensor(V[0, 0])])
    ref = torch.softmax(torch.tensor(Q[0, 0]) @ keys.T / d ** 0.5, dim=-1) @ vals
    err = (O[0, 0].float().cpu() - ref).abs()
    assert float(err.max()) <= 2e-2 and float(err.mean()) <= 2e-3


def test_unknown_variant_rejected():
    q = torch.zeros((1, 1, 64, 32), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mita.MitaError):
        mita.forward(q, q, q, (1, 64, 1, 4), 8, 1, variant="dense")


# ---------------------------------------------------------------------------
# routing-only ablation (no shared entries); k is the matched k + m / s
# ---------------------------------------------------------------------------
ROUTED = {
    # label: (B, H, grid_h, grid_w, d, land_h, land_w, k, s, kind, clusters, dtype)
    "ade_2d_matched": (2, 2, 32, 32, 64, 7, 7, 98, 1, "clustered", 16, "bf16"),
    "long_s2_matched": (1, 2, 1, 16384, 64, 1, 64, 96, 2, "runs", 64, "bf16"),
    "streaming_k600": (1, 1, 1, 12000, 64, 1, 64, 600, 1, "runs", 32, "bf16"),
    "streaming_s2": (1, 2, 1, 9000, 64, 1, 48, 700, 2, "clustered", 8, "bf16"),
    "f32_d32": (1, 3, 7, 9, 32, 2, 3, 13, 1, "clustered", 4, "f32"),
}


@pytest.mark.parametrize("label", list(ROUTED))
def test_routed_variant_parity(label):
    B, H, gh, gw, d, lh, lw, k, s, kind, nc, dtype = ROUTED[label]
    Q, K, V = synth.make(B, H, gh * gw, d, kind, nc, dtype, zlib.crc32(label.encode()) % 1000)
    gh_.run_and_check(Q, K, V, (gh, gw, lh, lw), k, s, dtype, label=label, variant="routed")


def test_routed_variant_long_1m_matched_sampled():
    """The N = 1M ablation shape: m = 512, k = 512 + 512 = 1024 keys per expert."""
    w = WORKLOADS["long_n1m"]
    Q, K, V = synth.make_from_workload(w)
    queries = np.sort(np.random.default_rng(4).choice(w.N, size=2048, replace=False))
    rows = np.sort(np.random.default_rng(5).choice(w.m, size=24, replace=False))
    gh_.run_and_check(Q, K, V, (w.grid_h, w.grid_w, w.land_h, w.land_w), w.k + w.m, w.s, w.dtype,
                      heads=[(0, 0)], queries=queries, rows=rows, label="long_n1m_routed", variant="routed")


def test_routed_closed_form_is_dense():
    """k = N, s = 1, no shared entries: the output is dense attention, which
    the dense baseline kernel computes independently."""
    B, H, N, d = 1, 2, 512, 64
    Q, K, V = synth.make(B, H, N, d, "clustered", 8, "bf16", 43)
    q, kk, v = (gh_.to_device(x, "bf16") for x in (Q, K, V))
    O = mita.forward(q, kk, v, (1, N, 1, 8), N, 1, variant="routed")
    D = mita.dense_attention(q, kk, v)
    torch.cuda.synchronize()
    err = (O.float() - D.float()).abs()
    assert float(err.max()) <= 2e-2 and float(err.mean()) <= 2e-3
