"""Seeded synthetic inputs for the MiTA forward pass.

This module is shared by the oracle-side tests, the GPU parity tests and the
benchmark.  It draws Q, K, V and rounds them to the working dtype; it holds
none of the method's arithmetic (no pooling, scoring, selection, routing or
softmax).

Value recipes (all drawn in float64 from NumPy's PCG64, then rounded once):

* ``iid``        Q, K, V ~ N(0, 1) independently.
* ``clustered``  per (b, h): G centres C[g] ~ N(0, I_d); every token n gets a
                 cluster z_n ~ U{0..G-1}; q_n = C[z_n] + 0.3 eps,
                 k_n = C[z_n] + 0.3 eps' (independent noise, shared centre and
                 cluster id); V ~ N(0, 1).
* ``runs``       as ``clustered`` but the cluster ids come in runs: the
                 sequence is cut into runs of length U{1..256}, each run
                 drawing one cluster id ~ U{0..G-1}.
* upstream gradients (``make_grad``) for the backward pass: dO ~ N(0, 1)
  independently, from their own seed.

The three shapes stand in for the workloads the MiTA pages evaluate on:
ImageNet-1K DeiT-S patches (14x14), ADE20K segmentation patches (32x32 and
40x40) and the long-sequence throughput test with m*k = N/4 (MiTA tutorial
(iwxt.cn), ch.7, paper section 4.3 / Fig. 5).  No dataset item is used.

Rounding: float64 -> float32 by NumPy's cast (round-to-nearest-even), then for
bf16 a round-to-nearest-even on the float32 bit pattern.  The result is kept
both as float32 values (exactly representable in the dtype) and, for bf16, as
the raw uint16 bit patterns used to fill device tensors.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SPREAD = 0.3
RUN_MAX = 256


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class HeadInputs:
    """Inputs of one (b, h) head, already rounded to the working dtype."""
    q: np.ndarray  # [N, d] float32 (dtype-exact)
    k: np.ndarray
    v: np.ndarray


def _round(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(x32))
    raise ValueError(dtype)


def _cluster_ids(rng: np.random.Generator, n: int, n_clusters: int, kind: str) -> np.ndarray:
    if kind == "clustered":
        return rng.integers(0, n_clusters, size=n)
    # runs of length U{1..RUN_MAX}, one cluster id per run
    ids = np.empty(n, dtype=np.int64)
    pos = 0
    while pos < n:
        n_runs = max(16, (n - pos) // 64)
        lens = rng.integers(1, RUN_MAX + 1, size=n_runs)
        labs = rng.integers(0, n_clusters, size=n_runs)
        for ln, lab in zip(lens, labs):
            if pos >= n:
                break
            e = min(n, pos + int(ln))
            ids[pos:e] = lab
            pos = e
    return ids


def make_head(rng: np.random.Generator, n: int, d: int, kind: str, n_clusters: int,
              dtype: str) -> HeadInputs:
    if kind == "iid":
        q = rng.standard_normal((n, d))
        k = rng.standard_normal((n, d))
        v = rng.standard_normal((n, d))
    elif kind in ("clustered", "runs"):
        centres = rng.standard_normal((n_clusters, d))
        z = _cluster_ids(rng, n, n_clusters, kind)
        q = centres[z] + SPREAD * rng.standard_normal((n, d))
        k = centres[z] + SPREAD * rng.standard_normal((n, d))
        v = rng.standard_normal((n, d))
    else:
        raise ValueError(kind)
    return HeadInputs(_round(q, dtype), _round(k, dtype), _round(v, dtype))


def make(B: int, H: int, N: int, d: int, kind: str, n_clusters: int, dtype: str,
         seed: int):
    """Return Q, K, V as float32 arrays [B, H, N, d] holding dtype-exact values.

    One ``SeedSequence(seed)`` per workload, spawned once per (b, h) head in
    row-major (b, h) order, so any single head can be regenerated alone with
    :func:`make_one_head`.
    """
    Q = np.empty((B, H, N, d), dtype=np.float32)
    K = np.empty_like(Q)
    V = np.empty_like(Q)
    children = np.random.SeedSequence(seed).spawn(B * H)
    for bh, ss in enumerate(children):
        b, h = divmod(bh, H)
        hi = make_head(np.random.Generator(np.random.PCG64(ss)), N, d, kind, n_clusters, dtype)
        Q[b, h], K[b, h], V[b, h] = hi.q, hi.k, hi.v
    return Q, K, V


def make_one_head(B: int, H: int, N: int, d: int, kind: str, n_clusters: int, dtype: str,
                  seed: int, b: int, h: int) -> HeadInputs:
    ss = np.random.SeedSequence(seed).spawn(B * H)[b * H + h]
    return make_head(np.random.Generator(np.random.PCG64(ss)), N, d, kind, n_clusters, dtype)


def make_from_workload(w, seed_offset: int = 0):
    return make(w.B, w.H, w.N, w.d, w.kind, w.n_clusters, w.dtype, w.seed + seed_offset)


def make_grad(B: int, H: int, N: int, d: int, dtype: str, seed: int) -> np.ndarray:
    """Upstream gradient dO [B, H, N, d] ~ N(0, 1) (float32, dtype-exact)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x6772])))
    return _round(rng.standard_normal((B, H, N, d)), dtype).astype(np.float32)
