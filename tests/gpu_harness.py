"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI binding, and compare with the CPU oracle.

Acceptance rules (floating point decides the index sets, so the comparison
is exact except within a relative band of 1e-4 around the decision value):

* Q~ bit-exact.
* I_i (top-k of landmark row i): if the oracle's relative gap between the
  k-th and (k+1)-th fp64 scores is >= 1e-4, the GPU set equals the oracle
  set; otherwise it must contain every key scoring above s_(k) + beta and no
  key scoring below s_(k) - beta, beta = 1e-4 max(|s_(k)|, |s_(k+1)|).
* e(n) (top-s routing): the same rule on q . q~, plus the GPU order is
  consistent with the fp64 scores up to beta.
* v~ and O: max-abs / mean-abs tolerances (bf16: 2e-2 / 2e-3; fp32: 1e-4
  max-abs).  O is compared with the oracle's joint softmax evaluated with the
  GPU's own (validated) I and e, and, on queries whose routing and experts
  are all outside the near-tie band, with the unconditional oracle as well.
"""
from __future__ import annotations

import math
import sys
import time
from dataclasses import dataclass, field

import numpy as np
import torch

from efficient_long_sequence_amd import mita, synth
from oracle import mita_oracle as mo

REL = 1e-4
TOL = {"bf16": dict(max=2e-2, mean=2e-3), "f32": dict(max=1e-4, mean=1e-4)}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x32: np.ndarray, dtype: str) -> torch.Tensor:
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(x32)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x32).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def run_gpu(Q, K, V, pool, k, s, dtype, variant="paper"):
    """Q, K, V: float32 arrays [B, H, N, d] (dtype-exact). Returns O and debug outputs."""
    q, kk, v = (to_device(x, dtype) for x in (Q, K, V))
    O, dbg = mita.forward(q, kk, v, pool, k, s, debug=True, variant=variant)
    torch.cuda.synchronize()
    return dict(O=to_host(O), topk=dbg.topk.cpu().numpy(), route=dbg.route.cpu().numpy(),
                vtilde=dbg.vtilde.cpu().numpy().astype(np.float64), qtilde=to_host(dbg.qtilde))


@dataclass
class Stats:
    rows: int = 0
    rows_exempt: int = 0
    routes: int = 0
    routes_exempt: int = 0
    o_max: float = 0.0
    o_mean: float = 0.0
    vt_max: float = 0.0
    vt_mean: float = 0.0
    o_strict_max: float = 0.0
    notes: list = field(default_factory=list)


def check_topk_row(srow: np.ndarray, got: np.ndarray, k: int) -> bool:
    """Returns True when the row was exempt (near tie); raises on a violation."""
    N = srow.size
    assert got.shape == (k,)
    assert np.all(np.diff(got) > 0), "top-k indices not strictly ascending"
    assert got[0] >= 0 and got[-1] < N
    if k == N:
        np.testing.assert_array_equal(got, np.arange(N))
        return False
    ref, gap, t = mo.topk_row(srow, k)
    if gap >= REL:
        np.testing.assert_array_equal(got, ref)
        return False
    srt = np.partition(srow, N - k - 1)
    t_next = srt[N - k - 1]
    beta = REL * max(abs(t), abs(t_next))
    must = np.flatnonzero(srow > t + beta)
    cannot = np.flatnonzero(srow < t - beta)
    gs = set(got.tolist())
    assert set(must.tolist()) <= gs, "near-tie row misses a key above the band"
    assert not (gs & set(cannot.tolist())), "near-tie row holds a key below the band"
    return True


def check_route_row(rrow: np.ndarray, got: np.ndarray, s: int) -> bool:
    m = rrow.size
    assert len(set(got.tolist())) == s and got.min() >= 0 and got.max() < m
    order = np.argsort(-rrow, kind="stable")
    ref = order[:s]
    exempt = False
    if s < m:
        a, b = rrow[order[s - 1]], rrow[order[s]]
        gap = (a - b) / max(abs(a), abs(b), 1e-30)
    else:
        gap = math.inf
    # order inside the list: descending up to the band
    for x, y in zip(got[:-1], got[1:]):
        bx = REL * max(abs(rrow[x]), abs(rrow[y]), 1e-30)
        assert rrow[x] >= rrow[y] - bx, "route list out of order"
    if gap >= REL:
        assert set(got.tolist()) == set(ref.tolist()), "route set differs"
        # exact order where consecutive oracle scores are well separated
        for i in range(s - 1):
            a, b = rrow[ref[i]], rrow[ref[i + 1]]
            if (a - b) / max(abs(a), abs(b), 1e-30) >= REL:
                assert got[i] == ref[i], "route order differs"
        return exempt
    t = rrow[order[s - 1]]
    t_next = rrow[order[s]]
    beta = REL * max(abs(t), abs(t_next))
    gs = set(got.tolist())
    assert set(np.flatnonzero(rrow > t + beta).tolist()) <= gs
    assert not (gs & set(np.flatnonzero(rrow < t - beta).tolist()))
    return True


def check_head(Qh, Kh, Vh, pool, k, s, dtype, gpu: dict, bh, stats: Stats,
               rows=None, queries=None, full_o=True, variant="paper"):
    """Compare one head; ``rows``/``queries`` sample landmark rows and queries
    (None = all)."""
    gh, gw, lh, lw = pool
    N, d = Qh.shape
    m = lh * lw
    b, h = bh
    Qt = mo.landmarks(Qh, gh, gw, lh, lw, dtype)
    np.testing.assert_array_equal(gpu["qtilde"][b, h], Qt, err_msg="Q~ not bit-exact")
    rows = np.arange(m) if rows is None else np.asarray(rows)
    I_gpu = gpu["topk"][b, h].astype(np.int64)
    e_gpu = gpu["route"][b, h].astype(np.int64)
    # landmark rows: top-k and v~ (every row's v~ is needed by the joint softmax)
    Vt = np.empty((m, d))
    I_or = np.empty((m, k), dtype=np.int64)
    row_exempt = np.zeros(m, dtype=bool)
    rowset = set(rows.tolist())
    full = rows.size == m and m * N <= (1 << 27)
    for r0 in range(0, m, 32):
        rr = np.arange(r0, min(m, r0 + 32))
        S = mo.landmark_scores(Qt, Kh, rows=rr)
        Vt[rr] = mo.shared_values(S, Vh)
        for j, r in enumerate(rr):
            if full:
                I_or[r] = mo.topk_row(S[j], k)[0]
            if r in rowset:
                row_exempt[r] = check_topk_row(S[j], I_gpu[r], k)
                stats.rows += 1
                stats.rows_exempt += int(row_exempt[r])
    if variant != "routed":  # the routing-only variant computes no shared values
        dv = np.abs(gpu["vtilde"][b, h][rows] - Vt[rows])
        stats.vt_max = max(stats.vt_max, float(dv.max()))
        stats.vt_mean = max(stats.vt_mean, float(dv.mean()))
    # routing
    qs = np.arange(N) if queries is None else np.asarray(queries)
    R = Qh[qs] @ Qt.T
    route_exempt = np.zeros(len(qs), dtype=bool)
    for j, n in enumerate(qs):
        route_exempt[j] = check_route_row(R[j], e_gpu[n], s)
    stats.routes += len(qs)
    stats.routes_exempt += int(route_exempt.sum())
    # output against the conditional oracle (GPU's I and e, oracle v~)
    O_c = mo.attend(Qh[qs], Kh, Vh, Qt, Vt, I_gpu, e_gpu[qs], variant=variant)
    do = np.abs(gpu["O"][b, h][qs] - O_c)
    stats.o_max = max(stats.o_max, float(do.max()))
    stats.o_mean = max(stats.o_mean, float(do.mean()))
    # and against the unconditional oracle where no decision was near a tie
    if full:
        sel = ~route_exempt & ~row_exempt[e_gpu[qs]].any(axis=1)
        if sel.any():
            e_or = mo.route(Qh[qs][sel], Qt, s)[0]
            O_u = mo.attend(Qh[qs][sel], Kh, Vh, Qt, Vt, I_or, e_or, variant=variant)
            stats.o_strict_max = max(stats.o_strict_max, float(np.abs(gpu["O"][b, h][qs][sel] - O_u).max()))
    return stats


def assert_tolerances(stats: Stats, dtype: str, scale: float = 1.0):
    """``scale``: the factor V was multiplied by (v~ and O scale with it, and
    so do their rounding errors)."""
    tol = {key: val * scale for key, val in TOL[dtype].items()}
    assert stats.vt_max <= tol["max"], f"v~ max-abs {stats.vt_max}"
    assert stats.o_max <= tol["max"], f"O max-abs {stats.o_max}"
    assert stats.o_strict_max <= tol["max"], f"O (unconditional) max-abs {stats.o_strict_max}"
    if dtype == "bf16":
        assert stats.vt_mean <= tol["mean"], f"v~ mean-abs {stats.vt_mean}"
        assert stats.o_mean <= tol["mean"], f"O mean-abs {stats.o_mean}"


def run_and_check(Q, K, V, pool, k, s, dtype, heads=None, rows=None, queries=None, label="", variant="paper",
                  tol_scale=1.0):
    """Run the whole batch on the GPU, check the listed heads (default all).
    ``tol_scale``: the tolerances' scale (the factor V was multiplied by)."""
    B, H = Q.shape[:2]
    t0 = time.time()
    say(f"[gpu] {label} B={B} H={H} N={Q.shape[2]} d={Q.shape[3]} pool={pool} k={k} s={s} {dtype} {variant}")
    gpu = run_gpu(Q, K, V, pool, k, s, dtype, variant)
    say(f"[gpu] {label} ran in {time.time() - t0:.2f}s; checking")
    # (a NaN would compare as no error below: every output must be finite)
    for key in ("O", "vtilde", "qtilde"):
        assert np.isfinite(gpu[key]).all(), f"{label}: non-finite values in {key}"
    stats = Stats()
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for (b, h) in heads:
        check_head(Q[b, h].astype(np.float64), K[b, h].astype(np.float64), V[b, h].astype(np.float64),
                   pool, k, s, dtype, gpu, (b, h), stats, rows=rows, queries=queries, variant=variant)
    assert_tolerances(stats, dtype, tol_scale)
    say(f"[gpu] {label} ok: rows {stats.rows} (exempt {stats.rows_exempt}), routes {stats.routes} "
        f"(exempt {stats.routes_exempt}), v~ max {stats.vt_max:.2e} mean {stats.vt_mean:.2e}, "
        f"O max {stats.o_max:.2e} mean {stats.o_mean:.2e}, O strict max {stats.o_strict_max:.2e}, "
        f"{time.time() - t0:.1f}s")
    return gpu, stats
