"""CPU oracle for the MiTA (Mixture-of-Top-k Attention) forward pass.

TEST INFRASTRUCTURE ONLY.  This module is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the CPU-baseline leg of ``bench.py``; the
product path (the HIP library and its Python binding) never imports, calls or
links it.  It shares no code with the GPU path: everything here is written in
plain NumPy float64 straight from the method's definition.

Sources (all describe Wen et al., "Mixture-of-Top-k Attention: Efficient
Attention via Scalable Fast Weights", arXiv 2602.01219 v6):

* [tutorial]  MiTA tutorial at iwxt.cn/tutorials/mita-attention, chapters 1-8;
  each chapter names the paper section it restates.
* [gist]      gist.science summary of arXiv 2602.01219, section 2.2-2.3
  ("MiTA core mechanism", "Algorithm 1").
* [article]   bit.fan republication of the 新智元 article on MiTA, section
  "MiTA 如何构造专家".

Per (b, h) head, with N tokens, head dim d, m landmarks, k keys per routed
expert and s experts per query, the method computes (tutorial ch.4, paper
section 3.2 eqs. 5-12):

1. q~_i = average of the queries in pooling window W_i (average pooling of Q,
   not of K);
2. s~_ij = q~_i . k_j / sqrt(d) for every key j;
3. I_i = indices of the k largest s~_i. (the i-th routed expert);
4. v~_i = sum_j softmax_j(s~_i.) v_j over all N keys (the shared expert's
   values; its keys are the q~_i);
5. e(n) = the s landmarks with the largest q_n . q~_i;
6. K*_n = [q~_1..q~_m, k_j (j in I_e1), ..., k_j (j in I_es)],
   V*_n = [v~_1..v~_m, v_j ...]; o_n = V*_n softmax(K*_n q_n / sqrt(d)).

Readings where the pages are silent (each listed in the design notes):

* Q~ precision: the exact window mean, rounded once (nearest, ties to even)
  to the input dtype, because Q~ is an operand of step 2's product.
* Windows: adaptive, half-open [floor(i G / P), ceil((i + 1) G / P)) per grid
  axis; token and landmark grids are row-major (tutorial ch.5: top row holds
  tokens 0-3 of the 2x4 grid).
* Ties in top-k (step 3) and top-s (step 5): the lowest index wins; I_i is
  returned in ascending index order, e(n) by score descending then index.
* The routing score is the unscaled q . q~ (the 1/sqrt(d) scale is monotone).
* With s >= 2, a key present in two chosen experts appears twice in K*_n
  (the pages count m + s k entries and let experts overlap).
* Every logit is scaled by 1/sqrt(d) (tutorial ch.5).  The tutorial's ch.8
  (third check) notes that the authors' code pre-scales the shared key by
  d^-1/2 before the d^-1/2 logit scale, so its shared logits are q . q~ / d
  while routed logits stay q . k / sqrt(d): ``variant="official"`` in
  attend() and forward() follows that path and changes nothing else.
* ``variant="routed"`` is the routing-only ablation the pages compare with
  (republication, "LRA" section): no shared entries, the softmax runs over
  the s k routed keys alone; entries per query are matched by the caller
  (k + m / s).

Parity pins (tests/test_oracle_*.py): the tutorial's worked softmax fact
(ch.1), the merge identity (ch.4), the m = k = N counterexample value
0.5577646447 (ch.8, paper Appendix A), the closed form m = 1 / k = N against a
library dense attention, brute force over every subset on the tutorial's
8-token 2x4 shape (ch.5), the similarity-score count N(2m + sk) (ch.6) and
invariants.  Nothing here is "parity unpinned" except as stated in the tests.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "round_to_dtype", "bf16_round", "pool_windows", "landmarks", "landmark_scores",
    "topk_row", "topk", "shared_values", "route", "attend_one", "attend", "forward",
    "DotCounter", "rel_gap", "ORACLE_IS_TEST_INFRASTRUCTURE",
]

ORACLE_IS_TEST_INFRASTRUCTURE = True


# ---------------------------------------------------------------------------
# rounding to the input dtype
# ---------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even).

    bfloat16 keeps 8 significant bits and float32's exponent range.  Write a
    finite x as f * 2**e with 0.5 <= |f| < 1 (numpy.frexp); the spacing of
    bf16 values around x is 2**(e - 8) (2**-133 below the smallest normal
    2**-126).  x / spacing is then exact, numpy.rint rounds it half-to-even,
    and scaling back is exact.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    q = np.ldexp(1.0, e - 8)
    r = np.rint(x / q) * q
    big = np.abs(r) > 3.3895313892515355e38  # largest finite bf16
    r = np.where(big, np.copysign(np.inf, x), r)
    return np.where(x == 0, x, r)


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round float64 to the input dtype's value set ("f32" or "bf16"; "f64"
    keeps every value, for finite-difference checks of the backward pass)."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64).copy()
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_round(x)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# step 1: landmark queries by average pooling of Q
# ---------------------------------------------------------------------------
def _axis_windows(G: int, P: int):
    return [(math.floor(i * G / P), math.ceil((i + 1) * G / P)) for i in range(P)]


def pool_windows(grid_h: int, grid_w: int, land_h: int, land_w: int):
    """Token index sets W_i of the m = land_h * land_w pooling windows.

    Tutorial ch.4 step 1 (paper section 3.2): each landmark query is an
    average of several queries; ch.5 pools the 8-token example over a 2x4
    grid whose top row holds tokens 0-3 (row-major tokens).  Adaptive windows
    [floor(i G / P), ceil((i + 1) G / P)) per axis; landmark i = r * land_w + c.
    """
    rows = _axis_windows(grid_h, land_h)
    cols = _axis_windows(grid_w, land_w)
    out = []
    for r0, r1 in rows:
        for c0, c1 in cols:
            idx = [r * grid_w + c for r in range(r0, r1) for c in range(c0, c1)]
            out.append(np.asarray(idx, dtype=np.int64))
    return out


def landmarks(Q: np.ndarray, grid_h: int, grid_w: int, land_h: int, land_w: int,
              dtype: str) -> np.ndarray:
    """Q~ [m, d]: exact window means rounded once to the input dtype.

    Tutorial ch.4 step 1; gist section 2.2 ("average pooling of Q").  The sum
    over a window is exact (math.fsum), divided once in float64, then rounded
    once to the dtype.
    """
    Q = np.asarray(Q, dtype=np.float64)
    d = Q.shape[1]
    wins = pool_windows(grid_h, grid_w, land_h, land_w)
    Qt = np.empty((len(wins), d))
    for i, w in enumerate(wins):
        for c in range(d):
            Qt[i, c] = math.fsum(Q[w, c]) / len(w)
    return round_to_dtype(Qt, dtype)


# ---------------------------------------------------------------------------
# step 2: landmark-key scores
# ---------------------------------------------------------------------------
@dataclass
class DotCounter:
    """Counts every d-length similarity dot product the oracle evaluates.

    Tutorial ch.6 (paper section 3.2, complexity): landmark-key scores Nm,
    query-landmark scores Nm (reused for routing and the shared logits) and
    routed raw-KV scores Nsk, N(2m + sk) per head.
    """
    landmark_key: int = 0
    query_landmark: int = 0
    query_raw: int = 0

    @property
    def total(self) -> int:
        return self.landmark_key + self.query_landmark + self.query_raw


def landmark_scores(Qt: np.ndarray, K: np.ndarray, rows=None, counter: DotCounter | None = None):
    """s~ [m, N] (or the given rows): q~_i . k_j / sqrt(d) in float64.

    Tutorial ch.4 step 2: every landmark scores all N keys.
    """
    Qt = np.asarray(Qt, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    if rows is not None:
        Qt = Qt[rows]
    d = K.shape[1]
    if counter is not None:
        counter.landmark_key += Qt.shape[0] * K.shape[0]
    return (Qt @ K.T) / math.sqrt(d)


def rel_gap(a: float, b: float) -> float:
    """(a - b) / max(|a|, |b|), floored at 1e-30 in the denominator."""
    return (a - b) / max(abs(a), abs(b), 1e-30)


# ---------------------------------------------------------------------------
# step 3: top-k per landmark (the routed experts)
# ---------------------------------------------------------------------------
def topk_row(srow: np.ndarray, k: int):
    """Indices of the k largest scores of one landmark row, ascending order.

    Tutorial ch.4 step 2: the top-k raw KV of landmark i form routed expert
    i; ch.3: the chosen keys need not be contiguous and experts may overlap.
    Ties at the k-th value go to the lowest indices.  Returns (I_i, gap, t)
    with t the k-th largest value and gap the relative distance from t to the
    (k+1)-th largest value (None when k = N).
    """
    srow = np.asarray(srow, dtype=np.float64)
    N = srow.shape[0]
    if not 1 <= k <= N:
        raise ValueError("k out of range")
    t = np.partition(srow, N - k)[N - k]  # k-th largest by value
    above = np.flatnonzero(srow > t)
    equal = np.flatnonzero(srow == t)
    idx = np.sort(np.concatenate([above, equal[: k - above.size]]))
    gap = None
    if k < N:
        t_next = np.partition(srow, N - k - 1)[N - k - 1]  # (k+1)-th largest
        gap = rel_gap(t, t_next)
    return idx.astype(np.int64), gap, t


def topk(S: np.ndarray, k: int):
    rows = [topk_row(S[i], k) for i in range(S.shape[0])]
    I = np.stack([r[0] for r in rows])
    gaps = [r[1] for r in rows]
    thr = np.asarray([r[2] for r in rows])
    return I, gaps, thr


# ---------------------------------------------------------------------------
# step 4: shared-expert values
# ---------------------------------------------------------------------------
def shared_values(S: np.ndarray, V: np.ndarray) -> np.ndarray:
    """v~_i = sum_j softmax_j(s~_ij) v_j over all N keys.

    Tutorial ch.4 step 3: the same global scores are soft-maxed over all N
    and weight all of V (not only the top-k); the shared key is q~_i.
    """
    S = np.asarray(S, dtype=np.float64)
    w = np.exp(S - S.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return w @ np.asarray(V, dtype=np.float64)


# ---------------------------------------------------------------------------
# step 5: routing each query to its top-s landmarks
# ---------------------------------------------------------------------------
def route(Q: np.ndarray, Qt: np.ndarray, s: int, counter: DotCounter | None = None):
    """e [N, s]: for each query the s landmarks with the largest q . q~_i.

    Tutorial ch.4 step 4: compare q . q~_i and keep the top-s landmarks; the
    score only selects (no gate weights the experts' outputs).  Order: score
    descending, then landmark index ascending.  Also returns the unscaled
    scores R [N, m] (reused for the shared logits, tutorial ch.6).
    """
    Q = np.asarray(Q, dtype=np.float64)
    Qt = np.asarray(Qt, dtype=np.float64)
    m = Qt.shape[0]
    if not 1 <= s <= m:
        raise ValueError("s out of range")
    R = Q @ Qt.T
    if counter is not None:
        counter.query_landmark += R.size
    # a stable sort of -R keeps equal scores in ascending landmark order
    order = np.argsort(-R, axis=1, kind="stable")
    e = order[:, :s].astype(np.int64)
    return e, R


# ---------------------------------------------------------------------------
# steps 6-7: concatenation and one joint softmax
# ---------------------------------------------------------------------------
def attend_one(q, Kstar, Vstar):
    """o = V*^T softmax(K* q / sqrt(d)) for one query (tutorial ch.1 and ch.4).

    Returns (o, w) with w the joint weights (they sum to one: shared and
    routed entries compete for one total weight, tutorial ch.4 step 6).
    """
    q = np.asarray(q, dtype=np.float64)
    l = np.asarray(Kstar, dtype=np.float64) @ q / math.sqrt(q.shape[0])
    w = np.exp(l - l.max())
    w /= w.sum()
    return w @ np.asarray(Vstar, dtype=np.float64), w


def _concat(Qt, Vt, K, V, I, experts):
    """K*, V* for one query: all m shared pairs, then each chosen expert's k rows.

    Tutorial ch.4 step 5 and the formula V* = [V~, V^(e1), ..., V^(es)];
    duplicates across overlapping experts are kept.
    """
    sel = np.concatenate([I[e] for e in experts])
    return np.concatenate([Qt, K[sel]]), np.concatenate([Vt, V[sel]])


def attend(Q, K, V, Qt, Vt, I, e, R=None, counter: DotCounter | None = None,
           check_weights: bool = True, variant: str = "paper"):
    """O [N, d] given landmarks, shared values, experts I [m, k] and routes e [N, s].

    This is the conditional form of steps 6-7: the GPU's own I and e can be
    passed in.  Queries that route to the same expert tuple share K*, V*, so
    they are evaluated together with one matrix product; each row is still
    exactly softmax(K* q / sqrt(d)) V*.  When R (the unscaled q . q~ scores
    of step 5) is given, the shared logits reuse it instead of recomputing.
    variant="official" divides the m shared logits by d instead of sqrt(d)
    (tutorial ch.8, third check); the routed logits keep 1/sqrt(d).
    variant="routed" drops the m shared entries (routing-only ablation).
    """
    if variant not in ("paper", "official", "routed"):
        raise ValueError("variant must be 'paper', 'official' or 'routed'")
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Qt = np.asarray(Qt, dtype=np.float64)
    Vt = np.asarray(Vt, dtype=np.float64)
    N, d = Q.shape
    m, k = I.shape
    s = e.shape[1]
    sq = math.sqrt(d)
    sh = sq if variant == "paper" else float(d)
    O = np.empty((N, d))
    tuples, inv = np.unique(np.asarray(e), axis=0, return_inverse=True)
    inv = inv.reshape(-1)
    for g, experts in enumerate(tuples):
        ns = np.flatnonzero(inv == g)
        Ks, Vs = _concat(Qt, Vt, K, V, I, experts)
        assert Ks.shape[0] == m + s * k
        raw = Q[ns] @ Ks[m:].T / sq
        if counter is not None:
            counter.query_raw += raw.size
        if variant == "routed":
            l, vals = raw, Vs[m:]
        else:
            shared = (R[ns] if R is not None else Q[ns] @ Qt.T) / sh
            l, vals = np.concatenate([shared, raw], axis=1), Vs
        w = np.exp(l - l.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        if check_weights:
            assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        O[ns] = w @ vals
    return O


# ---------------------------------------------------------------------------
# the whole forward pass of one head
# ---------------------------------------------------------------------------
@dataclass
class HeadResult:
    O: np.ndarray
    Qt: np.ndarray
    I: np.ndarray
    e: np.ndarray
    Vt: np.ndarray
    topk_gaps: list
    topk_thresholds: np.ndarray
    counter: DotCounter = field(default_factory=DotCounter)


def forward(Q, K, V, grid_h, grid_w, land_h, land_w, k, s, dtype="bf16", row_block=64, variant="paper"):
    """MiTA forward pass of one head, steps 1-7 in the pages' order
    (``variant`` as in attend()).

    Q, K, V [N, d] hold values exactly representable in ``dtype``.  Landmark
    scores are evaluated in blocks of ``row_block`` landmark rows only to
    bound memory; each block is the same formula.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    N, d = Q.shape
    if N != grid_h * grid_w:
        raise ValueError("N must equal grid_h * grid_w")
    m = land_h * land_w
    if not (1 <= land_h <= grid_h and 1 <= land_w <= grid_w):
        raise ValueError("landmark grid must fit in the token grid")
    if not 1 <= k <= N:
        raise ValueError("k out of range")
    cnt = DotCounter()
    Qt = landmarks(Q, grid_h, grid_w, land_h, land_w, dtype)
    I = np.empty((m, k), dtype=np.int64)
    Vt = np.empty((m, d))
    tk_gaps, thr = [], np.empty(m)
    for r0 in range(0, m, row_block):
        rows = np.arange(r0, min(m, r0 + row_block))
        S = landmark_scores(Qt, K, rows=rows, counter=cnt)
        Ib, gb, tb = topk(S, k)
        I[rows] = Ib
        tk_gaps += gb
        thr[rows] = tb
        Vt[rows] = shared_values(S, V)
    e, R = route(Q, Qt, s, counter=cnt)
    O = attend(Q, K, V, Qt, Vt, I, e, R=R, counter=cnt, variant=variant)
    return HeadResult(O, Qt, I, e, Vt, tk_gaps, thr, cnt)
