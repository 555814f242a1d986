"""Brute force on the tutorial's 8-token shape (MiTA tutorial (iwxt.cn), ch.5).

The chapter walks 8 tokens with d = 2 on a 2x4 grid (top row tokens 0-3,
bottom row 4-7), one head, s = 1, 1/sqrt(d) scaling, no projections.  Its
Q/K/V numbers sit in a collapsed widget that was not captured, so seeded
values stand in (parity of the page's own intermediate values is unpinned).

Everything below is written independently of the oracle's code: the pooling
windows are listed by hand from the grid, top-k is the lexicographically
smallest index set whose smallest score is at least every excluded score
(found by enumerating all subsets), routing enumerates landmarks, and each
output is an unstabilised sum of exponentials.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import mita_oracle as mo

# pooling layouts on the 2x4 grid: (land_h, land_w) -> windows listed by hand
LAYOUTS = {
    (1, 1): [[0, 1, 2, 3, 4, 5, 6, 7]],
    (1, 2): [[0, 1, 4, 5], [2, 3, 6, 7]],
    (2, 2): [[0, 1], [2, 3], [4, 5], [6, 7]],
    (1, 4): [[0, 4], [1, 5], [2, 6], [3, 7]],
    (2, 4): [[i] for i in range(8)],
}


def _nearest_bf16(x):
    """Nearest bfloat16 by searching the table of all bf16 values; ties to even bits."""
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    vals = bits.view(torch.bfloat16).to(torch.float64).numpy()
    b = np.arange(1 << 16)
    ok = np.isfinite(vals)
    vals, b = vals[ok], b[ok]
    d = np.abs(vals - x)
    best = np.flatnonzero(d == d.min())
    if best.size > 1:
        even = [i for i in best if b[i] % 2 == 0]
        best = np.asarray(even)
    return float(vals[best[0]])


def _topk_brute(scores, k):
    N = len(scores)
    valid = [c for c in itertools.combinations(range(N), k)
             if min(scores[j] for j in c) >= max([scores[j] for j in range(N) if j not in c],
                                                  default=-math.inf)]
    return list(min(valid))


def _route_brute(r, s):
    m = len(r)
    best = None
    for c in itertools.combinations(range(m), s):
        if min(r[i] for i in c) >= max([r[i] for i in range(m) if i not in c], default=-math.inf):
            best = c if best is None else min(best, c)
    return sorted(best, key=lambda i: (-r[i], i))


def _expsum_attention(q, keys, values):
    d = len(q)
    ws = [math.exp(sum(a * b for a, b in zip(q, kk)) / math.sqrt(d)) for kk in keys]
    z = sum(ws)
    return [sum(w * v[c] for w, v in zip(ws, values)) / z for c in range(len(values[0]))]


def _brute_head(Q, K, V, land, k, s, rounding):
    d = Q.shape[1]
    wins = LAYOUTS[land]
    Qt = [[rounding(sum(Q[t, c] for t in w) / len(w)) for c in range(d)] for w in wins]
    m = len(Qt)
    S = [[sum(a * b for a, b in zip(Qt[i], K[j])) / math.sqrt(d) for j in range(8)] for i in range(m)]
    I = [_topk_brute(S[i], k) for i in range(m)]
    Vt = []
    for i in range(m):
        ws = [math.exp(x) for x in S[i]]
        Vt.append([sum(w * V[j, c] for j, w in enumerate(ws)) / sum(ws) for c in range(d)])
    e, O = [], []
    for n in range(8):
        r = [sum(a * b for a, b in zip(Q[n], Qt[i])) for i in range(m)]
        en = _route_brute(r, s)
        e.append(en)
        keys = list(Qt) + [list(K[j]) for x in en for j in I[x]]
        vals = list(Vt) + [list(V[j]) for x in en for j in I[x]]
        O.append(_expsum_attention(list(Q[n]), keys, vals))
    return np.array(Qt), np.array(I), np.array(Vt), np.array(e), np.array(O)


def _cases():
    for land in LAYOUTS:
        m = land[0] * land[1]
        for k in range(1, 9):
            for s in range(1, m + 1):
                yield land, k, s


@pytest.mark.parametrize("values", ["random_bf16", "dyadic_ties"])
def test_tutorial_shape_bruteforce(values):
    rng = np.random.default_rng(2024 if values == "random_bf16" else 99)
    if values == "random_bf16":
        Q, K, V = (mo.bf16_round(rng.standard_normal((8, 2))) for _ in range(3))
        rounding, dtype = _nearest_bf16, "bf16"
    else:
        # small dyadic values: window means are exact and many scores tie
        Q, K, V = (rng.integers(-2, 3, size=(8, 2)) / 2.0 for _ in range(3))
        rounding, dtype = (lambda x: x), "bf16"
    n_checked = 0
    for land, k, s in _cases():
        Qt, I, Vt, e, O = _brute_head(Q, K, V, land, k, s, rounding)
        r = mo.forward(Q, K, V, 2, 4, land[0], land[1], k, s, dtype=dtype)
        np.testing.assert_array_equal(r.Qt, Qt)
        np.testing.assert_array_equal(r.I, I)
        np.testing.assert_allclose(r.Vt, Vt, rtol=1e-12, atol=1e-13)
        np.testing.assert_array_equal(r.e, e)
        np.testing.assert_allclose(r.O, O, rtol=1e-12, atol=1e-13)
        n_checked += 1
    assert n_checked == sum(8 * l[0] * l[1] for l in LAYOUTS)
