"""Pins of the CPU oracle against what the MiTA pages and the mathematics fix.

Every test here runs on the CPU.  Each one is chosen so that a plausible slip
in the oracle (a dropped term, a wrong sign or index, a transposed operand, a
wrong normalisation) fails it.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import mita_oracle as mo

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rand_head(rng, N, d, dtype="f32"):
    x = [rng.standard_normal((N, d)) for _ in range(3)]
    return [mo.round_to_dtype(a, dtype) for a in x]


# ---------------------------------------------------------------------------
# worked facts the pages print
# ---------------------------------------------------------------------------
def test_softmax_worked_example():
    g = _gold("softmax_worked_example.json")
    # logits q . k / sqrt(d) = 0 for both keys: q = 0
    q = np.zeros(1)
    Ks = np.array([[3.0], [-7.0]])
    o, w = mo.attend_one(q, Ks, np.array(g["values"])[:, None])
    assert np.allclose(w, g["weights"], atol=0, rtol=0)
    assert o[0] == g["output"]


def test_appendix_a_counterexample_value():
    g = _gold("appendix_a_counterexample.json")
    Q, K, V = (np.array(g[x]) for x in "QKV")
    r = mo.forward(Q, K, V, g["grid_h"], g["grid_w"], g["land_h"], g["land_w"], g["k"], g["s"],
                   dtype="f32")
    np.testing.assert_array_equal(r.Qt, Q)  # window of one token: Q~ = Q
    np.testing.assert_allclose(r.Vt[:, 0], g["shared_values"], rtol=0, atol=1e-15)
    o = r.O[g["query"], 0]
    assert abs(o - g["mita_output_printed"]) < 0.5 * 10 ** -g["printed_digits"]
    dense = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(Q[None, None]), torch.tensor(K[None, None]), torch.tensor(V[None, None]))
    assert float(dense[0, 0, g["query"], 0]) == g["dense_output"]
    assert abs(o - g["dense_output"]) > 0.05


def test_entries_per_query_and_weights_sum_to_one():
    g = _gold("entries_per_query.json")
    rng = np.random.default_rng(7)
    for case in g["cases"]:
        m, k, s = case["m"], case["k"], case["s"]
        assert m + s * k == case["entries"]
        N, d = 4 * m, 8
        Q, K, V = _rand_head(rng, N, d)
        r = mo.forward(Q, K, V, 1, N, 1, m, k, s, dtype="f32")
        n = 3
        experts = r.e[n]
        Ks, Vs = mo._concat(r.Qt, r.Vt, K, V, r.I, experts)
        assert Ks.shape[0] == case["entries"] and Vs.shape[0] == case["entries"]
        o, w = mo.attend_one(Q[n], Ks, Vs)
        assert abs(w.sum() - 1.0) < 1e-14
        np.testing.assert_allclose(o, r.O[n], rtol=0, atol=1e-13)


@pytest.mark.parametrize("N,d,gh,gw,lh,lw,k,s", [
    (64, 8, 8, 8, 2, 2, 5, 1),
    (64, 8, 8, 8, 4, 2, 7, 3),
    (96, 4, 1, 96, 1, 12, 9, 2),
    (196, 16, 14, 14, 5, 5, 25, 1),
])
def test_similarity_score_count(N, d, gh, gw, lh, lw, k, s):
    """Tutorial ch.6: the method evaluates N(2m + sk) similarity scores per head."""
    rng = np.random.default_rng(N + k)
    Q, K, V = _rand_head(rng, N, d, "bf16")
    r = mo.forward(Q, K, V, gh, gw, lh, lw, k, s, dtype="bf16")
    m = lh * lw
    assert r.counter.landmark_key == N * m
    assert r.counter.query_landmark == N * m
    assert r.counter.query_raw == N * s * k
    assert r.counter.total == N * (2 * m + s * k)


def test_merge_identity():
    """Tutorial ch.4: branch outputs merge as (Z1 o1 + Z2 o2) / (Z1 + Z2); o1 + o2 is wrong."""
    rng = np.random.default_rng(3)
    for trial in range(20):
        n_ent, d = int(rng.integers(2, 40)), int(rng.integers(1, 9))
        q = rng.standard_normal(d)
        Ks = rng.standard_normal((n_ent, d))
        Vs = rng.standard_normal((n_ent, d))
        o, _ = mo.attend_one(q, Ks, Vs)
        cut = rng.permutation(n_ent)
        a, b = cut[: n_ent // 2 or 1], cut[n_ent // 2 or 1:]
        if b.size == 0:
            continue
        o1, _ = mo.attend_one(q, Ks[a], Vs[a])
        o2, _ = mo.attend_one(q, Ks[b], Vs[b])
        Z1 = np.exp(Ks[a] @ q / math.sqrt(d)).sum()
        Z2 = np.exp(Ks[b] @ q / math.sqrt(d)).sum()
        np.testing.assert_allclose((Z1 * o1 + Z2 * o2) / (Z1 + Z2), o, rtol=1e-12, atol=1e-13)
        assert np.abs((o1 + o2) - o).max() > 1e-3


# ---------------------------------------------------------------------------
# closed forms and special cases that reduce to a library routine
# ---------------------------------------------------------------------------
def _dense_fp64(q, keys, values):
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(keys), t(values))[0, 0].numpy()


@pytest.mark.parametrize("gh,gw,lh,lw,d", [(1, 37, 1, 1, 8), (6, 6, 1, 1, 5), (4, 8, 2, 2, 4), (1, 50, 1, 5, 16)])
def test_closed_form_k_equals_n(gh, gw, lh, lw, d):
    """With k = N (and s = 1) every routed expert is all of K, V, so MiTA is dense
    softmax attention over keys [Q~; K] and values [V~; V], with
    V~ = softmax(Q~ K^T / sqrt(d)) V.  m = 1 is the case named for this check."""
    N = gh * gw
    rng = np.random.default_rng(N * d)
    Q, K, V = _rand_head(rng, N, d, "bf16")
    r = mo.forward(Q, K, V, gh, gw, lh, lw, N, 1, dtype="bf16")
    Vt_lib = _dense_fp64(r.Qt, K, V)
    np.testing.assert_allclose(r.Vt, Vt_lib, rtol=1e-12, atol=1e-13)
    O_lib = _dense_fp64(Q, np.concatenate([r.Qt, K]), np.concatenate([Vt_lib, V]))
    np.testing.assert_allclose(r.O, O_lib, rtol=1e-11, atol=1e-12)


def test_pool_matches_library_adaptive_average():
    """Landmark windows and means against torch.nn.functional.adaptive_avg_pool2d,
    whose windows are [floor(iG/P), ceil((i+1)G/P))."""
    rng = np.random.default_rng(11)
    for gh, gw, lh, lw in [(14, 14, 5, 5), (32, 32, 7, 7), (40, 40, 7, 7), (16, 16, 4, 4),
                           (1, 4096, 1, 8), (5, 9, 3, 4), (2, 4, 1, 2), (3, 3, 3, 3)]:
        d = 6
        Q = rng.standard_normal((gh * gw, d))
        ref = torch.nn.functional.adaptive_avg_pool2d(
            torch.tensor(Q.T.reshape(d, gh, gw)), (lh, lw)).numpy().reshape(d, lh * lw).T
        wins = mo.pool_windows(gh, gw, lh, lw)
        mean = np.stack([Q[w].mean(axis=0) for w in wins])
        np.testing.assert_allclose(mean, ref, rtol=1e-13, atol=1e-14)
        # the oracle's rounded landmarks are the nearest representable values
        Qt = mo.landmarks(Q, gh, gw, lh, lw, "f32")
        np.testing.assert_array_equal(Qt, ref.astype(np.float32).astype(np.float64))


def test_window_geometry_14_to_5():
    rows = mo._axis_windows(14, 5)
    assert rows == [(0, 3), (2, 6), (5, 9), (8, 12), (11, 14)]
    assert [b - a for a, b in mo._axis_windows(32, 7)] == [5, 6, 5, 6, 5, 6, 5]
    assert [b - a for a, b in mo._axis_windows(40, 7)] == [6, 7, 7, 6, 7, 7, 6]
    assert mo._axis_windows(65536, 128)[5] == (2560, 3072)


def test_window_one_token_gives_q():
    rng = np.random.default_rng(5)
    Q = mo.round_to_dtype(rng.standard_normal((12, 4)), "bf16")
    np.testing.assert_array_equal(mo.landmarks(Q, 3, 4, 3, 4, "bf16"), Q)


# ---------------------------------------------------------------------------
# rounding to bf16
# ---------------------------------------------------------------------------
def _all_bf16_values():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    vals = bits.view(torch.bfloat16).to(torch.float64).numpy()
    b = np.arange(1 << 16)
    ok = np.isfinite(vals)
    return vals[ok], b[ok]


def test_bf16_round_matches_library_on_float32_inputs():
    rng = np.random.default_rng(1)
    x32 = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-30,
                          rng.standard_normal(2000) * 1e30]).astype(np.float32)
    # exact ties: float32 values halfway between bf16 neighbours
    ties = (np.arange(1, 300, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x32 = np.concatenate([x32, ties, -ties])
    lib = torch.tensor(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(mo.bf16_round(x32.astype(np.float64)), lib)


def test_bf16_round_is_nearest_ties_even_on_float64_inputs():
    vals, bits = _all_bf16_values()
    order = np.argsort(vals, kind="stable")
    vals, bits = vals[order], bits[order]
    keep = np.concatenate([[True], np.diff(vals) > 0])  # drop -0 duplicate of +0
    vals, bits = vals[keep], bits[keep]
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-20, 20, 5000),
                        (vals[1000:1100] + vals[1001:1101]) / 2])  # exact midpoints
    got = mo.bf16_round(x)
    j = np.searchsorted(vals, x)
    lo, hi = vals[j - 1], vals[j]
    dlo, dhi = x - lo, hi - x
    even_lo = (bits[j - 1] & 1) == 0
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(even_lo, lo, hi)))
    want = np.where(np.isin(x, vals), x, want)
    np.testing.assert_array_equal(got, want)


# ---------------------------------------------------------------------------
# selection and routing against library routines and brute force
# ---------------------------------------------------------------------------
def test_topk_matches_library_on_distinct_scores():
    rng = np.random.default_rng(9)
    for N, k in [(100, 1), (100, 37), (513, 512), (4096, 200)]:
        s = rng.standard_normal(N)
        idx, gap, t = mo.topk_row(s, k)
        ref = np.sort(torch.topk(torch.tensor(s), k).indices.numpy())
        np.testing.assert_array_equal(idx, ref)
        assert t == np.sort(s)[::-1][k - 1]
        if k < N:
            srt = np.sort(s)[::-1]
            assert gap == pytest.approx((srt[k - 1] - srt[k]) / max(abs(srt[k - 1]), abs(srt[k])))


def test_topk_ties_go_to_lowest_index_bruteforce():
    rng = np.random.default_rng(4)
    for _ in range(200):
        N = int(rng.integers(1, 10))
        k = int(rng.integers(1, N + 1))
        s = rng.integers(-2, 3, size=N).astype(np.float64)  # many ties
        idx, _, _ = mo.topk_row(s, k)
        valid = [c for c in itertools.combinations(range(N), k)
                 if min(s[list(c)]) >= max(np.delete(s, list(c)), default=-np.inf)]
        assert list(idx) == list(min(valid))


def test_route_bruteforce_with_ties():
    rng = np.random.default_rng(6)
    for _ in range(100):
        m = int(rng.integers(1, 7))
        s = int(rng.integers(1, m + 1))
        Qt = rng.integers(-1, 2, size=(m, 3)).astype(np.float64)
        Q = rng.integers(-1, 2, size=(5, 3)).astype(np.float64)
        e, R = mo.route(Q, Qt, s)
        for n in range(5):
            r = Q[n] @ Qt.T
            order = sorted(range(m), key=lambda i: (-r[i], i))
            assert list(e[n]) == order[:s]


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def test_affine_values_map_to_affine_outputs():
    """V -> aV + b gives O -> aO + b: pins both softmax normalisations (V~ and O)."""
    rng = np.random.default_rng(12)
    Q, K, V = _rand_head(rng, 48, 4)
    a, b = 2.5, -0.75
    r1 = mo.forward(Q, K, V, 6, 8, 2, 2, 6, 2, dtype="f32")
    r2 = mo.forward(Q, K, a * V + b, 6, 8, 2, 2, 6, 2, dtype="f32")
    np.testing.assert_allclose(r2.O, a * r1.O + b, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r2.Vt, a * r1.Vt + b, rtol=1e-12, atol=1e-12)


def test_equal_keys_give_mean_values():
    rng = np.random.default_rng(13)
    Q, _, V = _rand_head(rng, 30, 4)
    K = np.tile(rng.standard_normal(4), (30, 1))
    r = mo.forward(Q, K, V, 5, 6, 1, 3, 4, 1, dtype="f32")
    np.testing.assert_allclose(r.Vt, np.tile(V.mean(axis=0), (3, 1)), rtol=1e-13, atol=1e-14)
    # all scores tie: every expert is the k lowest indices
    np.testing.assert_array_equal(r.I, np.tile(np.arange(4), (3, 1)))


def test_unselected_value_still_contributes_through_shared_expert():
    """Tutorial ch.5 quiz: a KV not chosen by any top-k still enters through V~."""
    rng = np.random.default_rng(14)
    Q, K, V = _rand_head(rng, 40, 4)
    r = mo.forward(Q, K, V, 5, 8, 1, 2, 3, 1, dtype="f32")
    unused = sorted(set(range(40)) - set(r.I.reshape(-1).tolist()))
    assert unused
    V2 = V.copy()
    V2[unused[0]] += 5.0
    r2 = mo.forward(Q, K, V2, 5, 8, 1, 2, 3, 1, dtype="f32")
    np.testing.assert_array_equal(r.I, r2.I)
    assert np.abs(r2.O - r.O).max() > 1e-6


def test_s_equals_m_counts_duplicates():
    """Overlapping experts keep duplicate keys: with s = m every query sees m + m k entries."""
    rng = np.random.default_rng(15)
    Q, K, V = _rand_head(rng, 12, 3)
    r = mo.forward(Q, K, V, 3, 4, 1, 2, 12, 2, dtype="f32")  # k = N: both experts are all keys
    for n in range(12):
        Ks, Vs = mo._concat(r.Qt, r.Vt, K, V, r.I, r.e[n])
        o, _ = mo.attend_one(Q[n], Ks, Vs)
        # keys counted twice: dense over [Q~; K; K] with [V~; V; V]
        ref = _dense_fp64(Q[n:n + 1], np.concatenate([r.Qt, K, K]), np.concatenate([r.Vt, V, V]))
        np.testing.assert_allclose(o, ref[0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(r.O[n], ref[0], rtol=1e-12, atol=1e-13)
