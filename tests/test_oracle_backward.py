"""Pins of the backward oracle (oracle/mita_backward.py).

The backward differentiates the forward with the experts I and routes e held
fixed.  Its torch restatement of the forward is checked against the numpy
oracle's forward, and its gradients against central differences of that
numpy forward (float64 inputs, no rounding of q~), on shapes whose pooling
windows overlap, with s = 2 and experts that share keys, for all three
variants.  Closed forms: the routing-only variant at k = N, s = 1 is dense
attention, whose gradient a library attention gives; value-shift invariance
(sum_j dV_j = sum_n dO_n) and, for the routing-only variant, sum_j dK_j = 0.
Planted mistakes (a frozen v~, no pooling path, the paper scale in the
official variant, experts deduplicated) must each fail a pin.
"""
import math

import numpy as np
import pytest
import torch

from oracle import mita_backward as mb
from oracle import mita_oracle as mo

VARIANTS = ["paper", "official", "routed"]


def _problem(seed, gh, gw, lh, lw, d, k, s, dtype="f64"):
    rng = np.random.default_rng(seed)
    N = gh * gw
    Q, K, V, dO = (mo.round_to_dtype(rng.standard_normal((N, d)), dtype) for _ in range(4))
    r = mo.forward(Q, K, V, gh, gw, lh, lw, k, s, dtype=dtype)
    return Q, K, V, dO, r.I, r.e


def _np_forward(Q, K, V, gh, gw, lh, lw, I, e, variant):
    """The numpy oracle's forward with I and e fixed and no rounding."""
    Qt = mo.landmarks(Q, gh, gw, lh, lw, "f64")
    Vt = mo.shared_values(mo.landmark_scores(Qt, K), V)
    return mo.attend(Q, K, V, Qt, Vt, I, e, variant=variant)


def _central_differences(Q, K, V, dO, gh, gw, lh, lw, I, e, variant, h=1e-5):
    grads = []
    args = [Q.copy(), K.copy(), V.copy()]
    for which in range(3):
        g = np.empty_like(args[which])
        for idx in np.ndindex(*g.shape):
            x0 = args[which][idx]
            args[which][idx] = x0 + h
            fp = float((_np_forward(*args, gh, gw, lh, lw, I, e, variant) * dO).sum())
            args[which][idx] = x0 - h
            fm = float((_np_forward(*args, gh, gw, lh, lw, I, e, variant) * dO).sum())
            args[which][idx] = x0
            g[idx] = (fp - fm) / (2 * h)
        grads.append(g)
    return grads


# (gh, gw, lh, lw, d, k, s): 11 tokens in 3 overlapping 1-D windows; a 3x4
# grid with 2x2 overlapping windows; s = 2 so keys appear in two experts
SHAPES = [(1, 11, 1, 3, 4, 5, 2), (3, 4, 2, 2, 3, 4, 2), (2, 5, 1, 4, 2, 6, 1)]


@pytest.mark.parametrize("variant", VARIANTS)
def test_restated_forward_matches_the_oracle(variant):
    for sh in SHAPES:
        gh, gw, lh, lw, d, k, s = sh
        Q, K, V, dO, I, e = _problem(3, gh, gw, lh, lw, d, k, s, dtype="bf16")
        r = mo.forward(Q, K, V, gh, gw, lh, lw, k, s, dtype="bf16", variant=variant)
        O = mb.forward_fixed(Q, K, V, gh, gw, lh, lw, r.I, r.e, dtype="bf16", variant=variant)
        np.testing.assert_allclose(O, r.O, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("shape", SHAPES)
def test_gradients_match_central_differences(variant, shape):
    gh, gw, lh, lw, d, k, s = shape
    Q, K, V, dO, I, e = _problem(11 + d, gh, gw, lh, lw, d, k, s)
    got = mb.backward(Q, K, V, dO, gh, gw, lh, lw, I, e, dtype="f64", variant=variant, chunk=5)
    ref = _central_differences(Q, K, V, dO, gh, gw, lh, lw, I, e, variant)
    for g, r_ in zip(got, ref):
        np.testing.assert_allclose(g, r_, rtol=1e-6, atol=1e-8)


def test_experts_share_keys_in_the_pinned_shapes():
    """The finite-difference shapes exercise duplicated keys (s = 2 with
    overlapping experts) and overlapping pooling windows."""
    gh, gw, lh, lw, d, k, s = SHAPES[0]
    Q, K, V, dO, I, e = _problem(11 + d, gh, gw, lh, lw, d, k, s)
    dup = [len(np.intersect1d(I[a], I[b])) for a, b in e]
    assert max(dup) > 0
    wins = mo.pool_windows(gh, gw, lh, lw)
    assert len(set(wins[0]) & set(wins[1])) > 0


@pytest.mark.parametrize("variant", VARIANTS)
def test_value_shift_invariance(variant):
    """Adding u to every value row adds u to every output (both softmaxes sum
    to one), so sum_j dV_j = sum_n dO_n."""
    Q, K, V, dO, I, e = _problem(5, 4, 8, 2, 2, 8, 6, 2, dtype="bf16")
    dQ, dK, dV = mb.backward(Q, K, V, dO, 4, 8, 2, 2, I, e, dtype="bf16", variant=variant)
    np.testing.assert_allclose(dV.sum(axis=0), dO.sum(axis=0), rtol=1e-12, atol=1e-12)


def test_routed_key_gradients_sum_to_zero():
    """Routing-only: adding u to every key shifts each query's logits by the
    same q . u / sqrt(d), which its softmax ignores."""
    Q, K, V, dO, I, e = _problem(6, 4, 8, 2, 2, 8, 6, 2, dtype="bf16")
    _, dK, _ = mb.backward(Q, K, V, dO, 4, 8, 2, 2, I, e, dtype="bf16", variant="routed")
    assert np.abs(dK.sum(axis=0)).max() < 1e-12 * max(1.0, np.abs(dK).max())


def test_routed_closed_form_is_dense_attention_gradient():
    """k = N, s = 1, routing only: every query attends to all keys once, so
    the gradient is dense attention's (library attention, float64 autograd)."""
    N, d = 40, 8
    Q, K, V, dO, I, e = _problem(8, 1, N, 1, 4, d, N, 1, dtype="bf16")
    got = mb.backward(Q, K, V, dO, 1, N, 1, 4, I, e, dtype="bf16", variant="routed")
    q, k_, v = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    o = torch.nn.functional.scaled_dot_product_attention(q[None, None], k_[None, None], v[None, None])[0, 0]
    (o * torch.tensor(dO)).sum().backward()
    for g, t in zip(got, (q, k_, v)):
        np.testing.assert_allclose(g, t.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_lse_helpers_match_definitions():
    Q, K, V, dO, I, e = _problem(9, 1, 30, 1, 3, 4, 7, 2, dtype="bf16")
    Qt = mo.landmarks(Q, 1, 30, 1, 3, "bf16")
    L = mb.joint_lse(Q, K, Qt, I, e)
    n = 13
    sel = np.concatenate([I[x] for x in e[n]])
    logits = np.concatenate([Qt @ Q[n], K[sel] @ Q[n]]) / 2.0
    assert abs(L[n] - math.log(np.exp(logits).sum())) < 1e-12
    Lm = mb.landmark_lse(Qt, K)
    assert abs(Lm[1] - math.log(np.exp(Qt[1] @ K.T / 2.0).sum())) < 1e-12


def test_pool_matrix_rows_average_their_windows():
    P = mb.pool_matrix(3, 4, 2, 2).numpy()
    np.testing.assert_allclose(P.sum(axis=1), 1.0)
    Q = np.random.default_rng(1).standard_normal((12, 3))
    np.testing.assert_allclose(P @ Q, mo.landmarks(Q, 3, 4, 2, 2, "f64"), rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# planted mistakes: each must fail a pin above
# ---------------------------------------------------------------------------
def _frozen_shared_values(Qt, K, V):
    return _orig_shared(Qt, K, V).detach()


def _no_pooling_path(Q, gh, gw, lh, lw, dtype):
    return _orig_landmarks(Q, gh, gw, lh, lw, dtype).detach()


def _official_as_paper(q, K, V, Qt, Vt, I, e_rows, variant):
    return _orig_joint(q, K, V, Qt, Vt, I, e_rows, "paper" if variant == "official" else variant)


def _dedup_experts(q, K, V, Qt, Vt, I, e_rows, variant):
    # a key chosen by both experts of a query counted once: replace a
    # duplicate by the first key of the row (a plausible "set union" slip)
    I = np.array(I)
    out = []
    for r in range(q.shape[0]):
        a, b = e_rows[r]
        Ib = I[b].copy()
        Ib[np.isin(Ib, I[a])] = I[a][0]
        II = I.copy()
        II[b] = Ib
        out.append(_orig_joint(q[r:r + 1], K, V, Qt, Vt, II, e_rows[r:r + 1], variant))
    return torch.cat(out)


_orig_shared = mb._shared_values
_orig_landmarks = mb._landmarks
_orig_joint = mb._joint


@pytest.mark.parametrize("name,fn,variant", [
    ("_shared_values", _frozen_shared_values, "paper"),
    ("_landmarks", _no_pooling_path, "paper"),
    ("_joint", _official_as_paper, "official"),
    ("_joint", _dedup_experts, "paper"),
])
def test_backward_pins_catch_planted_mistakes(monkeypatch, name, fn, variant):
    monkeypatch.setattr(mb, name, fn)
    with pytest.raises(AssertionError):
        test_gradients_match_central_differences(variant, SHAPES[0])
