"""Pins of the oracle's "official" variant: shared logits q . q~ / d.

The MiTA tutorial (chapter 8, third check) notes that the authors' code
pre-scales the shared key by d^-1/2 before the usual d^-1/2 logit scale, so
its shared logits are q . q~ / d while routed logits stay q . k / sqrt(d);
pooling, landmark scores, top-k, shared values and routing are unchanged.
These CPU tests pin that reading against a library dense attention and
against the paper variant, and check that plausible slips are caught.
"""
import math

import numpy as np
import pytest
import torch

from oracle import mita_oracle as mo


def _rand_head(rng, N, d, dtype="bf16"):
    return [mo.round_to_dtype(rng.standard_normal((N, d)), dtype) for _ in range(3)]


def _dense_fp64(q, keys, values):
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(keys), t(values))[0, 0].numpy()


@pytest.mark.parametrize("gh,gw,lh,lw,d", [(1, 37, 1, 1, 8), (4, 8, 2, 2, 4), (1, 50, 1, 5, 16)])
def test_official_closed_form_k_equals_n(gh, gw, lh, lw, d):
    """k = N, s = 1: dense softmax attention over keys [Q~ / sqrt(d); K] at the
    library's 1/sqrt(d) scale gives shared logits q . q~ / d and routed logits
    q . k / sqrt(d); values [V~; V] with the unchanged V~."""
    N = gh * gw
    rng = np.random.default_rng(7 * N + d)
    Q, K, V = _rand_head(rng, N, d)
    r = mo.forward(Q, K, V, gh, gw, lh, lw, N, 1, dtype="bf16", variant="official")
    Vt_lib = _dense_fp64(r.Qt, K, V)
    np.testing.assert_allclose(r.Vt, Vt_lib, rtol=1e-12, atol=1e-13)
    O_lib = _dense_fp64(Q, np.concatenate([r.Qt / math.sqrt(d), K]), np.concatenate([Vt_lib, V]))
    np.testing.assert_allclose(r.O, O_lib, rtol=1e-11, atol=1e-12)


def test_official_equals_paper_when_d_is_one():
    """1/d = 1/sqrt(d) at d = 1: both variants give the same output (here on
    the tutorial's m = k = N counterexample shape, output 0.5577646447)."""
    Q = K = V = np.array([[0.0], [1.0]])
    a = mo.forward(Q, K, V, 1, 2, 1, 2, 2, 1, dtype="f32")
    b = mo.forward(Q, K, V, 1, 2, 1, 2, 2, 1, dtype="f32", variant="official")
    np.testing.assert_array_equal(a.O, b.O)
    assert abs(b.O[0, 0] - 0.5577646447) < 5e-11


def test_official_changes_only_the_shared_logits():
    rng = np.random.default_rng(3)
    Q, K, V = _rand_head(rng, 96, 8)
    a = mo.forward(Q, K, V, 1, 96, 1, 6, 5, 2, dtype="bf16")
    b = mo.forward(Q, K, V, 1, 96, 1, 6, 5, 2, dtype="bf16", variant="official")
    for x, y in ((a.Qt, b.Qt), (a.I, b.I), (a.e, b.e), (a.Vt, b.Vt)):
        np.testing.assert_array_equal(x, y)
    assert np.abs(a.O - b.O).max() > 1e-3
    # per query: softmax over [q.q~/d, q.k/sqrt(d) of the routed keys]
    n = 17
    sel = np.concatenate([b.I[e] for e in b.e[n]])
    logits = np.concatenate([b.Qt @ Q[n] / 8.0, K[sel] @ Q[n] / math.sqrt(8.0)])
    w = np.exp(logits - logits.max())
    w /= w.sum()
    o = w @ np.concatenate([b.Vt, V[sel]])
    np.testing.assert_allclose(b.O[n], o, rtol=1e-12, atol=1e-13)


def test_unknown_variant_is_rejected():
    with pytest.raises(ValueError):
        mo.attend(np.zeros((2, 2)), np.zeros((2, 2)), np.zeros((2, 2)), np.zeros((1, 2)), np.zeros((1, 2)),
                  np.zeros((1, 1), dtype=np.int64), np.zeros((2, 1), dtype=np.int64), variant="dense")


# planted mistakes in the variant must fail a pin above
_orig_attend = mo.attend


def _ignores_variant(*a, **kw):
    kw["variant"] = "paper"
    return _orig_attend(*a, **kw)


def _scales_every_logit(Q, K, V, Qt, Vt, I, e, R=None, counter=None, check_weights=True, variant="paper"):
    if variant == "paper":
        return _orig_attend(Q, K, V, Qt, Vt, I, e, R=R, counter=counter, check_weights=check_weights)
    d = Q.shape[1]
    # 1/d on the routed logits too: same as scaling q by 1/sqrt(d) everywhere
    return _orig_attend(np.asarray(Q) / math.sqrt(d), K, V, Qt, Vt, I, e, R=None, counter=counter,
                        check_weights=check_weights)


@pytest.mark.parametrize("mistake", [_ignores_variant, _scales_every_logit])
def test_variant_pins_catch_planted_mistakes(monkeypatch, mistake):
    monkeypatch.setattr(mo, "attend", mistake)
    with pytest.raises(AssertionError):
        test_official_closed_form_k_equals_n(4, 8, 2, 2, 4)


# ---------------------------------------------------------------------------
# routing-only ablation: no shared entries
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("gh,gw,lh,lw,d", [(1, 37, 1, 1, 8), (4, 8, 2, 2, 4), (1, 50, 1, 5, 16)])
def test_routed_closed_form_is_dense_attention(gh, gw, lh, lw, d):
    """k = N, s = 1 and no shared entries: every query attends to all N keys,
    which is plain dense attention over K and V."""
    N = gh * gw
    rng = np.random.default_rng(11 * N + d)
    Q, K, V = _rand_head(rng, N, d)
    r = mo.forward(Q, K, V, gh, gw, lh, lw, N, 1, dtype="bf16", variant="routed")
    np.testing.assert_allclose(r.O, _dense_fp64(Q, K, V), rtol=1e-11, atol=1e-12)


def test_routed_softmax_runs_over_the_routed_keys_only():
    rng = np.random.default_rng(5)
    Q, K, V = _rand_head(rng, 96, 8)
    a = mo.forward(Q, K, V, 1, 96, 1, 6, 5, 2, dtype="bf16")
    b = mo.forward(Q, K, V, 1, 96, 1, 6, 5, 2, dtype="bf16", variant="routed")
    for x, y in ((a.Qt, b.Qt), (a.I, b.I), (a.e, b.e)):
        np.testing.assert_array_equal(x, y)
    for n in (0, 41, 95):
        sel = np.concatenate([b.I[e] for e in b.e[n]])
        logits = K[sel] @ Q[n] / math.sqrt(8.0)
        w = np.exp(logits - logits.max())
        np.testing.assert_allclose(b.O[n], (w / w.sum()) @ V[sel], rtol=1e-12, atol=1e-13)
    assert np.abs(a.O - b.O).max() > 1e-3


def _routed_keeps_shared(*a, **kw):
    if kw.get("variant") == "routed":
        kw["variant"] = "paper"
    return _orig_attend(*a, **kw)


def test_routed_pin_catches_a_kept_shared_branch(monkeypatch):
    monkeypatch.setattr(mo, "attend", _routed_keeps_shared)
    with pytest.raises(AssertionError):
        test_routed_closed_form_is_dense_attention(4, 8, 2, 2, 4)
