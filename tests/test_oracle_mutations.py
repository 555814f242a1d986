"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in the oracle (on the CPU, by monkeypatching a
single function) and checks that at least one pin in test_oracle_facts.py or
test_oracle_bruteforce.py then fails.  The oracle itself is not modified.
"""
import math

import numpy as np
import pytest

from oracle import mita_oracle as mo
from tests import test_oracle_bruteforce as tb
from tests import test_oracle_facts as tf

PINS = [
    tf.test_softmax_worked_example,
    tf.test_appendix_a_counterexample_value,
    tf.test_entries_per_query_and_weights_sum_to_one,
    lambda: tf.test_similarity_score_count(64, 8, 8, 8, 4, 2, 7, 3),
    tf.test_merge_identity,
    lambda: tf.test_closed_form_k_equals_n(4, 8, 2, 2, 4),
    lambda: tf.test_closed_form_k_equals_n(1, 37, 1, 1, 8),
    tf.test_pool_matches_library_adaptive_average,
    tf.test_window_geometry_14_to_5,
    tf.test_bf16_round_matches_library_on_float32_inputs,
    tf.test_topk_ties_go_to_lowest_index_bruteforce,
    tf.test_route_bruteforce_with_ties,
    tf.test_affine_values_map_to_affine_outputs,
    tf.test_equal_keys_give_mean_values,
    tf.test_s_equals_m_counts_duplicates,
    lambda: tb.test_tutorial_shape_bruteforce("random_bf16"),
    lambda: tb.test_tutorial_shape_bruteforce("dyadic_ties"),
]


def _some_pin_fails():
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


_orig = {n: getattr(mo, n) for n in ["landmark_scores", "shared_values", "topk_row", "route",
                                     "attend", "attend_one", "_concat", "_axis_windows",
                                     "bf16_round", "landmarks"]}


def _scores_no_scale(Qt, K, rows=None, counter=None):
    return _orig["landmark_scores"](Qt, K, rows, counter) * math.sqrt(K.shape[1])


def _shared_wrong_axis(S, V):
    w = np.exp(S - S.max(axis=1, keepdims=True))
    w /= w.sum(axis=0, keepdims=True)
    return w @ V


def _shared_topk_only(S, V):
    # averages only over the top-k, which the tutorial rules out
    k = max(1, S.shape[1] // 3)
    out = np.empty((S.shape[0], V.shape[1]))
    for i in range(S.shape[0]):
        idx, _, _ = _orig["topk_row"](S[i], k)
        w = np.exp(S[i, idx] - S[i, idx].max())
        out[i] = (w / w.sum()) @ V[idx]
    return out


def _topk_highest_index_ties(srow, k):
    idx, gap, t = _orig["topk_row"](srow[::-1], k)
    return np.sort(len(srow) - 1 - idx), gap, t


def _topk_off_by_one(srow, k):
    if k >= len(srow):
        return _orig["topk_row"](srow, k)
    idx, gap, t = _orig["topk_row"](srow, k + 1)
    return idx[:k], gap, t


def _route_lowest(Q, Qt, s, counter=None):
    e, R, g = _orig["route"](-np.asarray(Q), Qt, s, counter)
    return e, -R, g


def _route_ties_high(Q, Qt, s, counter=None):
    Qt = np.asarray(Qt)
    e, R, g = _orig["route"](Q, Qt[::-1], s, counter)
    return Qt.shape[0] - 1 - e, R[:, ::-1], g


def _concat_values_are_keys(Qt, Vt, K, V, I, experts):
    Ks, Vs = _orig["_concat"](Qt, Vt, K, V, I, experts)
    m = Qt.shape[0]
    Vs = Vs.copy()
    Vs[:m] = Qt
    return Ks, Vs


def _concat_no_shared(Qt, Vt, K, V, I, experts):
    sel = np.concatenate([I[e] for e in experts])
    return np.concatenate([Qt[:0], K[sel]]), np.concatenate([Vt[:0], V[sel]])


def _concat_dedup(Qt, Vt, K, V, I, experts):
    sel = np.unique(np.concatenate([I[e] for e in experts]))
    return np.concatenate([Qt, K[sel]]), np.concatenate([Vt, V[sel]])


def _attend_separate_softmax(Q, K, V, Qt, Vt, I, e, R=None, counter=None, check_weights=True, variant="paper"):
    # normalises the shared and routed parts separately and adds them: o1 + o2
    Q = np.asarray(Q, float)
    O = np.empty_like(Q)
    for n in range(Q.shape[0]):
        sel = np.concatenate([I[x] for x in e[n]])
        if counter is not None:
            counter.query_raw += sel.size
        o1, _ = _orig["attend_one"](Q[n], Qt, Vt)
        o2, _ = _orig["attend_one"](Q[n], K[sel], V[sel])
        O[n] = o1 + o2
    return O


def _attend_one_no_scale(q, Ks, Vs):
    return _orig["attend_one"](np.asarray(q) * math.sqrt(len(q)), Ks, Vs)


def _windows_floor_end(G, P):
    return [(math.floor(i * G / P), math.floor((i + 1) * G / P)) for i in range(P)]


def _bf16_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    return np.trunc(x / q) * q


def _landmarks_pool_k(Q, gh, gw, lh, lw, dtype):
    # pools with a column-major token order instead of row-major
    Q = np.asarray(Q).reshape(gh, gw, -1).transpose(1, 0, 2).reshape(gh * gw, -1)
    return _orig["landmarks"](Q, gw, gh, lw, lh, dtype)


MUTATIONS = {
    "scores without 1/sqrt(d)": ("landmark_scores", _scores_no_scale),
    "shared softmax over the wrong axis": ("shared_values", _shared_wrong_axis),
    "shared values only over the top-k": ("shared_values", _shared_topk_only),
    "top-k ties to the highest index": ("topk_row", _topk_highest_index_ties),
    "top-k off by one": ("topk_row", _topk_off_by_one),
    "routing picks the lowest score": ("route", _route_lowest),
    "routing ties to the highest index": ("route", _route_ties_high),
    "shared values replaced by shared keys": ("_concat", _concat_values_are_keys),
    "shared expert dropped": ("_concat", _concat_no_shared),
    "overlapping experts deduplicated": ("_concat", _concat_dedup),
    "separate softmax per branch, outputs added": ("attend", _attend_separate_softmax),
    "joint logits without 1/sqrt(d)": ("attend_one", _attend_one_no_scale),
    "windows end at floor": ("_axis_windows", _windows_floor_end),
    "bf16 rounding truncates": ("bf16_round", _bf16_truncate),
    "token grid read column-major": ("landmarks", _landmarks_pool_k),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(mo, attr, fn)
    assert _some_pin_fails(), f"no pin fails when the oracle has: {name}"
