"""The seeded input generator: determinism, dtype exactness and value structure."""
import numpy as np
import pytest

from efficient_long_sequence_amd import synth
from efficient_long_sequence_amd.configs import WORKLOADS
from oracle import mita_oracle as mo


def test_deterministic_and_per_head_regeneration():
    a = synth.make(2, 3, 64, 8, "clustered", 16, "bf16", seed=5)
    b = synth.make(2, 3, 64, 8, "clustered", 16, "bf16", seed=5)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    one = synth.make_one_head(2, 3, 64, 8, "clustered", 16, "bf16", 5, 1, 2)
    np.testing.assert_array_equal(one.q, a[0][1, 2])
    np.testing.assert_array_equal(one.v, a[2][1, 2])
    c = synth.make(2, 3, 64, 8, "clustered", 16, "bf16", seed=6)
    assert not np.array_equal(a[0], c[0])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_values_are_exact_in_dtype(dtype):
    Q, K, V = synth.make(1, 2, 300, 16, "iid", 0, dtype, seed=1)
    for x in (Q, K, V):
        x64 = x.astype(np.float64)
        np.testing.assert_array_equal(mo.round_to_dtype(x64, dtype), x64)


def test_bf16_bits_roundtrip():
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    b = synth.f32_to_bf16_bits(x)
    y = synth.bf16_bits_to_f32(b)
    np.testing.assert_array_equal(y.astype(np.float64), mo.bf16_round(x.astype(np.float64)))


def test_clustered_queries_and_keys_share_clusters():
    hi = synth.make_one_head(1, 1, 2000, 64, "clustered", 16, "f32", 3, 0, 0)
    # same-token q.k is large (shared centre), random pairs are not
    same = np.einsum("nd,nd->n", hi.q, hi.k).mean()
    rnd = np.einsum("nd,nd->n", hi.q, np.roll(hi.k, 1, axis=0)).mean()
    assert same > 50 and same > 2 * abs(rnd) + 10
    assert abs(hi.v.mean()) < 0.05 and abs(hi.v.std() - 1) < 0.05


def test_runs_have_bounded_length():
    rng = np.random.default_rng(1)
    z = synth._cluster_ids(rng, 100000, 64, "runs")
    change = np.flatnonzero(np.diff(z) != 0)
    lens = np.diff(np.concatenate([[-1], change, [len(z) - 1]]))
    assert lens.max() <= 256 * 3  # adjacent runs may draw the same id
    assert 80 < lens.mean() < 200


def test_workload_table():
    w = WORKLOADS["deit_s_n196"]
    assert (w.N, w.m, w.k, w.s, w.tokens) == (196, 25, 25, 1, 64 * 6 * 196)
    for name, w in WORKLOADS.items():
        assert w.m <= w.N and 1 <= w.k <= w.N and 1 <= w.s <= w.m
    assert WORKLOADS["long_n1m"].m * WORKLOADS["long_n1m"].k == WORKLOADS["long_n1m"].N // 4 * 1
    for name in ("long_n64k_s1", "long_n256k", "long_n1m"):
        w = WORKLOADS[name]
        assert w.m * w.k == w.N // 4  # m k = N / 4 as in the long-sequence test
