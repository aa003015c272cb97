"""Pins of the oracle's offline profiling and neuron index.

CSDN article, overall-architecture section: offline, activations are
profiled and a placement of neurons is computed under the hardware's
capacity; hada.io README summary: the hot set ("GPU index") is bounded by a
memory budget.  Reading: top-K neurons by activation count, ties to the
lower id, K = min(n, floor(budget / bytes per neuron)).
- brute force over all K-subsets of tiny layers: the hot set has the maximal
  total count, and among maximal sets it is the lexicographically smallest;
- numpy.lexsort((ids, -counts)) gives the same order (a library routine);
- the hot set for a smaller budget is a prefix of the larger one;
- activation counts against numpy float64 matmuls.
"""
import itertools

import numpy as np
import pytest

from oracle import oracle as O


@pytest.mark.parametrize("seed", range(6))
def test_index_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = 9
    counts = rng.integers(0, 4, n).astype(np.uint32)       # many ties
    for K in range(n + 1):
        perm, n_hot = O.build_neuron_index(counts, budget_bytes=K * 10 + 9, bytes_per_neuron=10)
        assert n_hot == K
        best = max(sum(int(counts[i]) for i in c) for c in itertools.combinations(range(n), K))
        cands = [c for c in itertools.combinations(range(n), K)
                 if sum(int(counts[i]) for i in c) == best]
        assert tuple(sorted(perm[:K].tolist())) == min(cands)


def test_index_matches_lexsort_and_prefix():
    rng = np.random.default_rng(1)
    n = 5000
    counts = rng.zipf(1.5, n).clip(max=1024).astype(np.uint32)
    perm, n_hot = O.build_neuron_index(counts, 10 ** 12, 7)
    assert n_hot == n
    ids = np.arange(n)
    assert np.array_equal(perm, np.lexsort((ids, -counts.astype(np.int64))))
    small, k1 = O.build_neuron_index(counts, 1300 * 7 + 6, 7)
    assert k1 == 1300 and np.array_equal(small, perm)


def test_index_budget_edge_cases():
    counts = np.array([3, 1, 2], np.uint32)
    assert O.build_neuron_index(counts, 0, 5)[1] == 0
    assert O.build_neuron_index(counts, 14, 5)[1] == 2
    assert O.build_neuron_index(counts, 10 ** 9, 5)[1] == 3
    perm, k = O.build_neuron_index(np.zeros(0, np.uint32), 100, 5)
    assert perm.size == 0 and k == 0


@pytest.mark.parametrize("act", ["relu", "reglu"])
def test_profile_counts_match_numpy(act):
    rng = np.random.default_rng(6)
    n, d, S = 120, 64, 50
    W = (rng.standard_normal((n, d)) / 8).astype(np.float16)
    D = rng.standard_normal((n, d)).astype(np.float16)
    b = rng.standard_normal(n).astype(np.float32) * 0.5
    X = rng.standard_normal((S, d)).astype(np.float16)
    if act == "relu":
        part = O.Part(d, W, D, act="relu", b_up=b)
    else:
        part = O.Part(d, D, D, act="reglu", W_gate=W, b_gate=b)
    c, c32, amb = O.profile_counts(part, X, band=1e-9)
    pre = X.astype(np.float64) @ W.astype(np.float64).T + b.astype(np.float64)
    assert amb.sum() == 0
    assert np.array_equal(c, (pre > 0).sum(axis=0).astype(np.uint32))
    assert np.array_equal(c32, c)
