"""Pins of the oracle's sparse FFN, merge and dense FFN.

Facts the pages fix (CSDN article, section on sparse activation: neurons
that do not fire contribute nothing to the output; section on the hybrid
design: the partitions' partial results merge into the layer output):
- dense FFN against numpy float64 matmuls (ReLU and ReGLU);
- the sparse FFN over the all-ones mask, over the true firing set, and over
  any superset of it equals the dense FFN bit for bit (the extra terms are
  exact zeros and the order is shared);
- brute force over all 2^n masks on tiny layers: y(M) == y(M & firing);
- rows outside the list may be NaN-poisoned without changing y;
- ReGLU with W_up row = e_k and x_k = 1 reduces to the ReLU FFN on the gate;
- squared ReLU equals ReGLU with the gate set to the up projection
  (max(0, a)^2 == max(0, a) * a), and an integer fixture gives h = a^2;
- Q4_0: the FFN on Q4_0 weights equals the FFN on the same weights decoded
  to float32 (the decode is exact);
- split + merge equals the unsplit layer bit for bit on integer fixtures,
  including the worked example of the hybrid-design figure (tests/golden).
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import oracle as O
from workload import synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _layer(rng, n, d, act="relu", dt=np.float32, integer=False, bias=True):
    if integer:
        W_up = rng.integers(-3, 4, (n, d)).astype(dt)
        W_gate = rng.integers(-3, 4, (n, d)).astype(dt)
        W_downT = rng.integers(-3, 4, (n, d)).astype(dt)
        b = rng.integers(-3, 4, n).astype(np.float32)
    else:
        W_up = (rng.standard_normal((n, d)) / np.sqrt(d)).astype(dt)
        W_gate = (rng.standard_normal((n, d)) / np.sqrt(d)).astype(dt)
        W_downT = (rng.standard_normal((n, d)) / np.sqrt(n)).astype(dt)
        b = (rng.standard_normal(n) * 0.5).astype(np.float32)
    if act in ("relu", "sqrelu"):
        return O.Part(d, W_up, W_downT, act=act, b_up=b if bias else None)
    return O.Part(d, W_up, W_downT, act="reglu", W_gate=W_gate, b_gate=b if bias else None)


def _np_ffn(part, x, act="relu"):
    W_up, W_gate, b_up, b_gate, W_downT = [None if a is None else a.astype(np.float64)
                                           for a in part.arrays]
    xx = x.astype(np.float64)
    up = xx @ W_up.T + (0 if b_up is None else b_up)
    if act == "sqrelu":
        h = np.maximum(up, 0) ** 2
    elif W_gate is None:
        h = np.maximum(up, 0)
    else:
        h = np.maximum(xx @ W_gate.T + (0 if b_gate is None else b_gate), 0) * up
    return h @ W_downT, up, h


def _firing(part, x, act="relu"):
    _, up, h = _np_ffn(part, x, act)
    return np.flatnonzero((h != 0).any(axis=0)).astype(np.int32)


@pytest.mark.parametrize("act", ["relu", "reglu", "sqrelu"])
@pytest.mark.parametrize("dt", [np.float32, np.float16])
def test_dense_matches_numpy(act, dt):
    rng = np.random.default_rng(11)
    part = _layer(rng, 150, 64, act, dt)
    x = rng.standard_normal((3, 64)).astype(dt)
    ref, _, _ = _np_ffn(part, x, act)
    np.testing.assert_allclose(O.dense_ffn(part, x), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act", ["relu", "reglu", "sqrelu"])
def test_sparse_equals_dense_on_full_true_and_superset(act):
    rng = np.random.default_rng(5)
    part = _layer(rng, 300, 64, act)
    x = rng.standard_normal((1, 64)).astype(np.float32)
    dense = O.dense_ffn(part, x)
    assert np.array_equal(O.sparse_ffn(part, x, np.arange(300)), dense)
    fire = _firing(part, x, act)
    assert 0 < fire.size < 300
    assert np.array_equal(O.sparse_ffn(part, x, fire), dense)
    extra = np.union1d(fire, rng.choice(300, 40, replace=False)).astype(np.int32)
    assert np.array_equal(O.sparse_ffn(part, x, extra), dense)


@pytest.mark.parametrize("act", ["relu", "reglu", "sqrelu"])
def test_brute_force_all_masks(act):
    rng = np.random.default_rng(9 + len(act))
    n, d = 10, 16
    part = _layer(rng, n, d, act)
    x = rng.standard_normal((1, d)).astype(np.float32)
    fire = set(_firing(part, x, act).tolist())
    assert 0 < len(fire) < n
    for bits in itertools.product([0, 1], repeat=n):
        M = [i for i in range(n) if bits[i]]
        MT = [i for i in M if i in fire]
        assert np.array_equal(O.sparse_ffn(part, x, M), O.sparse_ffn(part, x, MT))


def test_nan_poisoned_rows_outside_list():
    rng = np.random.default_rng(2)
    n, d = 90, 64
    part = _layer(rng, n, d, "reglu")
    x = rng.standard_normal((2, d)).astype(np.float32)
    L = np.sort(rng.choice(n, 20, replace=False)).astype(np.int32)
    y = O.sparse_ffn(part, x, L)
    W_up, W_gate, b_up, b_gate, W_downT = [None if a is None else a.copy() for a in part.arrays]
    out = np.setdiff1d(np.arange(n), L)
    for a in (W_up, W_gate, W_downT):
        a[out] = np.nan
    b_gate[out] = np.nan
    poisoned = O.Part(d, W_up, W_downT, act="reglu", W_gate=W_gate, b_gate=b_gate)
    assert np.array_equal(O.sparse_ffn(poisoned, x, L), y)


def test_reglu_reduces_to_relu_on_gate():
    rng = np.random.default_rng(4)
    n, d, k = 40, 32, 5
    W_gate = (rng.standard_normal((n, d)) / 6).astype(np.float32)
    b_gate = rng.standard_normal(n).astype(np.float32)
    W_downT = rng.standard_normal((n, d)).astype(np.float32)
    W_up = np.zeros((n, d), np.float32)
    W_up[:, k] = 1.0
    x = rng.standard_normal((1, d)).astype(np.float32)
    x[0, k] = 1.0
    reglu = O.Part(d, W_up, W_downT, act="reglu", W_gate=W_gate, b_gate=b_gate)
    relu = O.Part(d, W_gate, W_downT, act="relu", b_up=b_gate)
    assert np.array_equal(O.dense_ffn(reglu, x), O.dense_ffn(relu, x))


def test_squared_relu_is_reglu_with_gate_equal_to_up():
    """max(0, a)^2 == max(0, a) * a: the squared-ReLU FFN equals the ReGLU FFN of the
    same layer with W_gate := W_up and b_gate := b_up, bit for bit (the same dot
    product in the same order on both branches)."""
    rng = np.random.default_rng(23)
    n, d = 120, 64
    sq = _layer(rng, n, d, "sqrelu")
    W_up, _, b_up, _, W_downT = sq.arrays
    gl = O.Part(d, W_up, W_downT, act="reglu", W_gate=W_up, b_up=b_up, b_gate=b_up)
    x = rng.standard_normal((2, d)).astype(np.float32)
    assert np.array_equal(O.dense_ffn(sq, x), O.dense_ffn(gl, x))
    idx = np.sort(rng.choice(n, 40, replace=False)).astype(np.int32)
    assert np.array_equal(O.sparse_ffn(sq, x, idx), O.sparse_ffn(gl, x, idx))


def test_squared_relu_integer_fixture():
    """Integer fixture: a = W_up.x + b exactly, h = a^2 for a > 0, 0 otherwise."""
    d = 4
    W_up = np.array([[1, 2, 0, 0], [0, -1, 0, 0], [3, 0, 0, 1]], dtype=np.float32)
    b_up = np.array([0, 0, -5], dtype=np.float32)
    W_downT = np.eye(3, d, dtype=np.float32)          # y[i] = h_i for i < 3
    part = O.Part(d, W_up, W_downT, act="sqrelu", b_up=b_up)
    x = np.array([[1, 1, 7, 4]], dtype=np.float32)     # a = 3, -1, 2 -> h = 9, 0, 4
    assert O.dense_ffn(part, x).tolist() == [[9.0, 0.0, 4.0, 0.0]]


def test_q4_0_ffn_equals_decoded_fp32_ffn():
    wl = S.WORKLOADS["opt175b-q4_0"].scaled(d=256, n=96, r=16)
    L = S.make_layer(wl)
    q = O.Part.from_layer(L)
    up32 = O.dequant(L.W_up, wl.d, q4=True).astype(np.float32)
    dn32 = O.dequant(L.W_downT, wl.d, q4=True).astype(np.float32)
    assert np.array_equal(up32.astype(np.float64), O.dequant(L.W_up, wl.d, q4=True))
    f = O.Part(wl.d, up32, dn32, act="relu", b_up=L.b_up)
    x = S.make_x(wl, 0, 0, 2)
    assert np.array_equal(O.dense_ffn(q, x), O.dense_ffn(f, x))


def test_split_merge_equals_unsplit_integer():
    rng = np.random.default_rng(8)
    n, d, n_hot = 64, 32, 23
    full = _layer(rng, n, d, "relu", integer=True)
    W_up, _, b_up, _, W_downT = full.arrays
    hot = O.Part(d, W_up[:n_hot], W_downT[:n_hot], b_up=b_up[:n_hot])
    cold = O.Part(d, W_up[n_hot:], W_downT[n_hot:], b_up=b_up[n_hot:])
    x = rng.integers(-2, 3, (2, d)).astype(np.float32)
    L = np.sort(rng.choice(n, 30, replace=False)).astype(np.int32)
    y_un = O.sparse_ffn(full, x, L)
    y = O.merge(O.sparse_ffn(hot, x, L[L < n_hot]), O.sparse_ffn(cold, x, L[L >= n_hot] - n_hot))
    assert np.array_equal(y, y_un)
    assert np.array_equal(O.merge(y_un, None), y_un)


def test_worked_example_hybrid_figure():
    ex = json.load(open(os.path.join(GOLDEN, "hybrid_example.json")))
    n, d = ex["n"], 16
    rng = np.random.default_rng(12)
    # integer layer in which every neuron fires (large positive bias) so the
    # output depends on exactly the predicted set
    W_up = rng.integers(-2, 3, (n, d)).astype(np.float32)
    W_downT = rng.integers(-3, 4, (n, d)).astype(np.float32)
    b_up = np.full(n, 100.0, np.float32)
    x = rng.integers(-2, 3, (1, d)).astype(np.float32)
    perm = np.array(ex["hot_neurons"] + ex["cold_neurons"], np.int32)   # slot -> original id
    n_hot = len(ex["hot_neurons"])
    hot = O.Part(d, W_up[perm[:n_hot]], W_downT[perm[:n_hot]], b_up=b_up[perm[:n_hot]])
    cold = O.Part(d, W_up[perm[n_hot:]], W_downT[perm[n_hot:]], b_up=b_up[perm[n_hot:]])
    # predictor = identity-free stand-in: build the mask of the predicted set in slot ids
    slot = np.argsort(perm)
    words = np.zeros(1, np.uint64)
    for i in ex["predicted"]:
        words[0] |= np.uint64(1) << np.uint64(int(slot[i]))
    h_idx, c_idx = O.compact(words, n, n_hot)
    assert sorted(perm[h_idx].tolist()) == ex["expect_hot_computed"]
    assert sorted(perm[n_hot + c_idx].tolist()) == ex["expect_cold_computed"]
    y = O.merge(O.sparse_ffn(hot, x, h_idx), O.sparse_ffn(cold, x, c_idx))
    full = O.Part(d, W_up, W_downT, b_up=b_up)
    assert np.array_equal(y, O.sparse_ffn(full, x, np.array(ex["predicted"], np.int32)))


def test_layer_step_composes_the_steps():
    wl = S.WORKLOADS["opt30b-fp16"].scaled(d=128, n=300, r=32, hot_frac=0.26)
    L = S.make_layer(wl)
    n_hot = 78
    hot, cold = O.Part.from_layer(L, 0, n_hot), O.Part.from_layer(L, n_hot, wl.n)
    x = S.make_x(wl, 0, 1, 2)
    mask, h, c, y = O.layer_step(L.P1t, L.P2t, L.b2, 0.0, hot, cold, x)
    m2, _, _ = O.predict(L.P1t, L.P2t, L.b2, x)
    assert np.array_equal(mask, m2)
    h2, c2 = O.compact(m2, wl.n, n_hot)
    assert np.array_equal(h, h2) and np.array_equal(c, c2)
    assert np.array_equal(y, O.merge(O.sparse_ffn(hot, x, h2), O.sparse_ffn(cold, x, c2)))


def test_threaded_oracle_is_bit_identical():
    """The oracle's outer loops shared among threads (for timing on all host cores)
    give bit-identical results: each output is still computed by one thread with the
    same operations in the same order."""
    wl = S.WORKLOADS["opt175b-q4_0"].scaled(d=512, n=700, r=48, act="reglu")
    L = S.make_layer(wl)
    x = S.make_x(wl, 0, 1, 3)
    part = O.Part.from_layer(L)
    idx = np.arange(0, wl.n, 3, dtype=np.int32)
    X = S.make_profile_x(wl, 0, 40)
    runs = []
    try:
        for k in (1, 5):
            O.set_threads(k)
            assert O.get_threads() == k
            m, lg, m32 = O.predict(L.P1t, L.P2t, L.b2, x)
            y = O.sparse_ffn(part, x, idx)
            c, c32, amb = O.profile_counts(part, X, band=1e-4)
            runs.append((m, lg, m32, y, c, c32, amb))
    finally:
        O.set_threads(1)
    for a, b in zip(*runs):
        assert np.array_equal(a, b)
