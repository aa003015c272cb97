"""Pins of the oracle's predictor and compaction.

Predictor (CSDN article, section on sparse activation: a small per-layer
router predicts the neurons an input activates; read as the two-layer
low-rank MLP u = ReLU(P1^T x), logit = P2^T u + b2, active iff logit > t):
- against numpy float64 matmuls (a library routine) on random shapes;
- the identity construction P1 = [I, -I], P2 = [W; -W], b2 = b, for which
  ReLU(x) - ReLU(-x) = x makes the logit equal W x + b exactly, so the
  predicted set is the true ReLU firing set (integer fixtures, exact);
- an exact zero logit is inactive (strict comparison);
- over a batch the mask is the union (OR) of the per-token masks.
Compaction (the hybrid-design figure: predicted ids split between the
partitions): against numpy.flatnonzero, with ragged n and any split point.
"""
import numpy as np
import pytest

from oracle import oracle as O


def _bits(mask, n):
    words = np.asarray(mask, dtype=np.uint64)
    out = np.zeros(len(words) * 64, dtype=bool)
    for w, v in enumerate(words):
        for b in range(64):
            out[64 * w + b] = (int(v) >> b) & 1
    return out[:n], out[n:]


@pytest.mark.parametrize("d,n,r,B,dt", [(64, 100, 16, 1, np.float32), (128, 257, 32, 3, np.float16),
                                        (256, 64, 48, 2, np.float16)])
def test_predict_matches_numpy(d, n, r, B, dt):
    rng = np.random.default_rng(d + n)
    P1t = (rng.standard_normal((r, d)) / np.sqrt(d)).astype(dt)
    P2t = (rng.standard_normal((n, r)) / np.sqrt(r)).astype(dt)
    b2 = rng.standard_normal(n).astype(np.float32) * 0.3
    x = rng.standard_normal((B, d)).astype(dt)
    mask, logits, _ = O.predict(P1t, P2t, b2, x)
    u = np.maximum(x.astype(np.float64) @ P1t.astype(np.float64).T, 0.0)
    ref = u @ P2t.astype(np.float64).T + b2.astype(np.float64)
    np.testing.assert_allclose(logits, ref, rtol=1e-12, atol=1e-12)
    firing, tail = _bits(mask, n)
    assert not tail.any()
    clear = np.all(np.abs(ref) > 1e-9, axis=0)
    assert np.array_equal(firing[clear], (ref > 0).any(axis=0)[clear])


def test_predict_identity_construction_exact():
    rng = np.random.default_rng(7)
    d, n = 32, 77
    W = rng.integers(-3, 4, size=(n, d)).astype(np.float32)
    b = rng.integers(-4, 5, size=n).astype(np.float32)
    x = rng.integers(-2, 3, size=(1, d)).astype(np.float32)
    P1t = np.concatenate([np.eye(d), -np.eye(d)]).astype(np.float32)        # [2d][d]
    P2t = np.concatenate([W, -W], axis=1).astype(np.float32)                 # [n][2d]
    mask, logits, mask32 = O.predict(P1t, P2t, b, x)
    exact = (W.astype(np.int64) @ x[0].astype(np.int64)) + b.astype(np.int64)
    assert np.array_equal(logits[0], exact.astype(np.float64))
    firing, _ = _bits(mask, n)
    assert np.array_equal(firing, exact > 0)
    assert np.array_equal(mask, mask32)
    assert (exact == 0).any(), "fixture must contain an exact-zero logit (strict > pin)"


def test_strict_threshold_nonzero():
    # logit exactly equal to a nonzero threshold is inactive; just above is active
    P1t = np.array([[1.0]], np.float32)
    P2t = np.array([[1.0], [1.0], [1.0]], np.float32)
    b2 = np.array([0.0, 0.25, -0.25], np.float32)
    x = np.array([[0.5]], np.float32)   # u = 0.5; logits 0.5, 0.75, 0.25
    mask, logits, _ = O.predict(P1t, P2t, b2, x, threshold=0.5)
    assert list(logits[0]) == [0.5, 0.75, 0.25]
    assert int(mask[0]) == 0b010


def test_union_over_batch():
    rng = np.random.default_rng(3)
    d, n, r = 64, 200, 16
    P1t = (rng.standard_normal((r, d)) / 8).astype(np.float32)
    P2t = (rng.standard_normal((n, r)) / 4).astype(np.float32)
    b2 = np.full(n, -0.6, np.float32)
    x = rng.standard_normal((5, d)).astype(np.float32)
    m_all, _, _ = O.predict(P1t, P2t, b2, x)
    acc = np.zeros_like(m_all)
    for b in range(5):
        mb, _, _ = O.predict(P1t, P2t, b2, x[b:b + 1])
        acc |= mb
    assert np.array_equal(m_all, acc)


@pytest.mark.parametrize("n,n_hot", [(1, 1), (63, 63), (64, 20), (65, 0), (1000, 260), (4097, 4097)])
def test_compact_matches_flatnonzero(n, n_hot):
    rng = np.random.default_rng(n)
    bits = rng.random(n) < 0.3
    words = np.zeros((n + 63) // 64, np.uint64)
    for i in np.flatnonzero(bits):
        words[i // 64] |= np.uint64(1) << np.uint64(i % 64)
    hot, cold = O.compact(words, n, n_hot)
    ids = np.flatnonzero(bits)
    assert np.array_equal(hot, ids[ids < n_hot])
    assert np.array_equal(cold, ids[ids >= n_hot] - n_hot)


def test_compact_empty_and_full():
    n = 130
    hot, cold = O.compact(np.zeros(3, np.uint64), n, 50)
    assert hot.size == 0 and cold.size == 0
    full = np.array([~np.uint64(0)] * 2 + [np.uint64((1 << 2) - 1)], np.uint64)
    hot, cold = O.compact(full, n, 50)
    assert np.array_equal(hot, np.arange(50)) and np.array_equal(cold, np.arange(80))
