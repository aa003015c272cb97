"""Pins of the oracle's adaptive (recall-calibrated) predictor threshold.

The threshold (chatpaper.ai abstract: adaptive predictors; hada.io README
summary, hybrid-approach section): over the profiling samples, the largest
float32 tau such that at least ceil(target * N) of the N firing (sample, neuron)
pairs have a logit above tau.  Pinned against what the definition fixes, with
logits and firing computed independently by numpy on integer fixtures (exact):
- the recall at tau reaches the target and the next float32 above tau does not
  (tau is the largest such threshold);
- the counts N, m and the hits at tau;
- with the exact identity predictor (logit = the pre-activation itself) and
  target 1, the predicted set is exactly the firing set;
- a hand-worked example;
- no firing pair at all gives FLT_MAX.
"""
import numpy as np
import pytest

from oracle import oracle as O


def _int_layer(rng, n, d, r):
    W_up = rng.integers(-3, 4, (n, d)).astype(np.float32)
    W_down = rng.integers(-3, 4, (n, d)).astype(np.float32)
    b_up = rng.integers(-4, 5, n).astype(np.float32)
    P1t = rng.integers(-2, 3, (r, d)).astype(np.float32)
    P2t = rng.integers(-2, 3, (n, r)).astype(np.float32)
    b2 = rng.integers(-6, 7, n).astype(np.float32)
    return W_up, W_down, b_up, P1t, P2t, b2


def _numpy_pairs(W_up, b_up, P1t, P2t, b2, X):
    Xd = X.astype(np.float64)
    u = np.maximum(Xd @ P1t.astype(np.float64).T, 0)
    logits = (u @ P2t.astype(np.float64).T + b2).astype(np.float32)
    pre = (Xd @ W_up.astype(np.float64).T + b_up).astype(np.float32)
    return logits, pre > 0


@pytest.mark.parametrize("target", [0.5, 0.9, 0.99, 1.0])
def test_threshold_is_the_largest_meeting_the_recall(target):
    rng = np.random.default_rng(17)
    n, d, r, S = 37, 12, 8, 23
    W_up, W_down, b_up, P1t, P2t, b2 = _int_layer(rng, n, d, r)
    X = rng.integers(-3, 4, (S, d)).astype(np.float32)
    part = O.Part(d, W_up, W_down, act="relu", b_up=b_up)
    tau, N, m, hits = O.calibrate_threshold(P1t, P2t, b2, part, X, target)
    logits, fire = _numpy_pairs(W_up, b_up, P1t, P2t, b2, X)
    fl = logits[fire]
    assert N == fl.size > 0
    assert m == int(np.ceil(target * N))
    assert hits == int((fl > np.float32(tau)).sum())
    assert hits >= m                                       # recall at tau >= target
    above = np.nextafter(np.float32(tau), np.float32(np.inf))
    assert int((fl > above).sum()) < m                     # no larger threshold reaches it


def test_identity_predictor_at_full_recall_predicts_exactly_the_firing_set():
    """P1 = [I, -I], P2 = [W_up, -W_up], b2 = b_up: the logit is the pre-activation
    (relu(x) - relu(-x) = x), so target 1 keeps every firing pair and no other."""
    rng = np.random.default_rng(3)
    n, d, S = 29, 10, 31
    W_up, W_down, b_up, _, _, _ = _int_layer(rng, n, d, 4)
    P1t = np.concatenate([np.eye(d), -np.eye(d)]).astype(np.float32)
    P2t = np.concatenate([W_up, -W_up], axis=1).astype(np.float32)
    X = rng.integers(-3, 4, (S, d)).astype(np.float32)
    part = O.Part(d, W_up, W_down, act="relu", b_up=b_up)
    tau, N, m, hits = O.calibrate_threshold(P1t, P2t, b_up, part, X, 1.0)
    logits, fire = _numpy_pairs(W_up, b_up, P1t, P2t, b_up, X)
    predicted = logits > np.float32(tau)
    assert hits == N == m
    assert np.array_equal(predicted, fire)


def test_hand_worked_example():
    """d = 1, identity-like predictor scaled by 2 (logit = 2 * pre), one neuron per
    weight w in {1, 2, 3}, no biases; samples x in {1, 2, -1}.  Pre-activations
    w * x: x = 1 -> 1, 2, 3; x = 2 -> 2, 4, 6; x = -1 -> all negative.  Firing
    pairs: 6, logits 2, 4, 6, 4, 8, 12.  Target 0.5 -> m = 3: the third largest
    logit is 6, so tau is the float32 just below 6 and 3 pairs (12, 8, 6) are above."""
    W_up = np.array([[1.0], [2.0], [3.0]], np.float32)
    W_down = np.ones((3, 1), np.float32)
    P1t = np.array([[1.0], [-1.0]], np.float32)
    P2t = 2 * np.concatenate([W_up, -W_up], axis=1).astype(np.float32)
    X = np.array([[1.0], [2.0], [-1.0]], np.float32)
    part = O.Part(1, W_up, W_down, act="relu")
    tau, N, m, hits = O.calibrate_threshold(P1t, P2t, None, part, X, 0.5)
    assert (N, m, hits) == (6, 3, 3)
    assert tau == float(np.nextafter(np.float32(6.0), np.float32(-np.inf)))


def test_no_firing_pair_predicts_nothing():
    W_up = -np.ones((4, 3), np.float32)
    part = O.Part(3, W_up, np.ones((4, 3), np.float32), act="relu")
    P1t = np.ones((2, 3), np.float32)
    P2t = np.ones((4, 2), np.float32)
    X = np.ones((5, 3), np.float32)
    tau, N, m, hits = O.calibrate_threshold(P1t, P2t, None, part, X, 0.99)
    assert (N, m, hits) == (0, 0, 0)
    assert tau == float(np.finfo(np.float32).max)
