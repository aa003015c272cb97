"""Statistics and encodings of the seeded synthetic workloads.

CSDN article, section on sparse activation: about 10% of an OPT FFN's
neurons are needed per token; section on inference locality, figure (a):
26% (OPT-30B) / 43% (LLaMA(ReGLU)-70B) of one layer's neurons give 80% of
the activations.  The generator is checked against its own recipe (mean
probability exact, empirical firing rates within binomial bounds, predicted
density near the target); the skew figure is reported, not asserted.
"""
import numpy as np
import pytest

from oracle import oracle as O
from workload import synth as S


@pytest.mark.parametrize("name", list(S.WORKLOADS))
def test_zipf_mean_exact(name):
    wl = S.WORKLOADS[name]
    p = S.zipf_probs(wl.n, wl.mean)
    assert abs(p.mean() - wl.mean) < 1e-12
    assert p.max() <= S.P_CLIP and np.all(np.diff(p) <= 0)


def test_deterministic_and_distinct():
    wl = S.WORKLOADS["opt-fp32"].scaled(d=128, n=512, r=32)
    a, b = S.make_layer(wl, 0), S.make_layer(wl, 0)
    c = S.make_layer(wl, 1)
    assert np.array_equal(a.W_up, b.W_up) and np.array_equal(a.P2t, b.P2t)
    assert not np.array_equal(a.W_up, c.W_up)
    assert np.array_equal(S.make_x(wl, 0, 3, 2), S.make_x(wl, 0, 3, 2))
    assert not np.array_equal(S.make_x(wl, 0, 3, 2), S.make_x(wl, 0, 4, 2))


def test_firing_rates_follow_p():
    wl = S.WORKLOADS["opt-fp32"]
    L = S.make_layer(wl)
    X = S.make_profile_x(wl, 0, 2000).astype(np.float64)
    pre = X @ L.W_up.astype(np.float64).T + L.b_up.astype(np.float64)
    rate = (pre > 0).mean(axis=0)
    sigma = np.sqrt(L.p * (1 - L.p) / X.shape[0])
    z = np.abs(rate - L.p) / np.maximum(sigma, 1e-12)
    assert np.mean(z < 4) > 0.999
    assert abs(rate.mean() - wl.mean) < 0.005


def test_predicted_density_near_target():
    wl = S.WORKLOADS["opt-fp32"]
    L = S.make_layer(wl)
    dens = []
    for step in range(8):
        mask, _, _ = O.predict(L.P1t, L.P2t, L.b2, S.make_x(wl, 0, step, 1))
        dens.append(sum(bin(int(w)).count("1") for w in mask) / wl.n)
    assert abs(np.mean(dens) - wl.mean) < 0.01


def test_q4_0_pack_roundtrip():
    rng = np.random.default_rng(0)
    d = 512
    codes = rng.integers(0, 16, (3, d), dtype=np.uint8)
    scales = np.abs(rng.standard_normal((3, d // 32))).astype(np.float16)
    packed = S.q4_0_pack(codes, scales)
    assert packed.shape == (3, S.q4_0_row_bytes(d))
    for i in range(3):
        w = O.load_row(packed, d, i, q4=True)
        ref = (codes[i].astype(np.float64) - 8) * np.repeat(scales[i].astype(np.float64), 32)
        assert np.array_equal(w, ref)


def test_q4_0_bias_gives_target_rate():
    wl = S.WORKLOADS["opt175b-q4_0"].scaled(d=512, n=2048, r=64)
    L = S.make_layer(wl)
    W = O.dequant(L.W_up, wl.d, q4=True)
    X = S.make_profile_x(wl, 0, 400).astype(np.float64)
    rate = ((X @ W.T + L.b_up) > 0).mean()
    assert abs(rate - wl.mean) < 0.01


def test_skew_report():
    """Share of neurons giving 80% of activations (reported next to the pages' 26% / 43%)."""
    for name in ("opt30b-fp16", "llama70b-reglu-fp16"):
        wl = S.WORKLOADS[name]
        p = np.sort(S.zipf_probs(wl.n, wl.mean))[::-1]
        share = (np.searchsorted(np.cumsum(p) / p.sum(), 0.8) + 1) / wl.n
        assert 0.2 < share < 0.5


def test_budget_gives_hot_fraction():
    for name, k in (("opt30b-fp16", 7454), ("falcon40b-stack-fp16", 6553)):
        wl = S.WORKLOADS[name]
        assert S.budget_bytes(wl) // S.bytes_per_neuron(wl) == k
