"""Pins of the oracle's bandwidth- and capacity-aware hot/cold split.

The rule (CSDN article, overall-architecture section: placement from activation
frequencies and the hardware's bandwidth and capacity; hybrid-design section: the
partitions compute concurrently and merge): with K hot slots, per-step read times
T_hot = (counts of slots < K) / hbm_rate and T_cold = (counts of slots >= K) /
link_rate; K* is the smallest K minimising max(T_hot, T_cold); n_hot = min(K*,
budget / bytes_per_neuron).  Pinned by closed forms and limits, not by retyping it:
- uniform counts: K* = n * h / (h + l) when that is an integer (the two times equal);
- equal rates: the split where the hot counts first reach half the total;
- a slow link: every neuron that ever fired is hot, and nothing else;
- a fast link: K* = 0;
- the capacity budget caps n_hot, and a slower link never lowers n_hot.
"""
import numpy as np
import pytest

from oracle import oracle as O


def _plan(c, h, l, budget=None, bpn=1):
    c = np.asarray(c, dtype=np.uint32)
    return O.plan_hot_split(c, len(c) * bpn if budget is None else budget, bpn, h, l)


@pytest.mark.parametrize("n,h,l", [(8, 3.0, 1.0), (100, 9.0, 1.0), (1000, 99.0, 1.0),
                                   (30, 1.0, 2.0)])
def test_uniform_counts_balance_the_tiers(n, h, l):
    k = n * h / (h + l)
    assert k == int(k)
    assert _plan(np.ones(n), h, l) == int(k)


def test_equal_rates_split_at_half_the_activations():
    rng = np.random.default_rng(3)
    c = np.sort(rng.integers(0, 1000, 57))[::-1]
    k = _plan(c, 5.0, 5.0)
    hot = np.cumsum(np.concatenate([[0], c]))
    total = hot[-1]
    # max(hot, cold) is minimised where the hot sum crosses half of the total
    cost = np.maximum(hot, total - hot)
    assert cost[k] == cost.min() and np.all(cost[:k] > cost[k])


def test_slow_link_puts_every_firing_neuron_in_hbm():
    c = np.array([900, 50, 7, 3, 1, 0, 0, 0])
    assert _plan(c, 1e6, 1e-6) == 5


def test_fast_link_keeps_nothing_hot():
    assert _plan([5, 4, 3, 2, 1], 1.0, 1e9) == 0


def test_budget_caps_and_monotone_in_link_rate():
    rng = np.random.default_rng(5)
    c = np.sort(rng.zipf(1.3, 400).clip(max=10_000))[::-1]
    ks = [_plan(c, 5000.0, l) for l in (2000.0, 500.0, 50.0, 5.0)]
    assert ks == sorted(ks)
    full = _plan(c, 5000.0, 50.0)
    assert _plan(c, 5000.0, 50.0, budget=10 * 16, bpn=16) == min(full, 10)


def test_all_zero_counts_and_empty_layer():
    assert _plan([0, 0, 0], 10.0, 1.0) == 0
    assert _plan([], 10.0, 1.0) == 0
