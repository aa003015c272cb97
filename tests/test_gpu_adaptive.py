"""GPU parity of the adaptive predictor threshold and of the true firing mask.

The threshold (chatpaper.ai abstract: adaptive predictors; hada.io README
summary, hybrid-approach section) is chosen on profiling samples as the largest
float32 tau that keeps at least ceil(target * N) of the N firing (sample,
neuron) pairs above it.  The device computes the logits with the decode
predictor's kernels, decides firing in float32, and selects tau by an exact radix
selection; the oracle computes the logits and pre-activations in fp64.  Compared:

- the firing pairs: N equal up to pairs whose pre-activation is within 1e-4 of 0;
- tau against the oracle's order statistics: the selected logit (the float just
  above tau) lies within the logit tolerance of the oracle's m-th largest firing
  logit, the rank widened by the pairs whose firing is ambiguous; when no pair is
  ambiguous, tau itself is within the tolerance of the oracle's tau;
- recall: the device's own count of firing pairs above tau reaches m, and the
  oracle's pairs above tau reach the target up to the ambiguous ones;
- the selection step alone is exact: on the device's logits and firing
  decisions (read back), tau is the float32 just below the m-th largest, bit for bit.
- pi_true_mask against the oracle's firing union outside the ambiguity band.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import oracle as O  # noqa: E402
from parity import mask_bits, oracle_threads  # noqa: E402
from sparse_activation_ffn_amd import binding as pb  # noqa: E402
from sparse_activation_ffn_amd.layer import DeviceLayer  # noqa: E402
from workload import synth as S  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"
FIRE_BAND = 1e-4       # |pre-activation| within this of 0: float32 vs fp64 may disagree
LOGIT_TOL = 1e-4       # device logits vs the oracle's (both paths of pi_predict)


def log(*a):
    print(*a, flush=True)


def _np(t):
    return t.detach().cpu().numpy()


CASES = {
    # name: (workload, S samples)  -- S spans several batches of 64 and a ragged tail
    "f16": (S.WORKLOADS["opt30b-fp16"].scaled(d=512, n=1500, r=64), 200),
    "f32": (S.WORKLOADS["opt-fp32"].scaled(d=320, n=1000, r=32), 77),
    "q4": (S.WORKLOADS["opt175b-q4_0"].scaled(d=1280, n=700, r=64), 131),
    "reglu": (S.WORKLOADS["llama70b-reglu-fp16"].scaled(d=640, n=900, r=48), 65),
}


def _oracle_pairs(L, X):
    """fp64 logits [S][n] and deciding pre-activations [S][n] from the oracle."""
    wl = L.wl
    q4 = wl.wdtype == "q4_0"
    _, logits, _ = O.predict(L.P1t, L.P2t, L.b2, X, 0.0)
    W = L.W_gate if wl.act == "reglu" else L.W_up
    b = L.b_gate if wl.act == "reglu" else L.b_up
    pre = X.astype(np.float64) @ O.dequant(W, wl.d, q4).T
    if b is not None:
        pre = pre + b.astype(np.float64)
    return logits, pre


def _calibrate(dl, X, target):
    ws = torch.empty(pb.pi_calibrate_workspace_bytes(dl.d, dl.n, dl.r, X.shape[0]),
                     dtype=torch.uint8, device=DEV)
    tau = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    stats = torch.full((3,), 0x7fffffff, dtype=torch.int32, device=DEV)
    pb.pi_calibrate_threshold(dl.predictor(), dl.part(), X, target, tau, stats, ws)
    torch.cuda.synchronize()
    return float(_np(tau)[0]), [int(v) for v in _np(stats)]


@pytest.mark.parametrize("target", [0.9, 0.99, 1.0])
@pytest.mark.parametrize("name", list(CASES))
def test_calibrated_threshold_matches_oracle(name, target):
    wl, nS = CASES[name]
    log(f"calibration {name} S={nS} target={target}")
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    X_np = S.make_profile_x(wl, 0, nS)
    X = torch.from_numpy(X_np).to(DEV)
    tau, (N, m, hits) = _calibrate(dl, X, target)
    O.set_threads(oracle_threads())
    try:
        tau_o, N_o, m_o, hits_o = O.calibrate_threshold(L.P1t, L.P2t, L.b2, O.Part.from_layer(L),
                                                        X_np, target)
    finally:
        O.set_threads(1)
    logits, pre = _oracle_pairs(L, X_np)
    fire_o = pre.astype(np.float32) > 0
    assert int(fire_o.sum()) == N_o
    k_amb = int((np.abs(pre) <= FIRE_BAND).sum())
    log(f"  device tau {tau!r} N {N} m {m} hits {hits}; oracle tau {tau_o!r} N {N_o} m {m_o}; "
        f"{k_amb} ambiguous pairs")
    assert abs(N - N_o) <= k_amb
    assert m == int(np.ceil(target * N)) and hits >= m
    f = np.sort(logits[fire_o].astype(np.float32))[::-1]
    v = float(np.nextafter(np.float32(tau), np.float32(np.inf)))      # the selected logit
    lo_rank, hi_rank = min(m - 1 + k_amb, N_o - 1), max(m - 1 - k_amb, 0)
    assert f[lo_rank] - LOGIT_TOL <= v <= f[hi_rank] + LOGIT_TOL
    if k_amb == 0:
        assert (N, m) == (N_o, m_o)
        assert abs(tau - tau_o) <= LOGIT_TOL
    near = int((np.abs(logits[fire_o] - tau) <= LOGIT_TOL).sum())
    assert int((logits[fire_o] > tau).sum()) + near + k_amb >= m_o


@pytest.mark.parametrize("name", ["f16", "q4"])
def test_selection_is_exact_on_device_values(name):
    wl, nS = CASES[name]
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    X_np = S.make_profile_x(wl, 0, nS)
    X = torch.from_numpy(X_np).to(DEV)
    target = 0.97
    tau, (N, m, hits) = _calibrate(dl, X, target)
    # the device's own logits (same batches of 64 as the calibration) and firing
    ws = torch.zeros(pb.pi_workspace_bytes(wl.d, wl.n, wl.r, 64), dtype=torch.uint8, device=DEV)
    words = (wl.n + 63) // 64
    mask = torch.zeros(words, dtype=torch.int64, device=DEV)
    lg = torch.empty((nS, wl.n), dtype=torch.float32, device=DEV)
    for s0 in range(0, nS, 64):
        pb.pi_predict(dl.predictor(), X[s0:s0 + 64], mask, lg[s0:s0 + 64], None, ws)
    fire = np.zeros((nS, wl.n), bool)
    tm = torch.zeros(words, dtype=torch.int64, device=DEV)
    for s in range(nS):
        pb.pi_true_mask(dl.part(), X[s:s + 1], tm)
        torch.cuda.synchronize()
        fire[s] = mask_bits(_np(tm).view(np.uint64), wl.n)[0]
    torch.cuda.synchronize()
    g = _np(lg)
    logits_o, _ = _oracle_pairs(L, X_np)
    assert np.max(np.abs(g - logits_o)) <= LOGIT_TOL
    f = np.sort(g[fire])[::-1]
    assert N == f.size
    assert m == int(np.ceil(target * N))
    want = np.nextafter(f[m - 1], np.float32(-np.inf))
    assert np.float32(tau).view(np.uint32) == want.view(np.uint32)
    assert hits == int((f > want).sum())


def test_calibration_full_size_layer():
    """OPT-30B-shaped layer (d 7168, n 28672, r 1024), 96 profiling samples (one batch of
    64 and a ragged one of 32), target 0.99: tau against the oracle's order statistics."""
    wl = S.WORKLOADS["opt30b-fp16"]
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    X_np = S.make_profile_x(wl, 0, 96)
    X = torch.from_numpy(X_np).to(DEV)
    tau, (N, m, hits) = _calibrate(dl, X, 0.99)
    O.set_threads(oracle_threads())
    try:
        tau_o, N_o, m_o, _ = O.calibrate_threshold(L.P1t, L.P2t, L.b2, O.Part.from_layer(L), X_np, 0.99)
        logits, pre = _oracle_pairs(L, X_np)
    finally:
        O.set_threads(1)
    fire_o = pre.astype(np.float32) > 0
    k_amb = int((np.abs(pre) <= FIRE_BAND).sum())
    log(f"  device tau {tau!r} N {N} m {m} hits {hits}; oracle tau {tau_o!r} N {N_o} m {m_o}; "
        f"{k_amb} ambiguous pairs")
    assert abs(N - N_o) <= k_amb and hits >= m
    f = np.sort(logits[fire_o].astype(np.float32))[::-1]
    v = float(np.nextafter(np.float32(tau), np.float32(np.inf)))
    assert f[min(m - 1 + k_amb, N_o - 1)] - LOGIT_TOL <= v <= f[max(m - 1 - k_amb, 0)] + LOGIT_TOL


def test_no_firing_pair_gives_flt_max():
    wl = S.WORKLOADS["opt-fp32"].scaled(d=320, n=1000, r=32)
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    dl.b_up.fill_(-1e30)                       # no neuron can fire
    X = torch.from_numpy(S.make_profile_x(wl, 0, 9)).to(DEV)
    tau, stats = _calibrate(dl, X, 0.99)
    assert tau == float(np.finfo(np.float32).max)
    assert stats == [0, 0, 0]


@pytest.mark.parametrize("B", [1, 5])
@pytest.mark.parametrize("name", list(CASES))
def test_true_mask_matches_oracle(name, B):
    wl, _ = CASES[name]
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    x_np = S.make_x(wl, 0, 2, B)
    x = torch.from_numpy(x_np).to(DEV)
    words = (wl.n + 63) // 64
    tm = torch.full((words,), -1, dtype=torch.int64, device=DEV)
    pb.pi_true_mask(dl.part(), x, tm)
    torch.cuda.synchronize()
    got, tail = mask_bits(_np(tm).view(np.uint64), wl.n)
    assert not tail.any()
    _, pre = _oracle_pairs(L, x_np)
    want = (pre.astype(np.float32) > 0).any(axis=0)
    amb = (np.abs(pre) <= FIRE_BAND).any(axis=0)
    bad = np.flatnonzero((got != want) & ~amb)
    assert bad.size == 0, f"{bad.size} firing bits differ, e.g. {bad[:8]}"
