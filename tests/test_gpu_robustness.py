"""GPU robustness checks of the HIP path through the C ABI.

- Rows outside the active set are never used (CSDN article, section on sparse
  activation: neurons that do not fire contribute nothing): every weight row
  and bias of a neuron outside the step's predicted set is overwritten with
  NaN, and y, y_hot, y_cold and the lists must stay bit-identical, on every
  FFN path (fused batch-1 kernel for f32 / f16 / Q4_0, the gathered
  two-kernel path, the matrix-core path, with and without a cold partition).
- The matrix-core predictor (batch >= 2) keeps its decisions for inputs whose
  first-layer activations u are far above the f16 range or far below it.
- The read-stream kernel reads every word once.
"""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import oracle as O  # noqa: E402
from parity import (check_close, check_mask, mask_bits, oracle_ffn,  # noqa: E402
                    oracle_threads)
from sparse_activation_ffn_amd import binding as pb  # noqa: E402
from sparse_activation_ffn_amd.layer import DeviceLayer, StepBuffers  # noqa: E402
from workload import synth as S  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def log(*a):
    print(*a, flush=True)


def _np(t):
    return t.detach().cpu().numpy()


def _step(dl, buf, x_np, fused=True):
    x = torch.from_numpy(x_np).to(DEV)
    hot, cold = dl.parts()
    buf.hot_idx.fill_(-7)
    buf.cold_idx.fill_(-7)
    pb.pi_predict(dl.predictor(), x, buf.mask, None, None if fused else buf.lists, buf.ws)
    pb.pi_sparse_ffn_split(hot, cold, x, buf.lists, buf.y_hot,
                           buf.y_cold if cold is not None else None, buf.y, buf.ws,
                           mask=buf.mask if fused else None)
    torch.cuda.synchronize()
    c = _np(buf.counts)
    return dict(mask=_np(buf.mask).view(np.uint64).copy(), counts=c.copy(),
                hot=_np(buf.hot_idx)[:c[0]].copy(), cold=_np(buf.cold_idx)[:c[1]].copy(),
                y=_np(buf.y).copy(), y_hot=_np(buf.y_hot).copy(),
                y_cold=_np(buf.y_cold).copy() if cold is not None else None)


def _poison_rows(t: torch.Tensor, rows: torch.Tensor, q4: bool, d: int):
    """Rows `rows` of a per-neuron tensor set to NaN (f32 / f16), or for a Q4_0 row its
    fp16 scales set to NaN and its codes scrambled (codes are always finite)."""
    if t is None or rows.numel() == 0:
        return
    if q4:
        t[rows, : d // 2] = 0x5A
        sc = t[:, d // 2:].view(torch.int16)      # [rows][d / 32] fp16 scales
        sc[rows] = 0x7E00                          # binary16 quiet NaN
    elif t.dtype == torch.float16:
        t.view(torch.int16)[rows] = 0x7E00
    else:
        t[rows] = float("nan")


CASES = {
    # name: (workload, batch, n_hot)
    "f16-fused-split": (S.WORKLOADS["opt30b-fp16"].scaled(d=576, n=2085, r=64), 1, 700),
    "f32-fused": (S.WORKLOADS["opt-fp32"].scaled(d=320, n=1000, r=32), 1, None),
    "q4-fused": (S.WORKLOADS["opt175b-q4_0"].scaled(d=1280, n=1111, r=64), 1, None),
    "f16-reglu-fused": (S.WORKLOADS["llama70b-reglu-fp16"].scaled(d=640, n=1500, r=48), 1, 512),
    "f32-gathered": (S.WORKLOADS["opt-fp32"].scaled(d=320, n=1000, r=32), 6, 400),
    "q4-mfma": (S.WORKLOADS["opt175b-q4_0"].scaled(d=1280, n=1111, r=64), 8, 300),
    "f16-reglu-mfma": (S.WORKLOADS["llama70b-reglu-fp16"].scaled(d=768, n=1333, r=64), 16, None),
}


@pytest.mark.parametrize("name", list(CASES))
def test_nan_rows_outside_active_set(name):
    wl, B, n_hot = CASES[name]
    log(f"nan poisoning {name} B={B}")
    L = S.make_layer(wl)
    n_hot = wl.n if n_hot is None else n_hot
    dl = DeviceLayer.upload(L, DEV, n_hot=n_hot)
    buf = StepBuffers(dl, B, DEV)
    # a step whose predicted set leaves out the first row of every partition (the
    # row that unconditional, clamped loads fall back to)
    for step in range(64):
        x = S.make_x(wl, 0, step, B)
        ref = _step(dl, buf, x)
        bits = mask_bits(ref["mask"], wl.n)[0]
        if not bits[0] and (n_hot >= wl.n or not bits[n_hot]):
            break
    else:
        pytest.fail("no step leaves the first rows inactive")
    inactive = torch.from_numpy(np.flatnonzero(~bits)).to(DEV)
    q4 = wl.wdtype == "q4_0"
    for t in (dl.W_up, dl.W_gate, dl.W_downT):
        _poison_rows(t, inactive, q4, wl.d)
    for t in (dl.b_up, dl.b_gate):
        if t is not None:
            t[inactive] = float("nan")
    torch.cuda.synchronize()
    for fused in (True, False):
        out = _step(dl, buf, x, fused=fused)
        for k in ("mask", "counts", "hot", "cold", "y", "y_hot", "y_cold"):
            if ref[k] is not None:
                assert np.array_equal(out[k], ref[k]), f"{k} changed (fused={fused})"
    assert np.all(np.isfinite(out["y"]))
    log(f"  step {step}: {int(bits.sum())} active, {inactive.numel()} rows poisoned, y unchanged")


@pytest.mark.parametrize("B", [2, 20])
@pytest.mark.parametrize("scale_exp", [15, -8])
def test_matrix_core_predictor_extreme_magnitudes(scale_exp, B):
    """First-layer weights scaled by 2^e (so u scales by 2^e: up to ~1e5 for e = 15,
    beyond the largest f16, and ~1e-3 for e = -8), second layer by 2^-8 or 2^8 so the
    second layer's weights stay normal f16 numbers.  First-layer magnitudes are kept
    at least 1/sqrt(d) before scaling, so no stored weight is an f16 subnormal.  The
    matrix-core predictor's logits must match the oracle's within the band scaled like
    the logits, and its mask outside that band."""
    wl = S.WORKLOADS["opt30b-fp16"].scaled(d=512, n=1500, r=128)
    L = S.make_layer(wl)
    e2 = -8 if scale_exp > 0 else 8
    p1 = L.P1t.astype(np.float32)
    p1 = np.sign(p1) * (np.abs(p1) + np.float32(1.0 / np.sqrt(wl.d)))
    P1t = (p1 * np.float32(2.0 ** scale_exp)).astype(np.float16)
    P2t = (L.P2t.astype(np.float32) * np.float32(2.0 ** e2)).astype(np.float16)
    assert np.all(np.isfinite(P1t)) and np.all(np.isfinite(P2t))
    b2 = (L.b2 * np.float32(2.0 ** (scale_exp + e2))).astype(np.float32)
    Ls = dataclasses.replace(L, P1t=P1t, P2t=P2t, b2=b2)
    dl = DeviceLayer.upload(Ls, DEV)
    buf = StepBuffers(dl, B, DEV)
    x_np = S.make_x(wl, 0, 3, B)
    x = torch.from_numpy(x_np).to(DEV)
    lg = torch.empty((B, wl.n), dtype=torch.float32, device=DEV)
    pb.pi_predict(dl.predictor(), x, buf.mask, lg, None, buf.ws)
    torch.cuda.synchronize()
    mask_o, logits_o, _ = O.predict(Ls.P1t, Ls.P2t, Ls.b2, x_np, Ls.threshold)
    u_max = np.max(np.maximum(x_np.astype(np.float64) @ P1t.astype(np.float64).T, 0))
    scale = 2.0 ** (scale_exp + e2)
    err = np.max(np.abs(_np(lg) - logits_o))
    log(f"  e={scale_exp} B={B}: max u {u_max:.3g}, max |logit err| {err:.3g} (logit scale {scale})")
    assert err <= 1e-4 * scale
    check_mask(_np(buf.mask).view(np.uint64), mask_o, logits_o, wl.n, Ls.threshold, band=1e-5 * scale)


def test_stream_read_reads_every_word():
    n16 = 3 * 2048 * 256 * 4 + 77            # several passes and a ragged tail
    data = torch.randint(-2**31, 2**31 - 1, (n16 * 4,), dtype=torch.int32, device=DEV)
    sink = torch.zeros(pb.PI_STREAM_SINK_WORDS, dtype=torch.int32, device=DEV)
    pb.pi_stream_read(data, n16 * 16, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(_np(data).view(np.uint32))
    got = np.bitwise_xor.reduce(_np(sink).view(np.uint32))
    assert got == want


def test_threaded_oracle_matches_gpu_step():
    """The oracle's threaded run (used for the all-core CPU baseline and the large
    parity cases) against the GPU on one OPT-30B-shaped small step."""
    wl = S.WORKLOADS["opt30b-fp16"].scaled(d=576, n=2085, r=64)
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV, n_hot=600)
    buf = StepBuffers(dl, 1, DEV)
    x = S.make_x(wl, 0, 9, 1)
    out = _step(dl, buf, x)
    O.set_threads(oracle_threads())
    try:
        _, _, y = oracle_ffn(L, 600, x, out["hot"], out["cold"])
    finally:
        O.set_threads(1)
    check_close(out["y"], y, "f16")


def test_crossover_on_gathered_path():
    """The crossover on the gathered two-kernel path (f32 weights, batch 6): dense from
    the device count on, the oracle's dense FFN; below it, the sparse split."""
    wl = S.WORKLOADS["opt-fp32"].scaled(d=320, n=1000, r=32)
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV, n_hot=300)
    buf = StepBuffers(dl, 6, DEV)
    x_np = S.make_x(wl, 0, 4, 6)
    ref = _step(dl, buf, x_np)
    T = int(ref["counts"].sum())
    x = torch.from_numpy(x_np).to(DEV)
    hot, cold = dl.parts()
    for dense_from, want in ((T + 1, "sparse"), (T, "dense")):
        pb.pi_predict(dl.predictor(), x, buf.mask, None, None, buf.ws)
        pb.pi_sparse_ffn_crossover(hot, cold, x, buf.lists, dense_from, buf.y_hot, buf.y_cold,
                                   buf.y, buf.ws, mask=buf.mask)
        torch.cuda.synchronize()
        y = _np(buf.y)
        assert np.array_equal(_np(buf.counts), ref["counts"])
        if want == "sparse":
            assert np.array_equal(y, ref["y"])
        else:
            check_close(y, O.dense_ffn(O.Part.from_layer(L), x_np), "f32")
