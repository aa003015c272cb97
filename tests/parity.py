"""Parity protocol between the HIP path (through the C ABI) and the oracle.

Per decode step, on the same seeded inputs:
1. mask: the GPU's predicted bit equals the oracle's at every neuron that is
   not ambiguous; a neuron is ambiguous when no token's fp64 logit exceeds the
   threshold by more than BAND and some token's logit lies within BAND of it
   (those may take either value).
2. lists: the oracle compacts the GPU's mask; hot/cold lists and counts must
   match bit for bit.
3. FFN: the oracle recomputes each partition's sparse FFN over the GPU's lists
   and merges; the GPU output must match within the dtype's tolerance:
   fp32 weights: max_j |y - y_ref| / max_j |y_ref| <= 1e-5 (normwise, per token);
   fp16 / Q4_0 weights: ||y - y_ref||_2 / ||y_ref||_2 <= 2e-3 (per token).
"""
from __future__ import annotations

import numpy as np

from oracle import oracle as O

BAND = 1e-5
TOL = {"f32": ("max", 1e-5), "f16": ("l2", 2e-3), "q4_0": ("l2", 2e-3)}


def mask_bits(words: np.ndarray, n: int) -> np.ndarray:
    w = np.ascontiguousarray(words).view(np.uint64)
    bits = np.unpackbits(w.view(np.uint8), bitorder="little")
    return bits[:n].astype(bool), bits[n:]


def ambiguous(logits: np.ndarray, thr: float = 0.0, band: float = BAND) -> np.ndarray:
    clear_on = (logits > thr + band).any(axis=0)
    near = (np.abs(logits - thr) <= band).any(axis=0)
    return near & ~clear_on


def check_mask(gpu_words, oracle_words, oracle_logits, n, thr=0.0, band=BAND):
    """`band` is BAND unless a test scales the logits by a known power of two (then
    the band scales with them)."""
    g, gtail = mask_bits(gpu_words, n)
    o, _ = mask_bits(oracle_words, n)
    assert not gtail.any(), "mask tail bits must be 0"
    amb = ambiguous(oracle_logits, thr, band)
    bad = np.flatnonzero((g != o) & ~amb)
    assert bad.size == 0, f"{bad.size} predicted bits differ outside the band, e.g. {bad[:8]}"
    return int(amb.sum())


def rel_err(y, ref, kind, scale=None):
    """Per-token relative error, worst token.  `scale` (default: ref) is the
    output whose size the error is measured against."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    sc = ref if scale is None else np.asarray(scale, np.float64)
    out = []
    for b in range(ref.shape[0]):
        if kind == "max":
            den = np.max(np.abs(sc[b]))
            num = np.max(np.abs(y[b] - ref[b]))
        else:
            den = np.linalg.norm(sc[b])
            num = np.linalg.norm(y[b] - ref[b])
        out.append(num / den if den > 0 else num)
    return max(out) if out else 0.0


def check_close(y, ref, wdtype, scale=None):
    """y against the oracle's ref to the layer's tolerance.  The hot and cold
    partials are measured against the size of the merged layer output they add
    up to (`scale`): a partial with few active neurons can be much smaller
    than y, and its error is only meaningful on the output's scale."""
    kind, tol = TOL[wdtype]
    if np.all(ref == 0):
        assert np.all(np.asarray(y) == 0), "expected an exact zero output"
        return 0.0
    e = rel_err(y, ref, kind, scale)
    assert e <= tol, f"relative error {e:.3e} > {tol:.0e} ({kind})"
    return e


def permute_layer(L, perm):
    """Host copy of the layer with per-neuron rows in slot order (plain indexing)."""
    import dataclasses
    take = lambda a: None if a is None else np.ascontiguousarray(a[perm])  # noqa: E731
    return dataclasses.replace(L, p=take(L.p), W_up=take(L.W_up), W_gate=take(L.W_gate),
                               W_downT=take(L.W_downT), b_up=take(L.b_up), b_gate=take(L.b_gate),
                               P2t=take(L.P2t), b2=take(L.b2))


def oracle_ffn(Lh, n_hot, x, hot_idx, cold_idx):
    """Oracle sparse FFN per partition over the given lists, then merge."""
    hot = O.Part.from_layer(Lh, 0, n_hot)
    y_hot = O.sparse_ffn(hot, x, hot_idx) if n_hot > 0 else np.zeros((x.shape[0], Lh.d))
    if n_hot < Lh.n:
        cold = O.Part.from_layer(Lh, n_hot, Lh.n)
        y_cold = O.sparse_ffn(cold, x, cold_idx)
    else:
        y_cold = None
    return y_hot, y_cold, O.merge(y_hot, y_cold)


def oracle_threads():
    """Threads for the oracle's outer loops in the GPU tests (results are bit-identical
    for any count): the cores this process may use, at most 16."""
    import os
    try:
        k = len(os.sched_getaffinity(0))
    except AttributeError:
        k = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        k = min(k, int(env))
    return max(1, min(16, k))
