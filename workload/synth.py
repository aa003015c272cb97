"""Seeded synthetic inputs for the predictor-gated sparse FFN.

This module only draws and stores numbers: layer weights, predictor weights,
biases, inputs and profiling samples, with the shapes, distributions and
storage encodings of the five workloads below.  It computes nothing of the
method itself (no predictor, no FFN, no compaction, no index), so both the
CPU oracle and the GPU path can take their inputs from it without sharing
any of the method's arithmetic.

Sources (PowerInfer pages):
- chatpaper.ai abstract and the CSDN article, section on sparse activation:
  a dense OPT FFN needs only about 10% of its neurons per token, and a
  per-layer router predicts which ones.
- CSDN article, section on inference locality, figures (a)(b): activation
  frequencies follow a power law (26% / 43% of one layer's neurons give 80%
  of the activations in OPT-30B / LLaMA(ReGLU)-70B).
- hada.io README summary, quantisation section: INT4 models use Q4_0.

Recipe (each choice the pages leave open is a stated reading):
- Per-neuron firing probabilities p follow Zipf(s) over ranks 1..n,
  p_k = min(c * k**-s, 0.99), with c found by bisection so that mean(p) is the
  target exactly; ranks are dealt to neurons by a seeded permutation.
- x ~ N(0, 1); W_up, W_gate ~ N(0, 1/d); W_down ~ N(0, 1/n) stored
  transposed as W_downT[n][d]; P1 ~ N(0, 1/d) stored as P1t[r][d];
  P2 ~ N(0, 1/r) stored as P2t[n][r].
- The bias of the row that decides firing (W_up for ReLU, W_gate for ReGLU)
  is b_i = ||w_i||_2 * Phi^-1(p_i), computed from the row as stored, so that
  P(w_i . x + b_i > 0) = p_i exactly for Gaussian x.
- Predictor output bias b2_i = Phi^-1(p_i) / sqrt(2): the logit's standard
  deviation is 1/sqrt(2) for these draws, so the predictor fires with about
  the same marginal rate p_i.  Threshold 0.
- Q4_0 (blocks of 32 weights, fp16 scale s, 4-bit codes q, w = (q - 8) s):
  codes uniform on 0..15, s = fp16(|N(0, 1/fan_in)| * 0.25), fan_in = d for
  W_up / W_gate and n for W_downT.
- Floating draws are float32 normals scaled, then rounded once to the
  stored dtype (round to nearest even).

Storage encodings:
- f32 / f16 matrices: row-major [rows][cols], one row per neuron.
- Q4_0 matrix row (d elements, d % 256 == 0): d/2 code bytes followed by
  d/32 fp16 scales (9d/16 bytes per row).  Code byte 16*j + t (t < 16) holds
  element 32*j + t in its low nibble and element 32*j + t + 16 in its high
  nibble; scale j belongs to elements [32*j, 32*j + 32).

Seeds: numpy PCG64 from SeedSequence(20231216, spawn_key=(workload, layer,
tensor, step, block)); matrices are drawn in blocks of ROW_BLOCK rows so any
row block can be regenerated alone and blocks can be drawn in parallel.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np
from scipy.special import ndtri

SEED = 20231216
ROW_BLOCK = 2048
ZIPF_S = 1.1
P_CLIP = 0.99

# tensor ids of the spawn key
T_PERM, T_WUP, T_WGATE, T_WDOWN, T_P1, T_P2, T_X, T_PROF, T_QCODE, T_QSCALE = range(10)

F32, F16, Q4_0 = "f32", "f16", "q4_0"
RELU, REGLU, SQRELU = "relu", "reglu", "sqrelu"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: a layer shape plus how it is driven."""
    key: int                  # workload number in the spawn key
    name: str
    d: int                    # d_model
    n: int                    # d_ffn (neurons)
    r: int                    # predictor rank
    wdtype: str               # FFN weight storage: f32 / f16 / q4_0
    pdtype: str               # predictor weight storage: f32 / f16
    xdtype: str               # input storage: f32 / f16
    act: str                  # relu / reglu / sqrelu (squared ReLU: deciding row W_up, as ReLU)
    mean: float               # mean firing probability
    batches: tuple = (1,)
    steps: int = 64
    layers: int = 1
    hot_frac: Optional[float] = None   # hot partition budget as a fraction of neurons
    profile_samples: int = 1024

    def scaled(self, d, n, r, name=None, **kw):
        """Same recipe at a smaller shape (for tests the oracle finishes quickly)."""
        return dataclasses.replace(self, d=d, n=n, r=r, name=name or f"{self.name}-small", **kw)


WORKLOADS = {
    "opt-fp32": Workload(0, "opt-fp32", d=1024, n=4096, r=128, wdtype=F32, pdtype=F32,
                         xdtype=F32, act=RELU, mean=0.10, batches=(1,), steps=64),
    "opt30b-fp16": Workload(1, "opt30b-fp16", d=7168, n=28672, r=1024, wdtype=F16, pdtype=F16,
                            xdtype=F16, act=RELU, mean=0.10, batches=(1,), steps=64,
                            hot_frac=0.26, profile_samples=1024),
    "llama70b-reglu-fp16": Workload(2, "llama70b-reglu-fp16", d=8192, n=28672, r=1024, wdtype=F16,
                                    pdtype=F16, xdtype=F16, act=REGLU, mean=0.15,
                                    batches=(1, 4), steps=64),
    "falcon40b-stack-fp16": Workload(3, "falcon40b-stack-fp16", d=8192, n=32768, r=1024,
                                     wdtype=F16, pdtype=F16, xdtype=F16, act=RELU, mean=0.10,
                                     batches=(1,), steps=128, layers=60, hot_frac=0.20,
                                     profile_samples=1024),
    "opt175b-q4_0": Workload(4, "opt175b-q4_0", d=12288, n=49152, r=1024, wdtype=Q4_0,
                             pdtype=F16, xdtype=F16, act=RELU, mean=0.08, batches=(1, 8, 64),
                             steps=64),
}


def _rng(wl: Workload, layer: int, tensor: int, step: int = 0, block: int = 0):
    ss = np.random.SeedSequence(SEED, spawn_key=(wl.key, layer, tensor, step, block))
    return np.random.Generator(np.random.PCG64(ss))


def zipf_probs(n: int, mean: float, s: float = ZIPF_S, clip: float = P_CLIP) -> np.ndarray:
    """p_k = min(c * k**-s, clip) for ranks k = 1..n with mean(p) == mean (bisection on c)."""
    if not (0.0 < mean < clip):
        raise ValueError("mean must lie in (0, clip)")
    base = np.arange(1, n + 1, dtype=np.float64) ** (-s)
    lo, hi = 0.0, clip / base[-1]          # at hi every p is clipped -> mean == clip
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.minimum(mid * base, clip).mean() < mean:
            lo = mid
        else:
            hi = mid
    c = 0.5 * (lo + hi)
    return np.minimum(c * base, clip)


def neuron_probs(wl: Workload, layer: int = 0) -> np.ndarray:
    """Firing probability of each neuron: Zipf ranks dealt by a seeded permutation."""
    p_rank = zipf_probs(wl.n, wl.mean)
    perm = _rng(wl, layer, T_PERM).permutation(wl.n)
    p = np.empty(wl.n, dtype=np.float64)
    p[perm] = p_rank                       # neuron perm[k] has rank k+1
    return p


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F32:
        return a32.astype(np.float32, copy=False)
    if dtype == F16:
        return a32.astype(np.float16)
    raise ValueError(dtype)


def _normal_matrix(wl, layer, tensor, rows, cols, std, dtype, threads=8):
    """rows x cols of N(0, std^2), drawn per ROW_BLOCK block, stored as dtype."""
    out = np.empty((rows, cols), dtype=np.float32 if dtype == F32 else np.float16)

    def fill(b):
        r0, r1 = b * ROW_BLOCK, min(rows, (b + 1) * ROW_BLOCK)
        g = _rng(wl, layer, tensor, 0, b)
        a = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        a *= np.float32(std)
        out[r0:r1] = _store(a, dtype)

    nb = (rows + ROW_BLOCK - 1) // ROW_BLOCK
    with ThreadPoolExecutor(max(1, min(threads, nb))) as ex:
        list(ex.map(fill, range(nb)))
    return out


def q4_0_pack(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Store codes [rows][d] (0..15) and fp16 scales [rows][d/32] in the Q4_0 row encoding
    described in the module docstring: d/2 code bytes, then d/32 fp16 scales."""
    rows, d = codes.shape
    c = codes.reshape(rows, d // 32, 2, 16).astype(np.uint8)
    packed = (c[:, :, 0, :] | (c[:, :, 1, :] << 4)).reshape(rows, d // 2)
    sc = np.ascontiguousarray(scales.astype(np.float16)).view(np.uint8).reshape(rows, d // 16)
    return np.ascontiguousarray(np.concatenate([packed, sc], axis=1))


def q4_0_row_bytes(d: int) -> int:
    return d // 2 + d // 16


def _q4_0_matrix(wl, layer, which, rows, d, fan_in, threads=8):
    """Returns (packed bytes [rows][9d/16], row L2 norms of the represented weights)."""
    if d % 256:
        raise ValueError("Q4_0 rows need d % 256 == 0")
    out = np.empty((rows, q4_0_row_bytes(d)), dtype=np.uint8)
    norms = np.empty(rows, dtype=np.float64)

    def fill(b):
        r0, r1 = b * ROW_BLOCK, min(rows, (b + 1) * ROW_BLOCK)
        gc = _rng(wl, layer, T_QCODE, which, b)
        gs = _rng(wl, layer, T_QSCALE, which, b)
        codes = gc.integers(0, 16, size=(r1 - r0, d), dtype=np.uint8)
        s = np.abs(gs.standard_normal((r1 - r0, d // 32), dtype=np.float32))
        s *= np.float32(0.25 / math.sqrt(fan_in))
        s16 = s.astype(np.float16)
        out[r0:r1] = q4_0_pack(codes, s16)
        # ||w||^2 = sum_j s_j^2 * sum_t (q_t - 8)^2 over the block (generation-side bookkeeping)
        qq = ((codes.astype(np.int32) - 8) ** 2).reshape(r1 - r0, d // 32, 32).sum(axis=2)
        norms[r0:r1] = np.sqrt((s16.astype(np.float64) ** 2 * qq).sum(axis=1))

    nb = (rows + ROW_BLOCK - 1) // ROW_BLOCK
    with ThreadPoolExecutor(max(1, min(threads, nb))) as ex:
        list(ex.map(fill, range(nb)))
    return out, norms


@dataclasses.dataclass
class Layer:
    """One FFN layer plus its predictor, as stored on the device.

    f32 matrices are float32 arrays, f16 matrices float16 arrays, Q4_0 matrices
    uint8 arrays [rows][9d/16].  Biases are float32.
    """
    wl: Workload
    layer: int
    p: np.ndarray                 # firing probabilities (float64 [n])
    W_up: np.ndarray
    W_gate: Optional[np.ndarray]
    W_downT: np.ndarray
    b_up: Optional[np.ndarray]
    b_gate: Optional[np.ndarray]
    P1t: np.ndarray
    P2t: np.ndarray
    b2: np.ndarray
    threshold: float = 0.0

    @property
    def d(self): return self.wl.d

    @property
    def n(self): return self.wl.n

    @property
    def r(self): return self.wl.r


def _row_norms(W: np.ndarray) -> np.ndarray:
    out = np.empty(W.shape[0], dtype=np.float64)
    for r0 in range(0, W.shape[0], 4096):
        blk = W[r0:r0 + 4096].astype(np.float64)
        out[r0:r0 + 4096] = np.sqrt(np.einsum("ij,ij->i", blk, blk))
    return out


def make_layer(wl: Workload, layer: int = 0, predictor_bias: bool = True, threads: int = 8) -> Layer:
    """Draw one layer of workload wl (deterministic in (wl.key, layer))."""
    d, n, r = wl.d, wl.n, wl.r
    p = neuron_probs(wl, layer)
    z = ndtri(p)
    W_gate = b_gate = b_up = None
    if wl.wdtype == Q4_0:
        W_up, up_norm = _q4_0_matrix(wl, layer, T_WUP, n, d, fan_in=d, threads=threads)
        W_downT, _ = _q4_0_matrix(wl, layer, T_WDOWN, n, d, fan_in=n, threads=threads)
        if wl.act == REGLU:
            W_gate, gate_norm = _q4_0_matrix(wl, layer, T_WGATE, n, d, fan_in=d, threads=threads)
    else:
        W_up = _normal_matrix(wl, layer, T_WUP, n, d, 1.0 / math.sqrt(d), wl.wdtype, threads)
        W_downT = _normal_matrix(wl, layer, T_WDOWN, n, d, 1.0 / math.sqrt(n), wl.wdtype, threads)
        up_norm = _row_norms(W_up)
        if wl.act == REGLU:
            W_gate = _normal_matrix(wl, layer, T_WGATE, n, d, 1.0 / math.sqrt(d), wl.wdtype, threads)
            gate_norm = _row_norms(W_gate)
    if wl.act == REGLU:
        b_gate = (gate_norm * z).astype(np.float32)
    else:
        b_up = (up_norm * z).astype(np.float32)
    P1t = _normal_matrix(wl, layer, T_P1, r, d, 1.0 / math.sqrt(d), wl.pdtype, threads)
    P2t = _normal_matrix(wl, layer, T_P2, n, r, 1.0 / math.sqrt(r), wl.pdtype, threads)
    b2 = (z / math.sqrt(2.0)).astype(np.float32) if predictor_bias else np.zeros(n, np.float32)
    return Layer(wl, layer, p, W_up, W_gate, W_downT, b_up, b_gate, P1t, P2t, b2, 0.0)


def make_x(wl: Workload, layer: int, step: int, B: int) -> np.ndarray:
    """Decode inputs x[B][d] ~ N(0,1), stored in wl.xdtype."""
    a = _rng(wl, layer, T_X, step).standard_normal((B, wl.d), dtype=np.float32)
    return _store(a, wl.xdtype)


def make_profile_x(wl: Workload, layer: int, samples: Optional[int] = None) -> np.ndarray:
    """Profiling inputs [S][d] ~ N(0,1) from their own seed stream, stored in wl.xdtype."""
    S = wl.profile_samples if samples is None else samples
    a = _rng(wl, layer, T_PROF).standard_normal((S, wl.d), dtype=np.float32)
    return _store(a, wl.xdtype)


def bytes_per_neuron(wl: Workload) -> int:
    """Device bytes one neuron owns in the FFN: its weight rows plus fp32 biases."""
    m = 3 if wl.act == REGLU else 2
    row = q4_0_row_bytes(wl.d) if wl.wdtype == Q4_0 else wl.d * (4 if wl.wdtype == F32 else 2)
    return m * row + 4          # one fp32 bias: b_up (ReLU) or b_gate (ReGLU)


def budget_bytes(wl: Workload) -> int:
    """Device-memory budget of the hot partition: hot_frac of the layer's FFN bytes."""
    if wl.hot_frac is None:
        return wl.n * bytes_per_neuron(wl)
    return int(wl.hot_frac * wl.n * bytes_per_neuron(wl))


def make_layer_device(wl: Workload, layer: int, device="cuda"):
    """The same recipe drawn on the GPU with torch's generator (seeded per workload and
    layer), for timing runs over many layers where host generation would take minutes.
    Float workloads only.  Values differ from make_layer's (different generator); the
    shapes, distributions, biases and firing rates are the same.  Returns a dict of
    device tensors with the Layer field names."""
    import torch
    if wl.wdtype == Q4_0:
        raise ValueError("device generation covers f32/f16 workloads")
    d, n, r = wl.d, wl.n, wl.r
    g = torch.Generator(device=device)
    g.manual_seed(SEED * 1000003 + wl.key * 1009 + layer)
    dt = torch.float16 if wl.wdtype == F16 else torch.float32
    pdt = torch.float16 if wl.pdtype == F16 else torch.float32
    z = torch.from_numpy(ndtri(neuron_probs(wl, layer))).to(device)

    def normal(rows, cols, std, dtype):
        out = torch.empty(rows, cols, dtype=dtype, device=device)
        for r0 in range(0, rows, 4096):
            blk = torch.randn(min(4096, rows - r0), cols, generator=g, device=device)
            out[r0:r0 + blk.shape[0]] = (blk * std).to(dtype)
        return out

    W_up = normal(n, d, 1.0 / math.sqrt(d), dt)
    W_downT = normal(n, d, 1.0 / math.sqrt(n), dt)
    W_gate = b_up = b_gate = None
    if wl.act == REGLU:
        W_gate = normal(n, d, 1.0 / math.sqrt(d), dt)
        b_gate = (W_gate.float().norm(dim=1).double() * z).float()
    else:
        b_up = (W_up.float().norm(dim=1).double() * z).float()
    P1t = normal(r, d, 1.0 / math.sqrt(d), pdt)
    P2t = normal(n, r, 1.0 / math.sqrt(r), pdt)
    b2 = (z / math.sqrt(2.0)).float()
    return dict(W_up=W_up, W_gate=W_gate, W_downT=W_downT, b_up=b_up, b_gate=b_gate, P1t=P1t,
                P2t=P2t, b2=b2, threshold=0.0)
