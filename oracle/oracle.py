"""ctypes wrapper of the plain-C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the GPU library or its binding.
Every function here marshals numpy arrays to the C routines and back; the
arithmetic lives in oracle.c (double precision, scalar loops).

Parity pins: every routine is pinned by the CPU tests against something other
than itself (closed forms, invariants, brute force, numpy float64 routines);
the test module for each routine names the pins.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F32, F16, Q4_0 = 0, 1, 2
RELU, REGLU, SQRELU = 0, 1, 2
DT = {"f32": F32, "f16": F16, "q4_0": Q4_0}
ACT = {"relu": RELU, "reglu": REGLU, "sqrelu": SQRELU}


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (IEEE semantics: no fast-math, no contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC",
                               "-shared", "-Wall", "-Wextra", SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        P, I64, I, D = C.c_void_p, C.c_int64, C.c_int, C.c_double
        _lib.or_set_threads.argtypes = [I]
        _lib.or_set_threads.restype = None
        _lib.or_get_threads.argtypes = []
        _lib.or_get_threads.restype = I
        _lib.or_half_to_double.argtypes = [C.c_uint16]
        _lib.or_half_to_double.restype = D
        _lib.or_q4_0_element.argtypes = [P, I64, I64]
        _lib.or_q4_0_element.restype = D
        _lib.or_load_row.argtypes = [P, I, I64, I64, P]
        _lib.or_load_row.restype = None
        _lib.or_predict.argtypes = [I64, I64, I64, I, P, P, P, D, P, I, I64, P, P, P]
        _lib.or_compact.argtypes = [P, I64, I64, P, P, P]
        _lib.or_sparse_ffn.argtypes = [P, P, I, I64, P, I64, P]
        _lib.or_dense_ffn.argtypes = [P, P, I, I64, P]
        _lib.or_merge.argtypes = [P, P, I64, P]
        _lib.or_merge.restype = None
        _lib.or_profile_counts.argtypes = [P, P, I, I64, P, P, P, D]
        _lib.or_build_neuron_index.argtypes = [P, I64, I64, I64, P, P]
        _lib.or_plan_hot_split.argtypes = [P, I64, I64, I64, D, D, P]
        _lib.or_calibrate_threshold.argtypes = [I64, I64, I64, I, P, P, P, P, P, I, I64, D, P, P]
        _lib.or_layer_step.argtypes = [I64, I64, I64, I, P, P, P, D, P, P, P, I, I64, P, P, P, P,
                                       P]
    return _lib


class _Part(C.Structure):
    _fields_ = [("d", C.c_int64), ("rows", C.c_int64), ("wdtype", C.c_int), ("act", C.c_int),
                ("W_up", C.c_void_p), ("W_gate", C.c_void_p), ("b_up", C.c_void_p),
                ("b_gate", C.c_void_p), ("W_downT", C.c_void_p)]


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_code(a: np.ndarray, q4: bool = False) -> int:
    if q4:
        return Q4_0
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float16:
        return F16
    raise TypeError(f"unsupported dtype {a.dtype}")


class Part:
    """One FFN partition (row block of a layer) held as numpy arrays."""

    def __init__(self, d, W_up, W_downT, act="relu", W_gate=None, b_up=None, b_gate=None,
                 q4=False):
        self.d = d
        self.q4 = q4
        self.arrays = [np.ascontiguousarray(a) if a is not None else None
                       for a in (W_up, W_gate, b_up, b_gate, W_downT)]
        W_up, W_gate, b_up, b_gate, W_downT = self.arrays
        for b in (b_up, b_gate):
            if b is not None and b.dtype != np.float32:
                raise TypeError("biases are float32")
        self.rows = W_up.shape[0]
        self.s = _Part(d, self.rows, _dtype_code(W_up, q4), ACT[act] if isinstance(act, str) else act,
                       _ptr(W_up), _ptr(W_gate), _ptr(b_up), _ptr(b_gate), _ptr(W_downT))

    @classmethod
    def from_layer(cls, L, lo=0, hi=None):
        """Rows [lo, hi) of a workload Layer as a partition."""
        hi = L.n if hi is None else hi
        sl = lambda a: None if a is None else a[lo:hi]  # noqa: E731
        return cls(L.d, sl(L.W_up), sl(L.W_downT), act=L.wl.act, W_gate=sl(L.W_gate),
                   b_up=sl(L.b_up), b_gate=sl(L.b_gate), q4=(L.wl.wdtype == "q4_0"))


def set_threads(k: int) -> None:
    """Share the oracle's independent outer loops among k threads (1 = serial).
    Results are bit-identical for every k."""
    lib().or_set_threads(int(k))


def get_threads() -> int:
    return int(lib().or_get_threads())


def half_to_double(bits: int) -> float:
    return lib().or_half_to_double(bits)


def load_row(W: np.ndarray, d: int, row: int, q4: bool = False) -> np.ndarray:
    out = np.empty(d, dtype=np.float64)
    lib().or_load_row(_ptr(np.ascontiguousarray(W)), _dtype_code(W, q4), d, row, _ptr(out))
    return out


def dequant(W: np.ndarray, d: int, q4: bool = False) -> np.ndarray:
    """Whole matrix decoded to float64 [rows][d] via the row loader."""
    W = np.ascontiguousarray(W)
    return np.stack([load_row(W, d, i, q4) for i in range(W.shape[0])]) if W.shape[0] else \
        np.zeros((0, d))


def predict(P1t, P2t, b2, x, threshold=0.0):
    """Returns (mask uint64 [ceil(n/64)], logits float64 [B][n], mask decided in float32)."""
    P1t, P2t, x = (np.ascontiguousarray(a) for a in (P1t, P2t, x))
    r, d = P1t.shape
    n = P2t.shape[0]
    B = x.shape[0]
    words = (n + 63) // 64
    mask = np.zeros(words, np.uint64)
    mask32 = np.zeros(words, np.uint64)
    logits = np.zeros((B, n), np.float64)
    b2 = None if b2 is None else np.ascontiguousarray(b2, dtype=np.float32)
    rc = lib().or_predict(d, n, r, _dtype_code(P1t), _ptr(P1t), _ptr(P2t), _ptr(b2),
                          float(threshold), _ptr(x), _dtype_code(x), B, _ptr(mask), _ptr(logits),
                          _ptr(mask32))
    if rc:
        raise ValueError("or_predict rejected its arguments")
    return mask, logits, mask32


def compact(mask, n, n_hot=None):
    """Returns (hot ids, cold local ids) as int32 arrays."""
    n_hot = n if n_hot is None else n_hot
    mask = np.ascontiguousarray(mask, dtype=np.uint64)
    hot = np.zeros(max(n_hot, 1), np.int32)
    cold = np.zeros(max(n - n_hot, 1), np.int32)
    counts = np.zeros(2, np.int32)
    rc = lib().or_compact(_ptr(mask), n, n_hot, _ptr(hot), _ptr(cold), _ptr(counts))
    if rc:
        raise ValueError("or_compact rejected its arguments")
    return hot[:counts[0]].copy(), cold[:counts[1]].copy()


def sparse_ffn(part: Part, x, idx):
    x = np.ascontiguousarray(x)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B = x.shape[0]
    y = np.zeros((B, part.d), np.float64)
    rc = lib().or_sparse_ffn(C.byref(part.s), _ptr(x), _dtype_code(x), B, _ptr(idx), idx.size,
                             _ptr(y))
    if rc:
        raise ValueError("or_sparse_ffn rejected its arguments")
    return y


def dense_ffn(part: Part, x):
    x = np.ascontiguousarray(x)
    B = x.shape[0]
    y = np.zeros((B, part.d), np.float64)
    rc = lib().or_dense_ffn(C.byref(part.s), _ptr(x), _dtype_code(x), B, _ptr(y))
    if rc:
        raise ValueError("or_dense_ffn rejected its arguments")
    return y


def merge(y_hot, y_cold):
    y_hot = np.ascontiguousarray(y_hot, dtype=np.float64)
    y = np.empty_like(y_hot)
    yc = None if y_cold is None else np.ascontiguousarray(y_cold, dtype=np.float64)
    lib().or_merge(_ptr(y_hot), _ptr(yc), y_hot.size, _ptr(y))
    return y


def profile_counts(part: Part, X, band=0.0):
    """Returns (counts decided in fp64, counts decided in fp32, ambiguous-sample counts)."""
    X = np.ascontiguousarray(X)
    c = np.zeros(part.rows, np.uint32)
    c32 = np.zeros(part.rows, np.uint32)
    amb = np.zeros(part.rows, np.uint32)
    rc = lib().or_profile_counts(C.byref(part.s), _ptr(X), _dtype_code(X), X.shape[0], _ptr(c),
                                 _ptr(c32), _ptr(amb), float(band))
    if rc:
        raise ValueError("or_profile_counts rejected its arguments")
    return c, c32, amb


def build_neuron_index(counts, budget_bytes, bytes_per_neuron):
    counts = np.ascontiguousarray(counts, dtype=np.uint32)
    n = counts.size
    perm = np.zeros(max(n, 1), np.int32)
    n_hot = C.c_int64(0)
    rc = lib().or_build_neuron_index(_ptr(counts), n, int(budget_bytes), int(bytes_per_neuron),
                                     _ptr(perm), C.byref(n_hot))
    if rc:
        raise ValueError("or_build_neuron_index rejected its arguments")
    return perm[:n].copy(), int(n_hot.value)


def plan_hot_split(counts_slot, budget_bytes, bytes_per_neuron, hbm_rate, link_rate):
    """n_hot from the tiers' read rates and the capacity budget (counts in slot order)."""
    c = np.ascontiguousarray(counts_slot, dtype=np.uint32)
    out = C.c_int64(0)
    rc = lib().or_plan_hot_split(_ptr(c) if c.size else None, c.size, int(budget_bytes),
                                 int(bytes_per_neuron), float(hbm_rate), float(link_rate),
                                 C.byref(out))
    if rc:
        raise ValueError("or_plan_hot_split rejected its arguments")
    return int(out.value)


def calibrate_threshold(P1t, P2t, b2, part: Part, X, target):
    """Adaptive threshold: the largest float32 tau with recall >= target over the firing
    (sample, neuron) pairs of X.  Returns (tau, N firing pairs, m, firing pairs above tau)."""
    P1t, P2t, X = (np.ascontiguousarray(a) for a in (P1t, P2t, X))
    r, d = P1t.shape
    n = P2t.shape[0]
    b2 = None if b2 is None else np.ascontiguousarray(b2, dtype=np.float32)
    tau = np.zeros(1, np.float32)
    stats = np.zeros(3, np.int64)
    rc = lib().or_calibrate_threshold(d, n, r, _dtype_code(P1t), _ptr(P1t), _ptr(P2t), _ptr(b2),
                                      C.byref(part.s), _ptr(X), _dtype_code(X), X.shape[0],
                                      float(target), _ptr(tau), _ptr(stats))
    if rc:
        raise ValueError("or_calibrate_threshold rejected its arguments")
    return float(tau[0]), int(stats[0]), int(stats[1]), int(stats[2])


def layer_step(P1t, P2t, b2, threshold, hot: Part, cold, x):
    """predict -> compact -> sparse FFN per partition -> merge.  Returns (mask, hot, cold, y)."""
    P1t, P2t, x = (np.ascontiguousarray(a) for a in (P1t, P2t, x))
    r, d = P1t.shape
    n = P2t.shape[0]
    B = x.shape[0]
    mask = np.zeros((n + 63) // 64, np.uint64)
    hot_idx = np.zeros(max(hot.rows, 1), np.int32)
    cold_idx = np.zeros(max(n - hot.rows, 1), np.int32)
    counts = np.zeros(2, np.int32)
    y = np.zeros((B, d), np.float64)
    b2 = None if b2 is None else np.ascontiguousarray(b2, dtype=np.float32)
    rc = lib().or_layer_step(d, n, r, _dtype_code(P1t), _ptr(P1t), _ptr(P2t), _ptr(b2),
                             float(threshold), C.byref(hot.s),
                             None if cold is None else C.byref(cold.s), _ptr(x), _dtype_code(x),
                             B, _ptr(mask), _ptr(hot_idx), _ptr(cold_idx), _ptr(counts), _ptr(y))
    if rc:
        raise ValueError("or_layer_step rejected its arguments")
    return mask, hot_idx[:counts[0]].copy(), cold_idx[:counts[1]].copy(), y
