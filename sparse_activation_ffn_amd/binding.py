"""ctypes binding of libpi.so (the C ABI in include/pi.h).

Argument marshalling only: every function takes torch tensors (device memory)
or plain integers, converts them to pointers / sizes, calls the entry point of
the same name and raises PiError on a nonzero status.  All computation runs in
the library's HIP kernels.  There is no fallback: if libpi.so is missing or
cannot be loaded, `lib()` raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpi.so")

PI_OK, PI_ERR_ARG, PI_ERR_SHAPE, PI_ERR_ALIGN, PI_ERR_DTYPE, PI_ERR_WORKSPACE, PI_ERR_BUDGET, \
    PI_ERR_HIP = range(8)
PI_F32, PI_F16, PI_Q4_0 = 0, 1, 2
PI_RELU, PI_REGLU, PI_SQRELU = 0, 1, 2
PI_MAX_BATCH = 64
(PI_K_PRED_L1, PI_K_PRED_L2, PI_K_COMPACT, PI_K_UP, PI_K_DOWN, PI_K_MERGE, PI_K_PROFILE,
 PI_K_INDEX, PI_K_COPY, PI_K_REDUCE, PI_K_FFN, PI_K_ACCUMULATE, PI_K_STREAM, PI_K_UP_FINISH,
 PI_K_COUNT) = range(15)
PI_STREAM_SINK_WORDS = 2048
PI_SCRATCH_BYTES = 32 << 20

# every symbol include/pi.h declares
EXPORTS = ("pi_workspace_bytes", "pi_workspace_init", "pi_predict", "pi_compact_active",
           "pi_sparse_ffn", "pi_sparse_ffn_split", "pi_sparse_ffn_split_noalloc",
           "pi_sparse_ffn_crossover", "pi_merge",
           "pi_dense_ffn",
           "pi_profile_counts", "pi_build_neuron_index", "pi_plan_hot_split",
           "pi_calibrate_workspace_bytes", "pi_calibrate_threshold", "pi_true_mask",
           "pi_host_sparse_ffn", "pi_hybrid_host_bytes", "pi_sparse_ffn_hybrid",
           "pi_accumulate_mask", "pi_permute_rows",
           "pi_copy", "pi_stream_read",
           "pi_kernel_timer_start", "pi_kernel_timer_stop", "pi_kernel_name", "pi_status_string",
           "pi_last_error")


class PiError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class HybridInfo(C.Structure):
    _fields_ = [("cold_count", C.c_int32), ("threads", C.c_int32), ("wait_us", C.c_double),
                ("host_us", C.c_double)]


class Predictor(C.Structure):
    _fields_ = [("d", C.c_int32), ("n", C.c_int32), ("r", C.c_int32), ("wdtype", C.c_int32),
                ("P1t", C.c_void_p), ("P2t", C.c_void_p), ("b2", C.c_void_p),
                ("threshold", C.c_float)]


class FfnPart(C.Structure):
    _fields_ = [("d", C.c_int32), ("rows", C.c_int32), ("wdtype", C.c_int32), ("act", C.c_int32),
                ("W_up", C.c_void_p), ("W_gate", C.c_void_p), ("b_up", C.c_void_p),
                ("b_gate", C.c_void_p), ("W_downT", C.c_void_p)]


class ActiveLists(C.Structure):
    _fields_ = [("n_hot", C.c_int32), ("hot_idx", C.c_void_p), ("cold_idx", C.c_void_p),
                ("counts", C.c_void_p)]


_lib = None


def lib() -> C.CDLL:
    """Load libpi.so (built by sparse_activation_ffn_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sparse_activation_ffn_amd.build`")
    L = C.CDLL(LIB_PATH)
    P, I32, I64, SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    sig = {
        "pi_workspace_bytes": ([I32, I32, I32, I32], SZ),
        "pi_workspace_init": ([P, SZ, P], I32),
        "pi_predict": ([P, P, I32, I32, P, P, P, P, SZ, P], I32),
        "pi_compact_active": ([P, I32, P, P], I32),
        "pi_sparse_ffn": ([P, P, I32, I32, P, P, P, P, SZ, P], I32),
        "pi_sparse_ffn_split": ([P, P, P, I32, I32, P, P, P, P, P, P, SZ, P], I32),
        "pi_sparse_ffn_split_noalloc": ([P, P, P, I32, I32, P, P, P, P, P, P], I32),
        "pi_sparse_ffn_crossover": ([P, P, P, I32, I32, P, P, I32, P, P, P, P, SZ, P], I32),
        "pi_merge": ([P, P, I32, I32, P, P], I32),
        "pi_dense_ffn": ([P, P, I32, I32, P, P, SZ, P], I32),
        "pi_profile_counts": ([P, P, I32, I32, P, P], I32),
        "pi_build_neuron_index": ([P, I32, I64, I64, P, P, P], I32),
        "pi_plan_hot_split": ([P, I32, I64, I64, C.c_double, C.c_double, P], I32),
        "pi_calibrate_workspace_bytes": ([I32, I32, I32, I32], SZ),
        "pi_calibrate_threshold": ([P, P, P, I32, I32, C.c_double, P, P, P, SZ, P], I32),
        "pi_true_mask": ([P, P, I32, I32, P, P], I32),
        "pi_host_sparse_ffn": ([P, P, I32, I32, P, I32, P, I32], I32),
        "pi_hybrid_host_bytes": ([I32, I32, I32], SZ),
        "pi_sparse_ffn_hybrid": ([P, P, P, I32, I32, P, P, P, P, P, SZ, P, SZ, I32, P, P], I32),
        "pi_accumulate_mask": ([P, I32, P, P], I32),
        "pi_permute_rows": ([P, P, P, I32, I64, P], I32),
        "pi_copy": ([P, P, I64, P], I32),
        "pi_stream_read": ([P, I64, P, P], I32),
        "pi_kernel_timer_start": ([I32, I32], I32),
        "pi_kernel_timer_stop": ([I32, P, P], I32),
        "pi_kernel_name": ([I32], C.c_char_p),
        "pi_status_string": ([I32], C.c_char_p),
        "pi_last_error": ([], C.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def _check(status: int):
    if status != PI_OK:
        L = lib()
        raise PiError(status, f"{L.pi_status_string(status).decode()}: "
                              f"{L.pi_last_error().decode()}")


def ptr(t) -> Optional[int]:
    """Device pointer of a tensor (or an int passed through, None stays None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def stream_handle(stream=None) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return PI_F32
    if t.dtype == torch.float16:
        return PI_F16
    raise TypeError(f"no pi dtype for {t.dtype}")


# ---- the C entry points, same names -----------------------------------------

def pi_workspace_bytes(d: int, n: int, r: int, B: int) -> int:
    return int(lib().pi_workspace_bytes(d, n, r, B))


def pi_workspace_init(ws, stream=None):
    _check(lib().pi_workspace_init(ptr(ws), ws.numel() * ws.element_size(), stream_handle(stream)))


def pi_predict(pred: Predictor, x, mask, logits=None, lists: Optional[ActiveLists] = None,
               ws=None, stream=None):
    _check(lib().pi_predict(C.byref(pred), ptr(x), x.shape[0], dtype_code(x), ptr(mask),
                            ptr(logits), None if lists is None else C.byref(lists), ptr(ws),
                            0 if ws is None else ws.numel() * ws.element_size(),
                            stream_handle(stream)))


def pi_compact_active(mask, n: int, lists: ActiveLists, stream=None):
    _check(lib().pi_compact_active(ptr(mask), n, C.byref(lists), stream_handle(stream)))


def pi_sparse_ffn(part: FfnPart, x, idx, count, y, ws, stream=None):
    _check(lib().pi_sparse_ffn(C.byref(part), ptr(x), x.shape[0], dtype_code(x), ptr(idx),
                               ptr(count), ptr(y), ptr(ws), ws.numel() * ws.element_size(),
                               stream_handle(stream)))


def pi_sparse_ffn_split(hot: FfnPart, cold: Optional[FfnPart], x, lists: ActiveLists,
                        y_hot=None, y_cold=None, y=None, ws=None, stream=None, mask=None):
    """mask given: compaction fused, `lists` are outputs; mask None: `lists` are inputs."""
    _check(lib().pi_sparse_ffn_split(C.byref(hot), None if cold is None else C.byref(cold),
                                     ptr(x), x.shape[0], dtype_code(x), ptr(mask), C.byref(lists),
                                     ptr(y_hot), ptr(y_cold), ptr(y), ptr(ws),
                                     0 if ws is None else ws.numel() * ws.element_size(),
                                     stream_handle(stream)))


def pi_sparse_ffn_split_noalloc(hot: FfnPart, cold: Optional[FfnPart], x, lists: ActiveLists,
                                y_hot=None, y_cold=None, y=None, stream=None, mask=None):
    """pi_sparse_ffn_split with the library's static scratch instead of a workspace."""
    _check(lib().pi_sparse_ffn_split_noalloc(C.byref(hot), None if cold is None else C.byref(cold),
                                             ptr(x), x.shape[0], dtype_code(x), ptr(mask),
                                             C.byref(lists), ptr(y_hot), ptr(y_cold), ptr(y),
                                             stream_handle(stream)))


def pi_sparse_ffn_crossover(hot: FfnPart, cold: Optional[FfnPart], x, lists: ActiveLists,
                            dense_from: int, y_hot=None, y_cold=None, y=None, ws=None, stream=None,
                            mask=None):
    """pi_sparse_ffn_split, but every row is computed when the device active count
    reaches dense_from (the prompt-phase crossover)."""
    _check(lib().pi_sparse_ffn_crossover(C.byref(hot), None if cold is None else C.byref(cold),
                                         ptr(x), x.shape[0], dtype_code(x), ptr(mask),
                                         C.byref(lists), int(dense_from), ptr(y_hot), ptr(y_cold),
                                         ptr(y), ptr(ws),
                                         0 if ws is None else ws.numel() * ws.element_size(),
                                         stream_handle(stream)))


def pi_merge(y_hot, y_cold, y, stream=None):
    B, d = y_hot.shape
    _check(lib().pi_merge(ptr(y_hot), ptr(y_cold), B, d, ptr(y), stream_handle(stream)))


def pi_dense_ffn(part: FfnPart, x, y, ws, stream=None):
    _check(lib().pi_dense_ffn(C.byref(part), ptr(x), x.shape[0], dtype_code(x), ptr(y), ptr(ws),
                              ws.numel() * ws.element_size(), stream_handle(stream)))


def pi_profile_counts(part: FfnPart, X, counts, stream=None):
    _check(lib().pi_profile_counts(C.byref(part), ptr(X), X.shape[0], dtype_code(X), ptr(counts),
                                   stream_handle(stream)))


def pi_build_neuron_index(counts, budget_bytes: int, bytes_per_neuron: int, perm,
                          stream=None) -> int:
    n_hot = C.c_int32(0)
    _check(lib().pi_build_neuron_index(ptr(counts), counts.numel(), int(budget_bytes),
                                       int(bytes_per_neuron), ptr(perm), C.byref(n_hot),
                                       stream_handle(stream)))
    return int(n_hot.value)


def pi_plan_hot_split(counts_slot, budget_bytes: int, bytes_per_neuron: int, hbm_gbps: float,
                      link_gbps: float) -> int:
    """counts_slot: host array (numpy uint32) of activation counts in slot order."""
    import numpy as np
    c = np.ascontiguousarray(counts_slot, dtype=np.uint32)
    n_hot = C.c_int32(0)
    _check(lib().pi_plan_hot_split(c.ctypes.data if c.size else None, c.size, int(budget_bytes),
                                   int(bytes_per_neuron), float(hbm_gbps), float(link_gbps),
                                   C.byref(n_hot)))
    return int(n_hot.value)


def pi_calibrate_workspace_bytes(d: int, n: int, r: int, S: int) -> int:
    return int(lib().pi_calibrate_workspace_bytes(d, n, r, S))


def pi_calibrate_threshold(pred: Predictor, part: FfnPart, X, target_recall: float, tau, stats,
                           ws, stream=None):
    _check(lib().pi_calibrate_threshold(C.byref(pred), C.byref(part), ptr(X), X.shape[0],
                                        dtype_code(X), float(target_recall), ptr(tau), ptr(stats),
                                        ptr(ws), ws.numel() * ws.element_size(),
                                        stream_handle(stream)))


def pi_true_mask(part: FfnPart, x, mask, stream=None):
    _check(lib().pi_true_mask(C.byref(part), ptr(x), x.shape[0], dtype_code(x), ptr(mask),
                              stream_handle(stream)))


def pi_host_sparse_ffn(part: FfnPart, x, idx, count: int, y, threads: int = 0):
    """Every tensor here is a CPU tensor (host memory); runs on the host cores."""
    _check(lib().pi_host_sparse_ffn(C.byref(part), ptr(x), x.shape[0], dtype_code(x), ptr(idx),
                                    int(count), ptr(y), int(threads)))


def pi_hybrid_host_bytes(d: int, n: int, B: int) -> int:
    return lib().pi_hybrid_host_bytes(d, n, B)


def pi_sparse_ffn_hybrid(hot: FfnPart, cold: FfnPart, x, mask, lists: ActiveLists, y_cold, y, ws,
                         host_ws, threads: int = 0, stream=None) -> HybridInfo:
    """hot on the device, cold (host-memory weights) on the host cores; host_ws is a pinned
    CPU tensor of at least pi_hybrid_host_bytes bytes.  Returns the call's HybridInfo."""
    info = HybridInfo()
    _check(lib().pi_sparse_ffn_hybrid(C.byref(hot), C.byref(cold), ptr(x), x.shape[0],
                                      dtype_code(x), ptr(mask), C.byref(lists), ptr(y_cold),
                                      ptr(y), ptr(ws), ws.numel() * ws.element_size(),
                                      ptr(host_ws), host_ws.numel() * host_ws.element_size(),
                                      int(threads), C.byref(info), stream_handle(stream)))
    return info


def pi_accumulate_mask(mask, n: int, counts, stream=None):
    _check(lib().pi_accumulate_mask(ptr(mask), n, ptr(counts), stream_handle(stream)))


def pi_permute_rows(src, dst, perm, rows: int, row_bytes: int, stream=None):
    _check(lib().pi_permute_rows(ptr(src), ptr(dst), ptr(perm), rows, row_bytes,
                                 stream_handle(stream)))


def pi_copy(src, dst, nbytes: int, stream=None):
    _check(lib().pi_copy(ptr(src), ptr(dst), nbytes, stream_handle(stream)))


def pi_stream_read(src, nbytes: int, sink, stream=None):
    _check(lib().pi_stream_read(ptr(src), nbytes, ptr(sink), stream_handle(stream)))


def pi_kernel_timer_start(kid: int, max_launches: int):
    _check(lib().pi_kernel_timer_start(kid, max_launches))


def pi_kernel_timer_stop(kid: int):
    ms, k = C.c_float(0.0), C.c_int32(0)
    _check(lib().pi_kernel_timer_stop(kid, C.byref(ms), C.byref(k)))
    return float(ms.value), int(k.value)


def pi_kernel_name(kid: int) -> str:
    return lib().pi_kernel_name(kid).decode()


# ---- descriptors from device tensors ------------------------------------------

def make_predictor(P1t, P2t, b2, threshold: float = 0.0) -> Predictor:
    r, d = P1t.shape
    n = P2t.shape[0]
    p = Predictor(d, n, r, dtype_code(P1t), ptr(P1t), ptr(P2t), ptr(b2), float(threshold))
    p._keep = (P1t, P2t, b2)
    return p


def make_part(d: int, W_up, W_downT, act: int = PI_RELU, W_gate=None, b_up=None, b_gate=None,
              q4: bool = False) -> FfnPart:
    rows = W_up.shape[0]
    wdtype = PI_Q4_0 if q4 else dtype_code(W_up)
    p = FfnPart(d, rows, wdtype, act, ptr(W_up), ptr(W_gate), ptr(b_up), ptr(b_gate),
                ptr(W_downT))
    p._keep = (W_up, W_gate, b_up, b_gate, W_downT)
    return p


def make_lists(n_hot: int, hot_idx, cold_idx, counts) -> ActiveLists:
    L = ActiveLists(n_hot, ptr(hot_idx), ptr(cold_idx), ptr(counts))
    L._keep = (hot_idx, cold_idx, counts)
    return L


def row_slice(t, lo: int, hi: int):
    """Rows [lo, hi) of a per-neuron device tensor (a view, no copy)."""
    return None if t is None else t[lo:hi]
