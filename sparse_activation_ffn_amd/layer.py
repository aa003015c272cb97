"""One FFN layer with its predictor resident in device memory, driven through
the C ABI: offline profiling -> neuron index -> row permutation, and the
decode step predict(+compact) -> sparse FFN over hot and cold -> merge.

PowerInfer pages: CSDN article, overall-architecture section (offline
profiling and placement, online per-partition computation and merge) and
hybrid-design figure.  Only torch allocations and C calls happen here.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as pb


def _dev(a: Optional[np.ndarray], device) -> Optional[torch.Tensor]:
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceLayer:
    """Device tensors of one layer.  Per-neuron tensors are row-major [n][...]."""

    def __init__(self, d, n, r, act, wdtype_q4, W_up, W_gate, W_downT, b_up, b_gate, P1t, P2t,
                 b2, threshold=0.0, n_hot=None):
        self.d, self.n, self.r = d, n, r
        self.act = {"relu": pb.PI_RELU, "reglu": pb.PI_REGLU, "sqrelu": pb.PI_SQRELU}.get(act, act)
        self.q4 = wdtype_q4
        self.W_up, self.W_gate, self.W_downT = W_up, W_gate, W_downT
        self.b_up, self.b_gate = b_up, b_gate
        self.P1t, self.P2t, self.b2 = P1t, P2t, b2
        self.threshold = float(threshold)
        self.n_hot = n if n_hot is None else n_hot
        self.row_bytes = W_up.shape[1] * W_up.element_size()

    @classmethod
    def upload(cls, L, device="cuda", n_hot=None):
        """From a workload.synth.Layer (numpy) to device memory."""
        return cls(L.d, L.n, L.r, L.wl.act, L.wl.wdtype == "q4_0", _dev(L.W_up, device),
                   _dev(L.W_gate, device), _dev(L.W_downT, device), _dev(L.b_up, device),
                   _dev(L.b_gate, device), _dev(L.P1t, device), _dev(L.P2t, device),
                   _dev(L.b2, device), L.threshold, n_hot)

    @classmethod
    def from_tensors(cls, wl, t: dict, n_hot=None):
        """From device tensors with the Layer field names (workload.synth.make_layer_device)."""
        return cls(wl.d, wl.n, wl.r, wl.act, wl.wdtype == "q4_0", t["W_up"], t["W_gate"],
                   t["W_downT"], t["b_up"], t["b_gate"], t["P1t"], t["P2t"], t["b2"],
                   t["threshold"], n_hot)

    def clone(self):
        """Same values at new device addresses (another instance of the layer)."""
        c = lambda t: None if t is None else t.clone()  # noqa: E731
        return DeviceLayer(self.d, self.n, self.r, self.act, self.q4, c(self.W_up), c(self.W_gate),
                           c(self.W_downT), c(self.b_up), c(self.b_gate), c(self.P1t),
                           c(self.P2t), c(self.b2), self.threshold, self.n_hot)

    # ---- descriptors ---------------------------------------------------------
    def predictor(self) -> pb.Predictor:
        return pb.make_predictor(self.P1t, self.P2t, self.b2, self.threshold)

    def part(self, lo=0, hi=None) -> pb.FfnPart:
        hi = self.n if hi is None else hi
        s = lambda t: pb.row_slice(t, lo, hi)  # noqa: E731
        return pb.make_part(self.d, s(self.W_up), s(self.W_downT), self.act, s(self.W_gate),
                            s(self.b_up), s(self.b_gate), q4=self.q4)

    def parts(self):
        hot = self.part(0, self.n_hot)
        cold = None
        if self.n_hot < self.n:
            ch = getattr(self, "cold_host", None)
            if ch is None:
                cold = self.part(self.n_hot, self.n)
            else:
                s = lambda t: pb.row_slice(t, self.n_hot, self.n)  # noqa: E731
                cold = pb.make_part(self.d, ch["W_up"], ch["W_downT"], self.act, ch["W_gate"],
                                    s(self.b_up), s(self.b_gate), q4=self.q4)
        return hot, cold

    # ---- online index maintenance -------------------------------------------------
    def accumulate(self, mask: torch.Tensor, counts: torch.Tensor):
        """counts[i] += predicted bit i of this step's mask (current slot order)."""
        pb.pi_accumulate_mask(mask, self.n, counts)

    def reindex(self, counts: torch.Tensor, budget_bytes: int, bytes_per_neuron: int):
        """Online FFN splitting (hada.io README summary, recent updates; the FAQ
        rebuilds the GPU index): a new neuron index from counts gathered during
        decode, applied to the already-indexed layer.  counts is permuted with the
        rows, so it keeps describing the slots.  Returns (perm, n_hot), perm mapping
        each new slot to its slot before this call."""
        perm, n_hot = self.build_index(counts, budget_bytes, bytes_per_neuron)
        self.apply_index(perm, n_hot)
        moved = torch.empty_like(counts)
        pb.pi_permute_rows(counts, moved, perm, self.n, 4)
        counts.copy_(moved)
        if getattr(self, "cold_host", None) is not None:
            self.place_cold_on_host()
        return perm, n_hot

    # ---- capacity tiers ---------------------------------------------------------
    def place_cold_on_host(self):
        """Capacity-tiered placement (CSDN article, hybrid-design section: the hot
        neurons stay on the GPU, the cold ones live in host memory): the weight rows
        of the cold partition are copied into pinned host memory, which the GPU reads
        directly over the host link; the hot partition, the predictor and the biases
        stay in device memory.  parts() then describes the cold partition at its
        host addresses; the kernels are the same."""
        if self.n_hot >= self.n:
            return

        def host(t):
            if t is None:
                return None
            h = torch.empty(t[self.n_hot:].shape, dtype=t.dtype, pin_memory=True)
            h.copy_(t[self.n_hot:])
            return h
        self.cold_host = {"W_up": host(self.W_up), "W_gate": host(self.W_gate),
                          "W_downT": host(self.W_downT)}

    # ---- offline: profiling and neuron index ----------------------------------
    def profile_counts(self, X: torch.Tensor) -> torch.Tensor:
        counts = torch.empty(self.n, dtype=torch.int32, device=X.device)
        pb.pi_profile_counts(self.part(), X, counts)
        return counts

    def build_index(self, counts: torch.Tensor, budget_bytes: int, bytes_per_neuron: int):
        perm = torch.empty(self.n, dtype=torch.int32, device=counts.device)
        n_hot = pb.pi_build_neuron_index(counts, budget_bytes, bytes_per_neuron, perm)
        return perm, n_hot

    def apply_index(self, perm: torch.Tensor, n_hot: int):
        """Permute every per-neuron tensor by perm (slot -> original id)."""
        def permute(t):
            if t is None:
                return None
            out = torch.empty_like(t)
            rb = t[0].numel() * t.element_size() if t.dim() > 1 else t.element_size()
            pb.pi_permute_rows(t, out, perm, self.n, rb)
            return out
        self.W_up, self.W_gate, self.W_downT = (permute(self.W_up), permute(self.W_gate),
                                                permute(self.W_downT))
        self.b_up, self.b_gate = permute(self.b_up), permute(self.b_gate)
        self.P2t, self.b2 = permute(self.P2t), permute(self.b2)
        self.n_hot = n_hot


class StepBuffers:
    """Mask, active lists, outputs and workspace for decode steps of one shape."""

    def __init__(self, layer: DeviceLayer, B: int, device="cuda"):
        n, d = layer.n, layer.d
        self.B = B
        self.mask = torch.zeros((n + 63) // 64, dtype=torch.int64, device=device)
        self.hot_idx = torch.zeros(max(layer.n_hot, 1), dtype=torch.int32, device=device)
        self.cold_idx = torch.zeros(max(n - layer.n_hot, 1), dtype=torch.int32, device=device)
        self.counts = torch.zeros(2, dtype=torch.int32, device=device)
        self.y = torch.zeros((B, d), dtype=torch.float32, device=device)
        self.y_hot = torch.zeros((B, d), dtype=torch.float32, device=device)
        self.y_cold = torch.zeros((B, d), dtype=torch.float32, device=device)
        wsb = pb.pi_workspace_bytes(d, n, layer.r, B)
        self.ws = torch.empty(wsb, dtype=torch.uint8, device=device)
        pb.pi_workspace_init(self.ws)
        self.lists = pb.make_lists(layer.n_hot, self.hot_idx,
                                   self.cold_idx if layer.n_hot < n else None, self.counts)


def decode_step(layer: DeviceLayer, x: torch.Tensor, buf: StepBuffers, pred=None, parts=None,
                partials: bool = False, logits=None, stream=None):
    """predict -> (compaction fused into) sparse FFN on hot and cold -> merge, on one stream.
    buf.lists receives the active lists as a side output."""
    pred = layer.predictor() if pred is None else pred
    hot, cold = layer.parts() if parts is None else parts
    pb.pi_predict(pred, x, buf.mask, logits, None, buf.ws, stream)
    pb.pi_sparse_ffn_split(hot, cold, x, buf.lists, buf.y_hot if partials else None,
                           buf.y_cold if partials and cold is not None else None, buf.y, buf.ws,
                           stream, mask=buf.mask)
    return buf.y
