"""The no-allocation entry point (pi_sparse_ffn_split_noalloc) against the
workspace entry point (pi_sparse_ffn_split), through the C ABI.

Both run the same kernels with the same summation order, so their outputs
(y, y_hot, y_cold, the active lists and counts) must be bit-identical.  Two
calls in a row on one GPU, the second with a smaller input, so the second call
runs on scratch the first one left behind.  The too-large case is rejected
before anything is enqueued.
"""
import ctypes as C

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from sparse_activation_ffn_amd import binding as pb  # noqa: E402
from sparse_activation_ffn_amd.layer import DeviceLayer, StepBuffers  # noqa: E402
from workload import synth as S  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.detach().cpu().numpy().copy()


def _both(dl, B, x_np):
    """One step with the workspace entry point, then the same step with the static
    scratch; returns both outputs."""
    x = torch.from_numpy(x_np).to(DEV)
    hot, cold = dl.parts()
    res = []
    for noalloc in (False, True):
        buf = StepBuffers(dl, B, DEV)
        buf.hot_idx.fill_(-3)
        buf.cold_idx.fill_(-3)
        buf.y.fill_(7.0)
        pb.pi_predict(dl.predictor(), x, buf.mask, None, None, buf.ws)
        yc = buf.y_cold if cold is not None else None
        if noalloc:
            pb.pi_sparse_ffn_split_noalloc(hot, cold, x, buf.lists, buf.y_hot, yc, buf.y,
                                           mask=buf.mask)
        else:
            pb.pi_sparse_ffn_split(hot, cold, x, buf.lists, buf.y_hot, yc, buf.y, buf.ws,
                                   mask=buf.mask)
        torch.cuda.synchronize()
        c = _np(buf.counts)
        res.append(dict(counts=c, hot=_np(buf.hot_idx)[:c[0]], cold=_np(buf.cold_idx)[:c[1]],
                        y=_np(buf.y), y_hot=_np(buf.y_hot),
                        y_cold=_np(buf.y_cold) if cold is not None else None))
    return res


@pytest.mark.parametrize("first,second", [
    (("opt30b-fp16", 7168, 28672, 1024, 1, 7454), ("opt30b-fp16", 576, 2085, 64, 1, 700)),
    (("opt175b-q4_0", 1280, 1111, 128, 64, None), ("opt175b-q4_0", 1280, 1111, 128, 8, 300)),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    for name, d, n, r, B, n_hot in (first, second):
        wl = S.WORKLOADS[name]
        if d != wl.d:
            wl = wl.scaled(d=d, n=n, r=r)
        L = S.make_layer(wl)
        dl = DeviceLayer.upload(L, DEV, n_hot=n_hot)
        x = S.make_x(wl, 0, 2, B)
        ref, got = _both(dl, B, x)
        for k in ("counts", "hot", "cold", "y", "y_hot", "y_cold"):
            if ref[k] is not None:
                assert np.array_equal(got[k], ref[k]), f"{name} d={d} B={B}: {k} differs"
        print(f"  {name} d={d} B={B}: {int(ref['counts'].sum())} active, bit-identical", flush=True)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    L = pb.lib()
    FAKE = 0x10000        # never dereferenced: the call fails its size check first
    hot = pb.FfnPart(1024, 262144, pb.PI_F32, pb.PI_RELU, FAKE, None, None, None, FAKE)
    lists = pb.ActiveLists(262144, FAKE, None, FAKE)
    rc = L.pi_sparse_ffn_split_noalloc(C.byref(hot), None, FAKE, 64, pb.PI_F32, None,
                                       C.byref(lists), None, None, FAKE, None)
    assert rc == pb.PI_ERR_WORKSPACE
    assert b"static scratch" in L.pi_last_error()
