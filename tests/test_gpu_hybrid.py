"""GPU parity of the hybrid step: hot partition on the GPU, cold partition on the
host cores, merged on the GPU (CSDN article, section on the CPU/GPU hybrid design
and its figure; hada.io README summary, hybrid-approach section).

Per step, on seeded inputs: the predictor's mask comes from pi_predict; the
oracle compacts that mask into the hot and cold lists, and recomputes each
partition's sparse FFN over them in fp64.  Checked:
- the hot list and count the device writes equal the oracle's, bit for bit;
- the record's cold count equals the oracle's cold list length;
- y_cold (the host partial) and y (merged) match the oracle to the layer tolerance
  (partials measured on the scale of the merged output);
- y is close to the all-GPU split step (pi_sparse_ffn_split) on the same mask.
Edge cases: no hot rows, no cold rows, B = 5, repeated calls on one host workspace,
two host threads calling at once on two streams; and the errors the call detects
at run time (unpinned host workspace, cold weights in device memory).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import oracle as O  # noqa: E402
from parity import check_close  # noqa: E402
from sparse_activation_ffn_amd import binding as pb  # noqa: E402
from sparse_activation_ffn_amd.layer import DeviceLayer, StepBuffers  # noqa: E402
from workload import synth as S  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = {
    # name: (workload, n_hot)
    "f16": (S.WORKLOADS["opt30b-fp16"].scaled(d=512, n=1500, r=64), 400),
    "q4": (S.WORKLOADS["opt175b-q4_0"].scaled(d=1280, n=1111, r=64), 300),
    "f32-sqrelu": (S.WORKLOADS["opt-fp32"].scaled(d=320, n=1000, r=32, act="sqrelu"), 611),
    "reglu": (S.WORKLOADS["llama70b-reglu-fp16"].scaled(d=640, n=900, r=48), 128),
    "all-cold": (S.WORKLOADS["opt30b-fp16"].scaled(d=256, n=700, r=32), 0),
    "all-hot": (S.WORKLOADS["opt-fp32"].scaled(d=256, n=640, r=32), 640),
}


def log(*a):
    print(*a, flush=True)


def _np(t):
    return t.detach().cpu().numpy()


def _host_part(L, lo, hi):
    """Rows [lo, hi) in host memory (CPU tensors)."""
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a[lo:hi]))  # noqa: E731
    act = {"relu": pb.PI_RELU, "reglu": pb.PI_REGLU, "sqrelu": pb.PI_SQRELU}[L.wl.act]
    return pb.make_part(L.d, t(L.W_up), t(L.W_downT), act, t(L.W_gate), t(L.b_up), t(L.b_gate),
                        q4=L.wl.wdtype == "q4_0")


class Setup:
    def __init__(self, name, B):
        wl, n_hot = CASES[name]
        self.wl, self.n_hot, self.B = wl, n_hot, B
        self.L = S.make_layer(wl)
        self.dl = DeviceLayer.upload(self.L, DEV, n_hot=n_hot)
        self.buf = StepBuffers(self.dl, B, DEV)
        self.hot = self.dl.part(0, n_hot)
        self.cold = _host_part(self.L, n_hot, wl.n)
        self.y_cold = torch.zeros((B, wl.d), dtype=torch.float32, device=DEV)
        hb = pb.pi_hybrid_host_bytes(wl.d, wl.n, B)
        self.host_ws = torch.zeros(hb, dtype=torch.uint8, pin_memory=True)

    def step(self, s, threads=0):
        x_np = S.make_x(self.wl, 0, s, self.B)
        x = torch.from_numpy(x_np).to(DEV)
        b = self.buf
        pb.pi_predict(self.dl.predictor(), x, b.mask, None, None, b.ws)
        info = pb.pi_sparse_ffn_hybrid(self.hot, self.cold, x, b.mask, b.lists, self.y_cold, b.y,
                                       b.ws, self.host_ws, threads)
        torch.cuda.synchronize()
        return x, x_np, info


@pytest.mark.parametrize("B", [1, 5])
@pytest.mark.parametrize("name", list(CASES))
def test_hybrid_matches_oracle(name, B):
    log(f"hybrid {name} B={B}")
    st = Setup(name, B)
    wl, n_hot = st.wl, st.n_hot
    for s in range(3):                         # repeated calls on one host workspace
        x, x_np, info = st.step(s, threads=(0, 3, 1)[s])
        mask = _np(st.buf.mask).view(np.uint64)
        hot_o, cold_o = O.compact(mask, wl.n, n_hot)
        c = _np(st.buf.counts)
        if n_hot > 0:
            assert int(c[0]) == hot_o.size
            assert np.array_equal(_np(st.buf.hot_idx)[:c[0]], hot_o)
        assert info.cold_count == cold_o.size
        assert info.threads >= 1 and info.wait_us >= 0 and info.host_us >= 0
        y_hot_o = (O.sparse_ffn(O.Part.from_layer(st.L, 0, n_hot), x_np, hot_o) if n_hot > 0
                   else np.zeros((B, wl.d)))
        y_cold_o = (O.sparse_ffn(O.Part.from_layer(st.L, n_hot, wl.n), x_np, cold_o)
                    if n_hot < wl.n else np.zeros((B, wl.d)))
        y_o = O.merge(y_hot_o, y_cold_o)
        log(f"  step {s}: {hot_o.size} hot + {cold_o.size} cold active, host {info.host_us:.0f} us "
            f"on {info.threads} threads, wait {info.wait_us:.0f} us")
        check_close(_np(st.y_cold), y_cold_o, wl.wdtype, scale=y_o)
        check_close(_np(st.buf.y), y_o, wl.wdtype)
        # the all-GPU step over the same mask
        if n_hot < wl.n:
            dcold = st.dl.part(n_hot, wl.n)
            y_dev = torch.zeros_like(st.buf.y)
            pb.pi_sparse_ffn_split(st.hot, dcold, x, st.buf.lists, None, None, y_dev, st.buf.ws,
                                   mask=st.buf.mask)
            torch.cuda.synchronize()
            check_close(_np(st.buf.y), _np(y_dev), wl.wdtype)


def test_hybrid_runtime_errors():
    st = Setup("f16", 1)
    x = torch.from_numpy(S.make_x(st.wl, 0, 0, 1)).to(DEV)
    b = st.buf
    pb.pi_predict(st.dl.predictor(), x, b.mask, None, None, b.ws)
    # host workspace in pageable memory
    pageable = torch.zeros(st.host_ws.numel() + 64, dtype=torch.uint8)
    off = (-pageable.data_ptr()) % 64
    with pytest.raises(pb.PiError) as e:
        pb.pi_sparse_ffn_hybrid(st.hot, st.cold, x, b.mask, b.lists, st.y_cold, b.y, b.ws,
                                pageable[off:off + st.host_ws.numel()])
    assert e.value.status == pb.PI_ERR_ARG and "pinned" in str(e.value)
    # cold weights in device memory
    with pytest.raises(pb.PiError) as e:
        pb.pi_sparse_ffn_hybrid(st.hot, st.dl.part(st.n_hot, st.wl.n), x, b.mask, b.lists,
                                st.y_cold, b.y, b.ws, st.host_ws)
    assert e.value.status == pb.PI_ERR_ARG and "host memory" in str(e.value)
    torch.cuda.synchronize()
    # the call still works after the rejected ones
    x, x_np, info = st.step(1)
    hot_o, cold_o = O.compact(_np(b.mask).view(np.uint64), st.wl.n, st.n_hot)
    y_o = O.merge(O.sparse_ffn(O.Part.from_layer(st.L, 0, st.n_hot), x_np, hot_o),
                  O.sparse_ffn(O.Part.from_layer(st.L, st.n_hot, st.wl.n), x_np, cold_o))
    check_close(_np(b.y), y_o, st.wl.wdtype)


def test_hybrid_full_size_opt30b_shape():
    """OPT-30B-shaped layer (d 7168, n 28672) with the profiled neuron index and a 26 %
    hot partition on the GPU, the rest in host memory, batch 1: the output against
    the oracle's full-size result over the step's lists."""
    wl = S.WORKLOADS["opt30b-fp16"]
    L = S.make_layer(wl)
    base = DeviceLayer.upload(L, DEV)
    X = torch.from_numpy(S.make_profile_x(wl, 0)).to(DEV)
    counts = base.profile_counts(X)
    perm, n_hot = base.build_index(counts, S.budget_bytes(wl), S.bytes_per_neuron(wl))
    base.apply_index(perm, n_hot)
    del X
    p = _np(perm)
    import dataclasses
    take = lambda a: None if a is None else np.ascontiguousarray(a[p])  # noqa: E731
    Lh = dataclasses.replace(L, W_up=take(L.W_up), W_gate=take(L.W_gate), W_downT=take(L.W_downT),
                             b_up=take(L.b_up), b_gate=take(L.b_gate))
    buf = StepBuffers(base, 1, DEV)
    hot = base.part(0, n_hot)
    cold = _host_part(Lh, n_hot, wl.n)
    y_cold = torch.zeros((1, wl.d), dtype=torch.float32, device=DEV)
    host_ws = torch.zeros(pb.pi_hybrid_host_bytes(wl.d, wl.n, 1), dtype=torch.uint8, pin_memory=True)
    x_np = S.make_x(wl, 0, 3, 1)
    x = torch.from_numpy(x_np).to(DEV)
    pb.pi_predict(base.predictor(), x, buf.mask, None, None, buf.ws)
    info = pb.pi_sparse_ffn_hybrid(hot, cold, x, buf.mask, buf.lists, y_cold, buf.y, buf.ws, host_ws)
    torch.cuda.synchronize()
    hot_o, cold_o = O.compact(_np(buf.mask).view(np.uint64), wl.n, n_hot)
    assert info.cold_count == cold_o.size
    log(f"  n_hot {n_hot}: {hot_o.size} hot + {cold_o.size} cold active; host {info.host_us:.0f} us "
        f"on {info.threads} threads")
    y_o = O.merge(O.sparse_ffn(O.Part.from_layer(Lh, 0, n_hot), x_np, hot_o),
                  O.sparse_ffn(O.Part.from_layer(Lh, n_hot, wl.n), x_np, cold_o))
    check_close(_np(buf.y), y_o, "f16")


def test_hybrid_calls_from_two_threads_on_two_streams():
    """Two host threads, each with its own buffers and stream, run hybrid steps at the
    same time; each waits for its own mask and x (the arrival event is per thread) and
    gets its own step's result."""
    import threading
    st = [Setup("f16", 1), Setup("f16", 1)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    out = [None, None]
    errs = []

    def run(k):
        try:
            s = st[k]
            res = []
            with torch.cuda.stream(streams[k]):
                for step in range(4):
                    x_np = S.make_x(s.wl, 0, 10 * k + step, 1)
                    x = torch.from_numpy(x_np).to(DEV)
                    b = s.buf
                    pb.pi_predict(s.dl.predictor(), x, b.mask, None, None, b.ws, stream=streams[k])
                    pb.pi_sparse_ffn_hybrid(s.hot, s.cold, x, b.mask, b.lists, s.y_cold, b.y, b.ws,
                                            s.host_ws, 0, stream=streams[k])
                    streams[k].synchronize()
                    res.append((x_np, _np(b.mask).view(np.uint64).copy(), _np(b.y).copy()))
            out[k] = res
        except Exception as e:  # noqa: BLE001
            errs.append(e)

    th = [threading.Thread(target=run, args=(k,)) for k in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errs, errs
    for k in range(2):
        s = st[k]
        for x_np, mask, y in out[k]:
            hot_o, cold_o = O.compact(mask, s.wl.n, s.n_hot)
            y_o = O.merge(O.sparse_ffn(O.Part.from_layer(s.L, 0, s.n_hot), x_np, hot_o),
                          O.sparse_ffn(O.Part.from_layer(s.L, s.n_hot, s.wl.n), x_np, cold_o))
            check_close(y, y_o, s.wl.wdtype)
