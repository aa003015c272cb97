"""The host-core sparse FFN (pi_host_sparse_ffn) against the oracle, on the CPU.

This is the cold side of the hybrid step (CSDN article, section on the CPU/GPU
hybrid design and its figure: the CPU computes the predicted cold neurons next to
their weights in host memory).  The library's code runs on this machine's cores;
no GPU is used.  The oracle recomputes the same partition over the same list in
fp64; the host path accumulates in fp32, so the bar is the layer tolerance of the
GPU parity tests (fp32 weights: max-normwise 1e-5; fp16 / Q4_0: L2 2e-3).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import oracle as O  # noqa: E402
from parity import check_close  # noqa: E402
from sparse_activation_ffn_amd import binding as pb  # noqa: E402
from workload import synth as S  # noqa: E402

CASES = {
    # name: (workload, partition rows [lo, hi))
    "f32-relu": (S.WORKLOADS["opt-fp32"].scaled(d=320, n=700, r=32), (100, 700)),
    "f16-relu": (S.WORKLOADS["opt30b-fp16"].scaled(d=512, n=900, r=64), (233, 900)),
    "q4-relu": (S.WORKLOADS["opt175b-q4_0"].scaled(d=768, n=600, r=64), (0, 600)),
    "f16-reglu": (S.WORKLOADS["llama70b-reglu-fp16"].scaled(d=384, n=640, r=48), (64, 640)),
    "f32-sqrelu": (S.WORKLOADS["opt-fp32"].scaled(d=256, n=500, r=32, act="sqrelu"), (0, 500)),
    "q4-sqrelu": (S.WORKLOADS["opt175b-q4_0"].scaled(d=512, n=400, r=64, act="sqrelu"), (50, 400)),
}
_LAYERS = {}


def _layer(name):
    if name not in _LAYERS:
        _LAYERS[name] = S.make_layer(CASES[name][0])
    return _LAYERS[name]


def _host_part(L, lo, hi):
    """Rows [lo, hi) as a partition over CPU tensors (host memory)."""
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a[lo:hi]))  # noqa: E731
    act = {"relu": pb.PI_RELU, "reglu": pb.PI_REGLU, "sqrelu": pb.PI_SQRELU}[L.wl.act]
    return pb.make_part(L.d, t(L.W_up), t(L.W_downT), act, t(L.W_gate), t(L.b_up), t(L.b_gate),
                        q4=L.wl.wdtype == "q4_0")


def _ids(rows, seed, density=0.3):
    rng = np.random.default_rng(seed)
    ids = np.flatnonzero(rng.random(rows) < density).astype(np.int32)
    return np.unique(np.concatenate([ids, [0, rows - 1]]).astype(np.int32))


def _run(part, x, ids, threads, count=None):
    y = torch.full((x.shape[0], part.d), float("nan"), dtype=torch.float32)
    idx = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32))
    pb.pi_host_sparse_ffn(part, torch.from_numpy(x), idx, len(ids) if count is None else count, y,
                          threads)
    return y.numpy()


@pytest.mark.parametrize("threads", [1, 3, 0])
@pytest.mark.parametrize("B", [1, 3])
@pytest.mark.parametrize("name", list(CASES))
def test_host_sparse_ffn_matches_oracle(name, B, threads):
    wl, (lo, hi) = CASES[name]
    L = _layer(name)
    part = _host_part(L, lo, hi)
    x = S.make_x(wl, 0, 1, B)
    ids = _ids(hi - lo, seed=B * 7 + threads)
    y = _run(part, x, ids, threads)
    ref = O.sparse_ffn(O.Part.from_layer(L, lo, hi), x, ids)
    check_close(y, ref, wl.wdtype)


def test_reproducible_for_a_thread_count():
    name = "f16-relu"
    wl, (lo, hi) = CASES[name]
    L = _layer(name)
    part = _host_part(L, lo, hi)
    x = S.make_x(wl, 0, 2, 2)
    ids = _ids(hi - lo, seed=5, density=0.6)
    for threads in (1, 4):
        a, b = _run(part, x, ids, threads), _run(part, x, ids, threads)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    check_close(_run(part, x, ids, 4), _run(part, x, ids, 1), "f16")


def test_empty_list_and_ids_outside_the_partition():
    name = "f32-relu"
    wl, (lo, hi) = CASES[name]
    L = _layer(name)
    part = _host_part(L, lo, hi)
    x = S.make_x(wl, 0, 3, 2)
    # an empty list: y is all zeros (every token)
    y = _run(part, x, np.zeros(1, np.int32), threads=2, count=0)
    assert np.all(y == 0.0)
    # ids below 0 or at/after the partition's rows add nothing
    rows = hi - lo
    ids = _ids(rows, seed=11)
    mixed = np.concatenate([[-5, -1], ids, [rows, rows + 100]]).astype(np.int32)
    ref = O.sparse_ffn(O.Part.from_layer(L, lo, hi), x, ids)
    check_close(_run(part, x, mixed, threads=3), ref, "f32")
    # only the first `count` entries are read
    check_close(_run(part, x, np.concatenate([ids, [1, 2, 3]]).astype(np.int32), threads=2,
                     count=len(ids)), ref, "f32")


def test_more_threads_than_rows():
    name = "q4-relu"
    wl, (lo, hi) = CASES[name]
    L = _layer(name)
    part = _host_part(L, lo, hi)
    x = S.make_x(wl, 0, 4, 1)
    ids = np.array([7, 300], np.int32)
    ref = O.sparse_ffn(O.Part.from_layer(L, lo, hi), x, ids)
    check_close(_run(part, x, ids, threads=64), ref, "q4_0")


def test_host_sparse_ffn_validation():
    L = pb.lib()
    name = "f16-relu"
    wl, (lo, hi) = CASES[name]
    part = _host_part(_layer(name), lo, hi)
    x = torch.zeros((1, wl.d), dtype=torch.float16)
    y = torch.zeros((1, wl.d), dtype=torch.float32)
    idx = torch.zeros(4, dtype=torch.int32)
    C = pytest.importorskip("ctypes")
    call = lambda **kw: L.pi_host_sparse_ffn(  # noqa: E731
        C.byref(kw.get("part", part)), kw.get("x", x.data_ptr()), kw.get("B", 1),
        kw.get("xdt", pb.PI_F16), kw.get("idx", idx.data_ptr()), kw.get("count", 4),
        kw.get("y", y.data_ptr()), kw.get("threads", 1))
    assert call(B=0) == pb.PI_ERR_SHAPE
    assert call(B=pb.PI_MAX_BATCH + 1) == pb.PI_ERR_SHAPE
    assert call(xdt=7) == pb.PI_ERR_DTYPE
    assert call(count=-1) == pb.PI_ERR_SHAPE
    assert call(threads=-2) == pb.PI_ERR_ARG
    assert call(x=None) == pb.PI_ERR_ARG
    assert call(y=None) == pb.PI_ERR_ARG
    assert call(idx=None) == pb.PI_ERR_ARG
    bad = pb.FfnPart(wl.d, hi - lo, 9, pb.PI_RELU, part.W_up, None, None, None, part.W_downT)
    assert call(part=bad) == pb.PI_ERR_DTYPE
    assert call(idx=None, count=0) == pb.PI_OK
    assert np.all(y.numpy() == 0.0)


def test_portable_code_path_matches_oracle():
    """The same parity cases with the portable (non-AVX2) row code, selected by
    PI_HOST_PLAIN=1 in a fresh process (the choice is read once per process)."""
    import os
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    env = dict(os.environ, PI_HOST_PLAIN="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(here, "test_host_ffn.py"), "-k",
                        "matches_oracle and not portable"],
                       cwd=os.path.dirname(here), env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert " passed" in r.stdout


def test_forked_child_builds_its_own_pool():
    """A child forked after the pool exists (its worker threads are not copied) still
    computes: it starts a pool of its own."""
    import os
    name = "f16-relu"
    wl, (lo, hi) = CASES[name]
    L = _layer(name)
    part = _host_part(L, lo, hi)
    x = S.make_x(wl, 0, 5, 2)
    ids = _ids(hi - lo, seed=3)
    want = _run(part, x, ids, threads=4)            # the parent's pool now exists
    r, w = os.pipe()
    pid = os.fork()
    if pid == 0:                                    # child: same call, report bit equality
        ok = False
        try:
            ok = np.array_equal(_run(part, x, ids, threads=4).view(np.uint32), want.view(np.uint32))
        finally:
            os.write(w, b"1" if ok else b"0")
            os._exit(0)
    os.close(w)
    got = os.read(r, 1)
    os.waitpid(pid, 0)
    assert got == b"1"
