"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Workloads follow the five synthetic layer shapes (OPT-style fp32; OPT-30B fp16
with a 26% hot partition; LLaMA(ReGLU)-70B fp16 at batch 1 and 4; Falcon-40B
fp16 layer with a 20% hot partition from 1024 profiling samples; OPT-175B Q4_0
at batch 1, 8 and 64), at reduced sizes that span several tiles with ragged
tails and at full size.  The comparison protocol is in tests/parity.py.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import oracle as O  # noqa: E402
from parity import (check_close, check_mask, mask_bits, oracle_ffn,  # noqa: E402
                    oracle_threads, permute_layer)
from sparse_activation_ffn_amd import binding as pb  # noqa: E402
from sparse_activation_ffn_amd.layer import DeviceLayer, StepBuffers  # noqa: E402
from workload import synth as S  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _threaded_oracle():
    """The oracle's outer loops on the host's cores (bit-identical results) so the
    full-size cases finish in seconds."""
    O.set_threads(oracle_threads())
    yield
    O.set_threads(1)


def log(*a):
    print(*a, flush=True)


def _np(t):
    return t.detach().cpu().numpy()


def run_step(dl: DeviceLayer, buf: StepBuffers, x_np, logits=True, partials=True, fused=True):
    """One decode step through the C ABI.  fused: pi_predict writes the mask and
    pi_sparse_ffn_split compacts it (lists as side output); otherwise pi_predict
    compacts into lists and pi_sparse_ffn_split reads them."""
    x = torch.from_numpy(x_np).to(DEV)
    B = x_np.shape[0]
    lg = torch.empty((B, dl.n), dtype=torch.float32, device=DEV) if logits else None
    hot, cold = dl.parts()
    buf.hot_idx.fill_(-7)
    buf.cold_idx.fill_(-7)
    buf.counts.fill_(-7)
    pb.pi_predict(dl.predictor(), x, buf.mask, lg, None if fused else buf.lists, buf.ws)
    pb.pi_sparse_ffn_split(hot, cold, x, buf.lists, buf.y_hot if partials else None,
                           buf.y_cold if partials and cold is not None else None, buf.y, buf.ws,
                           mask=buf.mask if fused else None)
    torch.cuda.synchronize()
    c = _np(buf.counts)
    out = dict(mask=_np(buf.mask).view(np.uint64), counts=c, hot=_np(buf.hot_idx)[:c[0]],
               cold=_np(buf.cold_idx)[:c[1]], y=_np(buf.y))
    if lg is not None:
        out["logits"] = _np(lg)
    if partials:
        out["y_hot"] = _np(buf.y_hot)
        out["y_cold"] = _np(buf.y_cold) if cold is not None else None
    return out


def check_step(Lh, n_hot, x_np, out, tokens=None):
    """Full protocol for one step; Lh is the host layer in slot order."""
    n = Lh.n
    mask_o, logits_o, _ = O.predict(Lh.P1t, Lh.P2t, Lh.b2, x_np, Lh.threshold)
    namb = check_mask(out["mask"], mask_o, logits_o, n, Lh.threshold)
    if "logits" in out:
        assert np.max(np.abs(out["logits"] - logits_o)) < 1e-4
    hot_o, cold_o = O.compact(out["mask"], n, n_hot)
    assert np.array_equal(out["hot"], hot_o) and np.array_equal(out["cold"], cold_o)
    xs = x_np if tokens is None else x_np[tokens]
    yh, yc, y = oracle_ffn(Lh, n_hot, xs, hot_o, cold_o)
    sel = (lambda a: a) if tokens is None else (lambda a: a[tokens])  # noqa: E731
    e = check_close(sel(out["y"]), y, Lh.wl.wdtype)
    if "y_hot" in out:
        check_close(sel(out["y_hot"]), yh, Lh.wl.wdtype, scale=y)
        if out.get("y_cold") is not None:
            check_close(sel(out["y_cold"]), yc, Lh.wl.wdtype, scale=y)
    return e, namb, len(hot_o) + len(cold_o)


def index_layer(L, dl: DeviceLayer, samples: int, rows_checked=None, X=None):
    """Profile on the GPU, check counts, build + check the index, permute on the GPU.
    X: the profiling samples as a device tensor (default: drawn on the host)."""
    wl = L.wl
    if X is None:
        X_np = S.make_profile_x(wl, L.layer, samples)
        X = torch.from_numpy(X_np).to(DEV)
    else:
        X_np = _np(X)
    counts = dl.profile_counts(X)
    torch.cuda.synchronize()
    cg = _np(counts).astype(np.uint32)
    rows = np.arange(wl.n) if rows_checked is None else rows_checked
    sub = O.Part(wl.d, L.W_up[rows], L.W_downT[rows], act=wl.act,
                 W_gate=None if L.W_gate is None else L.W_gate[rows],
                 b_up=None if L.b_up is None else L.b_up[rows],
                 b_gate=None if L.b_gate is None else L.b_gate[rows], q4=(wl.wdtype == "q4_0"))
    _, c32, amb = O.profile_counts(sub, X_np, band=1e-4)
    diff = np.abs(cg[rows].astype(np.int64) - c32.astype(np.int64))
    assert np.all(diff <= amb), "activation counts differ beyond ambiguous samples"
    bpn, budget = S.bytes_per_neuron(wl), S.budget_bytes(wl)
    perm, n_hot = dl.build_index(counts, budget, bpn)
    torch.cuda.synchronize()
    perm_o, n_hot_o = O.build_neuron_index(cg, budget, bpn)
    assert n_hot == n_hot_o
    assert np.array_equal(_np(perm), perm_o)
    dl.apply_index(perm, n_hot)
    torch.cuda.synchronize()
    Lh = permute_layer(L, perm_o)
    for name in ("W_up", "W_downT", "P2t", "b2", "b_up", "b_gate", "W_gate"):
        a = getattr(Lh, name)
        if a is not None:
            assert np.array_equal(_np(getattr(dl, name)), a), f"{name} permuted wrongly"
    return Lh, n_hot


# --------------------------------------------------------------------------------
# reduced sizes (several tiles, ragged tails)
# --------------------------------------------------------------------------------

SMALL = {
    "opt-fp32": S.WORKLOADS["opt-fp32"].scaled(d=320, n=1000, r=32),
    "opt30b-fp16": S.WORKLOADS["opt30b-fp16"].scaled(d=576, n=2085, r=64),
    "llama70b-reglu-fp16": S.WORKLOADS["llama70b-reglu-fp16"].scaled(d=640, n=1500, r=48),
    "falcon40b-stack-fp16": S.WORKLOADS["falcon40b-stack-fp16"].scaled(d=512, n=1700, r=32),
    "opt175b-q4_0": S.WORKLOADS["opt175b-q4_0"].scaled(d=1280, n=1111, r=64),
}


@pytest.mark.parametrize("name,B", [("opt-fp32", 1), ("opt-fp32", 3), ("opt30b-fp16", 1),
                                    ("llama70b-reglu-fp16", 1), ("llama70b-reglu-fp16", 4),
                                    ("falcon40b-stack-fp16", 1), ("opt175b-q4_0", 1),
                                    ("opt175b-q4_0", 8), ("opt175b-q4_0", 64)])
def test_small_parity(name, B):
    wl = SMALL[name]
    log(f"small {name} B={B}")
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    if wl.hot_frac is not None:
        Lh, n_hot = index_layer(L, dl, 256)
    else:
        Lh, n_hot = L, wl.n
    buf = StepBuffers(dl, B, DEV)
    for step in range(4):
        x = S.make_x(wl, 0, step, B)
        e, namb, na = check_step(Lh, n_hot, x, run_step(dl, buf, x, fused=(step % 2 == 0)))
        log(f"  step {step}: active {na}, ambiguous {namb}, err {e:.2e}")


@pytest.mark.parametrize("base,d", [("opt-fp32", 1216), ("opt30b-fp16", 2368),
                                    ("llama70b-reglu-fp16", 2368), ("opt175b-q4_0", 9472),
                                    ("opt175b-q4_0", 16384)])
def test_fused_kernel_chunk_maps(base, d):
    """Batch-1 fused kernel with one 16-byte chunk per thread and between 256 and 512
    chunks per row: the down chunks start at the threads without an up chunk, so
    threads [0, 2 nch - 512) take both, [2 nch - 512, nch) up only and [nch, 512)
    down only.  d gives nch = 304 (f32), 296 (f16 and Q4_0): the boundaries fall
    inside waves; d = 16384 (Q4_0) gives 512 chunks, both on every thread."""
    wl = S.WORKLOADS[base].scaled(d=d, n=733, r=32, hot_frac=None)
    log(f"fused chunk map {base} d={d}")
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    buf = StepBuffers(dl, 1, DEV)
    for step in range(3):
        x = S.make_x(wl, 0, step, 1)
        e, namb, na = check_step(L, wl.n, x, run_step(dl, buf, x, fused=(step != 1)))
        log(f"  step {step}: active {na}, ambiguous {namb}, err {e:.2e}")


def test_gathered_path_with_more_than_64k_of_lds():
    """f32 weights at batch 6 take the gathered two-kernel path; at d = 2048 the
    token group of x (8 x 2048 fp32 = 64 KiB) plus the mask words and their scan
    exceed 64 KiB of dynamic LDS, which the kernel must be granted explicitly."""
    wl = S.WORKLOADS["opt-fp32"].scaled(d=2048, n=3000, r=64)
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    buf = StepBuffers(dl, 6, DEV)
    for step in range(2):
        x = S.make_x(wl, 0, step, 6)
        e, namb, na = check_step(L, wl.n, x, run_step(dl, buf, x, fused=(step == 0)))
        log(f"  step {step}: active {na}, ambiguous {namb}, err {e:.2e}")


SQRELU_SMALL = {
    "f16": S.WORKLOADS["opt30b-fp16"].scaled(d=576, n=2085, r=64, act="sqrelu"),
    "f32": S.WORKLOADS["opt-fp32"].scaled(d=320, n=1000, r=32, act="sqrelu"),
    "q4_0": S.WORKLOADS["opt175b-q4_0"].scaled(d=1280, n=1111, r=64, act="sqrelu"),
}


@pytest.mark.parametrize("name,B", [("f16", 1), ("f16", 16), ("f32", 1), ("f32", 3), ("f32", 6),
                                    ("q4_0", 1), ("q4_0", 8)])
def test_squared_relu(name, B):
    """Squared ReLU (h = max(0, a)^2) through the fused kernel (batch 1; f32 batch 3),
    the gathered two-kernel path (f32 batch 6) and the matrix-core path (batch 8, 16)."""
    wl = SQRELU_SMALL[name]
    log(f"squared relu {name} B={B}")
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    if wl.hot_frac is not None:
        Lh, n_hot = index_layer(L, dl, 256)
    else:
        Lh, n_hot = L, wl.n
    buf = StepBuffers(dl, B, DEV)
    for step in range(2):
        x = S.make_x(wl, 0, step, B)
        e, namb, na = check_step(Lh, n_hot, x, run_step(dl, buf, x, fused=(step == 0)))
        log(f"  step {step}: active {na}, ambiguous {namb}, err {e:.2e}")


MFMA_SMALL = {
    "reglu-f16": S.WORKLOADS["llama70b-reglu-fp16"].scaled(d=768, n=1333, r=64),
    "relu-f16-split": S.WORKLOADS["opt30b-fp16"].scaled(d=512, n=1500, r=32),
    "q4_0": S.WORKLOADS["opt175b-q4_0"].scaled(d=1280, n=1111, r=64),
    "q4_0-reglu-split": S.WORKLOADS["opt175b-q4_0"].scaled(d=768, n=900, r=32, act="reglu",
                                                           hot_frac=0.3, name="q4_0-reglu-small"),
}


@pytest.mark.parametrize("name,B", [("relu-f16-split", 2), ("reglu-f16", 3), ("q4_0", 5),
                                    ("reglu-f16", 16), ("reglu-f16", 33), ("relu-f16-split", 64),
                                    ("q4_0", 16), ("q4_0", 20), ("q4_0", 32), ("q4_0", 64),
                                    ("q4_0-reglu-split", 48)])
def test_matrix_core_batches(name, B):
    """Batches of 2..64 tokens (matrix-core path: token tiles of 16, 32 and 64; the
    Q4_0 up kernel in two K slices at 5, 20 and 32 tokens, four at 16, one at 64):
    union active set, f16-rounded h and dequantised weights, checked to the fp16 /
    Q4_0 tolerance."""
    wl = MFMA_SMALL[name]
    log(f"matrix-core {name} B={B}")
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    if wl.hot_frac is not None:
        Lh, n_hot = index_layer(L, dl, 256)
    else:
        Lh, n_hot = L, wl.n
    buf = StepBuffers(dl, B, DEV)
    for step in range(2):
        x = S.make_x(wl, 0, step, B)
        e, namb, na = check_step(Lh, n_hot, x, run_step(dl, buf, x, fused=(step == 0)))
        log(f"  step {step}: union active {na}, ambiguous {namb}, err {e:.2e}")


@pytest.mark.parametrize("B", [2, 20])
@pytest.mark.parametrize("thr", [1e30, -1e30])
def test_matrix_core_empty_and_full_active_sets(thr, B):
    """Matrix-core path with no active neuron (y = 0 exactly, zero counts) and with
    every neuron active (y = dense FFN), both partitions present."""
    import dataclasses
    wl = MFMA_SMALL["relu-f16-split"]
    L = dataclasses.replace(S.make_layer(wl), threshold=thr)
    dl = DeviceLayer.upload(L, DEV, n_hot=600)
    buf = StepBuffers(dl, B, DEV)
    x = S.make_x(wl, 0, 0, B)
    out = run_step(dl, buf, x)
    if thr > 0:
        assert out["counts"].tolist() == [0, 0] and not out["mask"].any()
        assert np.all(out["y"] == 0) and np.all(out["y_hot"] == 0) and np.all(out["y_cold"] == 0)
    else:
        assert out["counts"].tolist() == [600, wl.n - 600]
        check_close(out["y"], O.dense_ffn(O.Part.from_layer(L), x), "f16")
    check_step(L, 600, x, out)


def test_fp32_layer_all_decode_tokens():
    """OPT-style fp32 layer at full size (d 1024, n 4096, rank 128), all 64 decode tokens."""
    wl = S.WORKLOADS["opt-fp32"]
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    buf = StepBuffers(dl, 1, DEV)
    worst = 0.0
    for step in range(wl.steps):
        x = S.make_x(wl, 0, step, 1)
        e, _, _ = check_step(L, wl.n, x, run_step(dl, buf, x, fused=(step % 2 == 0)))
        worst = max(worst, e)
    log(f"  fp32 full: worst normwise max-rel error {worst:.2e} over {wl.steps} tokens")


# --------------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def small_f16():
    wl = S.WORKLOADS["opt30b-fp16"].scaled(d=320, n=777, r=32)
    L = S.make_layer(wl)
    return wl, L


@pytest.mark.parametrize("thr", [1e30, -1e30])
def test_empty_and_full_active_sets(small_f16, thr):
    wl, L = small_f16
    import dataclasses
    L2 = dataclasses.replace(L, threshold=thr)
    dl = DeviceLayer.upload(L2, DEV, n_hot=300)
    buf = StepBuffers(dl, 2, DEV)
    x = S.make_x(wl, 0, 0, 2)
    out = run_step(dl, buf, x)
    if thr > 0:
        assert out["counts"].tolist() == [0, 0] and not out["mask"].any()
        assert np.all(out["y"] == 0) and np.all(out["y_hot"] == 0) and np.all(out["y_cold"] == 0)
    else:
        assert out["counts"].tolist() == [300, wl.n - 300]
        dense = O.dense_ffn(O.Part.from_layer(L), x)
        check_close(out["y"], dense, "f16")
    check_step(L2, 300, x, out)


@pytest.mark.parametrize("n_hot", [0, 1, 776, 777])
def test_split_points(small_f16, n_hot):
    wl, L = small_f16
    dl = DeviceLayer.upload(L, DEV, n_hot=n_hot)
    buf = StepBuffers(dl, 1, DEV)
    for step in range(2):
        x = S.make_x(wl, 0, step, 1)
        check_step(L, n_hot, x, run_step(dl, buf, x, fused=(step == 0)))


def test_two_mask_words_per_thread_ragged():
    """32768 < n <= 65536 with n % 64 != 0: the fused kernel's prologue gives a
    thread two mask words, and the last word has one valid bit."""
    wl = S.WORKLOADS["opt30b-fp16"].scaled(d=256, n=40001, r=32)
    L = S.make_layer(wl)
    n_hot = 10000
    dl = DeviceLayer.upload(L, DEV, n_hot=n_hot)
    buf = StepBuffers(dl, 1, DEV)
    for step in range(2):
        x = S.make_x(wl, 0, step, 1)
        e, namb, na = check_step(L, n_hot, x, run_step(dl, buf, x, fused=True))
        log(f"  two words per thread, step {step}: active {na}, ambiguous {namb}, err {e:.2e}")


def test_wide_mask_compacted_before_fused_kernel():
    """n above the fused kernel's in-prologue mask bound (1024 words): the mask is
    compacted by its own kernel and the fused kernel reads the lists."""
    wl = S.WORKLOADS["opt30b-fp16"].scaled(d=256, n=66001, r=32)
    L = S.make_layer(wl)
    n_hot = 17160
    dl = DeviceLayer.upload(L, DEV, n_hot=n_hot)
    buf = StepBuffers(dl, 1, DEV)
    for step in range(2):
        x = S.make_x(wl, 0, step, 1)
        e, namb, na = check_step(L, n_hot, x, run_step(dl, buf, x, fused=(step == 0)))
        log(f"  wide mask step {step}: active {na}, ambiguous {namb}, err {e:.2e}")


def test_cold_partition_in_host_memory():
    """Cold partition's weight rows in pinned host memory, read by the same kernels
    over the host link: bit-identical to the all-device layer, and oracle parity."""
    wl = SMALL["opt30b-fp16"]
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    Lh, n_hot = index_layer(L, dl, 256)
    buf = StepBuffers(dl, 1, DEV)
    xs = [S.make_x(wl, 0, step, 1) for step in range(3)]
    ref = [run_step(dl, buf, x) for x in xs]
    dl.place_cold_on_host()
    hot, cold = dl.parts()
    assert cold is not None and not dl.cold_host["W_up"].is_cuda
    for step, x in enumerate(xs):
        out = run_step(dl, buf, x, fused=(step != 1))
        for k in ("y", "y_hot", "y_cold", "hot", "cold"):
            assert np.array_equal(out[k], ref[step][k]), k
        e, namb, na = check_step(Lh, n_hot, x, out)
        log(f"  cold on host, step {step}: active {na}, err {e:.2e}")


def test_online_counts_and_reindex():
    """Predicted activations counted on the device during decode (exact integer
    sums of the masks), then a new neuron index from them applied to the indexed
    layer: index equal to the oracle's for the same counts, and step parity after."""
    wl = SMALL["opt30b-fp16"]
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    Lh, n_hot = index_layer(L, dl, 256)
    buf = StepBuffers(dl, 1, DEV)
    counts = torch.zeros(wl.n, dtype=torch.int32, device=DEV)
    want = np.zeros(wl.n, dtype=np.int64)
    for step in range(6):
        x = S.make_x(wl, 0, 100 + step, 1)
        out = run_step(dl, buf, x, fused=(step % 2 == 0))
        check_step(Lh, n_hot, x, out)
        dl.accumulate(buf.mask, counts)
        want += mask_bits(out["mask"], wl.n)[0]
    torch.cuda.synchronize()
    got = _np(counts).astype(np.uint32)
    assert np.array_equal(got.astype(np.int64), want)
    bpn, budget = S.bytes_per_neuron(wl), S.budget_bytes(wl)
    perm, n_hot2 = dl.reindex(counts, budget, bpn)
    torch.cuda.synchronize()
    perm_o, n_hot_o = O.build_neuron_index(got, budget, bpn)
    assert n_hot2 == n_hot_o and np.array_equal(_np(perm), perm_o)
    assert np.array_equal(_np(counts).astype(np.uint32), got[perm_o])
    Lh2 = permute_layer(Lh, perm_o)
    buf2 = StepBuffers(dl, 1, DEV)
    for step in range(2):
        x = S.make_x(wl, 0, 200 + step, 1)
        e, namb, na = check_step(Lh2, n_hot2, x, run_step(dl, buf2, x))
        log(f"  after online reindex, step {step}: active {na}, err {e:.2e}")


def test_deterministic_reruns(small_f16):
    wl, L = small_f16
    dl = DeviceLayer.upload(L, DEV, n_hot=200)
    buf = StepBuffers(dl, 1, DEV)
    x = S.make_x(wl, 0, 5, 1)
    a = run_step(dl, buf, x)
    b = run_step(dl, buf, x)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["hot"], b["hot"])


def test_single_partition_and_dense_and_merge(small_f16):
    wl, L = small_f16
    dl = DeviceLayer.upload(L, DEV)
    part = dl.part()
    buf = StepBuffers(dl, 2, DEV)
    x_np = S.make_x(wl, 0, 3, 2)
    x = torch.from_numpy(x_np).to(DEV)
    pb.pi_predict(dl.predictor(), x, buf.mask, None, None, buf.ws)
    lists = pb.make_lists(wl.n, buf.hot_idx, None, buf.counts)
    pb.pi_compact_active(buf.mask, wl.n, lists)
    y = torch.empty((2, wl.d), dtype=torch.float32, device=DEV)
    pb.pi_sparse_ffn(part, x, buf.hot_idx, buf.counts, y, buf.ws)
    yd = torch.empty_like(y)
    pb.pi_dense_ffn(part, x, yd, buf.ws)
    torch.cuda.synchronize()
    mask = _np(buf.mask).view(np.uint64)
    hot_o, _ = O.compact(mask, wl.n, wl.n)
    assert np.array_equal(_np(buf.hot_idx)[:_np(buf.counts)[0]], hot_o)
    check_close(_np(y), O.sparse_ffn(O.Part.from_layer(L), x_np, hot_o), "f16")
    check_close(_np(yd), O.dense_ffn(O.Part.from_layer(L), x_np), "f16")
    # merge: fp32 a + b, correctly rounded, so bit-exact against the fp64 sum rounded once
    a = torch.randn(3, 333, device=DEV)
    b = torch.randn(3, 333, device=DEV)
    out = torch.empty_like(a)
    pb.pi_merge(a, b, out)
    pb.pi_merge(a, None, a.clone())
    torch.cuda.synchronize()
    ref = O.merge(_np(a).astype(np.float64), _np(b).astype(np.float64)).astype(np.float32)
    assert np.array_equal(_np(out), ref)


def test_compact_ignores_tail_bits():
    n = 130
    words = np.array([0xF0F0F0F0F0F0F0F0, 0x1, 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
    mask = torch.from_numpy(words.view(np.int64)).to(DEV)
    hot = torch.zeros(100, dtype=torch.int32, device=DEV)
    cold = torch.zeros(30, dtype=torch.int32, device=DEV)
    counts = torch.zeros(2, dtype=torch.int32, device=DEV)
    pb.pi_compact_active(mask, n, pb.make_lists(100, hot, cold, counts))
    torch.cuda.synchronize()
    ids = [i for i in range(n) if (int(words[i // 64]) >> (i % 64)) & 1]
    c = _np(counts)
    assert _np(hot)[:c[0]].tolist() == [i for i in ids if i < 100]
    assert _np(cold)[:c[1]].tolist() == [i - 100 for i in ids if i >= 100]


# --------------------------------------------------------------------------------
# full sizes
# --------------------------------------------------------------------------------

def test_opt30b_full_with_index():
    """OPT-30B-shaped layer (d 7168, n 28672, rank 1024, fp16), 26% hot partition from
    1024 profiling samples, split + merge, all 64 decode steps of the workload."""
    wl = S.WORKLOADS["opt30b-fp16"]
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    rows = np.random.default_rng(0).choice(wl.n, 256, replace=False)
    Lh, n_hot = index_layer(L, dl, wl.profile_samples, rows_checked=rows)
    assert n_hot == 7454
    buf = StepBuffers(dl, 1, DEV)
    for step in range(wl.steps):
        x = S.make_x(wl, 0, step, 1)
        e, namb, na = check_step(Lh, n_hot, x, run_step(dl, buf, x))
        if step % 8 == 0 or step == wl.steps - 1:
            log(f"  opt30b step {step}: active {na} (hot {int(buf.counts[0])}), ambiguous {namb}, "
                f"err {e:.2e}")


@pytest.mark.parametrize("B,steps", [(1, 64), (4, 24)])
def test_reglu70b_full(B, steps):
    """LLaMA(ReGLU)-70B-shaped layer (d 8192, n 28672, fp16) at batch 1 (the fused
    kernel) and 4 (the matrix-core path): the first `steps` decode steps."""
    wl = S.WORKLOADS["llama70b-reglu-fp16"]
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    buf = StepBuffers(dl, B, DEV)
    for step in range(steps):
        x = S.make_x(wl, 0, step, B)
        e, namb, na = check_step(L, wl.n, x, run_step(dl, buf, x))
        if step % 8 == 0 or step == steps - 1:
            log(f"  reglu70b B={B} step {step}: union active {na}, ambiguous {namb}, err {e:.2e}")


@pytest.mark.parametrize("layer", [0, 29, 59])
def test_falcon40b_layer_full(layer):
    """Layers 0, 29 and 59 of the Falcon-40B-shaped stack (host-drawn from their
    seeds): 20% hot partition from 1024 profiling samples, 16 decode steps spread over
    the 128 (fresh x per step and layer)."""
    wl = S.WORKLOADS["falcon40b-stack-fp16"]
    L = S.make_layer(wl, layer=layer)
    dl = DeviceLayer.upload(L, DEV)
    rows = np.random.default_rng(1 + layer).choice(wl.n, 64, replace=False)
    Lh, n_hot = index_layer(L, dl, wl.profile_samples, rows_checked=rows)
    assert n_hot == 6553
    buf = StepBuffers(dl, 1, DEV)
    worst = 0.0
    for step in range(0, 128, 8):
        x = S.make_x(wl, layer, step, 1)
        e, namb, na = check_step(Lh, n_hot, x, run_step(dl, buf, x, fused=(step % 16 == 0)))
        worst = max(worst, e)
    log(f"  falcon layer {layer}: 16 steps, last active {na}, worst err {worst:.2e}")


def test_falcon40b_device_drawn_layer():
    """A layer drawn on the GPU the way the stack benchmark draws its 60 layers
    (workload.synth.make_layer_device, device-drawn profiling samples and inputs),
    copied to the host and checked step by step against the oracle: the values the
    benchmark times."""
    wl = S.WORKLOADS["falcon40b-stack-fp16"]
    li = 29
    t = S.make_layer_device(wl, li, DEV)
    host = {k: (None if v is None or isinstance(v, float) else _np(v)) for k, v in t.items()}
    L = S.Layer(wl, li, None, host["W_up"], host["W_gate"], host["W_downT"], host["b_up"],
                host["b_gate"], host["P1t"], host["P2t"], host["b2"], 0.0)
    dl = DeviceLayer.from_tensors(wl, t)
    g = torch.Generator(device=DEV)
    g.manual_seed(S.SEED + 7 * li + 1)
    X = torch.randn(wl.profile_samples, wl.d, generator=g, device=DEV).to(torch.float16)
    rows = np.random.default_rng(7).choice(wl.n, 64, replace=False)
    Lh, n_hot = index_layer(L, dl, wl.profile_samples, rows_checked=rows, X=X)
    assert n_hot == 6553
    del X
    buf = StepBuffers(dl, 1, DEV)
    gx = torch.Generator(device=DEV)
    gx.manual_seed(S.SEED + 99)
    xs = torch.randn(16, 1, wl.d, generator=gx, device=DEV).to(torch.float16)
    worst = 0.0
    for step in range(16):
        x = _np(xs[step])
        e, namb, na = check_step(Lh, n_hot, x, run_step(dl, buf, x, fused=(step % 2 == 0)))
        worst = max(worst, e)
    log(f"  device-drawn falcon layer {li}: 16 steps, last active {na}, worst err {worst:.2e}")


@pytest.mark.parametrize("B,steps", [(1, 64), (8, 16), (64, 6)])
def test_opt175b_q4_full(B, steps):
    """OPT-175B-shaped Q4_0 layer, the first `steps` decode steps: the union mask of
    all B tokens against the oracle's predictor (ambiguity band), the list bit-exact,
    the FFN on up to four tokens over the GPU's union list."""
    wl = S.WORKLOADS["opt175b-q4_0"]
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    buf = StepBuffers(dl, B, DEV)
    tokens = None if B == 1 else sorted({0, B // 3, (2 * B) // 3, B - 1})
    for step in range(steps):
        x = S.make_x(wl, 0, step, B)
        out = run_step(dl, buf, x)
        e, namb, na = check_step(L, wl.n, x, out, tokens=tokens)
        if step % 8 == 0 or step == steps - 1:
            log(f"  q4_0 B={B} step {step}: union active {na}, ambiguous {namb}, err {e:.2e}")


def test_bandwidth_aware_split_with_cold_rows_in_host_memory():
    """The hot/cold split chosen from the measured read rates of HBM and of pinned host
    memory (pi_plan_hot_split) equals the oracle's rule on the same counts and rates; the
    layer then runs with its cold rows in host memory, checked against the oracle."""
    wl = SMALL["opt30b-fp16"]
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    X = torch.from_numpy(S.make_profile_x(wl, 0, 256)).to(DEV)
    counts = dl.profile_counts(X)
    perm, _ = dl.build_index(counts, S.budget_bytes(wl), S.bytes_per_neuron(wl))
    torch.cuda.synchronize()
    perm_np = _np(perm)
    counts_slot = _np(counts).astype(np.uint32)[perm_np]
    sink = torch.zeros(pb.PI_STREAM_SINK_WORDS, dtype=torch.int32, device=DEV)
    rates = []
    for host in (False, True):
        nb = 64 << 20
        buf = torch.empty(nb, dtype=torch.uint8, pin_memory=True) if host else \
            torch.empty(nb, dtype=torch.uint8, device=DEV)
        pb.pi_stream_read(buf, nb, sink)
        torch.cuda.synchronize()
        pb.pi_kernel_timer_start(pb.PI_K_STREAM, 2)
        pb.pi_stream_read(buf, nb, sink)
        pb.pi_stream_read(buf, nb, sink)
        ms, k = pb.pi_kernel_timer_stop(pb.PI_K_STREAM)
        rates.append(nb / (ms / k * 1e-3) / 1e9)
    bpn = S.bytes_per_neuron(wl)
    budget = wl.n * bpn
    n_hot = pb.pi_plan_hot_split(counts_slot, budget, bpn, rates[0], rates[1])
    assert n_hot == O.plan_hot_split(counts_slot, budget, bpn, rates[0], rates[1])
    log(f"  rates hbm {rates[0]:.0f} GB/s, host {rates[1]:.0f} GB/s -> n_hot {n_hot} of {wl.n}")
    dl.apply_index(perm, n_hot)
    dl.place_cold_on_host()
    Lh = permute_layer(L, perm_np)
    buf = StepBuffers(dl, 1, DEV)
    for step in range(3):
        x = S.make_x(wl, 0, 40 + step, 1)
        e, namb, na = check_step(Lh, n_hot, x, run_step(dl, buf, x, fused=(step != 1)))
        log(f"  split from rates, step {step}: active {na}, err {e:.2e}")


def _crossover_step(dl, buf, x_np, dense_from, fused_mask=True):
    x = torch.from_numpy(x_np).to(DEV)
    hot, cold = dl.parts()
    buf.hot_idx.fill_(-7)
    buf.cold_idx.fill_(-7)
    pb.pi_predict(dl.predictor(), x, buf.mask, None, None if fused_mask else buf.lists, buf.ws)
    yc = buf.y_cold if cold is not None else None
    pb.pi_sparse_ffn_crossover(hot, cold, x, buf.lists, dense_from, buf.y_hot, yc, buf.y, buf.ws,
                               mask=buf.mask if fused_mask else None)
    torch.cuda.synchronize()
    c = _np(buf.counts)
    return dict(mask=_np(buf.mask).view(np.uint64).copy(), counts=c.copy(),
                hot=_np(buf.hot_idx)[:c[0]].copy(), cold=_np(buf.cold_idx)[:c[1]].copy(),
                y=_np(buf.y).copy(), y_hot=_np(buf.y_hot).copy(),
                y_cold=_np(buf.y_cold).copy() if cold is not None else None)


@pytest.mark.parametrize("name,B,n_hot", [("reglu-f16", 4, 500), ("q4_0", 20, None),
                                          ("relu-f16-split", 64, 600), ("q4_0", 2, 400)])
def test_prompt_phase_crossover(name, B, n_hot):
    """pi_sparse_ffn_crossover: below the crossover it is the sparse split (bit for bit);
    from the crossover on, every row of both partitions is computed: the dense FFN of
    the oracle, with the lists and counts still naming the predicted set."""
    wl = MFMA_SMALL[name]
    L = S.make_layer(wl)
    n_hot = wl.n if n_hot is None else n_hot
    dl = DeviceLayer.upload(L, DEV, n_hot=n_hot)
    buf = StepBuffers(dl, B, DEV)
    x = S.make_x(wl, 0, 1, B)
    ref = run_step(dl, buf, x, logits=False)
    T = int(ref["counts"].sum())
    for fused_mask in (True, False):
        sparse = _crossover_step(dl, buf, x, T + 1, fused_mask)
        for k in ("counts", "hot", "cold", "y", "y_hot", "y_cold"):
            if ref.get(k) is not None:
                assert np.array_equal(sparse[k], ref[k]), f"sparse side: {k}"
        dense = _crossover_step(dl, buf, x, T, fused_mask)
        for k in ("counts", "hot", "cold"):
            assert np.array_equal(dense[k], ref[k]), f"dense side lists: {k}"
        yd = O.dense_ffn(O.Part.from_layer(L), x)
        check_close(dense["y"], yd, wl.wdtype)
        if n_hot < wl.n:
            yh = O.dense_ffn(O.Part.from_layer(L, 0, n_hot), x)
            check_close(dense["y_hot"], yh, wl.wdtype, scale=yd)
    log(f"  crossover {name} B={B}: {T} active of {wl.n}; dense from {T} matches the dense oracle")


@pytest.mark.parametrize("wname,B", [("llama70b-reglu-fp16", 4), ("opt175b-q4_0", 64)])
def test_dense_path_full_size(wname, B):
    """The dense side of the crossover at full size (LLaMA(ReGLU)-70B-shaped layer at
    batch 4, OPT-175B-shaped Q4_0 layer at batch 64) against the oracle's dense FFN on
    sampled tokens."""
    wl = S.WORKLOADS[wname]
    L = S.make_layer(wl)
    dl = DeviceLayer.upload(L, DEV)
    buf = StepBuffers(dl, B, DEV)
    x = S.make_x(wl, 0, 3, B)
    out = _crossover_step(dl, buf, x, 1)
    tokens = sorted({0, B - 1} | ({B // 2} if B > 2 else set()))
    yd = O.dense_ffn(O.Part.from_layer(L), x[tokens])
    e = check_close(out["y"][tokens], yd, wl.wdtype)
    log(f"  dense {wname} B={B}: tokens {tokens} err {e:.2e}")
