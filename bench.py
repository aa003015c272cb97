"""Benchmark of the predictor-gated sparse FFN decode step on one MI355X.

One step = one pass of the whole hot path over one token batch: predictor
(both layers, threshold, union -> mask; `pi_predict`), then
`pi_sparse_ffn_split` with the mask: compaction into hot/cold lists fused into
the fused FFN kernel (up/gate, activation and down over the hot and the cold
partition, one partial of y per workgroup), and the merge fused into the
reduction of those partials.  Four kernels at batch 1; six on the
matrix-core path at batch 2..64 (two predictor kernels and the slice sum, the
up and down kernels, the reduction), seven where the Q4_0 up kernel is split
over K; no host synchronisation.

Default workload: the OPT-30B-shaped ReLU layer (d_model 7168, d_ffn 28672,
predictor rank 1024, fp16 weights, fp32 accumulation, batch 1), hot partition
= top 26% of neurons by activation count over 1024 profiling samples (profiled,
indexed and permuted on the GPU before timing).  Steps rotate over INSTANCES
device copies of the layer (same values, distinct addresses) with a fresh
seeded x per step, so the 256 MB Infinity Cache cannot serve the weights.

Reported on one JSON line: mean microseconds per layer step (`value`, from a
replay of the timed steps captured in one HIP graph) and its p10/p50/p90 over
the steps (HIP events between eagerly launched steps), the
achieved GB/s on the bytes the step must touch, per-kernel durations from HIP
events recorded at each kernel's own dispatch, the roofline of the dominant
kernel against the 8 TB/s HBM peak and against the attainable read rate of a
plain read stream of the same size (`pi_stream_read`), the dense FFN of the
same layer, the literal bias-free predictor as a secondary row, the
Falcon-40B-shaped 60-layer stack (tokens/s of the FFN stack, default run
only), and the CPU oracle timed on all host cores and on one (the one-core leg
is skipped where a single step would take over a minute).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("sparse-FFN µs/layer + achieved HBM GB/s on touched weights vs peak, batch 1")
PEAK_HBM_GBPS = 8000.0
TARGET_FRAC = 0.70                 # the sustained fraction of peak the step aims for
INSTANCES = 8
COPY_CAL_BYTES = 512 << 20         # reads 512 MiB, writes 512 MiB
STREAM_BUF_BYTES = 1 << 30         # read-stream ceiling: offsets rotate through 1 GiB


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def esize(dt):
    return {"f32": 4, "f16": 2}[dt]


def wrow_bytes(wl):
    return wl.d // 2 + wl.d // 16 if wl.wdtype == "q4_0" else wl.d * esize(wl.wdtype)


def kernel_bytes(wl, B, active):
    """Algorithmic bytes per launch of each kernel for one step with `active` neurons:
    the weights and inputs the step must read and the results it must write."""
    ep = esize(wl.pdtype)
    ex = esize(wl.xdtype)
    m_up = 2 if wl.act == "reglu" else 1
    words = (wl.n + 63) // 64
    return {
        "k_pred_l1": wl.r * wl.d * ep + B * wl.d * ex + B * wl.r * 4,
        "k_pred_l2": wl.n * wl.r * ep + 4 * wl.n + B * wl.r * 4 + 8 * words,
        "k_compact": 8 * words + 4 * active + 8,
        "k_up": active * (m_up * wrow_bytes(wl) + 4 + 4) + B * wl.d * ex + 4 * B * active,
        "k_down": active * (wrow_bytes(wl) + 4) + 4 * B * active,
        "k_ffn": active * (m_up * wrow_bytes(wl) + wrow_bytes(wl) + 4) + B * wl.d * ex,
        "k_reduce": 4 * B * wl.d,
        "k_up_finish": 0,        # sum of the up kernel's K slices: implementation traffic only
    }


def step_bytes(wl, B, active):
    """Bytes one layer step must touch: predictor weights + b2, the active rows of the FFN
    (W_up / W_gate / W_downT rows and the fp32 bias), x in, y out."""
    m = 3 if wl.act == "reglu" else 2
    pred = (wl.d * wl.r + wl.r * wl.n) * esize(wl.pdtype) + 4 * wl.n
    return pred + active * (m * wrow_bytes(wl) + 4) + B * wl.d * esize(wl.xdtype) + 4 * B * wl.d


KERNEL_SOURCES = ("pi_device.h", "pi_kernels.h", "pi_ffn.h", "pi_mfma.h", "pi_api.hip")


def counter_traffic(wl_name, kernel, B=1):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter record
    (profiles/<workload>_traffic.json at batch 1, <workload>_b<B>_traffic.json
    otherwise: FETCH_SIZE and WRITE_SIZE passes scaled by a plain copy of known
    size), or None when there is no record or the kernel sources changed since the
    counters were taken."""
    import hashlib
    name = f"{wl_name}_traffic.json" if B == 1 else f"{wl_name}_b{B}_traffic.json"
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in rec.get("sources", KERNEL_SOURCES):   # the files the measured kernels come from
        h.update(open(os.path.join(ROOT, "sparse_activation_ffn_amd", "csrc", f), "rb").read())
    k = rec.get("kernels", {}).get(kernel)
    if rec.get("source_sha256") != h.hexdigest() or k is None:
        return None
    return k["read_bytes"] + k["write_bytes"]


def host_cpu():
    """(model name, logical CPUs, threads the oracle may use on this host)."""
    model = platform.processor() or "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    nproc = os.cpu_count() or 1
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = nproc
    env = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(avail, int(env)) if env.isdigit() and int(env) > 0 else avail
    return model, nproc, max(1, threads)


def hybrid_cpu_cold(pb, torch, wl, L, perm_np, layers, buf, xs, idxs, dev, threads):
    """The pages' hybrid step (CSDN article, CPU/GPU hybrid-design section and figure):
    the hot partition's rows in HBM computed by the GPU, the cold partition's rows in
    host memory computed by the host cores (pi_sparse_ffn_hybrid), predictor first.
    Eager steps (the call blocks the host), host clock around synchronised runs; one
    host copy of the cold rows per layer instance, so no step finds the previous
    instance's rows in the CPU caches."""
    n_hot = layers[0].n_hot
    rows = perm_np[n_hot:]
    take = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a[rows]))  # noqa: E731
    first = {k: take(getattr(L, k)) for k in ("W_up", "W_gate", "W_downT", "b_up", "b_gate")}
    copies = [first] + [{k: None if v is None else v.clone() for k, v in first.items()}
                        for _ in range(len(layers) - 1)]
    act = layers[0].act
    colds = [pb.make_part(wl.d, c["W_up"], c["W_downT"], act, c["W_gate"], c["b_up"], c["b_gate"],
                          q4=wl.wdtype == "q4_0") for c in copies]
    hots = [ly.parts()[0] for ly in layers]
    preds = [ly.predictor() for ly in layers]
    B = xs[0].shape[0]
    y_cold = torch.zeros((B, wl.d), dtype=torch.float32, device=dev)
    host_ws = torch.zeros(pb.pi_hybrid_host_bytes(wl.d, wl.n, B), dtype=torch.uint8,
                          pin_memory=True)

    def run(k, nthreads):
        infos = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for j, i in enumerate(idxs[:k]):
            li = i % len(layers)
            pb.pi_predict(preds[li], xs[i], buf.mask, None, None, buf.ws)
            infos.append(pb.pi_sparse_ffn_hybrid(hots[li], colds[li], xs[i], buf.mask, buf.lists,
                                                 y_cold, buf.y, buf.ws, host_ws, nthreads))
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / k, infos

    def hot_only(k):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in idxs[:k]:
            li = i % len(layers)
            pb.pi_predict(preds[li], xs[i], buf.mask, None, None, buf.ws)
            pb.pi_sparse_ffn_split(hots[li], None, xs[i], buf.lists, None, None, buf.y, buf.ws,
                                   mask=buf.mask)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / k

    # each timed run starts with the host caches holding none of the rows: a 512 MiB
    # pass evicts them (the runs repeat the same steps)
    flush = np.ones(64 << 20, np.float64)

    def evict():
        return float(flush.sum())

    K = len(idxs)
    run(K, threads)                              # warm the pool, the code, the page tables
    evict()
    us, infos = run(K, threads)
    sweep = {}
    for t in sorted({1, 4, 8, threads}):
        if t <= threads:
            evict()
            u, inf = run(K, t)
            sweep[str(t)] = {"us_per_step": round(u, 1),
                             "host_us": round(float(np.mean([q.host_us for q in inf])), 1)}
    del flush
    hot_us = hot_only(K)
    cold = np.array([q.cold_count for q in infos], np.float64)
    cold_bytes = float(cold.mean()) * ((3 if wl.act == "reglu" else 2) * wrow_bytes(wl) + 4)
    host_us = float(np.mean([q.host_us for q in infos]))
    return {"n_hot": n_hot, "threads": threads, "us_per_step": round(us, 1),
            "mean_cold_active": round(float(cold.mean()), 1),
            "host_us": round(host_us, 1),
            "host_us_p50": round(float(np.median([q.host_us for q in infos])), 1),
            "host_wait_us": round(float(np.mean([q.wait_us for q in infos])), 1),
            "host_gbps_cold_rows": round(cold_bytes / (host_us * 1e-6) / 1e9, 1),
            "gpu_hot_only_us_eager": round(hot_us, 1),
            "threads_sweep": sweep,
            "hbm_bytes_saved": int((wl.n - n_hot) * ((3 if wl.act == "reglu" else 2)
                                                     * wrow_bytes(wl) + 4)),
            "timing": "eager, host clock; predictor + hybrid call per step"}


def cpu_baseline(wl, L, n_hot, B, budget_s=8.0):
    """The oracle's layer step (predict, compact, sparse FFN per partition, merge) on the
    host: once single-threaded and once with its outer loops on all the cores this process
    may use.  Each leg runs for about budget_s seconds."""
    from oracle import oracle as O
    from workload import synth as S
    hot = O.Part.from_layer(L, 0, n_hot)
    cold = O.Part.from_layer(L, n_hot, wl.n) if n_hot < wl.n else None
    model, nproc, threads = host_cpu()

    def leg(k):
        O.set_threads(k)
        t0 = time.perf_counter()
        steps = 0
        while True:
            x = S.make_x(wl, 0, 10_000 + steps, B)
            O.layer_step(L.P1t, L.P2t, L.b2, L.threshold, hot, cold, x)
            steps += 1
            el = time.perf_counter() - t0
            if el >= budget_s or steps >= 400:
                break
        return el / steps * 1e6, steps

    try:
        log(f"[bench] oracle on {threads} threads ...")
        all_us, all_n = leg(threads)
        # one single-threaded step costs about threads times the threaded one: skipped
        # where that alone would exceed a minute (the large batches)
        one_us = one_n = None
        if all_us * threads * 1e-6 <= 60.0:
            log("[bench] oracle on 1 thread ...")
            one_us, one_n = leg(1)
    finally:
        O.set_threads(1)
    one = (f"single-threaded: {one_n} steps" if one_n is not None
           else "single-threaded leg skipped (one step would take over a minute)")
    return {"value": round(all_us, 1), "unit": "us/layer", "cores": threads, "kind": "oracle",
            "sample": f"{all_n} layer steps of the same {wl.name} layer (batch {B}), C oracle "
                      f"(fp64 accumulation) with its outer loops on {threads} threads; {one}",
            "single_thread_us": None if one_us is None else round(one_us, 1), "nproc": nproc,
            "cpu_model": model}


def time_stream(pb, torch, nbytes, dev, launches=16, host=False):
    """Attainable read rate of a plain stream of nbytes (per launch, HIP events at the
    kernel's own dispatch), offsets rotating through a 1 GiB buffer so no launch reads
    what the previous ones left in the caches.  host: the buffer is pinned host memory
    (read by the GPU over the host link), one buffer of 2 * nbytes."""
    nbytes = max(16, nbytes // 16 * 16)
    if host:
        total = 2 * nbytes
        buf = torch.empty(total, dtype=torch.uint8, pin_memory=True)
    else:
        total = max(STREAM_BUF_BYTES, 8 * nbytes)
        buf = torch.empty(total, dtype=torch.uint8, device=dev)
    sink = torch.empty(pb.PI_STREAM_SINK_WORDS, dtype=torch.int32, device=dev)
    slots = max(1, total // nbytes)
    for i in range(2):
        pb.pi_stream_read(buf[(i % slots) * nbytes:], nbytes, sink)
    torch.cuda.synchronize()
    pb.pi_kernel_timer_start(pb.PI_K_STREAM, launches)
    for i in range(launches):
        pb.pi_stream_read(buf[(i % slots) * nbytes:], nbytes, sink)
    ms, k = pb.pi_kernel_timer_stop(pb.PI_K_STREAM)
    del buf
    return nbytes / (ms / k * 1e-3) / 1e9


def per_step_us(torch, step, idxs):
    """Device time of each step: HIP events recorded on the stream between steps
    launched eagerly (the host enqueues a step faster than the GPU runs one, so the
    stream never idles between them)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(idxs) + 1)]
    ev[0].record()
    for i, e in zip(idxs, ev[1:]):
        step(i)
        e.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) * 1e3 for a, b in zip(ev[:-1], ev[1:])])


def adaptive_predictor(pb, torch, S, wl, layer, buf, xs, idxs, dev, target=0.99):
    """Recall-calibrated threshold on the workload's profiling samples (computed on the
    GPU by pi_calibrate_threshold), then, on held-out decode inputs, the predicted set
    against the true firing set (pi_true_mask) at that threshold and at the default one.
    layer: the whole layer in device memory (predictor and rows in the same order)."""
    X = torch.from_numpy(S.make_profile_x(wl, 0)).to(dev)
    nS = X.shape[0]
    ws = torch.empty(pb.pi_calibrate_workspace_bytes(wl.d, wl.n, wl.r, nS), dtype=torch.uint8,
                     device=dev)
    tau = torch.empty(1, dtype=torch.float32, device=dev)
    stats = torch.empty(3, dtype=torch.int32, device=dev)
    part = layer.part()
    pb.pi_calibrate_threshold(layer.predictor(), part, X, target, tau, stats, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    pb.pi_calibrate_threshold(layer.predictor(), part, X, target, tau, stats, ws)
    e1.record()
    torch.cuda.synchronize()
    cal_ms = e0.elapsed_time(e1)
    t = float(tau.item())
    N, m, hits = (int(v) for v in stats.cpu().numpy())
    del ws, X
    n = wl.n
    tm = torch.empty((n + 63) // 64, dtype=torch.int64, device=dev)

    def bits(words):
        return np.unpackbits(words.cpu().numpy().view(np.uint8), bitorder="little")[:n].astype(bool)

    preds = {"default_threshold": layer.predictor(),
             "adaptive": pb.make_predictor(layer.P1t, layer.P2t, layer.b2, t)}
    hot, cold = layer.parts()
    rows = {}
    for name, pred in preds.items():
        tp = npred = ntrue = 0
        for i in idxs:
            pb.pi_predict(pred, xs[i], buf.mask, None, None, buf.ws)
            pb.pi_true_mask(part, xs[i], tm)
            pm, tt = bits(buf.mask), bits(tm)
            tp += int((pm & tt).sum())
            npred += int(pm.sum())
            ntrue += int(tt.sum())

        def step(i, pred=pred):
            pb.pi_predict(pred, xs[i], buf.mask, None, None, buf.ws)
            pb.pi_sparse_ffn_split(hot, cold, xs[i], buf.lists, None, None, buf.y, buf.ws,
                                   mask=buf.mask)
        per = per_step_us(torch, step, idxs)
        rows[name] = {"threshold": preds[name].threshold,
                      "recall": round(tp / max(ntrue, 1), 5),
                      "precision": round(tp / max(npred, 1), 5),
                      "density": round(npred / (len(idxs) * n), 5),
                      "us_per_step_p50": round(float(np.median(per)), 3)}
    return {"target_recall": target, "samples": nS, "tau": t, "firing_pairs": N, "m": m,
            "calibration_recall": round(hits / max(N, 1), 6),
            "calibration_ms": round(cal_ms, 3), "decode_steps": len(idxs),
            "true_density": round(ntrue / (len(idxs) * n), 5), **rows,
            "note": "held-out decode inputs; the random-init predictor is independent of the "
                    "layer's firing beyond the per-neuron rates, so the density needed for a "
                    "recall target is far above a trained predictor's"}


def prompt_crossover(pb, torch, S, StepBuffers, wl, layer, dev, batches=(8, 16, 32, 64), steps=8):
    """The prompt-phase crossover on the indexed layer: per batch, the sparse split and
    the dense FFN taken through pi_sparse_ffn_crossover (dense_from = n + 1 and 1), the
    predictor alone, and the crossover count that the measured times give (the active
    count at which the sparse FFN's per-row cost reaches the dense FFN's time); then
    the same steps with that count, the device choosing per step."""
    hot, cold = layer.parts()
    pred = layer.predictor()
    rows = []
    for B in batches:
        buf = StepBuffers(layer, B, dev)
        xs = [torch.from_numpy(S.make_x(wl, 0, 100000 + s, B)).to(dev) for s in range(steps)]

        def predict(i):
            pb.pi_predict(pred, xs[i], buf.mask, None, None, buf.ws)

        def step(i, dense_from):
            predict(i)
            pb.pi_sparse_ffn_crossover(hot, cold, xs[i], buf.lists, dense_from, None, None, buf.y,
                                       buf.ws, mask=buf.mask)

        def timed(fn):
            fn(0)
            torch.cuda.synchronize()
            return float(np.median(per_step_us(torch, fn, list(range(steps)))))
        active = []
        for i in range(steps):
            step(i, wl.n + 1)
            active.append(int(buf.counts.sum().item()))
        t_pred = timed(predict)
        t_sparse = timed(lambda i: step(i, wl.n + 1))
        t_dense = timed(lambda i: step(i, 1))
        a = float(np.mean(active))
        per_row = max(t_sparse - t_pred, 1e-3) / max(a, 1.0)
        dense_from = max(1, min(wl.n + 1, int(np.ceil((t_dense - t_pred) / per_row))))
        t_chosen = timed(lambda i: step(i, dense_from))
        rows.append({"batch": B, "mean_active": round(a, 1), "density": round(a / wl.n, 4),
                     "predict_us": round(t_pred, 2), "sparse_us": round(t_sparse, 2),
                     "dense_us": round(t_dense, 2), "dense_from": dense_from,
                     "dense_steps": int(sum(c >= dense_from for c in active)),
                     "chosen_us": round(t_chosen, 2)})
        del buf, xs
    return {"workload": wl.name, "steps_per_batch": steps, "rows": rows,
            "note": "median step time from HIP events between eagerly launched steps; dense_from "
                    "= the active count where predict + per-row sparse cost reaches the dense "
                    "step, applied on the device per step"}


def draw_stack(wl, dev):
    """The Falcon-40B-shaped stack: 60 distinct layers drawn on the GPU
    (workload.synth.make_layer_device), each profiled on 1024 samples, indexed under its
    20% budget and permuted, all on the GPU."""
    import torch
    from sparse_activation_ffn_amd.layer import DeviceLayer
    from workload import synth as S
    layers = []
    for li in range(wl.layers):
        ly = DeviceLayer.from_tensors(wl, S.make_layer_device(wl, li, dev))
        g = torch.Generator(device=dev)
        g.manual_seed(S.SEED + 7 * li + 1)
        X = torch.randn(wl.profile_samples, wl.d, generator=g, device=dev).to(torch.float16)
        counts = ly.profile_counts(X)
        perm, n_hot = ly.build_index(counts, S.budget_bytes(wl), S.bytes_per_neuron(wl))
        ly.apply_index(perm, n_hot)
        layers.append(ly)
        del X
    torch.cuda.synchronize()
    return layers


def run_stack(wl, B, K, W, dev):
    """Decode steps over the whole stack (fresh x per step and layer).  Returns the
    summary dict: µs per layer step, tokens/s of the FFN stack, touched-byte rate, and
    per-kernel durations over the first timed step."""
    import torch
    from sparse_activation_ffn_amd import binding as pb
    from sparse_activation_ffn_amd.layer import StepBuffers
    NL = wl.layers
    t0 = time.perf_counter()
    layers = draw_stack(wl, dev)
    setup_s = time.perf_counter() - t0
    descs = [(ly.predictor(), ly.parts()) for ly in layers]
    buf = StepBuffers(layers[0], B, dev)
    gx = torch.Generator(device=dev)
    gx.manual_seed(20231216 + 99)
    xs = torch.randn(W + K, NL, B, wl.d, generator=gx, device=dev).to(torch.float16)

    def layer_step(s, li):
        pred, (hot, cold) = descs[li]
        x = xs[s, li]
        pb.pi_predict(pred, x, buf.mask, None, None, buf.ws)
        pb.pi_sparse_ffn_split(hot, cold, x, buf.lists, None, None, buf.y, buf.ws, mask=buf.mask)

    for s in range(W):
        for li in range(NL):
            layer_step(s, li)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(W, W + K):
            for li in range(NL):
                layer_step(s, li)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us_layer = e0.elapsed_time(e1) * 1e3 / (K * NL)
    kids = {"k_pred_l1": pb.PI_K_PRED_L1, "k_pred_l2": pb.PI_K_PRED_L2, "k_ffn": pb.PI_K_FFN,
            "k_reduce": pb.PI_K_REDUCE}
    for kid in kids.values():
        pb.pi_kernel_timer_start(kid, NL)
    active = []
    for li in range(NL):
        layer_step(W, li)
        active.append(int(buf.counts.sum().item()))
    kern = {name: pb.pi_kernel_timer_stop(kid) for name, kid in kids.items()}
    kern_us = {k: ms * 1e3 / max(n, 1) for k, (ms, n) in kern.items() if n}
    touched = float(np.mean([step_bytes(wl, B, a) for a in active]))
    gbps = touched / (us_layer * 1e-6) / 1e9
    del layers, descs, xs
    torch.cuda.empty_cache()
    return {"workload": wl.name, "layers": NL, "batch": B, "steps": K, "warmup": W,
            "us_per_layer": round(us_layer, 3), "ms_per_token": round(us_layer * NL / 1e3, 4),
            "tokens_per_s_ffn_stack": round(1e6 / (us_layer * NL), 1),
            "mean_active": round(float(np.mean(active)), 1),
            "touched_bytes_per_layer_step": round(touched),
            "achieved_gbps_touched": round(gbps, 1),
            "frac_of_peak_touched": round(gbps / PEAK_HBM_GBPS, 4),
            "kernels_us": {k: round(v, 3) for k, v in kern_us.items()},
            "dense_gemv_tokens_per_s_at_peak": round(
                PEAK_HBM_GBPS * 1e9 / (NL * (2 * wl.n * wrow_bytes(wl) + 4 * wl.n)), 1),
            "setup_s": round(setup_s, 1), "timing": "hip_graph",
            "data": "synthetic, layers drawn on the GPU"}


def stack_main(args, wl):
    """`--workload falcon40b-stack-fp16`: the stack on its own JSON line (µs per layer
    step as `value`)."""
    s = run_stack(wl, args.batch, args.steps, args.warmup, "cuda:0")
    out = {
        "metric": METRIC, "value": s["us_per_layer"], "unit": "us/layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": s["ms_per_token"],
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.layers, "d_model": wl.d, "d_ffn": wl.n,
                   "predictor_rank": wl.r, "batch": args.batch, "weights": wl.wdtype,
                   "accumulate": "f32", "hot_fraction": wl.hot_frac},
        "stack": s,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="opt30b-fp16")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--instances", type=int, default=INSTANCES)
    ap.add_argument("--stack-steps", type=int, default=16,
                    help="decode steps of the Falcon-40B-shaped stack in the default run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the step only (no per-step graphs, literal predictor, stream "
                         "ceiling): for profiler runs")
    ap.add_argument("--cold-host", action="store_true",
                    help="place the cold partition's weight rows in pinned host memory "
                         "(capacity tier), read by the kernels over the host link")
    ap.add_argument("--auto-split", action="store_true",
                    help="choose n_hot from the measured read rates of HBM and of pinned host "
                         "memory and a capacity budget (pi_plan_hot_split) instead of the "
                         "workload's fixed hot fraction")
    ap.add_argument("--budget-frac", type=float, default=1.0,
                    help="--auto-split: HBM capacity budget as a fraction of the layer's FFN bytes")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of a captured HIP graph")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the sparse FFN is a single-GPU path here "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_activation_ffn_amd import binding as pb
    from sparse_activation_ffn_amd.layer import DeviceLayer, StepBuffers
    from workload import synth as S

    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = S.WORKLOADS[args.workload]
    if wl.layers > 1:
        return stack_main(args, wl)
    B = args.batch
    K, W = args.steps, args.warmup
    log(f"[bench] generating {wl.name} layer ...")
    L = S.make_layer(wl)
    base = DeviceLayer.upload(L, dev)
    n_hot = wl.n
    perm_np = None
    if wl.hot_frac is not None:
        log("[bench] profiling + neuron index on the GPU ...")
        X = torch.from_numpy(S.make_profile_x(wl, 0)).to(dev)
        counts = base.profile_counts(X)
        perm, n_hot = base.build_index(counts, S.budget_bytes(wl), S.bytes_per_neuron(wl))
        base.apply_index(perm, n_hot)
        perm_np = perm.cpu().numpy()
        del X
    split = None
    if args.auto_split:
        if wl.hot_frac is None:
            raise SystemExit("--auto-split needs a workload with a neuron index")
        log("[bench] read rates of HBM and pinned host memory, bandwidth-aware split ...")
        counts_slot = counts.cpu().numpy().astype(np.uint32)[perm_np]
        r_h = time_stream(pb, torch, STREAM_BUF_BYTES // 2, dev, launches=8)
        r_l = time_stream(pb, torch, 256 << 20, dev, launches=4, host=True)
        bpn = S.bytes_per_neuron(wl)
        budget = int(args.budget_frac * wl.n * bpn)
        n_hot = pb.pi_plan_hot_split(counts_slot, budget, bpn, r_h, r_l)
        base.n_hot = n_hot
        c_hot = float(counts_slot[:n_hot].sum())
        c_all = float(counts_slot.sum())
        split = {"hbm_gbps": round(r_h, 1), "link_gbps": round(r_l, 1), "budget_bytes": budget,
                 "n_hot": n_hot, "fixed_fraction_n_hot": int(wl.hot_frac * wl.n),
                 "profiled_activation_share_hot": round(c_hot / max(c_all, 1.0), 5),
                 "hbm_bytes_saved": (wl.n - n_hot) * bpn,
                 "rule": "smallest n_hot minimising max(hot counts / hbm rate, cold counts / "
                         "link rate), capped by the budget"}
    layers = [base] + [base.clone() for _ in range(args.instances - 1)]
    if args.cold_host:
        log("[bench] placing the cold partition in pinned host memory ...")
        for ly in layers:
            ly.place_cold_on_host()
    descs = [(ly.predictor(), ly.parts()) for ly in layers]
    buf = StepBuffers(base, B, dev)
    xs = [torch.from_numpy(S.make_x(wl, 0, s, B)).to(dev) for s in range(W + K)]
    torch.cuda.synchronize()

    def step(i, literal=False):
        pred, (hot, cold) = descs[i % len(layers)]
        if literal:
            pred = lit_preds[i % len(layers)]
        x = xs[i]
        pb.pi_predict(pred, x, buf.mask, None, None, buf.ws)
        pb.pi_sparse_ffn_split(hot, cold, x, buf.lists, None, None, buf.y, buf.ws, mask=buf.mask)

    log(f"[bench] warmup {W} + timed {K} steps over {len(layers)} instances ...")
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # eager launches from Python: host-bound for kernels this short (reported aside)
    e0.record()
    for i in range(W, W + K):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    us_step_eager = e0.elapsed_time(e1) * 1e3 / K
    # the timed steps captured once into a HIP graph and replayed: device time only
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(W, W + K):
                step(i)
        graph.replay()
        torch.cuda.synchronize()
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        us_step = e0.elapsed_time(e1) * 1e3 / K
        del graph
    else:
        us_step = us_step_eager

    # second pass over the same steps: per-kernel durations from dispatch events, and the
    # active count of each step (deterministic, so identical to the first pass)
    kids = {"k_pred_l1": pb.PI_K_PRED_L1, "k_pred_l2": pb.PI_K_PRED_L2,
            "k_compact": pb.PI_K_COMPACT, "k_up": pb.PI_K_UP, "k_down": pb.PI_K_DOWN,
            "k_ffn": pb.PI_K_FFN, "k_reduce": pb.PI_K_REDUCE, "k_up_finish": pb.PI_K_UP_FINISH}
    for kid in kids.values():
        pb.pi_kernel_timer_start(kid, 2 * K)
    active = []
    hot_active = []
    for i in range(W, W + K):
        step(i)
        c = buf.counts.cpu().numpy()
        active.append(int(c[0] + c[1]))
        hot_active.append(int(c[0]))
    kern_ms = {name: pb.pi_kernel_timer_stop(kid) for name, kid in kids.items()}
    kern_us = {name: ms * 1e3 / max(k, 1) for name, (ms, k) in kern_ms.items()}
    mean_active = float(np.mean(active))
    kb = [kernel_bytes(wl, B, a) for a in active]
    kb_mean = {k: float(np.mean([b[k] for b in kb])) for k in kb[0]}
    touched = float(np.mean([step_bytes(wl, B, a) for a in active]))
    gbps_touched = touched / (us_step * 1e-6) / 1e9
    ran = {k for k in kern_us if kern_ms[k][1] > 0}
    dom = max(ran, key=lambda k: kern_us[k])
    dom_gbps = kb_mean[dom] / (kern_us[dom] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(dom_gbps, 1),
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(dom_gbps / PEAK_HBM_GBPS, 4),
                "algorithmic_bytes": round(kb_mean[dom]),
                "traffic": counter_traffic(wl.name, dom, B), "target_frac": TARGET_FRAC}

    extras = {}
    if not args.no_extras:
        log("[bench] per-step graphs, stream ceiling, literal predictor ...")
        per = per_step_us(torch, step, list(range(W, W + K)))
        extras["step_us_percentiles"] = {
            "p10": round(float(np.percentile(per, 10)), 3),
            "p50": round(float(np.percentile(per, 50)), 3),
            "p90": round(float(np.percentile(per, 90)), 3),
            "how": "HIP events between eagerly launched steps"}
        att = time_stream(pb, torch, int(kb_mean[dom]), dev)
        att_long = time_stream(pb, torch, STREAM_BUF_BYTES // 2, dev, launches=8)
        roofline["attainable"] = round(att, 1)
        roofline["frac_of_attainable"] = round(dom_gbps / att, 4)
        roofline["attainable_long_stream"] = round(att_long, 1)
        roofline["attainable_note"] = ("plain read stream (pi_stream_read) of the dominant "
                                       "kernel's algorithmic bytes per launch; the long stream "
                                       "reads 512 MiB per launch")
        extras["step_frac_of_attainable_long_stream"] = round(gbps_touched / att_long, 4)
        # the literal predictor: the configs' random predictor with no output bias and
        # threshold 0 fires for about half of the neurons
        lit_preds = [pb.make_predictor(ly.P1t, ly.P2t, None, ly.threshold) for ly in layers]
        for i in range(W, W + 3):
            step(i, literal=True)
        torch.cuda.synchronize()
        KL = max(10, K // 4)
        lit_active = []
        e0.record()
        for i in range(W, W + KL):
            step(i, literal=True)
        e1.record()
        torch.cuda.synchronize()
        lit_us = e0.elapsed_time(e1) * 1e3 / KL
        for i in range(W, W + 4):
            step(i, literal=True)
            lit_active.append(int(buf.counts.sum().item()))
        la = float(np.mean(lit_active))
        extras["literal_predictor"] = {
            "us_per_step_eager": round(lit_us, 3), "mean_active": round(la, 1),
            "density": round(la / wl.n, 4),
            "touched_bytes_per_step": round(step_bytes(wl, B, la)),
            "achieved_gbps_touched": round(step_bytes(wl, B, la) / (lit_us * 1e-6) / 1e9, 1),
            "note": "predictor without its output bias (b2 = 0, threshold 0), eager launches"}

        if B == 1 and not args.cold_host and wl.xdtype == "f16":
            log("[bench] prompt-phase crossover over batches ...")
            extras["prompt_crossover"] = prompt_crossover(pb, torch, S, StepBuffers, wl, base, dev)
        if wl.hot_frac is not None and not args.cold_host and B == 1:
            log("[bench] hybrid step: cold partition on the host cores ...")
            extras["hybrid_cpu_cold"] = hybrid_cpu_cold(pb, torch, wl, L, perm_np, layers, buf, xs,
                                                        list(range(W, W + K)), dev, host_cpu()[2])
        if wl.hot_frac is not None and not args.cold_host:
            log("[bench] adaptive predictor threshold ...")
            extras["adaptive_predictor"] = adaptive_predictor(pb, torch, S, wl, base, buf, xs,
                                                              list(range(W, W + K)), dev)

    dense = None
    if not args.no_dense:
        yd = torch.empty((B, wl.d), dtype=torch.float32, device=dev)
        parts = [ly.part() for ly in layers]
        for i in range(3):
            pb.pi_dense_ffn(parts[i % len(parts)], xs[i], yd, buf.ws)
        torch.cuda.synchronize()
        KD = max(10, K // 10)
        e0.record()
        for i in range(KD):
            pb.pi_dense_ffn(parts[i % len(parts)], xs[i], yd, buf.ws)
        e1.record()
        torch.cuda.synchronize()
        dense_us = e0.elapsed_time(e1) * 1e3 / KD
        dense_bytes = (3 if wl.act == "reglu" else 2) * wl.n * wrow_bytes(wl) + 4 * wl.n
        dense = {"us": round(dense_us, 2), "gbps": round(dense_bytes / (dense_us * 1e-6) / 1e9, 1),
                 "speedup_sparse_step_vs_dense_ffn": round(dense_us / us_step, 2),
                 "speedup_vs_dense_gemv_at_peak": round(
                     dense_bytes / (PEAK_HBM_GBPS * 1e3) / us_step, 2)}

    stack = None
    if (not args.no_stack and args.workload == "opt30b-fp16" and B == 1 and not args.cold_host
            and not args.eager):
        del layers, descs
        torch.cuda.empty_cache()
        log("[bench] Falcon-40B-shaped 60-layer stack ...")
        stack = run_stack(S.WORKLOADS["falcon40b-stack-fp16"], 1, args.stack_steps, 2, dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline ...")
        Lh = L
        if perm_np is not None:
            import dataclasses
            take = lambda a: None if a is None else np.ascontiguousarray(a[perm_np])  # noqa: E731
            Lh = dataclasses.replace(L, W_up=take(L.W_up), W_gate=take(L.W_gate),
                                     W_downT=take(L.W_downT), b_up=take(L.b_up),
                                     b_gate=take(L.b_gate), P2t=take(L.P2t), b2=take(L.b2))
        cpu = cpu_baseline(wl, Lh, n_hot, B)

    out = {
        "metric": METRIC, "value": round(us_step, 3), "unit": "us/layer", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(us_step / 1e3, 6),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "d_model": wl.d, "d_ffn": wl.n, "predictor_rank": wl.r,
                   "batch": B, "weights": wl.wdtype, "accumulate": "f32",
                   "hot_fraction": wl.hot_frac, "n_hot": n_hot, "instances": args.instances,
                   "mean_active": round(mean_active, 1),
                   "mean_hot_active": round(float(np.mean(hot_active)), 1)},
        "timing": "eager" if args.eager else "hip_graph",
        "us_per_step_eager_launch": round(us_step_eager, 3),
        "touched_bytes_per_step": round(touched),
        "achieved_gbps_touched": round(gbps_touched, 1),
        "frac_of_peak_touched": round(gbps_touched / PEAK_HBM_GBPS, 4),
        "kernels_us": {k: round(kern_us[k], 3) for k in sorted(ran)},
        "cold_tier": "host" if args.cold_host and n_hot < wl.n else "hbm",
        "cold_bytes_per_step": round(float(np.mean([a - h for a, h in zip(active, hot_active)]))
                                     * ((3 if wl.act == "reglu" else 2) * wrow_bytes(wl) + 4)),
        "kernel_bytes": {k: round(kb_mean[k]) for k in sorted(ran)},
        "auto_split": split,
        "roofline": roofline, **extras, "dense_ffn": dense, "falcon40b_stack": stack,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)

    # a plain copy of known size, whose hardware byte counters calibrate the
    # counter-based traffic figures taken from the same run
    nbytes = COPY_CAL_BYTES
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        pb.pi_copy(src, dst, nbytes)
    torch.cuda.synchronize()


if __name__ == "__main__":
    main()
