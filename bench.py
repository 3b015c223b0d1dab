#!/usr/bin/env python3
"""Route-sort benchmark on one MI355X.

One step = one complete route-sort call (FP32 conversion, correction bias,
grouped top-k, per-expert histogram, padded exclusive prefix, stable scatter,
expert per block) over one batch of seeded synthetic router logits already
resident in HBM.  The headline workload is the skewed prefill chunk (M=8192
tokens, E=896 experts, top-16, 8 groups keep 4, block 128, BF16 logits with
log-Zipf expert popularity).  To keep the logits out of the 256 MB last-level
cache the timed loop rotates over distinct copies of the input totalling at
least --rotate-mb megabytes.

The timed loop replays a HIP graph of consecutive calls, so the per-call time
is the GPU's (kernels and the gaps between them), not the Python launch
overhead; the eager host wall time per call (launch + synchronise) is
reported beside it for the small workloads.

Prints one JSON line on stdout; progress goes to stderr.
"""
import os

os.environ.setdefault("OMP_NUM_THREADS", "1")        # the CPU oracle leg uses one core
os.environ.setdefault("OPENBLAS_NUM_THREADS", "1")
os.environ.setdefault("MKL_NUM_THREADS", "1")

import argparse  # noqa: E402
import hashlib  # noqa: E402
import json  # noqa: E402
import math  # noqa: E402
import platform  # noqa: E402
import sys  # noqa: E402
import time  # noqa: E402

import numpy as np  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBPS = 8000.0
METRIC = "routes/sec (M*k) + achieved HBM GB/s at M=8192; µs/call at M=1, E=896, k=16"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(cfg, npp):
    """Bytes the method must move per call: logits in, bias in, ids + weights
    out, sorted rows, expert per block and the row count out."""
    sz = 2 if cfg.dtype == "bf16" else 4
    return (cfg.M * cfg.E * sz + 4 * cfg.E + 8 * cfg.M * cfg.k + 4 * npp + 4 * (npp // cfg.block) + 4)


def launch_bytes(cfg, npp, launches):
    """Algorithmic bytes attributed to each launch of one call.  One launch:
    everything.  Three launches: selection (logits + bias in, ids + weights
    out), column scan of the workgroup histograms (workspace only), scatter
    (sorted rows, expert per block, row count); two launches (few
    workgroups): the same without the column scan."""
    if launches == 1:
        return [algorithmic_bytes(cfg, npp)]
    sz = 2 if cfg.dtype == "bf16" else 4
    sel = cfg.M * cfg.E * sz + 4 * cfg.E + 8 * cfg.M * cfg.k
    sct = 4 * npp + 4 * (npp // cfg.block) + 4
    return [sel, sct] if launches == 2 else [sel, 0, sct]


def kernel_names(cfg, launches):
    """Names of a call's launches: one workgroup (k_small); selection then the
    scatter that folds the column scan in (k_scatter, at most 16 selection
    workgroups); or selection, column scan and scatter."""
    return {1: ["k_small"], 2: ["k_select", "k_scatter"]}.get(launches, ["k_select", "k_colscan", "k_scatter"])


def to_gpu(inp, torch):
    if inp.cfg.dtype == "bf16":
        x = torch.from_numpy(inp.logits_storage.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        x = torch.from_numpy(inp.logits_storage).cuda()
    return x, torch.from_numpy(inp.bias).cuda()


# calls timed for each workload besides the headline one: 5 replays of 50
# consecutive calls (at most ~25 ms of GPU time on the largest workload)
EXTRA_STEPS = 250


def graph_size(steps, cap=100, min_samples=5):
    """Calls per captured graph: the largest divisor of `steps` not above
    `cap` or steps / min_samples, so a run has at least that many replays.  A
    replay must hold enough GPU work that the host's replay submission does
    not pace the GPU: an empty one-workgroup kernel measured 4.6 us per call
    at 10 calls per replay, 2.0 at 20, 1.7 at 50 and 1.6 at 100; the 8192 x
    896 call 22.6 us at 4 calls per replay with an event between replays,
    21.5 without the events, 20.8 at 20 calls and 20.1 at 100."""
    cap = max(1, min(cap, steps // min_samples))
    return max(g for g in range(1, min(cap, steps) + 1) if steps % g == 0)


def time_workload(cfg, steps, warmup, rotate_mb, torch, amr, per_kernel=False):
    inp = workloads.make_inputs(cfg)
    x0, b = to_gpu(inp, torch)
    mb = x0.numel() * x0.element_size() / 1e6
    nrot = min(64, max(1, int(math.ceil(rotate_mb / mb)))) if rotate_mb > 0 else 1
    # distinct buffers with the same rows in a rotated order: same distribution,
    # no reuse of cached lines between consecutive steps
    xs = [x0] + [torch.roll(x0, shifts=(i * 997) % max(cfg.M, 1), dims=0).contiguous()
                 for i in range(1, nrot)]
    # Every call runs on one stream; its first call, outside the capture,
    # allocates the stream's workspace, so the graph holds route-sort launches
    # only.
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        out = amr.route_sort(x0, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block)
    torch.cuda.synchronize()
    # The timed steps replay a HIP graph of consecutive calls (rotating
    # inputs), so host-side launch overhead does not pace the GPU.
    def capture(G):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(G):
                amr.route_sort(xs[i % nrot], b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block, out=out)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for _ in range(max(1, warmup // G)):
                graph.replay()
        torch.cuda.synchronize()
        return graph
    # The value: exactly `steps` calls in graphs of up to 100 calls, events at
    # the two ends only (an event between replays costs time of its own).  One
    # untimed replay runs ahead of the start event, so the GPU is busy while
    # the host submits the timed replays and their submission latency stays
    # outside the timed region (which then holds exactly the timed calls).
    Gv = graph_size(steps, min_samples=1)
    graph = capture(Gv)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        graph.replay()
    start.record(stream)
    with torch.cuda.stream(stream):
        for i in range(steps // Gv):
            graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    del graph
    # The spread: another `steps` calls, split by events into at least five
    # samples of G calls (smaller graphs, so these samples run a little slower)
    G = graph_size(steps)
    graph = capture(G)
    nrep = steps // G
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(nrep + 1)]
    with torch.cuda.stream(stream):
        graph.replay()  # untimed, ahead of the first mark (as above)
    marks[0].record(stream)
    with torch.cuda.stream(stream):
        for i in range(nrep):
            graph.replay()
            marks[i + 1].record(stream)
    torch.cuda.synchronize()
    del graph
    per_call = np.array([marks[i].elapsed_time(marks[i + 1]) / G for i in range(nrep)]) * 1e3  # us
    npp = int(out.num_post_pad.item())
    # host wall time per call, launch + synchronise (latency view)
    t = time.perf_counter()
    reps = min(steps, 50)
    with torch.cuda.stream(stream):
        for i in range(reps):
            amr.route_sort(xs[i % nrot], b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block, out=out)
            torch.cuda.synchronize()
    wall_us = (time.perf_counter() - t) / reps * 1e6
    nbytes = algorithmic_bytes(cfg, npp)
    r = dict(ms=ms, npp=npp, nbytes=nbytes, rot=nrot, wall_us=wall_us,
             routes_per_s=cfg.M * cfg.k / (ms * 1e-3), gbps=nbytes / (ms * 1e-3) / 1e9,
             value_calls_per_graph=Gv, samples=nrep, calls_per_sample=G,
             us_per_call_p10_p50_p90=[round(float(v), 3) for v in np.percentile(per_call, [10, 50, 90])])
    if per_kernel:
        # HIP events stamped with each kernel's own start and end by the
        # library's launches (hipExtLaunchKernel), same rotation of inputs
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
        launches = 0
        with torch.cuda.stream(stream):
            for i in range(steps):
                _, launches = amr.route_sort(xs[i % nrot], b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block,
                                             out=out, events=evs[i])
        torch.cuda.synchronize()
        per = np.array([[evs[i][2 * j].elapsed_time(evs[i][2 * j + 1]) for j in range(launches)]
                        for i in range(steps)]) * 1e3  # us
        names = kernel_names(cfg, launches)
        r["kernels"] = [dict(name=names[j], avg_us=float(per[:, j].mean()),
                             algorithmic_bytes=launch_bytes(cfg, npp, launches)[j])
                        for j in range(launches)]
        r["launches"] = launches
    return r


def time_sort_from_ids(cfg, steps, torch, amr):
    """The sort-only entry point on the ids the full path chose for this
    workload (same skew), timed like the main loop (graph replay)."""
    inp = workloads.make_inputs(cfg)
    x0, b = to_gpu(inp, torch)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):  # the stream's workspace, allocated outside the capture
        ids = amr.route_sort(x0, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block).ids
        out = amr.sort_from_ids(ids, cfg.E, cfg.block)
    torch.cuda.synchronize()
    G = graph_size(steps)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(G):
            amr.sort_from_ids(ids, cfg.E, cfg.block, out=out)
    with torch.cuda.stream(stream):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(steps // G):
            graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    npp = int(out.num_post_pad.item())
    nbytes = 4 * cfg.M * cfg.k + 4 * npp + 4 * (npp // cfg.block) + 4
    return dict(us_per_call=round(ms * 1e3, 3), routes_per_s=cfg.M * cfg.k / (ms * 1e-3),
                algorithmic_gbps=round(nbytes / (ms * 1e-3) / 1e9, 1), algorithmic_bytes=nbytes)


def time_local(cfg, steps, ranks, torch, amr):
    """One expert-parallel rank's call (experts [0, E/ranks)) on this workload,
    timed like the main loop (graph replay of consecutive calls)."""
    inp = workloads.make_inputs(cfg)
    x0, b = to_gpu(inp, torch)
    rng_ = (0, cfg.E // ranks)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):  # the stream's workspace, allocated outside the capture
        out = amr.route_sort(x0, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block, local=rng_)
    torch.cuda.synchronize()
    G = graph_size(steps)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(G):
            amr.route_sort(x0, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block, local=rng_, out=out)
    with torch.cuda.stream(stream):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(steps // G):
            graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    return dict(ranks=ranks, local_experts=cfg.E // ranks, us_per_call=round(ms * 1e3, 3),
                routes_per_s=cfg.M * cfg.k / (ms * 1e-3), local_rows=int(out.num_post_pad.item()))


GATE_H = 7168  # Kimi-K3 model hidden size


def time_gate(steps, torch, amr):
    """Batch-1 gate projection + route-sort (decode shape: 1 token, 896
    experts, top-16, H = 7168), graph replay of consecutive calls, plus the
    gate kernel alone timed by its own HIP events."""
    cfg = workloads.CONFIGS["decode"]
    g = torch.Generator(device="cuda").manual_seed(0)
    h = torch.randn((1, GATE_H), generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn((cfg.E, GATE_H), generator=g, device="cuda") * GATE_H ** -0.5).to(torch.bfloat16)
    b = (torch.rand((cfg.E,), generator=g, device="cuda") * 0.2 - 0.1).float()
    logits, out = amr.gate_route_sort(h, w, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block)
    torch.cuda.synchronize()
    G = graph_size(steps)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(G):
            amr.gate_route_sort(h, w, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block, out=out, logits=logits)
    with torch.cuda.stream(stream):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(steps // G):
            graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    us = start.elapsed_time(end) / steps * 1e3
    wbytes = cfg.E * GATE_H * 2
    return dict(M=1, E=cfg.E, H=GATE_H, k=cfg.k, us_per_call=round(us, 3), weight_bytes=wbytes,
                weight_gbps_over_call=round(wbytes / (us * 1e-6) / 1e9, 1))


GEMM_K, GEMM_N = 3584, 768     # Kimi-K3 TP8 routed MoE: hidden 3584, 2 x intermediate 384
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 matrix peak


def time_gemm1(cfg, steps, torch, amr):
    """The grouped GEMM1 consumer on this workload's metadata (device-resident,
    straight from the route-sort call), random BF16 hidden states and expert
    weights of the Kimi-K3 TP8 shape; each launch timed by its own start/end
    events."""
    inp = workloads.make_inputs(cfg)
    x0, b = to_gpu(inp, torch)
    meta = amr.route_sort(x0, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block)
    K, N = GEMM_K, GEMM_N
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn((cfg.M, K), generator=g, device="cuda").to(torch.bfloat16)
    w = torch.empty((cfg.E, N, K), dtype=torch.bfloat16, device="cuda")
    for e0 in range(0, cfg.E, 64):  # in slices, so the FP32 draw stays small
        w[e0:e0 + 64] = (torch.randn((min(64, cfg.E - e0), N, K), generator=g, device="cuda")
                         * K ** -0.5).to(torch.bfloat16)
    y = amr.grouped_gemm1(x, w, meta.sorted_ids, meta.expert_of_block, meta.num_post_pad, cfg.k, cfg.block)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        amr.grouped_gemm1(x, w, meta.sorted_ids, meta.expert_of_block, meta.num_post_pad, cfg.k, cfg.block,
                          out=y, events=evs[i])
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(z) for a, z in evs])) * 1e3
    npp = int(meta.num_post_pad.item())
    counts = torch.bincount(meta.ids.reshape(-1).long(), minlength=cfg.E)
    active = int((counts > 0).sum().item())
    flops = 2.0 * cfg.M * cfg.k * N * K                  # routed rows only
    padded_flops = 2.0 * npp * N * K                     # what the tiles compute
    nbytes = active * N * K * 2 + cfg.M * K * 2 + npp * N * 2 + 4 * npp + 4 * (npp // cfg.block) + 4
    del w
    torch.cuda.empty_cache()
    tflops = flops / (us * 1e-6) / 1e12
    gbps = nbytes / (us * 1e-6) / 1e9
    t_mfma = padded_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e6
    t_hbm = nbytes / (HBM_PEAK_GBPS * 1e9) * 1e6
    return dict(kernel="k_gemm1", K=K, N=N, us_per_call=round(us, 2), num_post_pad=npp, active_experts=active,
                useful_tflops=round(tflops, 1), padded_tflops=round(padded_flops / (us * 1e-6) / 1e12, 1),
                algorithmic_bytes=nbytes, algorithmic_gbps=round(gbps, 1),
                roofline_us={"mfma_bf16": round(t_mfma, 2), "hbm": round(t_hbm, 2)},
                bound="hbm" if t_hbm > t_mfma else "mfma",
                frac_of_bound=round(max(t_mfma, t_hbm) / us, 4))


def traffic_record(kernel, workload):
    """HBM traffic per launch measured with rocprofv3 PMC counters and stored
    under profiles/, used only while the kernel source still has the hash the
    counters were taken with."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    src = os.path.join(ROOT, "align_moe_route_amd", "csrc", "moe_route_sort.hip")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("source_sha256") != h:
        return None
    return rec


def _pmc_medians(path, counter):
    """Median per dispatch of one counter, by kernel name, from a rocprofv3
    counter_collection.csv."""
    import csv
    vals = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter:
                vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: (float(np.median(v)), len(v)) for k, v in vals.items()}


def write_traffic_record(fetch_csv, write_csv, workload, calib_mb, commands):
    """HBM bytes per launch of this workload's kernels from two rocprofv3 PMC
    runs (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch), each scaled by
    what the same counter reads for the plain device copy of calib_mb MB that
    --calib-copy-mb runs first.  Writes profiles/traffic_<dominant>_<workload>.json
    (read back by traffic_record while the kernel source keeps its hash) and a
    markdown table of every kernel."""
    fetch = _pmc_medians(fetch_csv, "FETCH_SIZE")
    write = _pmc_medians(write_csv, "WRITE_SIZE")
    calib = int(calib_mb * 1e6) // 4 * 4
    copy = max((k for k in fetch if "copyBuffer" in k), key=lambda k: fetch[k][0])
    fscale = calib / (fetch[copy][0] * 1024)
    wscale = calib / (write[copy][0] * 1024)
    src = os.path.join(ROOT, "align_moe_route_amd", "csrc", "moe_route_sort.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    ours = [k for k in fetch if k.startswith(("void (anonymous namespace)::k_", "(anonymous namespace)::k_"))]
    dom = next(k for k in ours if "k_select" in k or "k_small" in k)
    name = "k_select" if "k_select" in dom else "k_small"
    rec = {"kernel": name, "workload": workload, "source_sha256": sha,
           "fetch_bytes": int(round(fetch[dom][0] * 1024 * fscale)),
           "write_bytes": int(round(write[dom][0] * 1024 * wscale)),
           "fetch_scale": fscale, "write_scale": wscale, "commands": commands}
    out = os.path.join(ROOT, "profiles", f"traffic_{name}_{workload}.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"# HBM traffic per launch, {workload} workload", "",
             "Commands (from the repository root):", ""] + ["    " + c for c in commands] + [
             "", f"Calibration: a plain device copy of {calib} bytes reads FETCH_SIZE = {fetch[copy][0]:.0f} KiB "
             f"and WRITE_SIZE = {write[copy][0]:.0f} KiB per dispatch; scale factors {fscale:.3f} x 1024 (fetch) "
             f"and {wscale:.3f} x 1024 (write).", f"Kernel source sha256: {sha}", "",
             "| kernel | dispatches | FETCH_SIZE KiB (median) | fetch MB (scaled) | WRITE_SIZE KiB (median) "
             "| write MB (scaled) |", "|---|---|---|---|---|---|"]
    for k in ours:
        fk, n = fetch[k]
        wk = write.get(k, (0.0, 0))[0]
        lines.append(f"| {k.replace('(anonymous namespace)::', '').split('((')[0]} | {n} | {fk:.0f} | "
                     f"{fk * 1024 * fscale / 1e6:.3f} | {wk:.0f} | {wk * 1024 * wscale / 1e6:.3f} |")
    md = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    with open(md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out, md


def copy_bandwidth(torch, nbytes=512 << 20, reps=5):
    """Measured device-to-device copy rate (bytes read + written per second),
    beside the 8 TB/s spec peak: what a plain streaming kernel reaches."""
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbps = 2 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return round(gbps, 1)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


_POOL_WORK = None  # (cfg, inputs) of the all-core figure, inherited by the forked workers


def _oracle_select_chunk(span):
    """Worker of the all-core figure: the oracle's per-token selection on one
    chunk of tokens (its metadata of the chunk is discarded)."""
    from oracle import route_sort as orc
    cfg, inp = _POOL_WORK
    r = orc.route_sort(inp.logits_storage, cfg.dtype, inp.bias, cfg.k, cfg.n_group, cfg.topk_group,
                       cfg.block, tokens=np.arange(span[0], span[1]))
    return r.ids


def cpu_baseline(cfg, reps=3):
    """The oracle as it stands, on the full workload: one complete call
    (selection of every token + sort metadata) timed with perf_counter_ns,
    median of `reps` (1 when a call exceeds 60 s), in this process with NumPy
    on one thread.  Also: the all-core figure (the per-token selection split
    over a pool of processes, one per affinity core, then the sort on one
    core; pool start-up not timed) and the oracle's near-tie gaps of the
    same inputs.  Run before the GPU is touched, so the pool forks a process
    that holds no GPU state."""
    from oracle import route_sort as orc
    inp = workloads.make_inputs(cfg)
    times, ref = [], None
    for _ in range(reps):
        t = time.perf_counter_ns()
        ref = orc.route_sort(inp.logits_storage, cfg.dtype, inp.bias, cfg.k, cfg.n_group,
                             cfg.topk_group, cfg.block)
        times.append((time.perf_counter_ns() - t) * 1e-9)
        if times[-1] > 60.0:
            break
    sec = float(np.median(times))
    ncore = len(os.sched_getaffinity(0))
    allcore = None
    if ncore > 1:
        import multiprocessing as mp
        global _POOL_WORK
        _POOL_WORK = (cfg, inp)
        edges = np.linspace(0, cfg.M, ncore + 1).astype(int)
        jobs = [(int(lo), int(hi)) for lo, hi in zip(edges[:-1], edges[1:]) if hi > lo]
        with mp.get_context("fork").Pool(len(jobs)) as pool:
            pool.map(_oracle_select_chunk, jobs[:1])  # workers up before the clock starts
            t = time.perf_counter_ns()
            parts = pool.map(_oracle_select_chunk, jobs)
            ids = np.concatenate(parts)
            orc.sort_metadata(ids, cfg.E, cfg.block)
            asec = (time.perf_counter_ns() - t) * 1e-9
        allcore = dict(value=cfg.M * cfg.k / asec, unit="routes/s", cores=len(jobs), s_per_call=asec,
                       method="per-token selection split over a process pool, sort metadata on one core")
    out = dict(value=cfg.M * cfg.k / sec, unit="routes/s", cores=1, kind="oracle", s_per_call=sec,
               samples_s=[round(x, 4) for x in times], host_cpu=cpu_model(), host_cpu_count=os.cpu_count(),
               host_affinity_cores=ncore,
               sample=f"one complete oracle call on the whole {cfg.name} workload ({cfg.M} tokens x {cfg.E} "
                      f"experts, top-{cfg.k}: selection + sort metadata), median of {len(times)}, one core "
                      f"of {cpu_model()}",
               all_cores=allcore)
    return out, ref


def near_ties(cfg, ref, limit=1e-6):
    """Tokens whose oracle gap between the k-th and (k+1)-th key (gap_k), or
    between the last kept and first dropped group score (gap_g), is below
    `limit`; they are still required to match exactly."""
    gk, gg = ref.gap_k, ref.gap_g
    near = np.flatnonzero((gk < limit) | (gg < limit))
    return dict(tokens=int(near.size), gap_k_below=int((gk < limit).sum()), gap_g_below=int((gg < limit).sum()),
                token_ids=[int(t) for t in near[:32]],
                gaps=[[float(gk[t]) if np.isfinite(gk[t]) else None,
                       float(gg[t]) if np.isfinite(gg[t]) else None] for t in near[:32]])


def gpu_ids(cfg, torch, amr):
    inp = workloads.make_inputs(cfg)
    x, b = to_gpu(inp, torch)
    out = amr.route_sort(x, b, cfg.k, cfg.n_group, cfg.topk_group, cfg.block)
    torch.cuda.synchronize()
    return out.ids.cpu().numpy()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill_skew", choices=list(workloads.CONFIGS))
    ap.add_argument("--rotate-mb", type=float, default=600.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--calib-copy-mb", type=float, default=0.0,
                    help="first run a plain device-to-device copy of this many MB three times "
                         "(reference dispatches for scaling PMC byte counters)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: turn two rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter_collection.csv "
                         "files of this workload (made with --calib-copy-mb) into profiles/traffic_*")
    args = ap.parse_args()
    if args.write_traffic:
        base = (f"python3 bench.py --workload {args.workload} --no-extra --no-cpu-baseline --steps 5 "
                f"--warmup 1 --calib-copy-mb {args.calib_copy_mb:g}")
        # the commands as they made the two files: output folder = each file's folder
        cmds = [f"rocprofv3 --pmc {c} --output-format csv -d {os.path.dirname(f) or '.'} -o run -- {base}"
                for c, f in (("FETCH_SIZE", args.write_traffic[0]), ("WRITE_SIZE", args.write_traffic[1]))]
        for path in write_traffic_record(args.write_traffic[0], args.write_traffic[1], args.workload,
                                         args.calib_copy_mb, cmds):
            print(path)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the route-sort path has no cross-GPU step "
              "(each rank routes its own tokens); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    cfg = workloads.CONFIGS[args.workload]
    # The CPU-baseline leg runs first, before anything touches the GPU: the
    # oracle timed on this workload, and the oracle's near-tie gaps of every
    # workload (reported separately; the GPU ids on those tokens are compared
    # with the oracle's after the GPU timing).
    cpu, near, near_ref = None, None, {}
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle: one complete call on {cfg.name}, median of 3")
        cpu, ref = cpu_baseline(cfg)
        log(f"[bench] oracle: {cpu['value']:.3e} routes/s on one core ({cpu['s_per_call']:.3f} s per call)"
            + (f", {cpu['all_cores']['value']:.3e} on {cpu['all_cores']['cores']} cores" if cpu["all_cores"] else ""))
        from oracle import route_sort as orc
        near = {}
        for name in workloads.CONFIG_ORDER:
            c = workloads.CONFIGS[name]
            if name == cfg.name:
                rr = ref
            else:
                inp = workloads.make_inputs(c)
                rr = orc.route_sort(inp.logits_storage, c.dtype, inp.bias, c.k, c.n_group, c.topk_group, c.block)
            near[name] = near_ties(c, rr)
            near_ref[name] = rr.ids
            log(f"[bench] near-tie tokens in {name}: {near[name]['tokens']}")

    import torch
    import align_moe_route_amd as amr
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    amr.lib()

    if args.calib_copy_mb > 0:
        n = int(args.calib_copy_mb * 1e6) // 4
        src = torch.arange(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: 3 x {4 * n} bytes read and written")
        del src, dst

    log(f"[bench] {cfg.name}: M={cfg.M} E={cfg.E} k={cfg.k} steps={args.steps} warmup={args.warmup}")
    torch.cuda.synchronize()
    r = time_workload(cfg, args.steps, args.warmup, args.rotate_mb, torch, amr, per_kernel=True)
    log(f"[bench] {cfg.name}: {r['ms']*1e3:.2f} us/call, {r['routes_per_s']:.3e} routes/s, "
        f"{r['gbps']:.1f} GB/s algorithmic, {r['rot']} rotating input copies")
    for kr in r["kernels"]:
        log(f"[bench]   {kr['name']}: {kr['avg_us']:.2f} us/launch, {kr['algorithmic_bytes']} algorithmic bytes")
    # warm: one input buffer, reused by every call (the logits stay in the caches)
    rw = time_workload(cfg, args.steps, args.warmup, 0.0, torch, amr)
    log(f"[bench] {cfg.name} warm (one input buffer): {rw['ms']*1e3:.2f} us/call")
    copy_gbps = copy_bandwidth(torch)
    log(f"[bench] measured device copy: {copy_gbps:.0f} GB/s (read + write)")
    dom = max(r["kernels"], key=lambda kr: kr["avg_us"])
    dom_gbps = dom["algorithmic_bytes"] / (dom["avg_us"] * 1e-6) / 1e9
    tr = traffic_record(dom["name"], cfg.name)

    extra = {}
    if not args.no_extra:
        for name in workloads.CONFIG_ORDER:
            if name == cfg.name:
                continue
            c = workloads.CONFIGS[name]
            e = time_workload(c, EXTRA_STEPS, 5, args.rotate_mb, torch, amr)
            extra[name] = dict(us_per_call=round(e["ms"] * 1e3, 3),
                               us_per_call_p10_p50_p90=e["us_per_call_p10_p50_p90"],
                               host_wall_us_per_call=round(e["wall_us"], 2),
                               routes_per_s=e["routes_per_s"], algorithmic_gbps=round(e["gbps"], 1),
                               frac_hbm_peak=round(e["gbps"] / HBM_PEAK_GBPS, 4))
            log(f"[bench] {name}: {e['ms']*1e3:.2f} us/call, {e['routes_per_s']:.3e} routes/s, "
                f"{e['gbps']:.1f} GB/s")

    if not args.no_extra:
        # batched decode on the decode shape (896 experts, top-16, 8 groups keep 4,
        # block 32, BF16): the batch sizes where the one-workgroup and the
        # three-launch paths trade places
        for mb in (32, 64):
            c = workloads.custom(mb, 896, 16, 8, 4, 32, "bf16", "normal", seed=0, name=f"decode_batch_{mb}")
            e = time_workload(c, EXTRA_STEPS, 5, args.rotate_mb, torch, amr)
            extra[c.name] = dict(us_per_call=round(e["ms"] * 1e3, 3), routes_per_s=e["routes_per_s"])
            log(f"[bench] {c.name}: {e['ms']*1e3:.2f} us/call")
        so = time_sort_from_ids(cfg, EXTRA_STEPS, torch, amr)
        extra["sort_from_ids_" + cfg.name] = so
        log(f"[bench] sort_from_ids on {cfg.name} ids: {so['us_per_call']:.2f} us/call, "
            f"{so['routes_per_s']:.3e} routes/s")
        lo = time_local(cfg, EXTRA_STEPS, 8, torch, amr)
        extra["local_rank_of_8_" + cfg.name] = lo
        log(f"[bench] one rank of 8 (experts [0, {lo['local_experts']})) on {cfg.name}: "
            f"{lo['us_per_call']:.2f} us/call, {lo['local_rows']} local rows")
        ga = time_gate(EXTRA_STEPS, torch, amr)
        extra["gate_route_sort_decode"] = ga
        log(f"[bench] gate projection (H={ga['H']}) + route-sort, 1 token: {ga['us_per_call']:.2f} us/call "
            f"({ga['weight_gbps_over_call']:.0f} GB/s of gate weights over the whole call)")
        gm = time_gemm1(cfg, 20, torch, amr)
        extra["grouped_gemm1_" + cfg.name] = gm
        log(f"[bench] grouped GEMM1 (K={gm['K']}, N={gm['N']}) on {cfg.name} metadata: {gm['us_per_call']:.1f} us, "
            f"{gm['useful_tflops']:.1f} TFLOP/s routed ({gm['padded_tflops']:.1f} with padding), "
            f"{gm['active_experts']} experts active, {gm['algorithmic_gbps']:.0f} GB/s, "
            f"{gm['frac_of_bound']:.3f} of the {gm['bound']} bound")

    if near is not None:
        # the GPU's ids on the near-tie tokens against the oracle's (every
        # other token is compared by the parity tests)
        for name, rec in near.items():
            toks = np.array(rec["token_ids"], dtype=np.int64)
            g = gpu_ids(workloads.CONFIGS[name], torch, amr)
            allnear = np.flatnonzero((near_ref[name] != g).any(axis=1))
            rec["gpu_ids_match_on_listed_tokens"] = bool(np.array_equal(g[toks], near_ref[name][toks]))
            rec["gpu_tokens_differing_from_oracle"] = int(allnear.size)

    res = {
        "metric": METRIC,
        "value": r["routes_per_s"],
        "unit": "routes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; BF16 logits N(0,1) + log-Zipf(1.1) expert offsets, bias U(-0.1,0.1))",
        "config": {"workload": cfg.name, "M": cfg.M, "E": cfg.E, "k": cfg.k, "n_group": cfg.n_group,
                   "topk_group": cfg.topk_group, "block": cfg.block, "logits": cfg.dtype},
        "hbm_gbps_algorithmic": r["gbps"],
        "us_per_call": r["ms"] * 1e3,
        "us_per_call_p10_p50_p90": r["us_per_call_p10_p50_p90"],
        "warm_us_per_call": rw["ms"] * 1e3,
        "timing": {"value_graph_calls": r["value_calls_per_graph"], "spread_graph_calls": r["calls_per_sample"],
                   "spread_samples": r["samples"], "untimed_replay_ahead": True},
        "launches_per_call": r["launches"],
        "decode_us_per_call": extra.get("decode", {}).get("us_per_call"),
        "hbm_copy_gbps_measured": copy_gbps,
        "roofline": {"bound": "hbm", "kernel": dom["name"], "achieved": dom_gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": dom_gbps / HBM_PEAK_GBPS,
                     "traffic": (tr["fetch_bytes"] + tr["write_bytes"]) if tr else None,
                     "algorithmic_bytes_per_launch": dom["algorithmic_bytes"],
                     "avg_launch_us": dom["avg_us"]},
        "kernels": r["kernels"],
        "whole_call": {"algorithmic_bytes": r["nbytes"], "achieved_gbps": r["gbps"],
                       "frac": r["gbps"] / HBM_PEAK_GBPS},
        "cpu_baseline": cpu,
        "near_tie": near,
        "other_workloads": extra,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
