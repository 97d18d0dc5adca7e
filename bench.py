#!/usr/bin/env python3
"""SPECTRA dequant-GEMV benchmark on one MI355X: effective HBM GB/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload cfg3] [--M 1]

Default workload (cfg3): the M = 1 decode step of a 4B-class decoder -- 36
layers x 7 linears (q/k/v/o/gate/up/down, hidden 2560, MLP 9728), every layer
distinct, so one step streams about 2.2 GB of packed weights from HBM.
Default mode `graph`: the products as 144 launches (q/k/v and gate/up
grouped) replayed as one captured HIP graph, each launch on its own
synthetic input.  Mode `step`: the whole step is one launch of the
persistent decode-step kernel (spectra_step_run): 144 dependent phases
(q/k/v, o, gate/up, down per layer), each phase reading the previous one's
output (o reads q, gate/up read o, down reads gate, the next q/k/v read
down, each scaled by a power of two; the attention, norms and activation
between them are outside the path).  Containers and inputs are resident in
HBM before timing starts.

value = algorithmic bytes per step / step time.  A linear's algorithmic bytes
are its container payload (codes + scales + zero nibbles + fp16 heavy-tailed
columns) + metadata (header, mask, perm) + x + y, each counted once (a
grouped launch counts x once).

Other workloads: cfg1 / cfg4 / cfg5 time one linear per step, rotating over
enough distinct packed copies to exceed 1 GiB so the last-level cache cannot
serve the weights (`--warm`: one container launched as often instead, the
cache-resident figure, labelled mode "warm"); cfg2 stacks the 1.5B-class
layer 28 deep.  `embed` times
the fused embedding gather instead (its own metric): --tokens random rows of
the 131072 x 3072 table per step, rotated over copies the same way; bytes =
the gathered rows' payload + the fp16 rows written + the ids.  `load` times
spectra_load of the 241 MB container file through the chunked staging path;
`kv` times decode attention over the Group-32 4-bit KV cache.

Prints ONE JSON line.  roofline: the dominant kernel (largest share of step
bytes) is replayed alone as a captured graph and timed with HIP events on its
launch stream; achieved = its algorithmic bytes per launch / average launch
time; traffic comes from a committed counter profile when it matches the
current kernel source.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "dequant-GEMV effective HBM GB/s and % of peak at M=1; weights-GB/s vs M"
PEAK_HBM_GBS = 8000.0      # MI355X published HBM3E bandwidth
PEAK_MFMA_F16_TFLOPS = 2500.0  # MI355X dense fp16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="cfg3", choices=["cfg1", "cfg2", "cfg3", "cfg4", "cfg5", "embed", "load", "kv"])
    ap.add_argument("--tokens", type=int, default=16384, help="embed: token ids gathered per step")
    ap.add_argument("--chunk-mib", type=int, default=8, help="load: staging chunk size")
    ap.add_argument("--context", type=int, default=8192, help="kv: cached tokens attended per step")
    ap.add_argument("--M", type=int, default=1)
    ap.add_argument("--kernel", default="auto", choices=["auto", "gemv", "mfma", "mfma_splitk", "mfma_tiled", "mfma_strip"])
    ap.add_argument("--mode", default="graph", choices=["step", "graph"],
                    help="cfg2/cfg3 at M = 1: a graph of 144 launches, or one persistent launch per step")
    ap.add_argument("--layers", type=int, default=None, help="cfg3: fewer layers (quick runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--warm", action="store_true",
                    help="cfg1/cfg4/cfg5: cache-resident figure, one container launched as many times per "
                         "replay as the rotation would launch distinct copies (labelled warm, not the headline)")
    ap.add_argument("--eager", action="store_true",
                    help="launch every unit directly instead of replaying graphs (for counter runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run plain 1 GiB device copies (counter calibration) and exit")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


GEMV_SOURCES = ("gemv.hip", "gemv_common.h")
MFMA_SOURCES = ("mfma.hip",)
STEP_SOURCES = ("step.hip", "gemv_common.h", "gemv.hip")  # gemv.hip picks the step's team width too


def kernel_sources_sha(files=GEMV_SOURCES):
    """Hash of a kernel's sources: stored counter figures are valid while it holds."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "dequant_gemv_spectra_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


class Linear:
    """One packed linear with resident x and y."""

    def __init__(self, sp, torch, lin, cfg, M, W=None, g=None, copy=0):
        import numpy as np
        from dequant_gemv_spectra_amd import synth
        W = synth.weights(lin, cfg) if W is None else W
        g = synth.gamma(lin, cfg) if g is None else g
        # rms gain of the product for unit-rms input (row norms of W): sets the
        # decode-step chain's power-of-two input scales
        w = W.astype(np.float32).ravel()
        self.gain = float(np.sqrt(np.dot(w, w) / lin.N))
        self.c = sp.spectra_pack(W, g)
        self.info = self.c.info()
        self.lin = lin
        self.x = torch.from_numpy(synth.activations(lin, cfg, M, salt=copy)).cuda()
        self.y = torch.empty((M, lin.N), dtype=torch.float16, device="cuda")
        self.bytes = (self.info["bytes_payload"] + self.info["bytes_meta"] + 2 * M * lin.K + 2 * M * lin.N)


def gemm_call(sp, p, kern):
    def f():
        sp.spectra_gemm(p.c, p.x, p.y, kernel=kern)
    return f


def grouped_call(sp, ps):
    cs = [p.c for p in ps]
    ys = [p.y for p in ps]
    x = ps[0].x

    def f():
        sp.spectra_gemm_grouped(cs, x, ys)
    return f


def layer_units(sp, packed, M, kern, tag):
    """Launch units of one decoder layer: (label, kind, callable, bytes, kernel run)."""
    by = {p.lin.name.split(".")[-1]: p for p in packed}
    plan = lambda p: sp.spectra_gemm_plan(p.c, M, kern)
    if M == 1 and kern in ("auto", "gemv"):
        qkv, gu = [by["q"], by["k"], by["v"]], [by["gate"], by["up"]]
        return [(f"{tag}.qkv", "qkv", grouped_call(sp, qkv), sum(p.bytes for p in qkv) - 2 * 2 * by["q"].lin.K,
                 "k_gemv_m1"),
                (f"{tag}.o", "o", gemm_call(sp, by["o"], kern), by["o"].bytes, plan(by["o"])),
                (f"{tag}.gate_up", "gate_up", grouped_call(sp, gu), sum(p.bytes for p in gu) - 2 * by["gate"].lin.K,
                 "k_gemv_m1"),
                (f"{tag}.down", "down", gemm_call(sp, by["down"], kern), by["down"].bytes, plan(by["down"]))]
    return [(f"{tag}.{nm}", nm, gemm_call(sp, by[nm], kern), by[nm].bytes, plan(by[nm]))
            for nm in ("q", "k", "v", "o", "gate", "up", "down")]


def build_units(args, sp, torch):
    from dequant_gemv_spectra_amd import synth
    cfg = int(args.workload[3:])
    wl = synth.workload(cfg, layers=args.layers if cfg == 3 else None)
    M, kern = args.M, args.kernel
    units = []
    args.layers_packed = []
    if cfg in (2, 3):
        by_layer = {}
        for lin in wl.linears:
            by_layer.setdefault(lin.layer, []).append(lin)
        depth = 28 if cfg == 2 else 1  # the 1.5B-class model is 28 layers deep
        cache = {}
        for layer in sorted(by_layer):
            for cp in range(depth):
                t0 = time.time()
                packed = []
                for lin in by_layer[layer]:
                    if lin.name not in cache:
                        cache[lin.name] = (synth.weights(lin, cfg), synth.gamma(lin, cfg))
                    W, g = cache[lin.name]
                    packed.append(Linear(sp, torch, lin, cfg, M, W, g, copy=cp))
                units.extend(layer_units(sp, packed, M, kern, f"L{layer if depth == 1 else cp}"))
                args.layers_packed.append({p.lin.name.split(".")[-1]: p for p in packed})
                if (layer if depth == 1 else cp) % 6 == 0:
                    log(f"layer {layer if depth == 1 else cp}: packed in {time.time() - t0:.1f}s")
            if depth == 1:
                cache.clear()
        name = wl.name if cfg == 3 else "decoder-1.5B-28-layers"
        return name, units, True
    lin = wl.linears[0]
    W, g = synth.weights(lin, cfg), synth.gamma(lin, cfg)
    first = Linear(sp, torch, lin, cfg, M, W, g)
    copies = max(1, int(args.rotate_gib * 2 ** 30 // first.bytes) + 1)
    if args.warm:  # the same container every launch: its bytes stay in the last-level cache
        packed = [first] * copies
        log(f"{wl.name}: warm, one container launched {copies} times per replay, {first.bytes / 1e6:.1f} MB")
    else:
        packed = [first] + [Linear(sp, torch, lin, cfg, M, W, g, copy=cp) for cp in range(1, copies)]
        log(f"{wl.name}: {copies} distinct copies, {first.bytes / 1e6:.1f} MB each")
    units = [(f"{lin.name}#{i}", lin.name, gemm_call(sp, p, kern), p.bytes, sp.spectra_gemm_plan(p.c, M, kern))
             for i, p in enumerate(packed)]
    return wl.name, units, False


EMBED_METRIC = "fused G32 embedding row gather: effective HBM GB/s (table rows read + fp16 rows written)"


def run_embed(args, sp, torch):
    """One step = gather args.tokens random rows of the 131072 x 3072 table
    (the LM-head shape read as a tied embedding), rotating over distinct
    packed copies (>= 1 GiB) so the rows come from HBM."""
    import numpy as np
    from dequant_gemv_spectra_amd import synth
    cfg = 4
    lin = synth.workload(cfg).linears[0]
    W, g = synth.weights(lin, cfg), synth.gamma(lin, cfg)
    first = sp.spectra_pack(W, g)
    info = first.info()
    copies = max(1, int(args.rotate_gib * 2 ** 30 // info["bytes_total"]) + 1)
    cs = [first] + [sp.spectra_pack(W, g) for _ in range(1, copies)]
    T = args.tokens
    rng = np.random.default_rng(2024)
    ids = [torch.from_numpy(rng.integers(0, lin.N, T).astype(np.int32)).cuda() for _ in cs]
    outs = [torch.empty((T, lin.K), dtype=torch.float16, device="cuda") for _ in cs]
    row_bytes = (info["bytes_payload"]) / lin.N  # codes + scales + zeros + fp16 channels of one row
    step_bytes = T * (row_bytes + 2 * lin.K + 4)
    log(f"embed: {copies} distinct copies of {lin.N} x {lin.K}, {T} ids per step, "
        f"{step_bytes / 1e6:.1f} MB per step")

    def mk(c, i, o):
        def f():
            sp.spectra_embed(c, i, out=o)
        return f
    fns = [mk(c, i, o) for c, i, o in zip(cs, ids, outs)]
    graph = capture(torch, fns)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // len(fns))
    ms = time_graph(torch, graph, reps) / len(fns)
    value = step_bytes / (ms * 1e-3) / 1e9
    dgraph = capture(torch, fns)
    dgraph.replay()
    dms = time_graph(torch, dgraph, 10) / len(fns)
    achieved = step_bytes / (dms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                "kernel": "k_embed", "avg_launch_us": round(dms * 1e3, 3),
                "bytes_per_launch": int(step_bytes), "launches_timed": 10 * len(fns)}
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import spectra_oracle as O
        img = sp.spectra_export(first)
        sample = rng.integers(0, lin.N, 2048)
        done, t_total, rounds = 0, 0.0, 0
        while t_total < 10.0:
            t0 = time.perf_counter()
            O.embed_ref(img, sample)
            t_total += time.perf_counter() - t0
            done += sample.size
            rounds += 1
        cpu = {"value": round(done * (row_bytes + 2 * lin.K + 4) / t_total / 1e9, 4), "unit": "GB/s",
               "cores": 1, "kind": "oracle",
               "sample": f"oracle row gather (unpack of the sampled rows + fp16 rounding) of 2048 random ids "
                         f"x {rounds} rounds in {t_total:.1f} s; single-threaded numpy"}
    out = {"metric": EMBED_METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
           "data": "synthetic",
           "config": {"workload": f"embedding-gather-{lin.N}x{lin.K}", "tokens": T,
                      "bytes_per_step": int(step_bytes), "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
                      "hip_graph": True, "parallelism": "single GPU"},
           "roofline": roofline, "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)


LOAD_METRIC = "container file streamed into HBM: GB/s (file bytes / wall time of spectra_load)"


def run_load(args, sp, torch):
    """One step = spectra_load of the 131072 x 3072 container (241 MB) from a
    file written by spectra_save (the file sits in the page cache after the
    save and the warmup loads: the rate is that of the staging path, not of a
    disk).  Synchronous calls, timed by the host clock."""
    import tempfile
    from dequant_gemv_spectra_amd import synth
    lin = synth.workload(4).linears[0]
    c = sp.spectra_pack(synth.weights(lin, 4), synth.gamma(lin, 4))
    total = c.info()["bytes_total"]
    chunk = args.chunk_mib << 20
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "lm_head.spectra")
        sp.spectra_save(c, path, chunk)
        for _ in range(args.warmup):
            sp.spectra_load(path, chunk).close()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            sp.spectra_load(path, chunk).close()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / max(1, args.steps)
    value = total / (ms * 1e-3) / 1e9
    out = {"metric": LOAD_METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bytes",
           "data": "synthetic",
           "config": {"workload": f"container-load-{lin.N}x{lin.K}", "bytes": int(total),
                      "chunk_bytes": chunk, "peak_host_staging_bytes": 2 * chunk, "parallelism": "single GPU"},
           "roofline": None, "cpu_baseline": None}
    print(json.dumps(out), flush=True)


KV_METRIC = "G32 4-bit KV-cache decode attention: effective HBM GB/s (quantized K and V read)"


def run_kv(args, sp, torch):
    """One step = decode attention of 32 query heads over 8 cache heads of 128
    channels (the 4B-class layer) with --context cached tokens, rotating over
    distinct caches (>= 1 GiB) so they stream from HBM."""
    import numpy as np
    H, rep_, D, L = 8, 4, 128, args.context
    per = 2 * L * H * (D // 32) * (16 + 2) + L * H * (D // 32)  # K and V records, scales, zero bytes
    copies = max(1, int(args.rotate_gib * 2 ** 30 // per) + 1)
    rng = np.random.default_rng(31)
    caches = []
    for i in range(copies):
        kv = sp.KvCache(L, H, D)
        k = torch.from_numpy(rng.standard_normal((L, H, D)).astype(np.float16)).cuda()
        v = torch.from_numpy((rng.standard_normal((L, H, D)) * 0.5).astype(np.float16)).cuda()
        kv.append(k, v)
        caches.append(kv)
    q = torch.from_numpy(rng.standard_normal((H * rep_, D)).astype(np.float16)).cuda()
    outs = [torch.empty_like(q) for _ in caches]
    step_bytes = per + 2 * 2 * H * rep_ * D
    log(f"kv: {copies} caches of {L} tokens, {per / 1e6:.2f} MB each")

    def mk(kv, o):
        def f():
            kv.attend(q, out=o)
        return f
    fns = [mk(kv, o) for kv, o in zip(caches, outs)]
    graph = capture(torch, fns)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // len(fns))
    ms = time_graph(torch, graph, reps) / len(fns)
    value = step_bytes / (ms * 1e-3) / 1e9
    out = {"metric": KV_METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
           "data": "synthetic",
           "config": {"workload": f"kv-attend-{H * rep_}q-{H}kv-{D}d-{L}ctx", "bytes_per_step": int(step_bytes),
                      "launches_per_step": 2, "hip_graph": True, "parallelism": "single GPU"},
           "roofline": {"bound": "hbm", "achieved": round(value, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(value / PEAK_HBM_GBS, 4), "traffic": None,
                        "kernel": "k_kv_split + k_kv_combine", "avg_launch_us": round(ms * 1e3, 3),
                        "bytes_per_launch": int(step_bytes)},
           "cpu_baseline": None}
    print(json.dumps(out), flush=True)


def run_step(args, sp, torch, name, units):
    """Mode `step`: the decoder stack as one persistent launch per step."""
    from dequant_gemv_spectra_amd import decoder
    layers, gains = [], []
    for L in args.layers_packed:
        layers.append({nm: (p.c, p.y.view(-1)) for nm, p in L.items()})
        gains += [L["q"].gain, L["o"].gain, L["gate"].gain, L["down"].gain]
    x0 = args.layers_packed[0]["q"].x.view(-1)
    phases = decoder.layer_phases(layers, x0, decoder.chain_scales(gains))
    plan = sp.StepPlan(phases)
    # algorithmic bytes: every container's payload + metadata, each phase's
    # input once, every output once
    step_bytes = 0
    for ph in phases:
        K = ph["containers"][0].info()["K"]
        step_bytes += 2 * K
        for c in ph["containers"]:
            inf = c.info()
            step_bytes += inf["bytes_payload"] + inf["bytes_meta"] + 2 * inf["N"]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(args.warmup):
            plan.run(stream=s)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    z = torch.cuda.Event(enable_timing=True)
    a.record(s)
    for _ in range(args.steps):
        plan.run(stream=s)
    z.record(s)
    torch.cuda.synchronize()
    ms = a.elapsed_time(z) / args.steps
    if plan.status(stream=s) != sp.SPECTRA_OK:
        print(json.dumps({"error": "a wait inside the decode step gave up; the run is invalid"}))
        sys.exit(3)
    value = step_bytes / (ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(value, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(value / PEAK_HBM_GBS, 4), "traffic": None,
                "kernel": "k_step (the whole step is one launch)", "avg_launch_us": round(ms * 1e3, 3),
                "bytes_per_launch": int(step_bytes), "launches_timed": args.steps}
    try:
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
        ent = tr.get("entries", {}).get(f"{args.workload}:M1:step")
        if ent and ent.get("source_sha") == kernel_sources_sha(STEP_SOURCES):
            roofline["traffic"] = int(ent["hbm_bytes_per_launch"])
    except (OSError, ValueError):
        pass
    plan.close()
    return ms, value, step_bytes, len(phases), roofline


_CAPTURE_STREAM = None


def capture(torch, fns):
    """Capture fns into a graph on one fixed side stream; an eager pass on the
    same stream first lets the library size its per-stream workspace outside
    capture."""
    global _CAPTURE_STREAM
    if _CAPTURE_STREAM is None:
        _CAPTURE_STREAM = torch.cuda.Stream()
    s = _CAPTURE_STREAM
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns:
            f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps):
    s = torch.cuda.current_stream()
    a = torch.cuda.Event(enable_timing=True)
    z = torch.cuda.Event(enable_timing=True)
    a.record(s)
    for _ in range(reps):
        g.replay()
    z.record(s)
    torch.cuda.synchronize()
    return a.elapsed_time(z) / reps  # ms


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _median(v):
    v = sorted(v)
    return v[len(v) // 2]


def cpu_baseline(cases, gemm_rounds=2):
    """The oracle as it stands, on a bounded sample: for each linear of the
    sample (name, W, gamma, x, algorithmic bytes) the oracle's pack (kurtosis
    split, G32 quantization, container image) once, then its product (unpack
    + float64 x W_hat^T) `gemm_rounds` times with every BLAS thread and once
    with one thread.  value = product GB/s on the algorithmic bytes (median
    round, all threads)."""
    from oracle import spectra_oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    blas = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    t_pack, w_bytes, imgs = 0.0, 0, []
    for name, W, g, x, nbytes in cases:
        t0 = time.perf_counter()
        imgs.append(O.pack(W, g))
        t_pack += time.perf_counter() - t0
        w_bytes += W.nbytes
    total = sum(c[4] for c in cases)

    def gemm_pass():
        t0 = time.perf_counter()
        for (name, W, g, x, nbytes), img in zip(cases, imgs):
            O.matmul_ref(O.unpack(img)["W_hat"], x)
        return time.perf_counter() - t0
    t_all = _median([gemm_pass() for _ in range(gemm_rounds)])
    with threadpool_limits(limits=1):
        t_one = gemm_pass()
    names = ", ".join(c[0] for c in cases)
    return {"value": round(total / t_all / 1e9, 4), "unit": "GB/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"oracle on {len(cases)} linear(s) ({names}): pack (kurtosis split, G32 quantization, "
                      f"image) once, then unpack + float64 product, {total / 1e6:.1f} MB algorithmic per pass; "
                      f"value = product pass, median of {gemm_rounds}, all BLAS threads",
            "cpu_model": _cpu_model(), "blas_threads": int(blas),
            "gemm_s_per_pass": round(t_all, 3), "gemm_s_per_pass_1thread": round(t_one, 3),
            "value_1thread": round(total / t_one / 1e9, 4),
            "pack_s": round(t_pack, 3), "pack_GBps_fp16_weights": round(w_bytes / t_pack / 1e9, 4)}


def cpu_baseline_for(args, sp, cfg):
    """The baseline's sample: the first layer's seven linears (cfg2, cfg3) or
    the one linear, with the workload's inputs."""
    from dequant_gemv_spectra_amd import synth
    wl = synth.workload(cfg, layers=1 if cfg == 3 else None)
    cases = []
    for lin in (wl.linears[:7] if cfg in (2, 3) else wl.linears[:1]):
        W, g = synth.weights(lin, cfg), synth.gamma(lin, cfg)
        x = synth.activations(lin, cfg, args.M)
        c = sp.spectra_pack(W, g)
        info = c.info()
        c.close()
        nbytes = info["bytes_payload"] + info["bytes_meta"] + 2 * args.M * (lin.K + lin.N)
        cases.append((lin.name, W, g, x, nbytes))
    return cpu_baseline(cases)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the dequant-GEMV path runs on one GPU; multi-GPU runs are not "
                                   "part of this benchmark (use --gpus 1)"}))
        sys.exit(2)
    import numpy as np
    import torch
    from dequant_gemv_spectra_amd import spectra as sp
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    sp.lib()  # fails loudly when the HIP library is missing
    torch.cuda.set_device(0)
    if args.calibrate_copy:  # plain copies of known size, for counter scale factors
        a = torch.empty(2 ** 29, dtype=torch.float16, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": a.numel() * 2, "written": b.numel() * 2, "copies": 5}))
        return
    if args.workload == "embed":
        run_embed(args, sp, torch)
        return
    if args.workload == "load":
        run_load(args, sp, torch)
        return
    if args.workload == "kv":
        run_kv(args, sp, torch)
        return
    cfg = int(args.workload[3:])
    t0 = time.time()
    name, units, layered = build_units(args, sp, torch)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f}s, {len(units)} launches per pass")

    pass_bytes = sum(u[3] for u in units)
    if layered and args.M == 1 and args.mode == "step" and not args.eager:
        ms_per_step, value, bytes_per_step, nph, roofline = run_step(args, sp, torch, name, units)
        cpu = None if args.no_cpu_baseline else cpu_baseline_for(args, sp, cfg)
        out = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
               "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
               "scaling": "weak", "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
               "config": {"workload": name, "M": 1, "launches_per_step": 1, "phases_per_step": nph,
                          "bytes_per_step": int(bytes_per_step),
                          "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2), "mode": "step",
                          "kernel": "k_step", "parallelism": "single GPU"},
               "roofline": roofline, "cpu_baseline": cpu}
        print(json.dumps(out), flush=True)
        return
    if args.eager:  # counter runs: plain launches, no graphs, no timing claims
        for _ in range(max(1, args.steps)):
            for u in units:
                u[2]()
        torch.cuda.synchronize()
        print(json.dumps({"eager_passes": max(1, args.steps), "launches_per_pass": len(units),
                          "bytes_per_pass": int(pass_bytes)}))
        return
    graph = capture(torch, [u[2] for u in units])
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    if layered:  # one step = one pass over every layer
        ms_per_step = time_graph(torch, graph, args.steps)
        bytes_per_step = pass_bytes
        launches = len(units)
    else:        # one step = one linear; a replay launches every rotated copy once
        reps = max(1, args.steps // len(units))
        ms_per_step = time_graph(torch, graph, reps) / len(units)
        bytes_per_step = pass_bytes / len(units)
        launches = 1
    value = bytes_per_step / (ms_per_step * 1e-3) / 1e9

    # roofline of the dominant kernel kind
    kinds = {}
    for _, kind, f, b, plan in units:
        kinds.setdefault(kind, []).append((f, b, plan))
    dom = max(kinds, key=lambda k: sum(b for _, b, _ in kinds[k]))
    dgraph = capture(torch, [f for f, _, _ in kinds[dom]])
    dgraph.replay()
    dms = time_graph(torch, dgraph, 10) / len(kinds[dom])
    dbytes = sum(b for _, b, _ in kinds[dom]) / len(kinds[dom])
    achieved = dbytes / (dms * 1e-3) / 1e9
    kernel_name = kinds[dom][0][2]  # as the library reports it (spectra_gemm_plan)
    if kernel_name != "k_gemv_m1":
        kernel_name = "k_xbulk + " + kernel_name
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                "kernel": f"{kernel_name} ({dom} launches)", "avg_launch_us": round(dms * 1e3, 3),
                "bytes_per_launch": int(dbytes), "launches_timed": 10 * len(kinds[dom])}
    if args.M > 1:  # past the ridge point the contraction is bound by the matrix cores
        from dequant_gemv_spectra_amd import synth
        lins = synth.workload(cfg, layers=1 if cfg == 3 else None).linears
        per = {l.name.split(".")[-1]: 2.0 * args.M * l.N * l.K for l in lins}
        dflops = per.get(dom, per[lins[0].name.split(".")[-1]])
        if dflops / dbytes > PEAK_MFMA_F16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
            tf = dflops / (dms * 1e-3) / 1e12
            roofline.update({"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_MFMA_F16_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(tf / PEAK_MFMA_F16_TFLOPS, 4)})
        roofline["arith_intensity_flop_per_byte"] = round(dflops / dbytes, 1)
    try:
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
        key = f"{args.workload}:M{args.M}:{dom}"
        ent = tr.get("entries", {}).get(key)
        srcs = GEMV_SOURCES if kernel_name == "k_gemv_m1" else MFMA_SOURCES
        if ent and ent.get("source_sha") == kernel_sources_sha(srcs) and not args.warm:
            roofline["traffic"] = int(ent["hbm_bytes_per_launch"])
    except (OSError, ValueError):
        pass

    cpu = None if args.no_cpu_baseline else cpu_baseline_for(args, sp, cfg)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": name, "M": args.M, "launches_per_step": launches,
                   "bytes_per_step": int(bytes_per_step),
                   "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
                   "hip_graph": True, "mode": "graph" if layered else ("warm" if args.warm else "launches"),
                   "kernel": args.kernel,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
