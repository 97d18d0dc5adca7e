#!/usr/bin/env python3
"""SPECTRA dequant-GEMV benchmark on one MI355X: effective HBM GB/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload cfg3]

Default workload (cfg3): the decode step of a 4B-class decoder -- 36 layers x
7 linears (q/k/v/o/gate/up/down, hidden 2560, MLP 9728), M = 1, every layer's
weights distinct, so one step streams about 2.2 GB of packed weights from HBM.
Same-input projections run as one grouped launch (q/k/v, gate/up): 4 launches
per layer.  One step = one pass over all 36 layers.  Inputs (containers and
x) are resident in HBM before the timed region.

value = algorithmic bytes per step / step time, where a linear's algorithmic
bytes are its container payload (codes + scales + zero nibbles + fp16
heavy-tailed columns) + metadata (header, mask, perm) + x + y, each counted
once.  Prints ONE JSON line.

Other workloads (--workload cfg1|cfg2|cfg4|cfg5, --M m) measure one linear (or
one decoder layer) rotated over enough distinct copies to exceed 1 GiB so the
last-level cache cannot serve the weights.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "dequant-GEMV effective HBM GB/s and % of peak at M=1; weights-GB/s vs M"
PEAK_HBM_GBS = 8000.0  # MI355X published HBM3E bandwidth


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="cfg3", choices=["cfg1", "cfg2", "cfg3", "cfg4", "cfg5"])
    ap.add_argument("--M", type=int, default=1)
    ap.add_argument("--kernel", default="auto", choices=["auto", "gemv", "mfma"])
    ap.add_argument("--layers", type=int, default=None, help="cfg3 only: fewer layers (smoke runs)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a hipGraph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Linear:
    """One packed linear with its resident x and y."""

    def __init__(self, sp, torch, lin, cfg, M, copy=0):
        from dequant_gemv_spectra_amd import synth
        W = synth.weights(lin, cfg)
        g = synth.gamma(lin, cfg)
        self.c = sp.spectra_pack(W, g)
        self.info = self.c.info()
        self.lin = lin
        self.x = torch.from_numpy(synth.activations(lin, cfg, M, salt=copy)).cuda()
        self.y = torch.empty((M, lin.N), dtype=torch.float16, device="cuda")
        self.M = M
        self.bytes = (self.info["bytes_payload"] + self.info["bytes_meta"] + 2 * M * lin.K + 2 * M * lin.N)


def build_units(args, sp, torch):
    """Launch units of one step: list of (label, callable, bytes)."""
    from dequant_gemv_spectra_amd import synth
    cfg = int(args.workload[3:])
    wl = synth.workload(cfg, layers=args.layers if cfg == 3 else None)
    M = args.M
    kern = args.kernel
    units = []
    if cfg in (2, 3):
        by_layer = {}
        for lin in wl.linears:
            by_layer.setdefault(lin.layer, []).append(lin)
        # the 1.5B-class layer (~28 MB) is stacked 28 deep, the depth of that model
        depth = 28 if cfg == 2 else 1
        for layer in sorted(by_layer):
            for cp in range(depth):
                t0 = time.time()
                packed = [Linear(sp, torch, lin, cfg, M, copy=cp) for lin in by_layer[layer]]
                tag = f"L{layer}" if depth == 1 else f"L{cp}"
                units.extend(layer_units(sp, packed, M, kern, tag))
                if layer % 6 == 0 or depth > 1 and cp % 7 == 0:
                    log(f"{tag}: packed {len(packed)} linears in {time.time() - t0:.1f}s")
        if cfg == 2:
            wl.name = "decoder-1.5B-28-layers"
        return wl, units
    # single linear: rotate distinct copies past the last-level cache
    lin = wl.linears[0]
    first = Linear(sp, torch, lin, cfg, M)
    copies = max(1, int(args.rotate_gib * 2 ** 30 // first.bytes) + 1)
    packed = [first] + [Linear(sp, torch, lin, cfg, M, copy=cp) for cp in range(1, copies)]
    log(f"{wl.name}: {copies} distinct copies, {first.bytes / 1e6:.1f} MB each")
    for i, p in enumerate(packed):
        units.append((f"{lin.name}#{i}", gemm_call(sp, p, kern), p.bytes))
    return wl, units


def gemm_call(sp, p, kern):
    def f():
        sp.spectra_gemm(p.c, p.x, p.y, kernel=kern)
    return f


def layer_units(sp, packed, M, kern, tag):
    by = {p.lin.name.split(".")[-1]: p for p in packed}
    units = []
    if M == 1 and kern in ("auto", "gemv"):
        qkv = [by["q"], by["k"], by["v"]]
        gu = [by["gate"], by["up"]]

        def grouped(ps):
            cs = [p.c for p in ps]
            ys = [p.y for p in ps]
            x = ps[0].x

            def f():
                sp.spectra_gemm_grouped(cs, x, ys)
            return f
        units.append((f"{tag}.qkv", grouped(qkv), sum(p.bytes for p in qkv) - 2 * 2 * qkv[0].lin.K))
        units.append((f"{tag}.o", gemm_call(sp, by["o"], kern), by["o"].bytes))
        units.append((f"{tag}.gate_up", grouped(gu), sum(p.bytes for p in gu) - 2 * gu[0].lin.K))
        units.append((f"{tag}.down", gemm_call(sp, by["down"], kern), by["down"].bytes))
    else:
        for nm in ("q", "k", "v", "o", "gate", "up", "down"):
            units.append((f"{tag}.{nm}", gemm_call(sp, by[nm], kern), by[nm].bytes))
    return units


def cpu_baseline(wl, units_meta, budget_s=20.0):
    """The oracle's product (unpack + float64 x W_hat^T) on a bounded sample."""
    import numpy as np
    from oracle import spectra_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    except Exception:
        blas = 1
    done_bytes = 0
    t_total = 0.0
    names = []
    for name, img, x, nbytes in units_meta:
        t0 = time.perf_counter()
        W_hat = O.unpack(img)["W_hat"]
        O.matmul_ref(W_hat, x)
        t_total += time.perf_counter() - t0
        done_bytes += nbytes
        names.append(name)
        if t_total > budget_s:
            break
    return {"value": round(done_bytes / t_total / 1e9, 4), "unit": "GB/s", "cores": int(blas),
            "kind": "oracle",
            "sample": f"oracle unpack + float64 product of {len(names)} linears "
                      f"({', '.join(names)}), {done_bytes / 1e6:.1f} MB algorithmic, {t_total:.1f} s; "
                      f"cores = BLAS threads of the product (unpack is single-threaded numpy)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the dequant-GEMV path "
                                   "has no multi-GPU mode (--gpus 1)"}))
        sys.exit(2)
    import numpy as np
    import torch
    from dequant_gemv_spectra_amd import spectra as sp
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    sp.lib()
    torch.cuda.set_device(0)
    t0 = time.time()
    wl, units = build_units(args, sp, torch)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f}s, {len(units)} launches per step")
    cfg = int(args.workload[3:])
    bytes_per_step = sum(b for _, _, b in units) if cfg in (2, 3) else None

    def run_step(i):
        if cfg in (2, 3):
            for _, f, _ in units:
                f()
        else:
            units[i % len(units)][1]()

    stream = torch.cuda.current_stream()
    use_graph = (cfg in (2, 3)) and not args.no_graph
    graph = None
    if use_graph:
        run_step(0)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_step(0)
        torch.cuda.synchronize()

    def step(i):
        if graph is not None:
            graph.replay()
        else:
            run_step(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / args.steps
    if cfg in (1, 4, 5):
        bytes_per_step = units[0][2]
    value = bytes_per_step / (ms_per_step * 1e-3) / 1e9

    # Roofline of the dominant kernel: per-launch HIP events (on the launch
    # stream) around each launch of the largest launch unit kind, eager.
    if cfg in (2, 3):
        kinds = {}
        for lab, f, b in units:
            kinds.setdefault(lab.split(".")[-1], []).append((f, b))
        dom = max(kinds, key=lambda k: sum(b for _, b in kinds[k]))
        dom_units = kinds[dom]
    else:
        dom = wl.linears[0].name
        dom_units = [(f, b) for _, f, b in units]
    durs = []
    nb = []
    reps = max(1, min(args.steps, 10))
    evs = []
    for r in range(reps):
        for f, b in dom_units:
            a = torch.cuda.Event(enable_timing=True)
            z = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            f()
            z.record(stream)
            evs.append((a, z, b))
    torch.cuda.synchronize()
    for a, z, b in evs:
        durs.append(a.elapsed_time(z))
        nb.append(b)
    avg_ms = float(np.mean(durs))
    avg_bytes = float(np.mean(nb))
    achieved = avg_bytes / (avg_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                "kernel": dom, "avg_launch_us": round(avg_ms * 1e3, 2),
                "bytes_per_launch": int(avg_bytes), "launches_timed": len(durs)}

    cpu = None
    if not args.no_cpu_baseline:
        from dequant_gemv_spectra_amd import synth
        sample = wl.linears[:7] if cfg in (2, 3) else wl.linears[:1]
        meta = []
        for lin in sample:
            c = sp.spectra_pack(synth.weights(lin, cfg), synth.gamma(lin, cfg))
            info = c.info()
            nbytes = info["bytes_payload"] + info["bytes_meta"] + 2 * args.M * (lin.K + lin.N)
            meta.append((lin.name, sp.spectra_export(c), synth.activations(lin, cfg, args.M), nbytes))
            c.close()
        cpu = cpu_baseline(wl, meta)

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
        "config": {"workload": wl.name, "M": args.M, "linears": len(wl.linears),
                   "launches_per_step": len(units) if cfg in (2, 3) else 1,
                   "bytes_per_step": int(bytes_per_step),
                   "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
                   "graph": graph is not None, "kernel": args.kernel,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
