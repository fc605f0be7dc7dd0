#!/usr/bin/env python3
"""Benchmark of the fused dequantise-and-multiply on one MI355X.

One step = one decode token through a Q4_0 SwiGLU FFN at batch 1 (the
Qwen2.5-0.5B FFN shape of the llamay pages: gate and up 4864x896, down
896x4864): quantise the 896-wide activation once, GEMV gate and up on it,
quantise the 4864-wide activation, GEMV down.  The three GEMVs are
independent here (down takes its own synthetic activation), so a step is one
grouped launch (qmv_launch_group) in which each GEMV quantises its activation
inside the kernel.  Inputs are seeded synthetic
weights/activations already resident in HBM; the weights are rotated over
copies totalling >= --rotate-mib so every step streams them from HBM rather
than from the 256 MB last-level cache.  Steps are replayed from a captured
HIP graph (the path is launch-bound at this size).

Prints ONE JSON line: metric/value (weight GB/s of the timed steps, wall
clock), the roofline of the dominant kernel (the GEMV; execution times from
HIP events on the stream it runs on), the CPU oracle timed on a bounded
sample of the same step, the metric's other halves (prefill GEMM TOPS at the
512-token Q4_0 FFN and the 8B-class Q4_K 14336x4096 shape, LM-head GEMV
GB/s; --no-extra leaves them out), and (with --suite) per-matrix GEMV/GEMM
figures for every workload shape.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--suite]

Counter collection helpers: --profile-steps N (eager steps only),
--profile-matrix WORKLOAD:INDEX:ROWS (one workload matrix, eagerly),
--copy-calib (a 256 MiB copy, the counters' byte calibration) and
--traffic-from DIR (turns their rocprofv3 --pmc output into
profiles/traffic.json).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, vendor figure
KERNEL_SRC = os.path.join(ROOT, "gguf_quantized_matvec_amd", "csrc", "qmv_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_src_sha() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def gemv_alg_bytes(fmt, N, K, B, g, fused=False) -> int:
    """Algorithmic bytes of one GEMV launch: weight blob + Q8_0 activation
    blocks (written, or read) + f32 output; a launch that quantises x itself
    also reads x (f32)."""
    return N * g.row_bytes(fmt, K) + B * (K // 32) * 34 + B * N * 4 + (B * K * 4 if fused else 0)


class GraphSteps:
    """`nsteps` calls of step(i) captured into one HIP graph."""

    def __init__(self, torch, step, nsteps):
        self.graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(self.graph, stream=s):
                for i in range(nsteps):
                    step(i, None)
        torch.cuda.current_stream().wait_stream(s)
        self.nsteps = nsteps

    def replay(self):
        self.graph.replay()


def graph_launch_us(torch, launch, n, reps=3):
    """Average time per launch of `n` back-to-back launches of one kernel
    (launch(i) enqueues launch i), captured into a HIP graph and replayed
    between two HIP events on the stream the kernels run on.  The figure is
    the kernel's execution time plus the short dispatch gap between
    consecutive graph nodes; the median over `reps` replays is returned."""
    G = GraphSteps(torch, lambda i, _: launch(i), n)
    G.replay()                               # warm
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    out = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        G.replay()
        e1.record(s)
        e1.synchronize()
        out.append(e0.elapsed_time(e1) * 1e3 / n)
    return sorted(out)[len(out) // 2]


def run_steps(graphs, make, n):
    """Replay graphs to run exactly n steps (graph sizes created on demand)."""
    full = graphs["full"]
    for _ in range(n // full.nsteps):
        full.replay()
    r = n % full.nsteps
    if r:
        if r not in graphs:
            graphs[r] = make(r)
        graphs[r].replay()


def ffn_workload(torch, g, synth, rotate_bytes):
    """The headline step's buffers: rotated weight copies, activations, outputs."""
    fmt = synth.Q4_0
    shapes = [("gate", 4864, 896), ("up", 4864, 896), ("down", 896, 4864)]
    blobs = {}
    for i, (name, N, K) in enumerate(shapes):
        blob, _ = synth.weights(fmt, N, K, synth.seed_for(1, i), dscale=0.02)
        blobs[name] = torch.from_numpy(blob).cuda()
    step_bytes = sum(int(b.numel()) for b in blobs.values())
    R = max(1, math.ceil(rotate_bytes / step_bytes))
    copies = {k: [v] + [v.clone() for _ in range(R - 1)] for k, v in blobs.items()}
    x1 = torch.from_numpy(synth.activations(1, 896, synth.act_seed_for(1, 1))).cuda()
    x2 = torch.from_numpy(synth.activations(1, 4864, synth.act_seed_for(1, 1) + 1)).cuda()
    xq1, xq2 = g.act_buffer(1, 896), g.act_buffer(1, 4864)
    ys = {n: torch.empty(1, N, dtype=torch.float32, device="cuda") for n, N, _ in shapes}
    return dict(fmt=fmt, shapes=shapes, copies=copies, R=R, x1=x1, x2=x2, xq1=xq1, xq2=xq2,
                ys=ys, step_bytes=step_bytes)


def make_ffn_step(torch, g, W):
    """One decode step = one grouped launch (qmv_launch_group) of the three
    GEMVs, each quantising its own activation inside the kernel; gate's and
    down's Q8_0 blocks are also written to their xq buffers."""
    L = g.lib()
    fmt = W["fmt"]
    R = W["R"]
    x1, x2 = W["x1"].data_ptr(), W["x2"].data_ptr()
    q1, q2 = W["xq1"].data_ptr(), W["xq2"].data_ptr()
    y = {k: v.data_ptr() for k, v in W["ys"].items()}
    groups = []
    for c in range(R):
        wp = {k: v[c].data_ptr() for k, v in W["copies"].items()}
        groups.append((g.Gemv * 3)(g.Gemv(wp["gate"], 4864, 896, x1, q1, y["gate"]),
                                   g.Gemv(wp["up"], 4864, 896, x1, None, y["up"]),
                                   g.Gemv(wp["down"], 896, 4864, x2, q2, y["down"])))

    def step(i, _unused=None):
        rc = L.qmv_launch_group(fmt, 1, groups[i % R], 3, torch.cuda.current_stream().cuda_stream)
        if rc:
            raise g.QmvError(rc, "qmv_launch_group")
    return step


def cpu_baseline(W, seconds):
    """The CPU oracle on the same step (both quantisations and the three
    products in f64), rows split over host threads, for ~`seconds`."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    import synth
    blobs = {k: v[0].cpu().numpy() for k, v in W["copies"].items()}
    x1, x2 = W["x1"].cpu().numpy(), W["x2"].cpu().numpy()
    fmt = W["fmt"]
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))
    rb = {n: synth.row_bytes(fmt, K) for n, _, K in W["shapes"]}

    def rows_job(name, N, K, xq, r0, r1):
        b = blobs[name][r0 * rb[name]: r1 * rb[name]]
        oracle.matmul_f64(fmt, b, r1 - r0, K, xq, 1, want_abs=False)

    oracle.lib()
    steps = 0
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(cores) as ex:
        while True:
            xq1 = oracle.quantize_act(x1)
            xq2 = oracle.quantize_act(x2)
            futs = []
            for name, N, K in W["shapes"]:
                xq = xq1 if K == 896 else xq2
                per = math.ceil(N / cores)
                for r0 in range(0, N, per):
                    futs.append(ex.submit(rows_job, name, N, K, xq, r0, min(N, r0 + per)))
            for f in futs:
                f.result()
            steps += 1
            if time.perf_counter() - t0 >= seconds:
                break
    dt = time.perf_counter() - t0
    return {"value": round(W["step_bytes"] * steps / dt / 1e9, 4), "unit": "GB/s",
            "cores": cores, "kind": "oracle",
            "sample": f"{steps} steps of the Q4_0 FFN decode step (quantise both activations, "
                      f"gate/up/down products in f64), rows split over {cores} threads, "
                      f"{dt:.1f} s; tok/s {steps / dt:.2f}"}


def suite(torch, g, synth, rotate_bytes, only=None):
    """Per-matrix figures for every workload shape: GEMV at each decode batch
    (weight GB/s) and GEMM at each prefill size (int8-equivalent TOPS), from
    the time per launch of back-to-back graph launches over rotated copies.
    only: a set of (workload, matrix index, rows) to restrict it to."""
    res = []
    L = g.lib()
    for wl, spec in synth.WORKLOADS.items():
        ci = list(synth.WORKLOADS).index(wl)
        for mi, (fmt, N, K, ds) in enumerate(spec["mats"]):
            batches = [B for B in spec["batches"] if only is None or (wl, mi, B) in only]
            if not batches:
                continue
            blob, _ = synth.weights(fmt, N, K, synth.seed_for(ci, mi), dscale=ds)
            wt = torch.from_numpy(blob).cuda()
            nbytes = int(wt.numel())
            R = max(1, min(64, math.ceil(rotate_bytes / nbytes)))
            copies = [wt] + [wt.clone() for _ in range(R - 1)]
            for B in batches:
                x = torch.from_numpy(synth.activations(B, K, synth.act_seed_for(ci, B))).cuda()
                xq = g.quantize(x)
                y = torch.empty(B, N, dtype=torch.float32, device="cuda")
                fn = L.qmv_launch if B <= 16 else L.qmm_launch

                def launch(i, fn=fn, B=B, xq=xq, y=y):
                    rc = fn(fmt, copies[i % R].data_ptr(), N, K, None, B, xq.data_ptr(),
                            y.data_ptr(), torch.cuda.current_stream().cuda_stream)
                    if rc:
                        raise g.QmvError(rc, "suite")
                launch(0)
                n = max(R, 20) if B <= 16 else max(min(R, 10), 5)
                med = graph_launch_us(torch, launch, n) * 1e-6
                row = {"workload": wl, "fmt": synth.NAMES[fmt], "N": N, "K": K, "rows": B,
                       "us": round(med * 1e6, 2), "weight_MB": round(nbytes / 1e6, 2)}
                if B <= 16:
                    gbs = nbytes / med / 1e9
                    row.update(weight_GBs=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
                               tok_s=round(B / med, 1))
                else:
                    tops = 2.0 * B * N * K / med / 1e12
                    row.update(int8_TOPS=round(tops, 1), mfma_frac=round(tops / INT8_PEAK_TOPS, 4))
                res.append(row)
                print(json.dumps({"suite_row": row}), file=sys.stderr, flush=True)
                del x, xq, y
            del copies, wt
            torch.cuda.empty_cache()
    return res


def other_halves(torch, g, synth):
    """The metric's other figures beside the headline decode step: the prefill
    GEMM (int8-equivalent TOPS) at the pages' 512-token prompt (Q4_0 gate/up
    and down) and at the 8B-class 2048-token shape (Q4_K 14336x4096), and the
    largest decode GEMV (the Q6_K 151936x1024 LM head, batch 1)."""
    rows = suite(torch, g, synth, 512 << 20,
                 only={("q4_0_prefill512", 0, 512), ("q4_0_prefill512", 1, 512),
                       ("8b_class", 2, 2048), ("kquant_lmhead", 0, 1)})
    by = {(r["workload"], r["N"], r["K"], r["rows"]): r for r in rows}
    gate, down = by[("q4_0_prefill512", 4864, 896, 512)], by[("q4_0_prefill512", 896, 4864, 512)]
    big = by[("8b_class", 14336, 4096, 2048)]
    lm = by[("kquant_lmhead", 151936, 1024, 1)]
    ops512 = 2.0 * 512 * 4864 * 896 * 2
    tops512 = ops512 / ((gate["us"] + down["us"]) * 1e-6) / 1e12
    return {
        "prefill": {
            "unit": "int8-equivalent TOPS", "peak": INT8_PEAK_TOPS,
            "q4_0_ffn_m512": {"TOPS": round(tops512, 1), "frac": round(tops512 / INT8_PEAK_TOPS, 4),
                              "us_gate_4864x896": gate["us"], "us_down_896x4864": down["us"]},
            "q4_k_14336x4096_m2048": {"TOPS": big["int8_TOPS"], "frac": big["mfma_frac"],
                                      "us": big["us"]},
            "timing": "HIP events around graph replays of back-to-back launches",
        },
        "lm_head": {"matrix": "Q6_K 151936x1024, batch 1", "weight_GBs": lm["weight_GBs"],
                    "frac": lm["hbm_frac"], "us": lm["us"]},
    }


def profile_matrix(torch, g, synth, spec, launches=20):
    """Launch one workload matrix (the suite's seeded weights, activations
    staged by quantize_act_q8_0) `launches` times back to back, eagerly."""
    wl, mi, rows = spec.split(":")
    mi, rows = int(mi), int(rows)
    ci = list(synth.WORKLOADS).index(wl)
    fmt, N, K, ds = synth.WORKLOADS[wl]["mats"][mi]
    blob, _ = synth.weights(fmt, N, K, synth.seed_for(ci, mi), dscale=ds)
    w = torch.from_numpy(blob).cuda()
    x = torch.from_numpy(synth.activations(rows, K, synth.act_seed_for(ci, rows))).cuda()
    xq = g.quantize(x)
    y = torch.empty(rows, N, dtype=torch.float32, device="cuda")
    L = g.lib()
    fn = L.qmv_launch if rows <= 16 else L.qmm_launch
    for _ in range(launches):
        rc = fn(fmt, w.data_ptr(), N, K, None, rows, xq.data_ptr(), y.data_ptr(),
                torch.cuda.current_stream().cuda_stream)
        if rc:
            raise g.QmvError(rc, "profile_matrix")
    torch.cuda.synchronize()
    print(json.dumps({"profile_matrix": spec, "fmt": synth.NAMES[fmt], "N": N, "K": K,
                      "rows": rows, "launches": launches}))


def traffic_from(pmc_dir):
    """profiles/traffic.json from four rocprofv3 --pmc runs under pmc_dir:
    fetch/ and write/ (FETCH_SIZE, WRITE_SIZE of `bench.py --profile-steps`),
    calib_fetch/ and calib_write/ (the same counters of `bench.py --copy-calib`).
    Each counter is scaled by true bytes / counted bytes of the plain copy."""
    import csv
    import glob

    def rows(sub, counter):
        out = []
        for f in glob.glob(os.path.join(pmc_dir, sub, "**", "*counter_collection.csv"),
                           recursive=True):
            for r in csv.DictReader(open(f)):
                if r.get("Counter_Name") == counter:
                    out.append((r["Kernel_Name"], float(r["Counter_Value"])))
        if not out:
            raise SystemExit(f"no {counter} rows under {os.path.join(pmc_dir, sub)}")
        return out

    def copy_kib(sub, counter):
        # the largest dispatch of the calibration run is the 256 MiB copy
        return max(v for _, v in rows(sub, counter))

    copy_bytes = 256 << 20
    f_scale = copy_bytes / (copy_kib("calib_fetch", "FETCH_SIZE") * 1024)
    w_scale = copy_bytes / (copy_kib("calib_write", "WRITE_SIZE") * 1024)
    fk = [v for k, v in rows("fetch", "FETCH_SIZE") if "k_dot" in k]
    wk = [v for k, v in rows("write", "WRITE_SIZE") if "k_dot" in k]
    fetch = sum(fk) / len(fk) * 1024 * f_scale
    write = sum(wk) / len(wk) * 1024 * w_scale
    out = {"kernel": "k_dot (grouped GEMV gate+up+down, Q4_0, batch 1)", "kernel_src_sha": kernel_src_sha(),
           "dispatches": [len(fk), len(wk)],
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
           "bytes_per_launch": round(fetch + write)}
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--rotate-mib", type=int, default=1024)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="leave out the prefill GEMM and LM-head figures")
    ap.add_argument("--suite", action="store_true",
                    help="also report every workload matrix (GEMV and GEMM) separately")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="only run this many eager steps (for counter collection)")
    ap.add_argument("--traffic-from", default=None,
                    help="write profiles/traffic.json from rocprofv3 --pmc output under DIR")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a 256 MiB device copy 10 times (counter calibration)")
    ap.add_argument("--profile-matrix", default=None, metavar="WORKLOAD:INDEX:ROWS",
                    help="only launch one workload matrix (e.g. 8b_class:2:2048) 20 times, "
                         "eagerly (for counter collection)")
    args = ap.parse_args()

    if args.traffic_from:
        traffic_from(args.traffic_from)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); the multiply shards by weight rows with no cross-GPU "
              f"reduction, so per-GPU throughput is the single-GPU figure", file=sys.stderr)
        sys.exit(2)

    import torch

    import gguf_quantized_matvec_amd as g
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    g.lib()

    if args.copy_calib:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": a.numel(), "launches": 10}))
        return

    if args.profile_matrix:
        profile_matrix(torch, g, synth, args.profile_matrix)
        return

    W = ffn_workload(torch, g, synth, args.rotate_mib << 20)
    step = make_ffn_step(torch, g, W)
    step(0, None)                       # eager run: device check, lazy init
    torch.cuda.synchronize()
    if args.profile_steps:
        for i in range(args.profile_steps):
            step(i, None)
        torch.cuda.synchronize()
        print(json.dumps({"profile_steps": args.profile_steps}))
        return

    graphs = {}

    def make(n):
        return GraphSteps(torch, step, n)

    graphs["full"] = make(W["R"])
    # capture the partial-replay graphs too before anything is timed
    for n in (args.warmup, args.steps):
        r = n % W["R"]
        if r and r not in graphs:
            graphs[r] = make(r)
    run_steps(graphs, make, args.warmup)
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    run_steps(graphs, make, args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0

    # the dominant (only) kernel: time per launch of the grouped GEMV, back to
    # back over every rotated copy
    per_launch_us = graph_launch_us(torch, lambda i: step(i), W["R"])
    # every GEMV reads its x; gate and down write their Q8_0 blocks, up does not
    alg = {"gate": gemv_alg_bytes(W["fmt"], 4864, 896, 1, g, fused=True),
           "up": gemv_alg_bytes(W["fmt"], 4864, 896, 1, g, fused=True) - (896 // 32) * 34,
           "down": gemv_alg_bytes(W["fmt"], 896, 4864, 1, g, fused=True)}
    alg_per_launch = alg["gate"] + alg["up"] + alg["down"]
    achieved = alg_per_launch / (per_launch_us * 1e-6) / 1e9

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tf = json.load(open(TRAFFIC_FILE))
        if tf.get("kernel_src_sha") == kernel_src_sha():
            traffic = tf.get("bytes_per_launch")

    value = W["step_bytes"] * args.steps / wall / 1e9
    out = {
        "metric": "decode GEMV weight-GB/s (% HBM peak); prefill int8 GEMM TOPS (% MFMA peak)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded GGUF Q4_0 blocks and N(0,1) activations)",
        "config": {"workload": "Q4_0 SwiGLU FFN decode, batch 1: gate+up 4864x896, down 896x4864 "
                               "(llamay Qwen2.5-0.5B shapes)",
                   "global_batch": 1, "weights_per_step_bytes": W["step_bytes"],
                   "rotated_copies": W["R"], "graph_replay": True,
                   "tok_s": round(args.steps / wall, 1),
                   "hbm_frac_of_value": round(value / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "k_dot<Q4_0, 1, fused> (grouped GEMV: gate, up, down)",
                     "avg_launch_us": round(per_launch_us, 3),
                     "launches_timed": W["R"],
                     "timing": "HIP events on the launch stream around a graph replay of the "
                               "step's grouped launch back to back over every rotated copy; "
                               "time per launch includes the inter-node dispatch gap",
                     "alg_bytes_per_launch": alg},
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(W, args.cpu_seconds)
    if not args.no_extra:
        del graphs
        W.clear()
        torch.cuda.empty_cache()
        graphs = None
        out.update(other_halves(torch, g, synth))
    if args.suite:
        graphs = None
        W.clear()
        torch.cuda.empty_cache()
        out["suite"] = suite(torch, g, synth, 512 << 20)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
