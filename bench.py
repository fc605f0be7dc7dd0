#!/usr/bin/env python3
"""Benchmark of the fused dequantise-and-multiply on one MI355X.

Headline step: one decoder layer of an 8B-class model in decode at batch 1,
built from the four 8B-class weight shapes (Q4_K 4096x4096, 1024x4096,
14336x4096, Q6_K 4096x14336) in the order a model runs them:

  A  q 4096x4096, k and v 1024x4096 on one activation (one grouped launch)
  B  o 4096x4096 on the attention output (a synthetic activation here)
  C  gate and up 14336x4096 on one activation, with the SwiGLU
     h = silu(gate) * up and the Q8_0 quantisation of h in the same launch
     (qmv_launch_gateup_swiglu_q8)
  D  down 4096x14336 (Q6_K) on the quantised h

A, B and C quantise their own activation to Q8_0 inside the GEMV; the
quantisation of h follows C's kernel as a launch of its own (at K = 4096 the
paired launch does not take it in: see qmv_launch_gateup_swiglu_q8).  Attention, norms and residuals are not part of the multiply and are
not run.  A step is replayed from a captured HIP graph; the weights are
rotated over copies totalling >= --rotate-mib, so every step streams them
from HBM rather than from the 256 MB last-level cache.  value = weight bytes
of the step / wall-clock time of the timed steps.

The same JSON line also carries: the roofline of the step's dominant kernel
(HIP-event time per launch on the stream it runs on), the layer step at batch
16, the prefill GEMMs of the four shapes at 2048 tokens (int8-equivalent
TOPS; Q8_0 activations on f16 MFMA, and Q8_K activations on int8 MFMA), the
four matrices as Q8_K-path GEMVs at batch 1 and 16, the LM-head GEMV (Q6_K 151936x1024) at batch 1/4/16, the pages' own
Qwen2.5-0.5B shapes (Q8_0 896x896, the Q4_0 SwiGLU FFN at batch 1, the Q4_0
prefill at 512 tokens), the measured ceilings of the chip (a streaming read,
int8 and f16 MFMA loops, the GEMM's f32 epilogue alone) and the CPU oracle
timed on the host's cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--suite] [--no-cpu]

Counter / trace helpers: --profile-stage NAME (eager launches of one stage),
--profile-matrix WORKLOAD:INDEX:ROWS, --copy-calib (a 256 MiB copy, the
counters' byte calibration), --traffic-from DIR (profiles/traffic.json from
rocprofv3 --pmc output) and --trace-summary DIR (per-kernel, per-grid
durations from a rocprofv3 kernel trace).
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
F16_PEAK_TFLOPS = 2500.0       # MI355X dense f16 MFMA, vendor figure
CSRC = os.path.join(ROOT, "gguf_quantized_matvec_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
MAX_HOST_THREADS = 16          # one GPU's share of the host CPUs (16 per GPU)

Q4_0, Q8_0, Q4_K, Q6_K = 2, 8, 12, 14
# (name, fmt, N, K) of one 8B-class decoder layer's projections
LAYER = [("q", Q4_K, 4096, 4096), ("k", Q4_K, 1024, 4096), ("v", Q4_K, 1024, 4096),
         ("o", Q4_K, 4096, 4096), ("gate", Q4_K, 14336, 4096), ("up", Q4_K, 14336, 4096),
         ("down", Q6_K, 4096, 14336)]
STAGES = {"A_qkv": ("q", "k", "v"), "B_o": ("o",), "C_gateup_swiglu": ("gate", "up"),
          "D_down": ("down",)}
# the multiply kernel of each stage at batch 1 (its rocprofv3 name: format,
# rows, fused quantisation, mode, Q8_K activations, lean loads): A, B and C
# quantise their activation inside the kernel; at K = 4096 the quantisation of
# h for D is a launch of its own after C's kernel; D reads it
STAGE_KERNEL = {"A_qkv": "k_dot<12, 1, true, 0, false, true>",
                "B_o": "k_dot<12, 1, true, 1, false, true>",
                "C_gateup_swiglu": "k_dot<12, 1, true, 2, false, true>",
                "D_down": "k_dot<14, 1, false, 1, false, false>"}
STAGE_KERNEL_WHAT = {"A_qkv": "grouped GEMV q, k, v (Q4_K)", "B_o": "GEMV o (Q4_K)",
                     "C_gateup_swiglu": "paired GEMV gate/up with the SwiGLU epilogue (Q4_K)",
                     "D_down": "GEMV down (Q6_K 4096x14336)"}


def kernel_src_sha() -> str:
    h = hashlib.sha256()
    for f in ("qmv_kernels.hip", "qmm_kernels.hip", "qmv_internal.h"):
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def row_bytes(fmt, K):
    qk, nb = {Q4_0: (32, 18), Q8_0: (32, 34), Q4_K: (256, 144), Q6_K: (256, 210)}[fmt]
    return K // qk * nb


class GraphSteps:
    """`nsteps` calls of step(i) captured into one HIP graph."""

    def __init__(self, torch, step, nsteps):
        self.graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(self.graph, stream=s):
                for i in range(nsteps):
                    step(i)
        torch.cuda.current_stream().wait_stream(s)
        self.nsteps = nsteps

    def replay(self):
        self.graph.replay()


def graph_launch_us(torch, launch, n, reps=3):
    """Average time per launch of `n` back-to-back launches (launch(i)
    enqueues launch i), captured into a HIP graph and replayed between two
    HIP events on the stream the kernels run on.  The figure is the kernel's
    execution time plus the short dispatch gap between consecutive graph
    nodes; the median over `reps` replays is returned."""
    G = GraphSteps(torch, launch, n)
    # warm: replays for at least 30 ms (the first milliseconds of a long
    # run are measurably slower than the rest)
    t0 = time.perf_counter()
    while True:
        G.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= 0.03:
            break
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


_WEIGHTS = {}


def weights(synth, fmt, N, K, seed, ds):
    """Seeded weight blob (generated once per process)."""
    key = (fmt, N, K, seed, ds)
    if key not in _WEIGHTS:
        _WEIGHTS[key] = synth.weights(fmt, N, K, seed, dscale=ds)[0]
    return _WEIGHTS[key]


def _check(g, rc, what):
    if rc:
        raise g.QmvError(rc, what)


# ------------------------------------------------------------ layer step --

class Layer:
    """Buffers of the 8B-class layer step at batch B: rotated weight copies,
    the stage activations, scratch and outputs."""

    def __init__(self, torch, g, synth, B, rotate_bytes, q8k=False):
        self.B = B
        self.q8k = q8k
        self.torch, self.g = torch, g
        blobs = {}
        for i, (name, fmt, N, K) in enumerate(LAYER):
            blob = weights(synth, fmt, N, K, synth.seed_for(4, 10 + i), 0.02)
            blobs[name] = torch.from_numpy(blob).cuda()
        self.step_bytes = sum(int(b.numel()) for b in blobs.values())
        self.R = max(1, math.ceil(rotate_bytes / self.step_bytes))
        self.w = {k: [v] + [v.clone() for _ in range(self.R - 1)] for k, v in blobs.items()}
        act = lambda K, j: torch.from_numpy(synth.activations(B, K, synth.act_seed_for(4, B) + j)).cuda()
        self.xa, self.xo, self.xc = act(4096, 0), act(4096, 1), act(4096, 2)
        if q8k:
            qb = lambda K: torch.empty(g.qmv_act_bytes_q8k(B, K), dtype=torch.uint8, device="cuda")
            self.xq_a, self.xq_o, self.xq_c, self.xq_d = qb(4096), qb(4096), qb(4096), qb(14336)
        else:
            self.xq_a = g.act_buffer(B, 4096)
            self.xq_o = g.act_buffer(B, 4096)
            self.xq_c = torch.empty(g.qmv_gateup_act_bytes(B, 14336, 4096), dtype=torch.uint8,
                                    device="cuda")
            self.xq_d = g.act_buffer(B, 14336)
        self.h = torch.empty(B, 14336, dtype=torch.float32, device="cuda")
        self.y = {n: torch.empty(B, N, dtype=torch.float32, device="cuda")
                  for n, _, N, _ in LAYER if n not in ("gate", "up")}
        self._groups = []
        self._groups_k = []  # the Q8_K path's q, k, v on one staged xq
        for c in range(self.R):
            P = lambda n: self.w[n][c].data_ptr()
            self._groups_k.append((g.Gemv * 3)(
                *[g.Gemv(P(n), N, 4096, None, self.xq_a.data_ptr(), self.y[n].data_ptr())
                  for n, N in (("q", 4096), ("k", 1024), ("v", 1024))]))
            fused = B <= 4
            xa = self.xa.data_ptr() if fused else None
            xq_k = None if fused else self.xq_a.data_ptr()
            self._groups.append((g.Gemv * 3)(
                g.Gemv(P("q"), 4096, 4096, xa, self.xq_a.data_ptr(), self.y["q"].data_ptr()),
                g.Gemv(P("k"), 1024, 4096, xa, xq_k, self.y["k"].data_ptr()),
                g.Gemv(P("v"), 1024, 4096, xa, xq_k, self.y["v"].data_ptr())))

    def kernel(self, name, c):
        """Enqueue the multiply kernel of stage `name` alone: the stage itself
        for A, B and D (one kernel each at batch <= 4); for C the paired
        gate/up GEMV without the quantisation of h that follows it."""
        if name != "C_gateup_swiglu":
            self.stage(name, c)
            return
        g = self.g
        s = self.torch.cuda.current_stream().cuda_stream
        _check(g, g.lib().qmv_launch_gateup_swiglu(
            Q4_K, self.w["gate"][c].data_ptr(), self.w["up"][c].data_ptr(), 14336, 4096,
            self.xc.data_ptr(), self.B, self.xq_c.data_ptr(), self.h.data_ptr(), s), "gate/up")

    def kernel_alg_bytes(self, name):
        """Algorithmic bytes of one kernel(): as stage_alg_bytes, without the
        quantisation of h for C."""
        b = self.stage_alg_bytes(name)
        if name == "C_gateup_swiglu":
            b -= self.B * (14336 // 32) * 34
        return b

    def stage(self, name, c):
        """Enqueue stage `name` with weight copy c on the current stream."""
        torch, g, B = self.torch, self.g, self.B
        L = g.lib()
        s = torch.cuda.current_stream().cuda_stream
        W = lambda n: self.w[n][c].data_ptr()
        if self.q8k:
            self._stage_q8k(name, W, s, c)
            return
        if name == "A_qkv":
            if B > 4:   # the group runs its GEMVs one after another: quantise once
                _check(g, L.quantize_act_q8_0(self.xa.data_ptr(), self.xq_a.data_ptr(), B, 4096, s),
                       "quantize")
            _check(g, L.qmv_launch_group(Q4_K, B, self._groups[c], 3, s), "qkv")
        elif name == "B_o":
            _check(g, L.qmv_launch(Q4_K, W("o"), 4096, 4096, self.xo.data_ptr(), B,
                                   self.xq_o.data_ptr(), self.y["o"].data_ptr(), s), "o")
        elif name == "C_gateup_swiglu":
            # h = silu(gate) * up, and its Q8_0 quantisation into D's scratch
            _check(g, L.qmv_launch_gateup_swiglu_q8(Q4_K, W("gate"), W("up"), 14336, 4096,
                                                    self.xc.data_ptr(), B, self.xq_c.data_ptr(),
                                                    self.h.data_ptr(), self.xq_d.data_ptr(), s),
                   "gate/up")
        else:
            _check(g, L.qmv_launch(Q6_K, W("down"), 4096, 14336, None, B, self.xq_d.data_ptr(),
                                   self.y["down"].data_ptr(), s), "down")

    def _stage_q8k(self, name, W, s, c):
        """The stage on the Q8_K path: A quantises x once for q, k, v, one
        grouped launch; C is the paired gate/up launch with the SwiGLU; B and
        D quantise their x."""
        g, B, L = self.g, self.B, self.g.lib()
        if name == "A_qkv":
            _check(g, L.quantize_act_q8_k(self.xa.data_ptr(), self.xq_a.data_ptr(), B, 4096, s),
                   "quantize q8k")
            _check(g, L.qmv_launch_group_q8k(Q4_K, B, self._groups_k[c], 3, s), "qkv q8k")
        elif name == "B_o":
            _check(g, L.qmv_launch_q8k(Q4_K, W("o"), 4096, 4096, self.xo.data_ptr(), B,
                                       self.xq_o.data_ptr(), self.y["o"].data_ptr(), s), "o")
        elif name == "C_gateup_swiglu":
            _check(g, L.qmv_launch_gateup_swiglu_q8k(Q4_K, W("gate"), W("up"), 14336, 4096,
                                                     self.xc.data_ptr(), B, self.xq_c.data_ptr(),
                                                     self.h.data_ptr(), s), "gate/up")
        else:
            _check(g, L.qmv_launch_q8k(Q6_K, W("down"), 4096, 14336, self.h.data_ptr(), B,
                                       self.xq_d.data_ptr(), self.y["down"].data_ptr(), s), "down")

    def step(self, i):
        c = i % self.R
        for name in STAGES:
            self.stage(name, c)

    def stage_alg_bytes(self, name):
        """Algorithmic bytes of one launch of a stage: weight blobs; A, B, C:
        the f32 activation read and its Q8_0 blocks written; D: the Q8_0
        blocks of h read; the f32 outputs (C: h, and its Q8_0 blocks)."""
        B = self.B
        wb = {n: row_bytes(f, K) * N for n, f, N, K in LAYER}
        Kd = {n: K for n, _, _, K in LAYER}
        Nd = {n: N for n, _, N, _ in LAYER}
        mats = STAGES[name]
        K = Kd[mats[0]]
        w = sum(wb[n] for n in mats)
        if name == "D_down":
            return w + B * (K // 32) * 34 + B * Nd["down"] * 4
        act = B * K * 4 + B * (K // 32) * 34
        if name == "C_gateup_swiglu":
            Nh = Nd["gate"]
            return w + act + B * Nh * 4 + B * (Nh // 32) * 34
        return w + act + sum(B * Nd[n] * 4 for n in mats)


def time_layer(torch, g, synth, B, steps, warmup, rotate_bytes, q8k=False):
    Lw = Layer(torch, g, synth, B, rotate_bytes, q8k)
    Lw.step(0)
    torch.cuda.synchronize()
    graphs = {}

    def make(n):
        return GraphSteps(torch, Lw.step, n)

    graphs["full"] = make(Lw.R)
    for n in (warmup, steps):
        r = n % Lw.R
        if r and r not in graphs:
            graphs[r] = make(r)
    run_steps(graphs, make, warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(graphs, make, steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # each stage alone, back to back over every rotated copy
    n = max(Lw.R, 32)
    stage_us = {name: graph_launch_us(torch, lambda i, name=name: Lw.stage(name, i % Lw.R), n)
                for name in STAGES}
    res = {"wall_s": wall, "step_bytes": Lw.step_bytes, "R": Lw.R, "stage_us": stage_us,
           "stage_alg_bytes": {n_: Lw.stage_alg_bytes(n_) for n_ in STAGES}}
    if B <= 4:
        # each stage's multiply kernel alone
        res["kernel_us"] = {
            name: graph_launch_us(torch, lambda i, name=name: Lw.kernel(name, i % Lw.R), n)
            for name in STAGES}
        res["kernel_alg_bytes"] = {n_: Lw.kernel_alg_bytes(n_) for n_ in STAGES}
        res["kernel_launches"] = n
    del graphs, Lw
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------- per-matrix rows --

def matrix_us(torch, g, synth, fmt, N, K, rows, seed, ds, rotate_bytes, n_min=20, q8k=False,
              prepared=False):
    """Time per launch of qmv_launch (rows <= 16) or qmm_launch on one
    seeded matrix, activations staged in xq, weights rotated; q8k: the same
    on the Q8_K path (qmv_launch_q8k / qmm_launch_q8k); prepared: the Q8_K
    GEMM on weights repacked by qmv_prepare beforehand (untimed, as at load).
    Returns (us, GGUF weight bytes, copies)."""
    blob = weights(synth, fmt, N, K, seed, ds)
    wt = torch.from_numpy(blob).cuda()
    nbytes = int(wt.numel())
    if prepared:
        wt = g.prepare(fmt, wt, N, K)
    R = max(1, math.ceil(rotate_bytes / int(wt.numel())))
    copies = [wt] + [wt.clone() for _ in range(R - 1)]
    x = torch.from_numpy(synth.activations(rows, K, seed + 1)).cuda()
    xq = g.quantize_q8k(x) if (q8k or prepared) else g.quantize(x)
    y = torch.empty(rows, N, dtype=torch.float32, device="cuda")
    L = g.lib()
    if prepared:
        fn = L.qmm_launch_q8k_prepared
    elif q8k:
        fn = L.qmv_launch_q8k if rows <= 16 else L.qmm_launch_q8k
    else:
        fn = L.qmv_launch if rows <= 16 else L.qmm_launch

    def launch(i):
        _check(g, fn(fmt, copies[i % R].data_ptr(), N, K, None, rows, xq.data_ptr(),
                     y.data_ptr(), torch.cuda.current_stream().cuda_stream), "matrix")
    launch(0)
    n = max(R, n_min) if rows <= 16 else max(R, 5)
    us = graph_launch_us(torch, launch, n)
    touched = min(n, R) * int(wt.numel())
    del copies, wt, x, xq, y
    torch.cuda.empty_cache()
    return us, nbytes, (R, touched)


def gemv_row(us, nbytes, B):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 2), "weight_MB": round(nbytes / 1e6, 2), "weight_GBs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "tok_s": round(B / (us * 1e-6), 1)}


def gemm_row(us, M, N, K):
    tops = 2.0 * M * N * K / (us * 1e-6) / 1e12
    return {"us": round(us, 2), "TOPS": round(tops, 1), "frac": round(tops / INT8_PEAK_TOPS, 4)}


SHAPES_8B = [("q,o", Q4_K, 4096, 4096, 2), ("k,v", Q4_K, 1024, 4096, 2),
             ("gate,up", Q4_K, 14336, 4096, 2), ("down", Q6_K, 4096, 14336, 1)]


def prefill_8b(torch, g, synth, M=2048, q8k=False, prepared=False):
    """GEMMs of the four 8B-class shapes at M tokens, and the layer's seven
    (Q8_0 activations: f16 MFMA; Q8_K: int8 MFMA, on the GGUF blob or on the
    load-time repacked weights)."""
    out, tot_ops, tot_us = {}, 0.0, 0.0
    for i, (name, fmt, N, K, cnt) in enumerate(SHAPES_8B):
        us, _, _ = matrix_us(torch, g, synth, fmt, N, K, M, synth.seed_for(4, i), 0.02, 512 << 20,
                             q8k=q8k, prepared=prepared)
        out[f"{name} {N}x{K}"] = gemm_row(us, M, N, K)
        tot_ops += cnt * 2.0 * M * N * K
        tot_us += cnt * us
    tops = tot_ops / (tot_us * 1e-6) / 1e12
    out["layer (7 GEMMs)"] = {"us": round(tot_us, 1), "TOPS": round(tops, 1),
                              "frac": round(tops / INT8_PEAK_TOPS, 4)}
    return out


def decode_8b_q8k(torch, g, synth):
    """The four 8B-class matrices as single GEMVs on the Q8_K path, batch 1 and
    16, activations staged, weights rotated over >= 1 GiB."""
    res = {}
    for B in (1, 16):
        for i, (name, fmt, N, K, _) in enumerate(SHAPES_8B):
            us, nb, _ = matrix_us(torch, g, synth, fmt, N, K, B, synth.seed_for(4, i), 0.02, 1 << 30,
                                  q8k=True)
            res[f"B{B} {name} {N}x{K}"] = gemv_row(us, nb, B)
    return res


def lm_head(torch, g, synth):
    """The LM head at batch 1, 4, 16 (Q8_0 activations) and on the Q8_K path
    at 4 and 16."""
    res = {}
    for B in (1, 4, 16):
        us, nb, R = matrix_us(torch, g, synth, Q6_K, 151936, 1024, B, synth.seed_for(2, 0), 0.01,
                              1 << 30)
        res[f"B{B}"] = gemv_row(us, nb, B)
    for B in (4, 16):
        us, nb, R = matrix_us(torch, g, synth, Q6_K, 151936, 1024, B, synth.seed_for(2, 0), 0.01,
                              1 << 30, q8k=True)
        res[f"B{B}_q8k"] = gemv_row(us, nb, B)
    return res


def qwen_ffn(torch, g, synth, rotate_bytes):
    """The pages' Qwen2.5-0.5B FFN at batch 1 (Q4_0 gate/up 4864x896, down
    896x4864) as a model runs it: gate/up with the SwiGLU, then down on h."""
    L = g.lib()
    ws = {}
    for i, (n, N, K) in enumerate([("gate", 4864, 896), ("up", 4864, 896), ("down", 896, 4864)]):
        blob, _ = synth.weights(Q4_0, N, K, synth.seed_for(1, i), dscale=0.02)
        ws[n] = torch.from_numpy(blob).cuda()
    step_bytes = sum(int(v.numel()) for v in ws.values())
    R = max(1, math.ceil(rotate_bytes / step_bytes))
    cp = {k: [v] + [v.clone() for _ in range(R - 1)] for k, v in ws.items()}
    x = torch.from_numpy(synth.activations(1, 896, synth.act_seed_for(1, 1))).cuda()
    xq = torch.empty(g.qmv_gateup_act_bytes(1, 4864, 896), dtype=torch.uint8, device="cuda")
    xq2 = g.act_buffer(1, 4864)
    h = torch.empty(1, 4864, dtype=torch.float32, device="cuda")
    y = torch.empty(1, 896, dtype=torch.float32, device="cuda")

    def step(i):
        # gate/up + SwiGLU + the quantisation of h in one launch, then down
        c = i % R
        s = torch.cuda.current_stream().cuda_stream
        _check(g, L.qmv_launch_gateup_swiglu_q8(Q4_0, cp["gate"][c].data_ptr(),
                                                cp["up"][c].data_ptr(), 4864, 896, x.data_ptr(), 1,
                                                xq.data_ptr(), h.data_ptr(), xq2.data_ptr(), s),
               "qwen gate/up")
        _check(g, L.qmv_launch(Q4_0, cp["down"][c].data_ptr(), 896, 4864, None, 1,
                               xq2.data_ptr(), y.data_ptr(), s), "qwen down")
    step(0)
    us = graph_launch_us(torch, step, R)
    del cp, ws
    torch.cuda.empty_cache()
    gbs = step_bytes / (us * 1e-6) / 1e9
    return {"us_per_step": round(us, 2), "weight_MB": round(step_bytes / 1e6, 2),
            "weight_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "tok_s": round(1e6 / us, 1), "launches_per_step": 2,
            "note": "latency-bound: 7.35 MB of weights per step"}


def qwen_small(torch, g, synth):
    us, nb, _ = matrix_us(torch, g, synth, Q8_0, 896, 896, 1, synth.seed_for(0, 0), 0.01, 1 << 30)
    q8 = gemv_row(us, nb, 1)
    q8["note"] = "latency-bound: 0.85 MB of weights"
    pre = {}
    tot_us = 0.0
    for i, (N, K) in enumerate([(4864, 896), (896, 4864)]):
        us, _, _ = matrix_us(torch, g, synth, Q4_0, N, K, 512, synth.seed_for(3, i), 0.02, 512 << 20)
        pre[f"{N}x{K}"] = gemm_row(us, 512, N, K)
        tot_us += us * (2 if N == 4864 else 1)
    tops = 3 * 2.0 * 512 * 4864 * 896 / (tot_us * 1e-6) / 1e12
    pre["ffn (gate, up, down)"] = {"us": round(tot_us, 1), "TOPS": round(tops, 1),
                                   "frac": round(tops / INT8_PEAK_TOPS, 4)}
    return {"q8_0_896x896_b1": q8, "q4_0_prefill_m512": pre}


# --------------------------------------------------------------- ceilings --

def ceilings(torch):
    """Measured ceilings of this chip (libqmv_ceilings.so)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "gguf_quantized_matvec_amd", "libqmv_ceilings.so"))
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.qmv_ceil_stream_read.argtypes = [P, ctypes.c_size_t, P, P]
    lib.qmv_ceil_stream_read_nt.argtypes = [P, ctypes.c_size_t, P, P]
    for f in ("qmv_ceil_mfma_i8", "qmv_ceil_mfma_f16", "qmv_ceil_epilogue"):
        getattr(lib, f).argtypes = [P, I, I, P]
    s = lambda: torch.cuda.current_stream().cuda_stream

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            t = e0.elapsed_time(e1) * 1e-3
            best = t if best is None else min(best, t)
        return best

    nbytes = 1 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.empty(nbytes // 128, dtype=torch.int32, device="cuda")  # the larger of the two sinks
    # 4 reads of the 1 GiB back to back per timing (a lone launch also pays
    # its dispatch and ramp-up, some 20 % of it here)
    def reads(fn):
        for _ in range(4):
            fn(buf.data_ptr(), nbytes, sink.data_ptr(), s())
    t = timed(lambda: reads(lib.qmv_ceil_stream_read)) / 4
    out = {"stream_read_GBs": round(nbytes / t / 1e9, 1)}
    t = timed(lambda: reads(lib.qmv_ceil_stream_read_nt)) / 4
    out["stream_read_nt_GBs"] = round(nbytes / t / 1e9, 1)
    # the nontemporal read at the size of the headline's dominant launch
    # (66.1 MB), rotated over the 16 slices of the buffer so none is cached
    part = (66138368 // 32768) * 32768
    copies = nbytes // part

    def rotated():
        for i in range(32):
            lib.qmv_ceil_stream_read_nt(buf.data_ptr() + (i % copies) * part, part,
                                        sink.data_ptr(), s())
    t = timed(rotated) / 32
    out["stream_read_nt_66MB_us"] = round(t * 1e6, 2)
    out["stream_read_nt_66MB_GBs"] = round(part / t / 1e9, 1)
    # the decode GEMV's own load pattern over the same bytes as the headline's
    # dominant launch (gate + up: 28672 Q4_K rows of 16 chunks of 144 bytes),
    # every lane one chunk, nothing else
    lib.qmv_ceil_chunk_read.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P, P]
    crows, cpart = 28672, 28672 * 16 * 144
    ccopies = nbytes // cpart

    def chunk_launch(i):
        rc = lib.qmv_ceil_chunk_read(buf.data_ptr() + (i % ccopies) * cpart, crows, 16, 144,
                                     sink.data_ptr(), s())
        assert rc == 0, rc
    # timed as the GEMVs are: graph replays of back-to-back launches
    t = graph_launch_us(torch, chunk_launch, 32) * 1e-6
    out["chunk_read_66MB_us"] = round(t * 1e6, 2)
    out["chunk_read_66MB_GBs"] = round(cpart / t / 1e9, 1)
    del buf, sink
    blocks, iters = 256 * 8, 2000
    o = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    t = timed(lambda: lib.qmv_ceil_mfma_i8(o.data_ptr(), blocks, iters, s()))
    out["mfma_i8_TOPS"] = round(blocks * 4 * 4 * iters * 65536 / t / 1e12, 1)
    t = timed(lambda: lib.qmv_ceil_mfma_f16(o.data_ptr(), blocks, iters, s()))
    out["mfma_f16_TFLOPS"] = round(blocks * 4 * 4 * iters * 32768 / t / 1e12, 1)
    t = timed(lambda: lib.qmv_ceil_epilogue(o.data_ptr(), blocks, iters, s()))
    fma_s = blocks * 256 * 16 * iters / t
    out["epilogue_Tfma_s"] = round(fma_s / 1e12, 2)
    # one fma per output and 32-element block = 32 int8 MACs = 64 int8 ops
    out["epilogue_bound_int8_TOPS"] = round(fma_s * 64 / 1e12, 1)
    out["how"] = ("libqmv_ceilings.so (qmv_ceilings.hip): 4 back-to-back reads of 1 GiB with "
                  "16-byte loads, 16 in flight per thread, and with the nontemporal hint, 8 in "
                  "flight per thread (also 32 back-to-back 66.1 MB reads over rotated slices), "
                  "time per read; the decode GEMV's load pattern alone over the same 66.1 MB "
                  "(28672 Q4_K rows, each lane one 144-byte chunk), rotated likewise and timed "
                  "by graph replays as the GEMVs are; "
                  "2048 workgroups x 4 waves of 4 independent MFMA chains; "
                  "16 f32 fma chains per thread; best of 5 launches by HIP events")
    return out


# ----------------------------------------------------------- CPU baseline --

def host_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    return {"nproc": os.cpu_count(), "affinity": aff, "model": model}


def cpu_baseline(synth, seconds):
    """The CPU oracle (plain C, f64 products, f32 quantisation) on the
    headline step (the 8B-class layer at batch 1: quantise, seven products,
    SwiGLU), rows split over the host threads this process may use (at most
    16: the machine's host CPUs per GPU), for about `seconds`; plus single-thread
    figures for the pages' own shapes."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    info = host_info()
    threads = max(1, min(info["affinity"], MAX_HOST_THREADS))
    oracle.lib()
    blobs = {}
    for i, (name, fmt, N, K) in enumerate(LAYER):
        blobs[name] = weights(synth, fmt, N, K, synth.seed_for(4, 10 + i), 0.02)
    rb = {n: row_bytes(f, K) for n, f, _, K in LAYER}
    spec = {n: (f, N, K) for n, f, N, K in LAYER}
    xs = [synth.activations(1, 4096, synth.act_seed_for(4, 1) + j) for j in range(3)]
    step_bytes = sum(int(b.size) for b in blobs.values())

    def rows_job(name, xq, r0, r1):
        f, _, K = spec[name]
        y, _ = oracle.matmul_f64(f, blobs[name][r0 * rb[name]: r1 * rb[name]], r1 - r0, K, xq, 1,
                                 want_abs=False)
        return r0, y

    def product(ex, name, xq):
        N = spec[name][1]
        per = math.ceil(N / threads)
        y = np.zeros(N)
        for f in [ex.submit(rows_job, name, xq, r0, min(N, r0 + per)) for r0 in range(0, N, per)]:
            r0, part = f.result()
            y[r0: r0 + part.shape[1]] = part[0]
        return y

    steps = 0
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(threads) as ex:
        while True:
            xa = oracle.quantize_act(xs[0])
            for n in ("q", "k", "v"):
                product(ex, n, xa)
            product(ex, "o", oracle.quantize_act(xs[1]))
            xc = oracle.quantize_act(xs[2])
            gt = product(ex, "gate", xc).astype(np.float32)
            up = product(ex, "up", xc).astype(np.float32)
            h = oracle.swiglu(gt, up).reshape(1, -1)
            product(ex, "down", oracle.quantize_act(h))
            steps += 1
            if time.perf_counter() - t0 >= seconds:
                break
    dt = time.perf_counter() - t0

    # single thread, the pages' shapes at batch 1 (configs 1-3)
    single = {}

    def one(tag, fmt, N, K, seed, ds, rows=None):
        blob = weights(synth, fmt, N, K, seed, ds)
        xq = oracle.quantize_act(synth.activations(1, K, seed + 1))
        n = rows or N
        part = blob[: n * row_bytes(fmt, K)]
        t = time.perf_counter()
        oracle.matmul_f64(fmt, part, n, K, xq, 1, want_abs=False)
        el = (time.perf_counter() - t) * N / n
        single[tag] = {"s_per_call": round(el, 4), "weight_GBs": round(blob.size / el / 1e9, 3)}
        if rows:
            single[tag]["sample"] = f"first {n} of {N} rows, scaled to all rows"

    one("q8_0_896x896", Q8_0, 896, 896, synth.seed_for(0, 0), 0.01)
    one("q4_0_4864x896", Q4_0, 4864, 896, synth.seed_for(1, 0), 0.02)
    one("q4_0_896x4864", Q4_0, 896, 4864, synth.seed_for(1, 2), 0.02)
    one("q6_k_151936x1024", Q6_K, 151936, 1024, synth.seed_for(2, 0), 0.01, rows=16384)
    one("q4_k_4864x1024", Q4_K, 4864, 1024, synth.seed_for(2, 1), 0.01)
    return {"value": round(step_bytes * steps / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"{steps} headline steps (8B-class layer, batch 1: 3 activation "
                       f"quantisations, 7 products in f64, SwiGLU) in {dt:.1f} s with rows split "
                       f"over {threads} threads; tok/s {steps / dt:.3f}"),
            "host": {**info, "threads_used": threads,
                     "why_threads": "at most 16: one GPU's share of the host CPUs"},
            "single_thread_b1": single}


# --------------------------------------------------------- profile helpers --

def profile_stage(torch, g, synth, name, launches=20):
    Lw = Layer(torch, g, synth, 1, 1 << 30)
    for i in range(launches):
        Lw.stage(name, i % Lw.R)
    torch.cuda.synchronize()
    print(json.dumps({"profile_stage": name, "launches": launches}))


def profile_kernel(torch, g, synth, name, launches=20):
    """Launch one stage's multiply kernel (Layer.kernel) `launches` times,
    eagerly, over the rotated weight copies."""
    Lw = Layer(torch, g, synth, 1, 1 << 30)
    Lw.step(0)   # (D reads the h quantised by C)
    torch.cuda.synchronize()
    for i in range(launches):
        Lw.kernel(name, i % Lw.R)
    torch.cuda.synchronize()
    print(json.dumps({"profile_kernel": name, "kernel": STAGE_KERNEL[name], "launches": launches}))


def profile_matrix(torch, g, synth, spec, launches=20):
    """Launch one workload matrix (the suite's seeded weights, activations
    staged) `launches` times back to back, eagerly.  spec WORKLOAD:INDEX:ROWS
    (Q8_0 activations), WORKLOAD:INDEX:ROWS:q8k (the Q8_K path) or
    WORKLOAD:INDEX:ROWS:q8kp (the Q8_K GEMM on repacked weights)."""
    parts = spec.split(":")
    wl, mi, rows = parts[:3]
    q8k = parts[3:] in (["q8k"], ["q8kp"])
    prepared = parts[3:] == ["q8kp"]
    mi, rows = int(mi), int(rows)
    ci = list(synth.WORKLOADS).index(wl)
    fmt, N, K, ds = synth.WORKLOADS[wl]["mats"][mi]
    blob, _ = synth.weights(fmt, N, K, synth.seed_for(ci, mi), dscale=ds)
    w = torch.from_numpy(blob).cuda()
    if prepared:
        w = g.prepare(fmt, w, N, K)
    x = torch.from_numpy(synth.activations(rows, K, synth.act_seed_for(ci, rows))).cuda()
    xq = g.quantize_q8k(x) if q8k else g.quantize(x)
    y = torch.empty(rows, N, dtype=torch.float32, device="cuda")
    L = g.lib()
    if prepared:
        fn = L.qmm_launch_q8k_prepared
    elif q8k:
        fn = L.qmv_launch_q8k if rows <= 16 else L.qmm_launch_q8k
    else:
        fn = L.qmv_launch if rows <= 16 else L.qmm_launch
    for _ in range(launches):
        _check(g, fn(fmt, w.data_ptr(), N, K, None, rows, xq.data_ptr(), y.data_ptr(),
                     torch.cuda.current_stream().cuda_stream), "profile_matrix")
    torch.cuda.synchronize()
    print(json.dumps({"profile_matrix": spec, "fmt": synth.NAMES[fmt], "N": N, "K": K,
                      "rows": rows, "launches": launches}))


def suite(torch, g, synth, rotate_bytes):
    """Every workload matrix at each of its batch sizes: GEMV weight GB/s and
    GEMM int8-equivalent TOPS, weights rotated over >= rotate_bytes."""
    res = []
    for wl, spec in synth.WORKLOADS.items():
        ci = list(synth.WORKLOADS).index(wl)
        for mi, (fmt, N, K, ds) in enumerate(spec["mats"]):
            for B in spec["batches"]:
                us, nb, (R, touched) = matrix_us(torch, g, synth, fmt, N, K, B,
                                                 synth.seed_for(ci, mi), ds, rotate_bytes)
                # weights the timed launches read: past the 256 MB last-level
                # cache they stream from HBM, else they may be served from it
                row = {"workload": wl, "fmt": synth.NAMES[fmt], "N": N, "K": K, "rows": B,
                       "rotated_copies": R, "weights_read_MB": round(touched / 1e6, 1),
                       "weights_from": "HBM" if touched > 512e6 else "last-level cache"}
                row.update(gemv_row(us, nb, B) if B <= 16 else gemm_row(us, B, N, K))
                res.append(row)
                print(json.dumps({"suite_row": row}), file=sys.stderr, flush=True)
    return res


def traffic_from(pmc_dir, kernel_filter, stage):
    """profiles/traffic.json from four rocprofv3 --pmc runs under pmc_dir:
    stage_FETCH_SIZE/ and stage_WRITE_SIZE/ (`bench.py --profile-stage S`),
    calib_FETCH_SIZE/ and calib_WRITE_SIZE/ (`bench.py --copy-calib`).
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

    copy_bytes = 256 << 20
    f_scale = copy_bytes / (max(v for _, v in rows("calib_FETCH_SIZE", "FETCH_SIZE")) * 1024)
    w_scale = copy_bytes / (max(v for _, v in rows("calib_WRITE_SIZE", "WRITE_SIZE")) * 1024)
    fk = [v for k, v in rows("stage_FETCH_SIZE", "FETCH_SIZE") if kernel_filter in k]
    wk = [v for k, v in rows("stage_WRITE_SIZE", "WRITE_SIZE") if kernel_filter in k]
    fetch = sum(fk) / len(fk) * 1024 * f_scale
    write = sum(wk) / len(wk) * 1024 * w_scale
    out = {"stage": stage, "kernel_filter": kernel_filter, "kernel_src_sha": kernel_src_sha(),
           "dispatches": [len(fk), len(wk)],
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
           "bytes_per_launch": round(fetch + write)}
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(out))


def trace_summary(trace_dir):
    """Per (kernel, grid) launch counts and durations from a rocprofv3
    --kernel-trace run (its *kernel_trace.csv files)."""
    import csv
    import glob
    import statistics
    groups = {}
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            key = (r["Kernel_Name"][:90], r.get("Grid_Size_X", r.get("Grid_Size", "")),
                   r.get("Grid_Size_Y", ""), r.get("Workgroup_Size_X", r.get("Workgroup_Size", "")))
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            groups.setdefault(key, []).append(dur)
    print("| kernel | grid x | grid y | workgroup | launches | mean us | median us | min us |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|")
    for key, d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{key[0]}` | {key[1]} | {key[2]} | {key[3]} | {len(d)} | "
              f"{statistics.mean(d):.2f} | {statistics.median(d):.2f} | {min(d):.2f} |")


# ------------------------------------------------------------------- main --

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--rotate-mib", type=int, default=1024)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="only the headline step (no batch-16 step, prefill, LM head, ceilings)")
    ap.add_argument("--suite", action="store_true",
                    help="also report every workload matrix (GEMV and GEMM) separately")
    ap.add_argument("--profile-stage", default=None, choices=list(STAGES),
                    help="only launch one stage of the layer step 20 times, eagerly")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the M = 2048 GEMMs of the four 8B-class shapes (Q8_0 activations, "
                         "Q8_K, Q8_K on repacked weights)")
    ap.add_argument("--profile-kernel", default=None, choices=list(STAGES),
                    help="only launch one stage's multiply kernel 20 times, eagerly")
    ap.add_argument("--profile-matrix", default=None, metavar="WORKLOAD:INDEX:ROWS",
                    help="only launch one workload matrix 20 times, eagerly")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a 256 MiB device copy 10 times (counter calibration)")
    ap.add_argument("--traffic-from", default=None, metavar="DIR")
    ap.add_argument("--traffic-stage", default="D_down", choices=list(STAGES),
                    help="the stage whose kernel (--profile-kernel) the counters under "
                         "--traffic-from were taken on")
    ap.add_argument("--trace-summary", default=None, metavar="DIR")
    args = ap.parse_args()

    if args.traffic_from:
        traffic_from(args.traffic_from, STAGE_KERNEL[args.traffic_stage], args.traffic_stage)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
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
    if args.profile_stage:
        profile_stage(torch, g, synth, args.profile_stage)
        return
    if args.prefill_only:
        print(json.dumps({"prefill_m2048": prefill_8b(torch, g, synth),
                          "prefill_m2048_q8k": prefill_8b(torch, g, synth, q8k=True),
                          "prefill_m2048_q8k_repacked": prefill_8b(torch, g, synth, q8k=True,
                                                                   prepared=True)}))
        return
    if args.profile_kernel:
        profile_kernel(torch, g, synth, args.profile_kernel)
        return
    if args.profile_matrix:
        profile_matrix(torch, g, synth, args.profile_matrix)
        return

    rot = args.rotate_mib << 20
    print("step: headline layer, batch 1", file=sys.stderr, flush=True)
    r1 = time_layer(torch, g, synth, 1, args.steps, args.warmup, rot)
    wall = r1["wall_s"]
    value = r1["step_bytes"] * args.steps / wall / 1e9
    # roofline: the step's slowest multiply kernel, timed alone (as a kernel
    # trace sees it)
    dom = max(r1["kernel_us"], key=r1["kernel_us"].get)
    dom_us = r1["kernel_us"][dom]
    achieved = r1["kernel_alg_bytes"][dom] / (dom_us * 1e-6) / 1e9

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tf = json.load(open(TRAFFIC_FILE))
        if tf.get("kernel_src_sha") == kernel_src_sha() and tf.get("stage") == dom:
            traffic = tf.get("bytes_per_launch")

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
        "data": "synthetic (seeded GGUF Q4_K / Q6_K blocks, N(0,1) activations)",
        "config": {
            "workload": ("8B-class decoder layer, decode batch 1: [q 4096x4096, k/v 1024x4096] "
                         "-> o 4096x4096 -> [gate, up 14336x4096 + SwiGLU] -> down 4096x14336; "
                         "Q4_K, down Q6_K; 5 launches per step in dependency order"),
            "global_batch": 1, "weights_per_step_bytes": r1["step_bytes"],
            "rotated_copies": r1["R"], "graph_replay": True,
            "tok_s": round(args.steps / wall, 1),
            "hbm_frac_of_value": round(value / HBM_PEAK_GBS, 4),
            "stage_us": {k: round(v, 2) for k, v in r1["stage_us"].items()},
            "kernel_us": {k: round(v, 2) for k, v in r1["kernel_us"].items()},
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "stage": dom, "kernel": STAGE_KERNEL[dom],
                     "kernel_does": STAGE_KERNEL_WHAT[dom],
                     "avg_launch_us": round(dom_us, 3), "launches_timed": r1["kernel_launches"],
                     "alg_bytes_per_launch": r1["kernel_alg_bytes"][dom],
                     "timing": "HIP events on the launch stream around graph replays of the "
                               "kernel's launches back to back over the rotated weight copies; "
                               "time per launch includes the dispatch gap between graph nodes"},
    }
    if not args.no_cpu:
        print("step: cpu baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(synth, args.cpu_seconds)
    if not args.no_extra:
        print("step: layer batch 16", file=sys.stderr, flush=True)
        n16 = max(20, args.steps // 4)
        r16 = time_layer(torch, g, synth, 16, n16, max(2, args.warmup // 4), rot)
        v16 = r16["step_bytes"] * n16 / r16["wall_s"] / 1e9
        out["decode_b16"] = {"value_GBs": round(v16, 1), "hbm_frac": round(v16 / HBM_PEAK_GBS, 4),
                             "ms_per_step": round(r16["wall_s"] / n16 * 1e3, 5),
                             "tok_s": round(16 * n16 / r16["wall_s"], 1), "steps": n16,
                             "stage_us": {k: round(v, 2) for k, v in r16["stage_us"].items()}}
        print("step: layer batch 16, Q8_K activations", file=sys.stderr, flush=True)
        r16k = time_layer(torch, g, synth, 16, n16, max(2, args.warmup // 4), rot, q8k=True)
        v16k = r16k["step_bytes"] * n16 / r16k["wall_s"] / 1e9
        out["decode_b16_q8k"] = {
            "value_GBs": round(v16k, 1), "hbm_frac": round(v16k / HBM_PEAK_GBS, 4),
            "ms_per_step": round(r16k["wall_s"] / n16 * 1e3, 5),
            "tok_s": round(16 * n16 / r16k["wall_s"], 1), "steps": n16,
            "stage_us": {k: round(v, 2) for k, v in r16k["stage_us"].items()},
            "path": "the same step with Q8_K activations: A quantises once, then q, k, v in "
                    "one qmv_launch_group_q8k; B, D qmv_launch_q8k; C "
                    "qmv_launch_gateup_swiglu_q8k; the batched int8-MFMA kernel, one f32 term "
                    "per superblock"}
        print("step: prefill M=2048", file=sys.stderr, flush=True)
        out["prefill_m2048"] = {"unit": "int8-equivalent TOPS", "peak": INT8_PEAK_TOPS,
                                **prefill_8b(torch, g, synth)}
        print("step: prefill M=2048, Q8_K activations", file=sys.stderr, flush=True)
        out["prefill_m2048_q8k"] = {"unit": "int8-equivalent TOPS", "peak": INT8_PEAK_TOPS,
                                    **prefill_8b(torch, g, synth, q8k=True)}
        print("step: prefill M=2048, Q8_K activations, repacked weights", file=sys.stderr,
              flush=True)
        out["prefill_m2048_q8k_repacked"] = {
            "unit": "int8-equivalent TOPS", "peak": INT8_PEAK_TOPS,
            "repack": "qmv_prepare at load (untimed): int8 digit pairs, 3.7x Q4_K / 2.5x Q6_K bytes",
            **prefill_8b(torch, g, synth, q8k=True, prepared=True)}
        print("step: decode GEMVs, Q8_K activations", file=sys.stderr, flush=True)
        out["decode_8b_q8k"] = decode_8b_q8k(torch, g, synth)
        print("step: lm head", file=sys.stderr, flush=True)
        out["lm_head_q6_k_151936x1024"] = lm_head(torch, g, synth)
        print("step: qwen shapes", file=sys.stderr, flush=True)
        out["qwen_ffn_b1"] = qwen_ffn(torch, g, synth, rot)
        out.update(qwen_small(torch, g, synth))
        print("step: ceilings", file=sys.stderr, flush=True)
        out["ceilings"] = ceilings(torch)
    if args.suite:
        out["suite"] = suite(torch, g, synth, rot)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
