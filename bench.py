#!/usr/bin/env python3
"""Benchmark of the routed MoE layer on 4-bit packed weights, one MI355X.

One step = one MoE-layer forward (router, top-k, grouping, gate_up + SwiGLU,
down, weighted combine) over one batch of T synthetic tokens, on the next of
`layers` independently seeded layers (rotated so the weights are not
cache-resident). Prints ONE JSON line.

Default run: the OLMoE-1B-7B-shaped layer (E=64, top_k=8, H=2048, I=1024, NF4
blocksize 64) at batch-1 decode (T=1, 64 layers) as the headline, plus a
`prefill` object for the same layer at T=4096 (8 layers): the two halves of the
metric. Timing: a HIP graph of one rotation over the layers is replayed; each
replay is timed by HIP events, a process's figure is the median over >= 5
replays, and a second, independent set of replays is reported beside it (the
self-pair). The default run repeats the two step times in fresh processes (3 in
all, one after another) and reports each, their median (the line's figure) and
the worst.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "MoE-layer tokens/s + effective packed-weight HBM GB/s (decode T=1, prefill)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 / f16 MFMA, published
RIDGE_FLOP_PER_BYTE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # 312.5
MIN_REPLAYS = 5


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="olmoe_decode",
                    choices=["olmoe_decode", "olmoe_prefill", "qwen3_zipf", "gptoss_mxfp4", "tiny"])
    ap.add_argument("--tokens", type=int, default=None, help="T per step (workload default if unset)")
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--path", default="auto", choices=["auto", "small", "mfma"])
    ap.add_argument("--graph", type=int, default=1, help="1: time HIP-graph replays as well")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="default workload only: leave out the T=4096 prefill object")
    ap.add_argument("--profile-steps", type=int, default=None,
                    help="event-timed steps of the dominant kernel (default: 8 rotations, at most 512)")
    ap.add_argument("--absmax-bf16", action="store_true",
                    help="NF4 workloads: bf16-source weights stored with bf16 absmax")
    ap.add_argument("--gptoss-form", action="store_true",
                    help="the gpt-oss expert form: clamped GLU (alpha 1.702, limit 7), per-expert "
                         "biases, interleaved gate / up rows")
    ap.add_argument("--op", default="forward", choices=["forward", "dgrad"],
                    help="forward: the routed MoE layer (default). dgrad: the input gradients "
                         "of the layer's two grouped GEMMs (gate_up and down) on the forward's "
                         "routing, for training-shaped token counts")
    ap.add_argument("--fresh-processes", type=int, default=3, metavar="N",
                    help="default workload: time the decode and prefill steps in N fresh processes "
                         "in all (this one and N - 1 children, one after another); the line's step "
                         "times are the median over the processes")
    ap.add_argument("--rep-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise copy of MIB MiB (read + write once) five "
                         "times, for scaling the FETCH_SIZE / WRITE_SIZE counters, and exit")
    return ap.parse_args()


def copy_calibration(mib):
    """A plain copy kernel of known size: torch.neg reads n fp32 and writes n fp32."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"kernel": "torch.neg fp32", "read_bytes": 4 * n,
                                           "write_bytes": 4 * n, "launches": 5}}), flush=True)


ROOT = os.path.dirname(os.path.abspath(__file__))
# Sources a kernel's code depends on; their hash ties a stored counter record
# (profiles/traffic.json) to the kernel it was measured on.
KERNEL_SOURCES = {"small": ["gemv.hip", "common.h", "internal.h"],
                  "mfma": ["mfma.hip", "common.h", "internal.h"]}


def kernel_source_hash(kind):
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "bit_quantized_moe_expert_amd", "csrc")
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kind):
    """HBM bytes per launch of the dominant kernel from the committed FETCH_SIZE /
    WRITE_SIZE counter record, or None when there is none or the kernel's
    sources changed since it was taken."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
            rec = json.load(fh)[workload]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash(kind):
        return None
    return float(rec["hbm_bytes_per_launch"])


def spin_cycles_for(seconds, stream):
    """Cycles of torch.cuda._sleep's spin kernel that last about `seconds` on
    this GPU: the counter's rate from two spins of different lengths (their
    difference cancels the launch overhead), after one call that loads the
    kernel."""
    import torch
    torch.cuda._sleep(1 << 10)
    lens, secs = (1 << 20, 1 << 23), []
    for c in lens:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        torch.cuda._sleep(c)
        b.record(stream)
        torch.cuda.synchronize()
        secs.append(a.elapsed_time(b) * 1e-3)
    rate = (lens[1] - lens[0]) / max(secs[1] - secs[0], 1e-6)  # cycles per second
    return int(min(max(seconds, 0.001), 1.0) * rate)


def workload(name, absmax_bf16=False):
    import moe_synth as S
    wl = S.WORKLOADS[name]
    if absmax_bf16:
        if wl.fmt != 0:
            raise SystemExit("--absmax-bf16 applies to NF4 workloads")
        import dataclasses
        wl = dataclasses.replace(wl, fmt=2, name=wl.name + "_bf16abs")
    return wl


def bf16_source(w, wl):
    """The bf16-absmax workloads stand for a bf16 checkpoint: weights rounded to bf16."""
    import torch
    return w.to(torch.bfloat16).to(torch.float32) if wl.fmt == 2 else w


def packed_bytes_per_expert(wl):
    """Algorithmic bytes of one expert: codes + scales of gate_up and down."""
    blk = 32 if wl.fmt == 1 else 64
    sbytes = {0: 4, 1: 1, 2: 2}[wl.fmt]
    g = 2 * wl.I * (wl.H // 2 + (wl.H // blk) * sbytes)
    d = wl.H * (wl.I // 2 + (wl.I // blk) * sbytes)
    return g, d


def roofline_class(wl, T, active):
    """'hbm' or 'mfma' from the workload's arithmetic intensity: algorithmic flops
    (6 R H I) over the packed bytes of the experts the batch touches (`active`,
    counted from the routing), against the ridge point of the published peaks
    (2.5 PFLOP/s / 8 TB/s = 312.5 flop/B)."""
    g, d = packed_bytes_per_expert(wl)
    intensity = 6.0 * T * wl.top_k * wl.H * wl.I / (active * (g + d))
    return ("mfma" if intensity > RIDGE_FLOP_PER_BYTE else "hbm"), intensity


def cpu_info():
    cores = len(os.sched_getaffinity(0))
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


class Run:
    """The layers of one workload on the device, the forward call and its timings."""

    def __init__(self, wl, T, nlayers, path, dev, gptoss_form=False):
        import ctypes
        import numpy as np
        import torch
        import moe_synth as S
        import bit_quantized_moe_expert_amd as M
        self.wl, self.T, self.nlayers, self.dev = wl, T, nlayers, dev
        self.M, self.gptoss_form = M, gptoss_form
        self.layers, self.xs, self.xb = [], [], []
        t0 = time.time()
        for l in range(nlayers):
            W_r, b_r = S.make_router(wl, l)
            w13 = bf16_source(S.make_stack_torch(wl, l, "w13", dev), wl)
            p13, s13 = M.quantize(w13, wl.fmt)
            del w13
            w2 = bf16_source(S.make_stack_torch(wl, l, "w2", dev), wl)
            p2, s2 = M.quantize(w2, wl.fmt)
            del w2
            form = {}
            if gptoss_form:
                b13, b2 = S.make_biases(wl, l)
                form = dict(glu=M.GLU_CLAMPED, glu_alpha=GPTOSS_ALPHA, glu_limit=GPTOSS_LIMIT,
                            glu_interleaved=1, b13=torch.from_numpy(b13).to(dev),
                            b2=torch.from_numpy(b2).to(dev))
            self.layers.append(M.MoELayer(
                fmt=wl.fmt, E=wl.E, H=wl.H, I=wl.I, top_k=wl.top_k, w13=p13, w13_scale=s13, w2=p2,
                w2_scale=s2, router_w=torch.from_numpy(W_r).to(dev),
                router_b=None if b_r is None else torch.from_numpy(b_r).to(dev),
                renormalize=wl.renormalize, path=path, **form))
            xb = S.make_x(wl, T, l)
            self.xb.append(xb)
            self.xs.append(torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16))
        torch.cuda.synchronize()
        self.setup_s = time.time() - t0
        self.fwd = M.Forward(self.layers[0], T, dev)
        self.structs = [lay.struct() for lay in self.layers]
        self.out = torch.empty(T, wl.H, dtype=torch.bfloat16, device=dev)
        self.L = M.lib()
        self.stream = torch.cuda.current_stream()
        self.sp = ctypes.c_void_p(self.stream.cuda_stream)
        self.xptr = [ctypes.c_void_p(x.data_ptr()) for x in self.xs]
        self.optr = ctypes.c_void_p(self.out.data_ptr())
        self.srefs = [ctypes.byref(s) for s in self.structs]
        R = T * wl.top_k
        self.small = (path == M.PATH_SMALL_M) or (path == M.PATH_AUTO and
                                                   M.auto_path(wl.fmt, R, max(wl.H, wl.I)) == M.PATH_SMALL_M)

    def step(self, i, stream_ptr=None):
        n = self.nlayers
        st = self.L.nf4moe_moe_forward(self.srefs[i % n], self.xptr[i % n], self.T, self.optr, None, None,
                                       self.fwd.wsp, self.fwd.nb, stream_ptr or self.sp)
        if st != 0:
            self.M._check(st)

    def time_eager(self, steps, warmup):
        """W untimed steps, then exactly K timed steps between two synchronisations."""
        import torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for i in range(steps):
            self.step(warmup + i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def time_graph(self, replays):
        """A HIP graph of one rotation (one call per layer), replayed: two
        independent sets of `replays` event-timed replays after one untimed
        replay. Returns per-step times (ms) of each replay of both sets."""
        import ctypes
        import torch
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(self.stream)
        with torch.cuda.stream(cs):
            with torch.cuda.graph(g, stream=cs):
                csp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                for i in range(self.nlayers):
                    self.step(i, csp)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        sets = []
        for _ in range(2):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(replays)]
            for a, b in evs:
                a.record(self.stream)
                g.replay()
                b.record(self.stream)
            torch.cuda.synchronize()
            sets.append([a.elapsed_time(b) / self.nlayers for a, b in evs])
        del g
        return sets

    def profile_gate_up(self, prof_steps, step_ms):
        """The gate_up kernel's own durations from two HIP events handed to its
        launch, over `prof_steps` profiled steps on the forward's stream; steps
        shorter than 0.2 ms are queued behind a spin kernel so they run back
        to back, as in the timed loops."""
        import numpy as np
        import torch
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(prof_steps)]
        for row in evs:
            for ev in row:
                ev.record(self.stream)
        torch.cuda.synchronize()
        spin_ev = None
        if step_ms < 0.2:
            spin = spin_cycles_for(0.0003 * prof_steps + 0.02, self.stream)
            spin_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            spin_ev[0].record(self.stream)
            torch.cuda._sleep(spin)
            spin_ev[1].record(self.stream)
        t_enq = time.perf_counter()
        for i in range(prof_steps):
            self.fwd.set_layer(self.layers[i % self.nlayers])
            self.fwd.profiled(self.xs[i % self.nlayers], self.out, [ev.cuda_event for ev in evs[i]])
        enqueue_ms = (time.perf_counter() - t_enq) * 1e3
        torch.cuda.synchronize()
        spin_ms = spin_ev[0].elapsed_time(spin_ev[1]) if spin_ev is not None else None
        stage = np.array([[r[0].elapsed_time(r[1]), r[1].elapsed_time(r[2]), r[2].elapsed_time(r[3])]
                          for r in evs])
        gate = np.array([r[4].elapsed_time(r[5]) for r in evs])
        return dict(stage=np.median(stage, axis=0), gate=gate, spin_ms=spin_ms, enqueue_ms=enqueue_ms)

    def routing(self):
        """Each layer's GPU routing (topk ids) for its batch."""
        import torch
        ids = []
        for i in range(self.nlayers):
            t = torch.empty(self.T, self.wl.top_k, dtype=torch.int32, device=self.dev)
            self.fwd.set_layer(self.layers[i])
            self.fwd(self.xs[i], out=self.out, topk_ids=t)
            ids.append(t.cpu().numpy())
        return ids


def near_ties(run, gpu_ids, max_layers):
    """Routing near-ties: tokens whose k-th and (k+1)-th fp64 logits are within
    tau = 1e-5 (1 + max|L|), and tokens whose GPU (fp32 logits) selection differs
    from the fp64 selection (allowed only at such a near-tie). Logits in fp64
    with numpy; selection by a stable sort (logit descending, id ascending)."""
    import numpy as np
    import moe_synth as S
    wl = run.wl
    k = wl.top_k
    n_near = n_diff = n_tok = 0
    for l in range(min(max_layers, run.nlayers)):
        W_r, b_r = S.make_router(wl, l)
        xb = run.xb[l].astype(np.uint32) << 16
        x = xb.view(np.float32).astype(np.float64)
        L = x @ W_r.astype(np.float64).T
        if b_r is not None:
            L = L + b_r.astype(np.float64)
        order = np.argsort(-L, axis=1, kind="stable")
        srt = np.take_along_axis(L, order, axis=1)
        tau = 1e-5 * (1.0 + np.abs(L).max(axis=1))
        near = (srt[:, k - 1] - srt[:, k] <= tau) if k < wl.E else np.zeros(len(L), bool)
        diff = np.any(np.sort(order[:, :k], axis=1) != np.sort(gpu_ids[l], axis=1), axis=1)
        n_near += int(near.sum())
        n_diff += int(diff.sum())
        n_tok += len(L)
        if np.any(diff & ~near):
            raise SystemExit(f"layer {l}: GPU routing differs from the fp64 selection away from a near-tie")
    return {"tokens": n_tok, "near_tie_tokens": n_near, "selection_differs": n_diff,
            "tau": "1e-5 * (1 + max|logit|)"}


def measure(wl, T, nlayers, args, dev, headline_steps, warmup, gptoss_form=False, path_name="auto"):
    """One workload's numbers: eager and graph step times, the dominant (gate_up)
    kernel's event-timed duration and roofline, routing near-ties, CPU baseline."""
    import numpy as np
    import bit_quantized_moe_expert_amd as M
    path = {"auto": M.PATH_AUTO, "small": M.PATH_SMALL_M, "mfma": M.PATH_MFMA}[path_name]
    run = Run(wl, T, nlayers, path, dev, gptoss_form)
    print(f"[bench] {wl.name} T={T} layers={nlayers} setup {run.setup_s:.1f}s", file=sys.stderr, flush=True)
    steps = max(headline_steps, 1)
    eager_ms = run.time_eager(steps, warmup)
    graph_sets = None
    if args.graph:
        try:
            replays = max(MIN_REPLAYS, -(-steps // nlayers))
            graph_sets = run.time_graph(replays)
        except Exception as ex:  # graph capture is optional for the line
            print(f"[bench] graph capture skipped: {ex}", file=sys.stderr, flush=True)
    if graph_sets is not None:
        med = [float(np.median(s)) for s in graph_sets]
        ms = med[0]
        timing = {"mode": "hip_graph", "replays_per_set": len(graph_sets[0]), "steps_per_replay": nlayers,
                  "median_ms_per_step": med[0], "min_ms_per_step": float(np.min(graph_sets[0])),
                  "max_ms_per_step": float(np.max(graph_sets[0])),
                  "self_pair": {"a_ms": med[0], "b_ms": med[1], "a_over_b": med[0] / med[1]}}
    else:
        ms = eager_ms
        timing = {"mode": "eager"}
    prof_steps = args.profile_steps or min(512, 8 * nlayers)
    prof = run.profile_gate_up(prof_steps, ms)
    gate = prof["gate"]
    ids = run.routing()
    active = float(np.mean([np.unique(i).size for i in ids]))
    g_b, d_b = packed_bytes_per_expert(wl)
    R = T * wl.top_k
    bound, intensity = roofline_class(wl, T, active)
    gate_ms = float(np.mean(gate))
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": active * g_b / (gate_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "per_launch": f"{active:.1f} active experts x {g_b} B (gate_up codes + scales)"}
    else:
        roof = {"bound": "mfma", "achieved": 4.0 * R * wl.H * wl.I / (gate_ms * 1e-3) / 1e12,
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "per_launch": f"4 R H I = {4.0 * R * wl.H * wl.I:.4g} flop"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    kind = "small" if run.small else "mfma"
    roof["traffic"] = measured_traffic(wl.name if T == wl.tokens[0] else f"{wl.name}_T{T}", kind)
    roof["kernel"] = "k_gemv<SwiGLU> (gate_up)" if run.small else "k_mfma<SwiGLU> (gate_up)"
    roof["kernel_ms_mean"] = gate_ms
    roof["kernel_ms_median"] = float(np.median(gate))
    roof["intensity_flop_per_byte"] = intensity
    roof["kernel_timing"] = {"launches": prof_steps, "queued_behind_spin_ms": prof["spin_ms"],
                             "host_enqueue_ms": prof["enqueue_ms"]}
    roof["kernel_source_hash"] = kernel_source_hash(kind)
    step_bytes = active * (g_b + d_b)
    flops = 6.0 * R * wl.H * wl.I
    res = {
        "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "eager_ms_per_step": eager_ms,
        "eager_steps": steps, "timing": timing,
        "effective_packed_GBps": step_bytes / (ms * 1e-3) / 1e9,
        "algorithmic_TFLOPs": flops / (ms * 1e-3) / 1e12,
        "layer_roofline_frac": (step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS) if bound == "hbm"
        else (flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS),
        "active_experts_per_step": active,
        "stage_ms_median": {"route": float(prof["stage"][0]), "gate_up_kernel": float(np.median(gate)),
                            "down_combine": float(prof["stage"][2])},
        "roofline": roof,
        "routing": near_ties(run, ids, max_layers=nlayers if T <= 64 else 2),
        "path": "small_m" if run.small else "mfma",
    }
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, T, run, args.cpu_seconds, gptoss_form)
    res["cpu_baseline"] = cpu
    return run, res


def retime(res, ms, T):
    """Put a new step time into a result and rescale the figures derived from it."""
    f = res["ms_per_step"] / ms
    for k in ("effective_packed_GBps", "algorithmic_TFLOPs", "layer_roofline_frac"):
        res[k] *= f
    res["ms_per_step"] = ms
    res["tokens_per_s"] = T / (ms * 1e-3)


def graph_step_ms(wl, T, nlayers, dev, steps, warmup):
    """The graph-timed step of one workload alone (median of the first set of
    replays), after the same eager warm-up as measure()."""
    import numpy as np
    import bit_quantized_moe_expert_amd as M
    run = Run(wl, T, nlayers, M.PATH_AUTO, dev)
    run.time_eager(max(steps, 1), warmup)
    sets = run.time_graph(max(MIN_REPLAYS, -(-steps // nlayers)))
    del run
    return float(np.median(sets[0]))


def rep_child(args):
    """One fresh-process repetition of the default line's two step times."""
    import torch
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    d, p = workload("olmoe_decode"), workload("olmoe_prefill")
    out = {"decode_ms": graph_step_ms(d, d.tokens[0], d.layers, dev, args.steps, args.warmup),
           "prefill_ms": graph_step_ms(p, p.tokens[0], p.layers, dev, p.layers, p.layers)}
    print(json.dumps(out), flush=True)


def fresh_process_reps(n, steps, warmup):
    """Run n - 1 child processes, one after another, each timing the default
    line's decode and prefill steps afresh (new process, new weights of the
    same seeds, new graph). Called before this process touches the GPU."""
    import subprocess
    reps = []
    for i in range(n - 1):
        cmd = [sys.executable, os.path.abspath(__file__), "--rep-child", "--steps", str(steps),
               "--warmup", str(warmup)]
        print(f"[bench] fresh-process repetition {i + 1} of {n - 1}", file=sys.stderr, flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        if r.returncode != 0:
            raise RuntimeError(f"fresh-process repetition failed ({r.returncode}): {r.stderr[-2000:]}")
        reps.append(json.loads([x for x in r.stdout.splitlines() if x.startswith("{")][-1]))
    return reps


def mfma_ceiling(dev, workgroups=2048, iters=1024, launches=5):
    """Measured bf16 matrix-core rate under full load (nf4moe_mfma_peak: every
    wave back-to-back MFMAs on random finite register operands, no memory
    traffic): the median of `launches` event-timed launches after one untimed."""
    import numpy as np
    import torch
    import bit_quantized_moe_expert_amd as M
    sink = torch.empty(workgroups * 512, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    M.mfma_peak(workgroups, iters, sink)
    times, flops = [], 0
    for _ in range(launches):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        flops = M.mfma_peak(workgroups, iters, sink)
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = float(np.median(times))
    tf = flops / (ms * 1e-3) / 1e12
    del sink
    return {"bf16_TFLOPs": tf, "frac_of_spec": tf / BF16_PEAK_TFLOPS, "ms": ms, "flops_per_launch": flops,
            "launch": f"{workgroups} workgroups x 8 waves x {iters} rounds of 8 v_mfma_f32_32x32x16_bf16, "
                      "random finite bf16 register operands, median of 5"}


def stream_ceiling(dev, sizes, launches=32, shapes=(2, 4, 8, 16)):
    """Measured single-launch HBM read rate (nf4moe_stream_read) at given byte
    counts, the fastest of several launch shapes (16-byte loads per thread):
    each launch reads a different slice of a 2 GiB buffer (so the bytes are not
    cache-resident), queued back to back behind a spin kernel, each timed by its
    own HIP events; the median per shape, the best shape per size."""
    import numpy as np
    import torch
    import bit_quantized_moe_expert_amd as M
    buf = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    stream = torch.cuda.current_stream()
    out = {}
    for name, nbytes in sizes.items():
        nbytes = nbytes // 16 * 16
        nslice = max(1, (1 << 31) // nbytes)
        per_shape = {}
        for loads in shapes:
            sink = torch.empty(M.stream_read_sink_words(nbytes, loads), dtype=torch.int32, device=dev)
            views = [buf[(i % nslice) * nbytes:(i % nslice + 1) * nbytes] for i in range(launches + 4)]
            for v in views[:4]:
                M.stream_read(v, nbytes, sink, loads)
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(launches)]
            torch.cuda._sleep(spin_cycles_for(0.0002 * launches + 0.01, stream))
            for (a, b), v in zip(evs, views[4:]):
                a.record(stream)
                M.stream_read(v, nbytes, sink, loads)
                b.record(stream)
            torch.cuda.synchronize()
            per_shape[loads] = float(np.median([a.elapsed_time(b) for a, b in evs]))
        best = min(per_shape, key=per_shape.get)
        t = per_shape[best]
        out[name] = {"bytes": nbytes, "ms": t, "GBps": nbytes / (t * 1e-3) / 1e9,
                     "frac_of_spec": nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, "loads_per_thread": best,
                     "ms_by_loads_per_thread": per_shape}
    del buf
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "this library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.op == "dgrad":
        bench_dgrad(args)
        return
    if args.rep_child:
        rep_child(args)
        return

    wl = workload(args.workload, args.absmax_bf16)
    T = args.tokens or wl.tokens[0]
    nlayers = args.layers or wl.layers
    steps = args.steps or (nlayers * 20 if T <= 16 else nlayers * 4)
    warmup = args.warmup if args.warmup is not None else min(steps, nlayers * 2)
    default_run = (args.workload == "olmoe_decode" and args.tokens is None and not args.absmax_bf16
                   and args.path == "auto" and not args.gptoss_form)
    # The fresh-process repetitions run first, while this process has not yet
    # touched the GPU: the children are separate programs, one at a time.
    reps = None
    if default_run and args.graph and not args.no_prefill and args.fresh_processes > 1:
        reps = fresh_process_reps(args.fresh_processes, steps, warmup)

    import torch
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] {wl.name} T={T} layers={nlayers} steps={steps} warmup={warmup}", file=sys.stderr, flush=True)
    run, res = measure(wl, T, nlayers, args, dev, steps, warmup, args.gptoss_form, args.path)
    small = run.small
    g_b, d_b = packed_bytes_per_expert(wl)
    del run
    torch.cuda.empty_cache()

    ceiling = None
    if small:
        act = res["active_experts_per_step"]
        ceiling = stream_ceiling(dev, {"gate_up_bytes": int(act * g_b), "down_bytes": int(act * d_b),
                                       "layer_bytes": int(act * (g_b + d_b))})
        print(f"[bench] stream ceiling {json.dumps(ceiling)}", file=sys.stderr, flush=True)

    prefill = None
    if default_run and not args.no_prefill:
        pwl = workload("olmoe_prefill")
        pT, pl = pwl.tokens[0], pwl.layers
        prun, pres = measure(pwl, pT, pl, args, dev, pl, pl, False, "auto")
        del prun
        torch.cuda.empty_cache()
        prefill = {"config": {"workload": pwl.name, "format": "nf4_b64", "E": pwl.E, "top_k": pwl.top_k,
                              "H": pwl.H, "I": pwl.I, "T": pT, "layers": pl},
                   "value": pres["tokens_per_s"], "unit": "tokens/s", "dtype": "bf16 (split operands), fp32 acc",
                   **pres}
        ceil = mfma_ceiling(dev)
        print(f"[bench] mfma ceiling {json.dumps(ceil)}", file=sys.stderr, flush=True)
        prefill["mfma_ceiling"] = ceil
        # the gate_up kernel's MFMA work (two bf16 products per useful one: B as
        # hi + lo) and its useful flops, each against the measured ceiling
        prefill["roofline"]["frac_of_measured_ceiling"] = prefill["roofline"]["achieved"] / ceil["bf16_TFLOPs"]
        prefill["roofline"]["mfma_work_frac_of_measured_ceiling"] = (2.0 * prefill["roofline"]["achieved"]
                                                                    / ceil["bf16_TFLOPs"])

    if reps is not None and res["timing"]["mode"] == "hip_graph":
        # the pages' discipline: the same measurement in several fresh processes,
        # reported with the median and the worst; the line takes the median
        import numpy as np
        dms = [res["ms_per_step"]] + [r["decode_ms"] for r in reps]
        res["fresh_processes"] = {"n": len(dms), "ms_per_step": dms, "median_ms": float(np.median(dms)),
                                  "worst_ms": float(np.max(dms)), "this_process_ms": res["ms_per_step"]}
        retime(res, float(np.median(dms)), T)
        if prefill is not None:
            pms = [prefill["ms_per_step"]] + [r["prefill_ms"] for r in reps]
            prefill["fresh_processes"] = {"n": len(pms), "ms_per_step": pms, "median_ms": float(np.median(pms)),
                                          "worst_ms": float(np.max(pms)),
                                          "this_process_ms": prefill["ms_per_step"]}
            retime(prefill, float(np.median(pms)), prefill["config"]["T"])
            prefill["value"] = prefill["tokens_per_s"]

    line = {
        "metric": METRIC, "value": res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if small else "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights quantized on device)",
        "config": {"workload": wl.name, "format": {0: "nf4_b64", 1: "mxfp4_b32", 2: "nf4_b64_bf16abs"}[wl.fmt],
                   "E": wl.E, "top_k": wl.top_k, "H": wl.H, "I": wl.I, "T": T, "layers": nlayers,
                   "path": res["path"], "timing": res["timing"]["mode"],
                   "epilogue": "clamped_glu+biases" if args.gptoss_form else "swiglu"},
        **{k: v for k, v in res.items() if k not in ("ms_per_step", "tokens_per_s", "path")},
        "stream_read_ceiling": ceiling,
        "prefill": prefill,
    }
    print(json.dumps(line), flush=True)


def bench_dgrad(args):
    """One step = the input gradients of one layer's two grouped GEMMs
    (grouped_dgrad through gate_up [E, 2I, H] and down [E, H, I]) on the routing
    the forward computes for a synthetic batch, with random bf16 output
    gradients, rotating over independently seeded layers."""
    import ctypes
    import numpy as np
    import torch
    import moe_synth as S
    import bit_quantized_moe_expert_amd as M

    wl = S.WORKLOADS[args.workload if args.workload != "olmoe_decode" else "olmoe_prefill"]
    T = args.tokens or wl.tokens[-1]
    nlayers = args.layers or wl.layers
    steps = args.steps or 4 * nlayers
    warmup = args.warmup if args.warmup is not None else nlayers
    dev = torch.device("cuda", 0)
    R = T * wl.top_k
    L = M.lib()
    setups = []
    for l in range(nlayers):
        W_r, b_r = S.make_router(wl, l)
        w13 = bf16_source(S.make_stack_torch(wl, l, "w13", dev), wl)
        p13, s13 = M.quantize(w13, wl.fmt)
        del w13
        w2 = bf16_source(S.make_stack_torch(wl, l, "w2", dev), wl)
        p2, s2 = M.quantize(w2, wl.fmt)
        del w2
        xb = S.make_x(wl, T, l)
        x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
        logits = M.router_logits(x, torch.from_numpy(W_r).to(dev),
                                 None if b_r is None else torch.from_numpy(b_r).to(dev))
        off = M.route_permute(logits, wl.top_k, bool(wl.renormalize))["expert_offsets"]
        g = torch.Generator(device=dev).manual_seed(7000 + l)
        dc13 = torch.randn(R, 2 * wl.I, generator=g, device=dev).to(torch.bfloat16)
        dc2 = torch.randn(R, wl.H, generator=g, device=dev).to(torch.bfloat16)
        setups.append((p13, s13, p2, s2, off, dc13, dc2))
    G = wl.E
    need = L.nf4moe_gemm_workspace_bytes(G, R)
    ws = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    wsp = ctypes.c_void_p((ws.data_ptr() + 255) // 256 * 256)
    da13 = torch.empty(R, wl.H, dtype=torch.float32, device=dev)
    da2 = torch.empty(R, wl.I, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    p = M._ptr

    def call(i, which):
        p13, s13, p2, s2, off, dc13, dc2 = setups[i % nlayers]
        if which == 0:
            st = L.nf4moe_grouped_dgrad(wl.fmt, p(dc13), p(p13), p(s13), wl.E, 2 * wl.I, wl.H, G, p(off),
                                        None, R, p(da13), M.DT_F32, wsp, need, sp)
        else:
            st = L.nf4moe_grouped_dgrad(wl.fmt, p(dc2), p(p2), p(s2), wl.E, wl.H, wl.I, G, p(off),
                                        None, R, p(da2), M.DT_F32, wsp, need, sp)
        if st != 0:
            M._check(st)

    for i in range(warmup):
        call(i, 0)
        call(i, 1)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record(stream)
    for i in range(steps):
        call(i, 0)
        call(i, 1)
    e[1].record(stream)
    torch.cuda.synchronize()
    ms = e[0].elapsed_time(e[1]) / steps
    # per-GEMM split on a second pass
    per = [[], []]
    for i in range(min(steps, 4 * nlayers)):
        for which in (0, 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            call(i, which)
            b.record(stream)
            per[which].append((a, b))
    torch.cuda.synchronize()
    gu_ms = float(np.mean([a.elapsed_time(b) for a, b in per[0]]))
    dn_ms = float(np.mean([a.elapsed_time(b) for a, b in per[1]]))
    flops = 6.0 * R * wl.H * wl.I
    gu_flops = 4.0 * R * wl.H * wl.I
    line = {
        "metric": "grouped dgrad TFLOP/s (input gradients of gate_up and down on 4-bit weights)",
        "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (forward routing of seeded N(0,1) tokens, N(0,1) bf16 output gradients)",
        "config": {"workload": wl.name + "_dgrad", "format": {0: "nf4_b64", 1: "mxfp4_b32", 2: "nf4_b64_bf16abs"}[wl.fmt],
                   "E": wl.E, "top_k": wl.top_k, "H": wl.H, "I": wl.I, "T": T, "R": R, "layers": nlayers,
                   "timing": "eager"},
        "gate_up_dgrad_ms_mean": gu_ms, "down_dgrad_ms_mean": dn_ms,
        "roofline": {"bound": "mfma", "achieved": gu_flops / (gu_ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": gu_flops / (gu_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                     "traffic": None, "kernel": "k_dgrad (gate_up, events around the call)"},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


# gpt-oss's published clamped-GLU constants
GPTOSS_ALPHA, GPTOSS_LIMIT = 1.702, 7.0


def cpu_baseline(wl, T, run, seconds, gptoss_form=False):
    """Time oracle.moe_forward (fp64, numpy) on the host cores for a bounded
    sample of this workload: layer calls of up to 16 tokens (each layer's own
    batch, the first layers of the rotation), cycled until `seconds` of oracle
    time. The oracle's quantization of the experts the calls need is done
    first, untimed, on a thread pool. BLAS may use every core the process is
    allowed, up to 16."""
    import torch
    import moe_synth as S
    import oracle as O
    from concurrent.futures import ThreadPoolExecutor
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_info = threadpool_limits = None
    cores, model = cpu_info()
    blas_threads = min(cores, 16)
    Tc = min(T, 16)                                         # bounded token sample per call
    n_prep = min(run.nlayers, 8 if Tc == 1 else 1)          # layers whose experts are prepared

    class Pick:
        def __init__(self, q, i):
            self.q, self.i = q, i

        def __getitem__(self, e):
            return self.q[int(e)][self.i]

    prepared = []
    for l in range(n_prep):
        W_r, b_r = S.make_router(wl, l)
        xb = run.xb[l][:Tc]
        ids, _ = O.topk_route(O.router_logits(xb, W_r, b_r), wl.top_k, bool(wl.renormalize))
        need = sorted(set(ids.reshape(-1).tolist()))
        w13 = bf16_source(S.make_stack_torch(wl, l, "w13", run.dev), wl)
        w2 = bf16_source(S.make_stack_torch(wl, l, "w2", run.dev), wl)
        src13 = {e: w13[e].cpu().numpy() for e in need}
        src2 = {e: w2[e].cpu().numpy() for e in need}
        del w13, w2
        torch.cuda.empty_cache()
        with ThreadPoolExecutor(blas_threads) as ex:
            q13 = dict(zip(need, ex.map(lambda e: O.quantize(wl.fmt, src13[e]), need)))
            q2 = dict(zip(need, ex.map(lambda e: O.quantize(wl.fmt, src2[e]), need)))
        layer = dict(fmt=wl.fmt, E=wl.E, H=wl.H, I=wl.I, top_k=wl.top_k, renormalize=wl.renormalize,
                     w13=Pick(q13, 0), w13_scale=Pick(q13, 1), w2=Pick(q2, 0), w2_scale=Pick(q2, 1),
                     router_w=W_r, router_b=b_r)
        if gptoss_form:
            b13, b2 = S.make_biases(wl, l)
            layer.update(glu=O.GLU_CLAMPED, glu_alpha=GPTOSS_ALPHA, glu_limit=GPTOSS_LIMIT,
                         glu_interleaved=1, b13=b13, b2=b2)
        prepared.append((layer, xb))
    ctx = threadpool_limits(limits=blas_threads, user_api="blas") if threadpool_limits else None
    info = None
    if threadpool_info:
        info = [{"api": d.get("user_api"), "lib": d.get("internal_api"), "threads": d.get("num_threads")}
                for d in threadpool_info()]
    total, calls = 0.0, 0
    try:
        while total < seconds or calls == 0:
            layer, xb = prepared[calls % n_prep]
            t = time.perf_counter()
            O.moe_forward(layer, xb)
            total += time.perf_counter() - t
            calls += 1
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return {"value": calls * Tc / total, "unit": "tokens/s", "cores": blas_threads, "kind": "oracle",
            "host_cores_allowed": cores, "blas_threads": blas_threads, "blas": info, "cpu_model": model,
            "sample": f"{calls} layer calls of {Tc} token(s) ({wl.name}, cycling over the batches of "
                      f"{n_prep} layer(s)), {total:.1f}s of fp64 numpy (BLAS on up to {blas_threads} "
                      f"threads, elementwise steps on one); the oracle's quantization untimed"}


if __name__ == "__main__":
    main()
