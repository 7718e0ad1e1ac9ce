#!/usr/bin/env python3
"""Benchmark of the routed MoE layer on 4-bit packed weights, one MI355X.

One step = one MoE-layer forward (router, top-k, grouping, gate_up + SwiGLU,
down, weighted combine) over one batch of T synthetic tokens, on the next of
`layers` independently seeded layers (rotated so the weights are not
cache-resident). Prints ONE JSON line.

Default workload: OLMoE-1B-7B-shaped decode, E=64, top_k=8, H=2048, I=1024,
T=1, NF4 blocksize 64, 64 layers.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "MoE-layer tokens/s + effective packed-weight HBM GB/s (decode T=1, prefill)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


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
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--absmax-bf16", action="store_true",
                    help="NF4 workloads: bf16-source weights stored with bf16 absmax")
    ap.add_argument("--gptoss-form", action="store_true",
                    help="the gpt-oss expert form: clamped GLU (alpha 1.702, limit 7), per-expert "
                         "biases, interleaved gate / up rows")
    ap.add_argument("--op", default="forward", choices=["forward", "dgrad"],
                    help="forward: the routed MoE layer (default). dgrad: the input gradients "
                         "of the layer's two grouped GEMMs (gate_up and down) on the forward's "
                         "routing, for training-shaped token counts")
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


def workload(args):
    import moe_synth as S
    wl = S.WORKLOADS[args.workload]
    if args.absmax_bf16:
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

    import numpy as np
    import torch
    import moe_synth as S
    import bit_quantized_moe_expert_amd as M

    wl = workload(args)
    T = args.tokens or wl.tokens[0]
    nlayers = args.layers or wl.layers
    path = {"auto": M.PATH_AUTO, "small": M.PATH_SMALL_M, "mfma": M.PATH_MFMA}[args.path]
    steps = args.steps or (nlayers * 20 if T <= 16 else nlayers * 4)
    warmup = args.warmup if args.warmup is not None else min(steps, nlayers * 2)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] {wl.name} T={T} layers={nlayers} steps={steps} warmup={warmup}", file=sys.stderr,
          flush=True)

    # ---- inputs: weights drawn on the device and quantized by the library (untimed)
    layers, xs = [], []
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
        if args.gptoss_form:
            b13, b2 = S.make_biases(wl, l)
            form = dict(glu=M.GLU_CLAMPED, glu_alpha=GPTOSS_ALPHA, glu_limit=GPTOSS_LIMIT, glu_interleaved=1,
                        b13=torch.from_numpy(b13).to(dev), b2=torch.from_numpy(b2).to(dev))
        layers.append(M.MoELayer(
            fmt=wl.fmt, E=wl.E, H=wl.H, I=wl.I, top_k=wl.top_k, w13=p13, w13_scale=s13, w2=p2,
            w2_scale=s2, router_w=torch.from_numpy(W_r).to(dev),
            router_b=None if b_r is None else torch.from_numpy(b_r).to(dev),
            renormalize=wl.renormalize, path=path, **form))
        xb = S.make_x(wl, T, l)
        xs.append(torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16))
    torch.cuda.synchronize()
    print(f"[bench] setup {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    fwd = M.Forward(layers[0], T, dev)
    structs = [lay.struct() for lay in layers]
    out = torch.empty(T, wl.H, dtype=torch.bfloat16, device=dev)
    L = M.lib()
    import ctypes
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    xptr = [ctypes.c_void_p(x.data_ptr()) for x in xs]
    optr = ctypes.c_void_p(out.data_ptr())
    srefs = [ctypes.byref(s) for s in structs]

    def step(i):
        st = L.nf4moe_moe_forward(srefs[i % nlayers], xptr[i % nlayers], T, optr, None, None,
                                  fwd.wsp, fwd.nb, sp)
        if st != 0:
            M._check(st)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region (eager)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / steps

    # ---- HIP graph of one rotation over all layers, replayed
    graph_ms = None
    if args.graph:
        try:
            g = torch.cuda.CUDAGraph()
            cs = torch.cuda.Stream()
            cs.wait_stream(stream)
            with torch.cuda.stream(cs):
                csp = ctypes.c_void_p(cs.cuda_stream)
                with torch.cuda.graph(g, stream=cs):
                    for i in range(nlayers):
                        st = L.nf4moe_moe_forward(srefs[i], xptr[i], T, optr, None, None, fwd.wsp,
                                                  fwd.nb, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
                        if st != 0:
                            M._check(st)
            torch.cuda.synchronize()
            reps = max(1, steps // nlayers)
            g.replay()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            graph_ms = e0.elapsed_time(e1) / (reps * nlayers)
        except Exception as ex:  # graph capture is optional for the line
            print(f"[bench] graph capture skipped: {ex}", file=sys.stderr, flush=True)

    # ---- dominant kernel (gate_up + SwiGLU): HIP events around its launch on the same stream
    prof_steps = min(steps, 8 * nlayers)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(prof_steps)]
    for row in evs:
        for ev in row:
            ev.record(stream)
    torch.cuda.synchronize()
    # The host records the events and launches of a profiled step in about
    # 0.1 ms (0.3 ms allowed below); shorter steps are queued behind a spin kernel, so that the stream
    # runs them back to back, as in the timed loops, instead of each starting on
    # an idle GPU.
    step_ms = graph_ms if graph_ms is not None else eager_ms
    spin_ev = None
    if step_ms < 0.2:
        spin = spin_cycles_for(0.0003 * prof_steps + 0.02, stream)
        spin_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        spin_ev[0].record(stream)
        torch.cuda._sleep(spin)
        spin_ev[1].record(stream)
    t_enq = time.perf_counter()
    for i in range(prof_steps):
        fwd.set_layer(layers[i % nlayers])
        fwd.profiled(xs[i % nlayers], out, [ev.cuda_event for ev in evs[i]])
    enqueue_ms = (time.perf_counter() - t_enq) * 1e3
    torch.cuda.synchronize()
    spin_ms = spin_ev[0].elapsed_time(spin_ev[1]) if spin_ev is not None else None
    stage = np.array([[r[0].elapsed_time(r[1]), r[1].elapsed_time(r[2]), r[2].elapsed_time(r[3])]
                      for r in evs])
    route_ms, gate_ms, down_ms = (float(v) for v in np.median(stage, axis=0))
    # the gate_up kernel's own duration (events taken by its launch)
    gate_kernel = np.array([r[4].elapsed_time(r[5]) for r in evs])
    gate_mean_ms = float(np.mean(gate_kernel))

    # ---- work per step
    g_b, d_b = packed_bytes_per_expert(wl)
    R = T * wl.top_k
    # experts actually active per step, from the routing of every layer
    act = []
    for i in range(nlayers):
        ids = torch.empty(T, wl.top_k, dtype=torch.int32, device=dev)
        fwd.set_layer(layers[i])
        fwd(xs[i], out=out, topk_ids=ids)
        act.append(int(torch.unique(ids).numel()))
    active = float(np.mean(act))
    step_bytes = active * (g_b + d_b)
    flops = 6.0 * R * wl.H * wl.I
    ms = graph_ms if graph_ms is not None else eager_ms
    value = T / (ms * 1e-3)
    small = (path == M.PATH_SMALL_M) or (path == M.PATH_AUTO and R <= 64 and max(wl.H, wl.I) <= 4096)
    if small:
        gate_bytes = active * g_b
        roof = {"bound": "hbm", "achieved": gate_bytes / (gate_mean_ms * 1e-3) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        gate_flops = 4.0 * R * wl.H * wl.I
        roof = {"bound": "mfma", "achieved": gate_flops / (gate_mean_ms * 1e-3) / 1e12,
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    kind = "small" if small else "mfma"
    roof["traffic"] = measured_traffic(wl.name if T == wl.tokens[0] else f"{wl.name}_T{T}", kind)
    roof["kernel"] = "k_gemv<SwiGLU> (gate_up)" if small else "k_mfma<SwiGLU> (gate_up)"
    roof["kernel_ms_mean"] = gate_mean_ms
    roof["kernel_timing"] = {"launches": prof_steps, "queued_behind_spin_ms": spin_ms,
                             "host_enqueue_ms": enqueue_ms}
    roof["kernel_source_hash"] = kernel_source_hash(kind)

    # ---- CPU baseline: the fp64 oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, T, layers, xs, dev, args.cpu_seconds, args.gptoss_form)

    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if small else "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights quantized on device)",
        "config": {"workload": wl.name, "format": {0: "nf4_b64", 1: "mxfp4_b32", 2: "nf4_b64_bf16abs"}[wl.fmt],
                   "E": wl.E, "top_k": wl.top_k, "H": wl.H, "I": wl.I, "T": T, "layers": nlayers,
                   "path": "small_m" if small else "mfma", "timing": "hip_graph" if graph_ms else "eager",
                   "epilogue": "clamped_glu+biases" if args.gptoss_form else "swiglu"},
        "eager_ms_per_step": eager_ms, "graph_ms_per_step": graph_ms,
        "effective_packed_GBps": step_bytes / (ms * 1e-3) / 1e9,
        "algorithmic_TFLOPs": flops / (ms * 1e-3) / 1e12,
        "active_experts_per_step": active,
        "stage_ms_median": {"route": route_ms, "gate_up_kernel": float(np.median(gate_kernel)),
                            "down_combine": down_ms},
        "roofline": roof,
        "cpu_baseline": cpu,
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
    t_gu, t_dn = 0.0, 0.0
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


def cpu_baseline(wl, T, layers, xs, dev, seconds, gptoss_form=False):
    """Time oracle.moe_forward (fp64, numpy) on host cores for a bounded sample:
    whole layer calls of this workload, one token batch each, until `seconds`."""
    import numpy as np
    import torch
    import moe_synth as S
    import oracle as O
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = 1
    total, calls, toks = 0.0, 0, 0
    ctx = threadpool_limits(limits=cores) if threadpool_limits else None
    try:
        l = 0
        while total < seconds and l < len(layers):
            W_r, b_r = S.make_router(wl, l)
            xb = S.make_x(wl, T, l)
            Tc = min(T, 16)                                     # bounded token sample per call
            xb = xb[:Tc]
            L64 = O.router_logits(xb, W_r, b_r)
            ids, _ = O.topk_route(L64, wl.top_k, bool(wl.renormalize))
            need = sorted(set(ids.reshape(-1).tolist()))
            w13 = bf16_source(S.make_stack_torch(wl, l, "w13", dev), wl)
            w2 = bf16_source(S.make_stack_torch(wl, l, "w2", dev), wl)
            E = wl.E
            q13 = {e: O.quantize(wl.fmt, w13[e].cpu().numpy()) for e in need}
            q2 = {e: O.quantize(wl.fmt, w2[e].cpu().numpy()) for e in need}
            del w13, w2
            torch.cuda.empty_cache()

            class Pick:
                def __init__(self, q, i):
                    self.q, self.i = q, i

                def __getitem__(self, e):
                    return self.q[int(e)][self.i]
            layer = dict(fmt=wl.fmt, E=E, H=wl.H, I=wl.I, top_k=wl.top_k, renormalize=wl.renormalize,
                         w13=Pick(q13, 0), w13_scale=Pick(q13, 1), w2=Pick(q2, 0), w2_scale=Pick(q2, 1),
                         router_w=W_r, router_b=b_r)
            if gptoss_form:
                b13, b2 = S.make_biases(wl, l)
                layer.update(glu=O.GLU_CLAMPED, glu_alpha=GPTOSS_ALPHA, glu_limit=GPTOSS_LIMIT,
                             glu_interleaved=1, b13=b13, b2=b2)
            t = time.perf_counter()
            O.moe_forward(layer, xb)
            total += time.perf_counter() - t
            calls += 1
            toks += Tc
            l += 1
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    return {"value": toks / total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{calls} layer calls of {min(T, 16)} token(s) each ({wl.name}), "
                      f"{total:.1f}s of fp64 numpy on 1 host thread; quantization untimed"}


if __name__ == "__main__":
    main()
