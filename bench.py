"""Benchmark of the routed FP4 MoE FFN on one MI355X.

Default workload: Qwen-shaped decode, 48 MoE layers x 512 NVFP4 experts
(63.3 GiB resident in HBM) + one bf16 shared expert per layer, top-10, hidden
2560, intermediate 640, one token per step with a fresh seeded activation
vector per (step, layer). A step is one token through all 48 layers: one
moe_layer_decode per layer (router GEMV + softmax + top-k on the device,
expert SwiGLU GEMVs, weighted combine, shared expert). The K timed steps are
captured once as a HIP graph and replayed; inputs are resident in HBM before
the timer starts.

The roofline member covers the expert GEMV (moe_expert_decode: the gate/up
and down kernels that stream the chosen experts' FP4 blocks): HIP events on
the launch stream bracket each call while the GPU is still busy with a graph
replay, so the host's enqueue time is not in the measured interval.

Prints ONE JSON line (see the "roofline" and "cpu_baseline" members).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "MoE layer tokens/s and achieved HBM GB/s (decode), MFMA TFLOP/s (prefill)"

# HBM bytes per call of the roofline's kernels from rocprofv3 --pmc
# (FETCH_SIZE x 2 + WRITE_SIZE x 1 KiB, the factors a plain 1 GiB copy gives;
# profiles/*_hbm_traffic.md), per workload, with the fingerprint of the kernel
# sources the counters were taken on. A figure whose sources have changed
# since is not reported (traffic: null).
# qwen_decode: k_gateup<1,5,2,0> + k_down_combine<1,16,5,true,true>;
# qwen_layer_decode (no shared expert): k_down_combine<1,16,5,false,true>.
# deepseek_decode: k_gateup_stream<2,2,false> + k_down_stream_pair<2,2>.
# *_prefill: every kernel of one moe_expert_prefill call.
# fp8_act_quant / fp8_gemv: the one kernel of each call.
TRAFFIC: dict = {  # workload: (HBM bytes per call, sources fingerprint)
    "qwen_decode": (38256128, "4036827fbed01d9d"),
    "qwen_layer_decode": (28344013, "4036827fbed01d9d"),
    "deepseek_decode": (114368512, "4036827fbed01d9d"),
    "qwen_prefill": (2574034842, "5acc77f42e0b0790"),
    "deepseek_prefill": (7298760090, "5acc77f42e0b0790"),
    "fp8_act_quant": (21128192, "4d7a263804fc10fd"),
    "fp8_gemv": (21209088, "4d7a263804fc10fd"),
}
TRAFFIC_SOURCES = {  # kernel sources behind each workload's figure
    "decode": ["kernels_decode.hip", "moe_device.h", "moe_internal.h"],
    "prefill": ["kernels_prefill.hip", "moe_device.h", "moe_internal.h"],
    "fp8": ["kernels_fp8.hip", "moe_device.h", "moe_internal.h"],
}


def sources_fingerprint(kind: str) -> str:
    """sha256 (first 16 hex digits) of the kernel sources of a workload kind."""
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[kind]:
        with open(os.path.join(ROOT, "block_scaled_fp4_route_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def traffic_for(workload: str, kind: str):
    """The counted HBM bytes per call if they were taken on the current sources."""
    t = TRAFFIC.get(workload)
    if t is None or t[1] != sources_fingerprint(kind):
        return None
    return t[0]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def phase_marker(torch):
    """A tiny, uniquely named kernel (torch's spin kernel) that separates the
    phases of a --profile-run in a rocprofv3 trace."""
    torch.cuda._sleep(100)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measure_copy_bandwidth(torch, nbytes=4 << 30, iters=10):
    """Device-to-device copy of a 4 GiB buffer: bytes read + written per second."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / 1e3 / iters
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / s / 1e9


class DecodeModel:
    """All layers of a decode workload resident on the GPU."""

    def __init__(self, m, sg, wl, replicas=1):
        import torch
        self.m, self.wl = m, wl
        self.L = wl.layers * replicas
        self.d = m.desc(wl.H, wl.I, wl.E, wl.k, wl.fmt)
        B = wl.block_bytes
        t0 = time.time()
        self.blocks = torch.empty((self.L * wl.E, B), dtype=torch.uint8, device="cuda")
        for l in range(self.L):
            sg.fill_layer_blocks(wl, l % wl.layers if replicas == 1 else l, self.blocks[l * wl.E:(l + 1) * wl.E])
        self.Wr = torch.stack([sg.router_weights(wl, l, device="cuda") for l in range(self.L)])
        self.shared = ([[t.contiguous() for t in sg.shared_expert(wl, l, device="cuda")] for l in range(self.L)]
                       if wl.shared else [None] * self.L)
        base = self.blocks.data_ptr()
        self.ptrs = torch.tensor([[base + (l * wl.E + e) * B for e in range(wl.E)] for l in range(self.L)],
                                 dtype=torch.int64, device="cuda")
        self.ws_d = m.alloc_workspace(self.d, 1, m.MOE_MODE_DECODE)
        self.idx = torch.empty((self.L, wl.k), dtype=torch.int32, device="cuda")
        self.w = torch.empty((self.L, wl.k), dtype=torch.float32, device="cuda")
        self.y = torch.empty((self.L, wl.H), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        log(f"[bench] resident: {self.blocks.numel() / 2**30:.2f} GiB experts in {self.L} layers, "
            f"generated in {time.time() - t0:.1f} s")

    def inputs(self, sg, steps):
        import torch
        wl = self.wl
        return torch.stack([torch.stack([sg.activations(wl, s, l % wl.layers, T=1, device="cuda").view(-1)
                                         for l in range(wl.layers)]) for s in range(steps)])

    def layer(self, x, l):
        self.m.moe_layer_decode(self.d, x, self.Wr[l], self.ptrs[l], self.shared[l], self.y[l], self.idx[l],
                                self.w[l], self.ws_d)

    def experts(self, x, l):
        """The expert GEMV alone, on the routing the last layer call left."""
        self.m.moe_expert_decode(self.d, x, self.ptrs[l], self.idx[l], self.w[l], self.shared[l], self.y[l],
                                 self.ws_d)

    def step(self, xs, s, replica_offset=0):
        for l in range(self.wl.layers):
            self.layer(xs[s, l], replica_offset + l)


def bytes_per_layer(wl):
    experts = wl.k * wl.block_bytes
    router = wl.E * wl.H * 4
    shared = 3 * wl.H * wl.I * 2 if wl.shared else 0
    act = wl.H * 4 * 2  # x in, y out (the router and the experts read the same x)
    return experts, router, shared, act


def cpu_baseline_decode(sg, wl, model, budget_s=20.0, budget_1t_s=8.0):
    """The oracle on a bounded sample: the first layers of one token, with all
    host cores, then with one thread; inputs copied to the host before the
    timer starts."""
    import numpy as np
    import torch
    from oracle import oracle as O
    O.build(force=False)
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    L = wl.layers
    x = [sg.activations(wl, 0, l, T=1).numpy().reshape(-1) for l in range(L)]
    Wr = [model.Wr[l].cpu().numpy() for l in range(L)]
    sh = [None if s is None else [t.view(torch.int16).cpu().numpy().view(np.uint16) for t in s]
          for s in model.shared[:L]]

    def run(nthreads, budget):
        done, t_total = 0, 0.0
        while done < L and (done == 0 or t_total < budget):
            l = done
            _, oi, ow = O.route(x[l], Wr[l], wl.k)
            blks = [model.blocks[l * wl.E + int(e)].cpu().numpy() for e in oi[0]]
            t0 = time.perf_counter()
            O.route(x[l], Wr[l], wl.k)
            O.moe_decode(wl.fmt, wl.H, wl.I, x[l], blks, ow[0], shared=sh[l], nthreads=nthreads)
            t_total += time.perf_counter() - t0
            done += 1
        return 1.0 / (t_total / done * L), done, t_total

    v, done, t = run(max(1, cores), budget_s)
    v1, done1, t1 = run(1, budget_1t_s)
    what = f"fp64 router + {wl.k} experts" + (" + shared" if wl.shared else "")
    return {"value": v, "unit": "tokens/s", "cores": max(1, cores), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"layers 0..{done - 1} of token 0 ({done} of {L} layers, each: {what}), "
                      f"timed {t:.1f} s, extrapolated to {L} layers",
            "value_1_thread": v1,
            "sample_1_thread": f"layers 0..{done1 - 1} of token 0 on one thread, timed {t1:.1f} s, "
                               f"extrapolated to {L} layers"}


def run_decode(args, m, sg, torch):
    wl = sg.get(args.workload)
    replicas = args.replicas if args.replicas else (16 if wl.layers == 1 else 1)
    model = DecodeModel(m, sg, wl, replicas=replicas)
    K, W = args.steps, args.warmup
    xs = model.inputs(sg, W + K)
    nrep = replicas

    def step(s):
        model.step(xs, s, replica_offset=(s % nrep) * wl.layers if nrep > 1 else 0)

    # eager warmup (also checks the calls)
    for s in range(W):
        step(s)
    torch.cuda.synchronize()

    g = None
    if args.eager:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(W, W + K):
            step(s)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        mode = "eager"
    else:
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            with torch.cuda.graph(g, stream=cs):
                for s in range(W, W + K):
                    step(s)
        torch.cuda.current_stream().wait_stream(cs)
        g.replay()  # one untimed replay
        torch.cuda.synchronize()
        if args.profile_run:
            phase_marker(torch)
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        mode = "hip_graph"
        if args.profile_run:
            phase_marker(torch)

    # Per-call durations with HIP events on the launch stream. The calls are
    # enqueued behind a replay of the whole step graph (or a run of eager
    # steps), so the GPU reaches each one with the next already queued.
    nprobe = min(2 * wl.layers, 96) if wl.layers > 1 else 32
    ev_x = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nprobe)]
    ev_l = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nprobe)]

    def probe(fn, evs):
        if g is not None:
            g.replay()
        else:
            for s in range(W, W + K):
                step(s)
        if args.profile_run:
            phase_marker(torch)  # the calls that follow are the trace's probe phase
        for i in range(nprobe):
            l = i % wl.layers
            li = (i % nrep) * wl.layers + l if nrep > 1 else l
            evs[i][0].record()
            fn(xs[W + (i // wl.layers) % K, l], li)
            evs[i][1].record()
        torch.cuda.synchronize()
        return [e[0].elapsed_time(e[1]) * 1e3 for e in evs]

    expert_samples = probe(model.experts, ev_x)
    if args.profile_run:
        phase_marker(torch)
        torch.cuda.synchronize()
    layer_samples = probe(model.layer, ev_l) if not args.profile_run else expert_samples
    expert_us = statistics.median(expert_samples)
    layer_us_call = statistics.median(layer_samples)

    ms_per_step = elapsed / K * 1e3
    tok_s = 1e3 / ms_per_step
    experts, router, shared, act = bytes_per_layer(wl)
    layer_bytes = experts + router + shared + act
    step_bytes = layer_bytes * wl.layers
    expert_call_bytes = experts + shared + act
    achieved = expert_call_bytes / (expert_us * 1e-6) / 1e9
    copy_gbps = measure_copy_bandwidth(torch) if not args.profile_run else 0.0
    pair = "k_gateup + k_down_combine" if wl.fmt == "nvfp4" else "k_gateup_stream + k_down_stream_pair"
    res = {
        "metric": METRIC, "value": round(tok_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded SplitMix64; random-code FP4 experts, no trained weights)",
        "config": {"workload": wl.name, "layers": wl.layers, "experts": wl.E, "top_k": wl.k, "hidden": wl.H,
                   "intermediate": wl.I, "weights": wl.fmt, "shared_expert": "bf16" if wl.shared else None,
                   "tokens_per_step": 1, "replicas": replicas, "launch": mode, "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "expert GEMV: moe_expert_decode (" + pair + ")", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_for(wl.name, "decode"),
                     "bytes_per_launch": expert_call_bytes, "median_us": round(expert_us, 3),
                     "mean_us": round(statistics.fmean(expert_samples), 3), "samples": nprobe},
        "layer_us": round(ms_per_step * 1e3 / wl.layers, 3),
        "layer_us_per_call": round(layer_us_call, 3),
        "layer_GBps": round(layer_bytes / (ms_per_step * 1e-3 / wl.layers) / 1e9, 1),
        "step_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "hbm_copy_GBps_measured": round(copy_gbps, 1),
    }
    if args.profile_run:
        res["profile_run"] = True
    elif not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(sg, wl, model)
    return res


def prefill_flops_bytes(wl, idx, out_bf16):
    """Algorithmic work of one prefill layer: 2 * (assignments) * 3 * H * I
    flops; bytes = every expert that receives a token read once + x in + out."""
    import numpy as np
    n = idx.numel()
    touched = int(np.unique(idx.cpu().numpy()).size)
    flops = 2.0 * n * 3 * wl.H * wl.I
    byts = touched * wl.block_bytes + wl.T * wl.H * 4 + wl.T * wl.H * (2 if out_bf16 else 4)
    return flops, byts, touched


def cpu_baseline_prefill(sg, wl, blocks, x, idx, w, budget_tokens=16, tokens_1t=4):
    import numpy as np
    from oracle import oracle as O
    O.build(force=False)
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()

    def run(ntok, nthreads):
        toks = np.linspace(0, wl.T - 1, ntok).astype(int)
        ih = idx.cpu().numpy()[toks]
        hb = {int(e): blocks[int(e)].cpu().numpy() for e in np.unique(ih)}
        xh = x.cpu().numpy()[toks]
        wh = w.cpu().numpy()[toks]
        t0 = time.perf_counter()
        O.moe_prefill(wl.fmt, wl.H, wl.I, wl.E, xh, hb, ih, wh, act=1 if wl.fmt == "nvfp4" else 2,
                      out_bf16=wl.out_bf16, nthreads=nthreads)
        return len(toks), time.perf_counter() - t0

    n, dt = run(budget_tokens, cores)
    n1, dt1 = run(tokens_1t, 1)
    return {"value": n / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{n} of {wl.T} prompt tokens (evenly spaced) through the layer with their "
                      f"{wl.k} experts each, fp64, one thread per token, timed {dt:.1f} s",
            "value_1_thread": n1 / dt1,
            "sample_1_thread": f"{n1} of {wl.T} prompt tokens on one thread, timed {dt1:.1f} s"}


def run_prefill(args, m, sg, torch):
    wl = sg.get(args.workload)
    d = m.desc(wl.H, wl.I, wl.E, wl.k, wl.fmt)
    t0 = time.time()
    blocks = torch.empty((wl.E, wl.block_bytes), dtype=torch.uint8, device="cuda")
    sg.fill_layer_blocks(wl, 0, blocks)
    ptrs = m.expert_ptr_table(blocks)
    x = sg.activations(wl, 0, 0, device="cuda")
    idx, w = sg.routing(wl)
    idx, w = idx.cuda(), w.cuda()
    out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16 if wl.out_bf16 else torch.float32, device="cuda")
    ws = m.alloc_workspace(d, wl.T, m.MOE_MODE_PREFILL)
    od = m.MOE_OUT_BF16 if wl.out_bf16 else m.MOE_OUT_F32
    log(f"[bench] {wl.name}: {wl.E} experts resident ({blocks.numel() / 2**30:.2f} GiB), "
        f"{wl.T} tokens, set up in {time.time() - t0:.1f} s")
    K, W = args.steps, args.warmup
    # warmup: at least W calls and at least 0.5 s of them (a few calls leave
    # the GPU short of its steady clocks: 3 calls after 3 warmup calls time
    # 20% slower than calls after half a second of work)
    t_w, n_w = time.perf_counter(), 0
    while n_w < W or time.perf_counter() - t_w < 0.5:
        m.moe_expert_prefill(d, x, wl.T, ptrs, idx, w, out, od, ws)
        n_w += 1
        if n_w % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    if args.profile_run:
        phase_marker(torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        m.moe_expert_prefill(d, x, wl.T, ptrs, idx, w, out, od, ws)
    e1.record()
    torch.cuda.synchronize()
    if args.profile_run:
        phase_marker(torch)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    flops, byts, touched = prefill_flops_bytes(wl, idx, wl.out_bf16)
    tflops = flops / (ms * 1e-3) / 1e12
    gbps = byts / (ms * 1e-3) / 1e9
    mfma_peak = 2500.0 if wl.fmt == "nvfp4" else 10100.0
    res = {
        "metric": METRIC, "value": round(wl.T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": n_w, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16 (gate/up) and bf16 (down) MFMA, f32 accumulate" if wl.fmt == "nvfp4" else "mxfp4 MFMA, f32 accumulate",
        "data": "synthetic (seeded SplitMix64; random-code FP4 experts, no trained weights)",
        "config": {"workload": wl.name, "experts": wl.E, "top_k": wl.k, "hidden": wl.H, "intermediate": wl.I,
                   "weights": wl.fmt, "tokens": wl.T, "assignments": int(idx.numel()), "experts_touched": touched,
                   "routing": f"{wl.routing} (s={wl.zipf_s})" if wl.routing == "zipf" else wl.routing,
                   "out": "bf16" if wl.out_bf16 else "f32", "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "moe_expert_prefill (grouping + quantise + grouped GEMMs + combine)",
                     "bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic_for(wl.name, "prefill"),
                     "bytes_per_launch": int(byts), "avg_us": round(ms * 1e3, 2)},
        "mfma_TFLOPs": round(tflops, 2), "mfma_peak_TFLOPs": mfma_peak,
        "mfma_frac": round(tflops / mfma_peak, 4), "flops_per_call": flops,
        # the fp32 expert outputs Y [assignments][H], written by the down GEMM
        # and read back by the combine: bytes beyond the algorithmic ones
        "y_round_trip": {"bytes": 2 * int(idx.numel()) * wl.H * 4,
                         "share_of_algorithmic": round(2 * int(idx.numel()) * wl.H * 4 / byts, 4)},
    }
    if args.profile_run:
        res["profile_run"] = True
    elif not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(sg, wl, blocks, x, idx, w)
    return res


FP8_WORKLOADS = {
    # rows = tokens of the DeepSeek-shaped hidden size; the pages check the
    # quantiser at 1, 17, 300 and 1024 rows ([D] "Three bugs", item 2)
    "fp8_act_quant": {"rows": 1024, "cols": 4096, "block": 32, "rule": "floor"},
    # a dense FP8 matrix of the Qwen-shaped hidden size (the pages give no
    # shape for their FP8 matrices; 8192 x 2560 stands in for them)
    "fp8_gemv": {"rows": 8192, "cols": 2560},
}


def run_fp8(args, m, sg, torch):
    """The FP8 kernels beside the MoE path: K calls captured in a HIP graph,
    rotating over input replicas that together exceed the 256 MB MALL, so
    every call reads HBM."""
    cfg = dict(FP8_WORKLOADS[args.workload])
    K, W = args.steps, args.warmup
    rows, cols = cfg["rows"], cfg["cols"]
    if args.workload == "fp8_act_quant":
        block, rule = cfg["block"], (m.MOE_SCALE_FLOOR if cfg["rule"] == "floor" else m.MOE_SCALE_CEIL)
        in_bytes = rows * cols * 4
        nrep = max(2, -(-384 * 2**20 // in_bytes))
        xs = [sg.fp8_activations(rows, cols, r, device="cuda") for r in range(nrep)]
        codes = [torch.empty((rows, cols), dtype=torch.uint8, device="cuda") for _ in range(nrep)]
        scales = [torch.empty((rows, cols // block), dtype=torch.uint8, device="cuda") for _ in range(nrep)]

        def call(i):
            j = i % nrep
            m.moe_act_quant_fp8(xs[j], rows, cols, block, rule, codes[j], scales[j])
        nbytes = in_bytes + rows * cols + rows * cols // block
        kernel, unit_name = "k_act_quant_fp8", "rows/s"
    else:
        mat_bytes = rows * cols
        nrep = max(2, -(-384 * 2**20 // mat_bytes))
        Ws = [sg.fp8_matrix(rows, cols, r, device="cuda") for r in range(nrep)]
        ss = [sg.fp8_row_scales(rows, r, device="cuda") for r in range(nrep)]
        x = sg.fp8_vector(cols, 0, device="cuda")
        ys = [torch.empty(rows, device="cuda") for _ in range(nrep)]

        def call(i):
            j = i % nrep
            m.moe_gemv_fp8(Ws[j], ss[j], x, rows, cols, ys[j])
        nbytes = mat_bytes + 8 * rows + 4 * cols
        kernel, unit_name = "k_gemv_fp8", "GEMV/s"
    for i in range(W):
        call(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            for i in range(K):
                call(i)
    torch.cuda.current_stream().wait_stream(cs)
    g.replay()
    torch.cuda.synchronize()
    if args.profile_run:
        phase_marker(torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    if args.profile_run:
        phase_marker(torch)
        torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / K
    gbps = nbytes / (us * 1e-6) / 1e9
    res = {
        "metric": METRIC, "value": round((rows if args.workload == "fp8_act_quant" else 1) / (us * 1e-6), 1),
        "unit": unit_name, "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 in, e4m3 out" if args.workload == "fp8_act_quant" else "e4m3 weights, f32 accumulate",
        "data": "synthetic (seeded SplitMix64)",
        "config": {"workload": args.workload, **cfg, "replicas": nrep, "launch": "hip_graph",
                   "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": kernel, "bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic_for(args.workload, "fp8"),
                     "bytes_per_launch": nbytes, "avg_us": round(us, 3)},
    }
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        t0 = time.perf_counter()
        if args.workload == "fp8_act_quant":
            n = 64
            O.quant_fp8_rows(xs[0][:n].cpu().numpy(), block=block, rule=rule)
            el = time.perf_counter() - t0
            res["cpu_baseline"] = {"value": n / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
                                   "sample": f"{n} of {rows} rows, {cols} values each"}
        else:
            O.gemv_fp8(Ws[0].cpu().numpy(), ss[0].cpu().numpy(), x.cpu().numpy())
            el = time.perf_counter() - t0
            res["cpu_baseline"] = {"value": 1.0 / el, "unit": "GEMV/s", "cores": 1, "kind": "oracle",
                                   "sample": f"one full {rows} x {cols} product (fp64)"}
    return res


def run_tier(args, m, sg, torch):
    """Qwen-shaped decode with every expert in pinned host memory behind an
    HBM slot cache (moe_tier): per token, the layers read through the tier's
    tables (misses over PCIe, in place), the routing is read back, and the
    tier promotes the step's misses. Reported for a slot pool of
    --tier-slots experts (default a quarter of all) and with no slots (every
    expert read from host memory)."""
    import numpy as np
    wl = sg.get("qwen_decode")
    L = args.tier_layers
    E, k, bb = wl.E, wl.k, wl.block_bytes
    d = m.desc(wl.H, wl.I, E, k, wl.fmt)
    t0 = time.time()
    host = torch.empty((L * E, bb), dtype=torch.uint8, pin_memory=True)
    buf = torch.empty((E, bb), dtype=torch.uint8, device="cuda")
    for l in range(L):
        sg.fill_layer_blocks(wl, l, buf)
        host[l * E:(l + 1) * E].copy_(buf)
    del buf
    Wr = [sg.router_weights(wl, l, device="cuda") for l in range(L)]
    # skewed routing: the router rows of a seeded set of hot experts per layer
    # scaled by tier_hot_scale, so those experts win the top-k more often
    # (the synthetic router alone routes almost uniformly)
    hot = max(0, args.tier_hot)
    Wr_hot = []
    for l in range(L):
        perm = torch.argsort(sg.words(sg.stream_key(77, l), E, device="cuda"))
        sc = torch.ones(E, device="cuda")
        sc[perm[:hot]] = args.tier_hot_scale
        Wr_hot.append((Wr[l] * sc[:, None]).contiguous())
    shared = [[t.contiguous() for t in sg.shared_expert(wl, l, device="cuda")] for l in range(L)]
    K, W = args.steps, args.warmup
    xs = [[sg.activations(wl, s, l, T=1, device="cuda").view(-1) for l in range(L)] for s in range(W + K)]
    log(f"[bench] tier: {L} layers x {E} experts in pinned host memory ({host.numel() / 2**30:.1f} GiB), "
        f"set up in {time.time() - t0:.1f} s")
    # host -> device copy rate of pinned memory (1 GiB)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    src = host.view(-1)[:1 << 30]
    dst.copy_(src)
    torch.cuda.synchronize()
    c0 = time.perf_counter()
    for _ in range(3):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    h2d = 3 * (1 << 30) / (time.perf_counter() - c0) / 1e9
    del dst

    def run(n_slots, Wr):
        slots = torch.empty((n_slots, bb), dtype=torch.uint8, device="cuda") if n_slots else None
        table = torch.empty(L * E, dtype=torch.int64, device="cuda")
        tier = m.ExpertTier(d, L, host, slots, n_slots, table)
        ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
        y = torch.empty(wl.H, device="cuda")
        idx = torch.empty((L, k), dtype=torch.int32, device="cuda")
        w = torch.empty((L, k), device="cuda")
        idx_h = torch.empty((L, k), dtype=torch.int32, pin_memory=True)
        try:
            def step(s):
                for l in range(L):
                    m.moe_layer_decode(d, xs[s][l], Wr[l], tier.table(l), shared[l], y, idx[l], w[l], ws)
                idx_h.copy_(idx, non_blocking=True)
                torch.cuda.current_stream().synchronize()  # the routing reaches the host
                tier.update(idx_h.numpy(), args.tier_promote)
            for s in range(W):
                step(s)
            torch.cuda.synchronize()
            st0 = tier.stats()
            c0 = time.perf_counter()
            for s in range(W, W + K):
                step(s)
            torch.cuda.synchronize()
            el = time.perf_counter() - c0
            st = tier.stats()
        finally:
            tier.close()
        hits, misses = st["hits"] - st0["hits"], st["misses"] - st0["misses"]
        return {"tokens_per_s": round(K / el, 2), "ms_per_token": round(el / K * 1e3, 3),
                "hit_rate": round(hits / max(1, hits + misses), 4),
                "host_read_GBps": round(misses * bb / el / 1e9, 2),
                "promoted_GBps": round((st["promotions"] - st0["promotions"]) * bb / el / 1e9, 2),
                "slots": n_slots}
    n_slots = args.tier_slots if args.tier_slots >= 0 else (L * E) // 4
    tiered = run(n_slots, Wr)
    host_only = run(0, Wr)
    skewed = {"hot_experts_per_layer": hot, "hot_router_scale": args.tier_hot_scale,
              "tiered": run(n_slots, Wr_hot), "host_only": run(0, Wr_hot)}
    pcie_peak = 64.0  # PCIe 5.0 x16, one direction
    res = {
        "metric": METRIC, "value": tiered["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": tiered["ms_per_token"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded SplitMix64; random-code FP4 experts, no trained weights)",
        "config": {"workload": "qwen_tier", "layers": L, "experts": E, "top_k": k, "hidden": wl.H,
                   "intermediate": wl.I, "weights": "nvfp4", "shared_expert": "bf16 (HBM)",
                   "expert_store": "pinned host memory + HBM slot cache", "slots": n_slots,
                   "max_promote_per_token": args.tier_promote, "routing_readback": "per token",
                   "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "decode layers reading missed experts from pinned host memory", "bound": "pcie",
                     "achieved": host_only["host_read_GBps"], "peak": pcie_peak, "unit": "GB/s",
                     "frac": round(host_only["host_read_GBps"] / pcie_peak, 4), "traffic": None,
                     "bytes_per_launch": k * bb, "note": "achieved = expert bytes read over the host link per second "
                     "with no slots (every routed expert a miss)"},
        "tiered": tiered, "host_only": host_only, "skewed_routing": skewed,
        "h2d_copy_GBps_measured": round(h2d, 2),
    }
    return res


def run_speculate(args, m, sg, torch):
    """Speculative next-layer routing on the 48-layer Qwen-shaped decode: while
    layer l runs, a second stream routes layer l+1's router on layer l's input
    and reads the guessed experts' blocks (moe_expert_prefetch) so they sit in
    the MALL when layer l+1 needs them. The layer inputs are a synthetic
    residual stream, x_l = x_(l-1) + 0.5 e_l with fresh N(0, 1) draws e_l, so
    that consecutive layers' inputs are correlated (with independent inputs
    per layer any guess would hit by chance only). Both runs (with and without
    speculation) are HIP graphs of the same K steps."""
    import numpy as np
    wl = sg.get("qwen_decode")
    model = DecodeModel(m, sg, wl)
    L, K, W = wl.layers, args.steps, args.warmup
    d = model.d
    xs = []
    for s in range(W + K):
        row, prev = [], None
        for l in range(L):
            e = sg.activations(wl, s, l, T=1, device="cuda").view(-1)
            prev = e if prev is None else prev + 0.5 * e
            row.append(prev.contiguous())
        xs.append(row)
    ws = m.alloc_workspace(d, 1, m.MOE_MODE_DECODE)
    wsr = m.alloc_workspace(d, 1, m.MOE_MODE_ROUTE)
    y = torch.empty(wl.H, device="cuda")
    idx = torch.empty((W + K, L, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((L, wl.k), device="cuda")
    guess = torch.full((W + K, L, wl.k), -1, dtype=torch.int32, device="cuda")
    gw = torch.empty((L, wl.k), device="cuda")
    sink = torch.empty(m.moe_prefetch_sink_bytes(d, wl.k) // 4 * L, dtype=torch.int32, device="cuda")
    nsink = m.moe_prefetch_sink_bytes(d, wl.k) // 4
    s2 = torch.cuda.Stream()

    def step(s, spec):
        cs = torch.cuda.current_stream()
        for l in range(L):
            if spec and l + 1 < L:
                ev = torch.cuda.Event()
                ev.record(cs)  # layer l's input exists from here on
                s2.wait_event(ev)
                m.moe_route(d, xs[s][l], 1, model.Wr[l + 1], guess[s, l + 1], gw[l + 1], None, wsr, stream=s2)
                m.moe_expert_prefetch(d, model.ptrs[l + 1], guess[s, l + 1], wl.k, sink[l * nsink:(l + 1) * nsink],
                                      stream=s2)
            m.moe_layer_decode(d, xs[s][l], model.Wr[l], model.ptrs[l], model.shared[l], y, idx[s, l], w[l], ws)
        if spec:
            cs.wait_stream(s2)

    def timed(spec):
        for s in range(W):
            step(s, spec)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            with torch.cuda.graph(g, stream=cs):
                for s in range(W, W + K):
                    step(s, spec)
        torch.cuda.current_stream().wait_stream(cs)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    ms_plain = timed(False)
    ms_spec = timed(True)
    gi, ai = guess[W:, 1:].cpu().numpy(), idx[W:, 1:].cpu().numpy()
    hit = np.mean([len(set(gi[s, l]) & set(ai[s, l])) / wl.k for s in range(K) for l in range(L - 1)])
    experts, router, shared, act = bytes_per_layer(wl)
    layer_bytes = experts + router + shared + act
    res = {
        "metric": METRIC, "value": round(1e3 / ms_spec, 2), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_spec, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded SplitMix64; residual-stream inputs x_l = x_(l-1) + 0.5 e_l)",
        "config": {"workload": "qwen_speculate", "layers": L, "experts": wl.E, "top_k": wl.k, "hidden": wl.H,
                   "intermediate": wl.I, "weights": "nvfp4", "shared_expert": "bf16", "launch": "hip_graph",
                   "speculation": "moe_route(x_l, Wr_(l+1)) + moe_expert_prefetch on a second stream",
                   "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "48 decode layers (moe_layer_decode) with speculative prefetch beside them",
                     "bound": "hbm", "achieved": round(layer_bytes * L / (ms_spec * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(layer_bytes * L / (ms_spec * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None,
                     "bytes_per_launch": layer_bytes * L},
        "without_speculation": {"tokens_per_s": round(1e3 / ms_plain, 2), "ms_per_step": round(ms_plain, 4)},
        "guess_hit_rate": round(float(hit), 4),
    }
    return res


def summarize(root: str) -> None:
    """Per-phase kernel tables from rocprofv3 CSV output (kernel trace or
    counter collection) of a --profile-run: the phases are the intervals
    between the marker kernels (phase 1: the timed region; decode phase 3: the
    expert-call probes); a run without markers is one phase."""
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True) +
                   glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        print(f"no rocprofv3 CSV under {root}")
        return
    for fn in files:
        disp = {}  # dispatch id -> [name, start, end, {counter: value}]
        with open(fn) as f:
            for r in csv.DictReader(f):
                d = disp.setdefault(r["Dispatch_Id"], [r["Kernel_Name"], int(r["Start_Timestamp"]),
                                                       int(r["End_Timestamp"]), {}])
                if "Counter_Name" in r:
                    d[3][r["Counter_Name"]] = d[3].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        rows = sorted(disp.values(), key=lambda d: d[1])
        marks = [d[1] for d in rows if "spin_kernel" in d[0]]
        bounds = list(zip(marks, marks[1:])) if len(marks) >= 2 else [(rows[0][1] - 1, rows[-1][2] + 1)]
        outside = sum(1 for d in rows if not any(lo < d[1] < hi for lo, hi in bounds))
        print(f"### {os.path.relpath(fn, root)}\n")
        print(f"{len(marks)} phase markers; {outside} dispatches outside the phases (set-up, warmup)\n")
        for ph, (lo, hi) in enumerate(bounds, 1):
            sel = [d for d in rows if lo < d[1] < hi and "spin_kernel" not in d[0]]
            if not sel:
                continue
            by = {}
            for d in sel:
                by.setdefault(d[0], []).append(d)
            counters = sorted({c for d in sel for c in d[3]})
            print(f"phase {ph}: {len(sel)} dispatches, {(max(d[2] for d in sel) - min(d[1] for d in sel)) / 1e3:.1f} us "
                  f"first start to last end\n")
            if counters:
                print("| kernel | dispatches | " + " | ".join(f"{c} (mean)" for c in counters) + " |")
                print("|---|---|" + "---|" * len(counters))
            else:
                print("| kernel | dispatches | avg us | min us | max us | total us |")
                print("|---|---|---|---|---|---|")
            for name, ds in sorted(by.items(), key=lambda kv: -sum(d[2] - d[1] for d in kv[1])):
                if counters:
                    vals = [statistics.fmean([d[3].get(c, 0.0) for d in ds]) for c in counters]
                    print(f"| `{name[:90]}` | {len(ds)} | " + " | ".join(f"{v:,.1f}" for v in vals) + " |")
                else:
                    us = [(d[2] - d[1]) / 1e3 for d in ds]
                    print(f"| `{name[:90]}` | {len(ds)} | {statistics.fmean(us):.2f} | {min(us):.2f} | "
                          f"{max(us):.2f} | {sum(us):.1f} |")
            print()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen_decode")
    ap.add_argument("--replicas", type=int, default=0, help="layer replicas to rotate through (cold timing)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tier-layers", type=int, default=8, help="qwen_tier: layers in pinned host memory")
    ap.add_argument("--tier-slots", type=int, default=-1, help="qwen_tier: HBM slots (default: a quarter)")
    ap.add_argument("--tier-promote", type=int, default=16, help="qwen_tier: promotions per token at most")
    ap.add_argument("--tier-hot", type=int, default=48, help="qwen_tier: hot experts per layer (skewed run)")
    ap.add_argument("--tier-hot-scale", type=float, default=3.0, help="qwen_tier: router scale of hot experts")
    ap.add_argument("--profile-run", action="store_true",
                    help="for rocprofv3: marker kernels around the timed region (phase 1) and, in a decode "
                         "run, around the expert-call probes (phase 3, after the replay that precedes them); "
                         "no copy-bandwidth probe and no CPU baseline")
    ap.add_argument("--summarize", metavar="DIR",
                    help="print per-phase kernel tables from the rocprofv3 CSVs under DIR (no GPU needed)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run 4 device copies of 1 GiB (calibrates the FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path, and each "
              "step computes the whole MoE layer on that GPU.", file=sys.stderr)
        sys.exit(2)
    import torch

    import block_scaled_fp4_route_amd as m
    import synthgen as sg
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        a = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": 1 << 30, "copies": 4}), flush=True)
        return
    if args.workload in FP8_WORKLOADS:
        res = run_fp8(args, m, sg, torch)
    elif args.workload == "qwen_tier":
        res = run_tier(args, m, sg, torch)
    elif args.workload == "qwen_speculate":
        res = run_speculate(args, m, sg, torch)
    else:
        wl = sg.get(args.workload)
        res = run_prefill(args, m, sg, torch) if wl.is_prefill else run_decode(args, m, sg, torch)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
