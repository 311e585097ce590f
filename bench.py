#!/usr/bin/env python3
"""Benchmark of the routed-MoE layer (ds4moe) on one MI355X.

Headline (one JSON line on stdout): decode throughput of one DeepSeek V4
Flash-shaped MoE layer at batch 1 -- d_model 4096, 256 routed experts, top-6
+ 1 shared, expert intermediate 2048, CB2 gate/up + Q2K down, F16 router and
shared expert, bf16 activations -- in layer-tokens per second.

  * inputs are resident in HBM before timing; each step is one
    ds4moe_forward_decode (router, top-k, grouping, gate/up, down, combine);
  * the packed layer is replicated into --copies device copies used round
    robin, each step with a fresh seeded token, so the 256 MB Infinity Cache
    cannot serve the shared/router weights from one step to the next;
  * the K timed steps are captured once into a HIP graph and replayed (the
    launch sequence a decode loop would submit), bracketed by events on the
    capture stream; the headline is the median of --repeats replays after an
    untimed first one; the eager (host-launched) median is reported beside it;
  * "roofline" covers the dominant decode kernel (the longest of the three
    stages): algorithmic bytes per launch / its mean duration from the
    start/stop events the library attaches to each kernel dispatch
    (hipExtLaunchKernel) during an eager pass over the same steps;
  * "measured_peaks" gives a device copy rate and a library fp16 GEMM rate
    on the same GPU beside the vendor peaks;
  * "prefill" times ds4moe_forward_prefill on a 2048-token chunk with
    Zipf-like expert loads against the dense fp16 MFMA peak;
  * "decode16" times the 16-token batched decode (about 60 distinct experts);
  * "decode_small" times speculative-verify shapes, T = 2, 4, 8 tokens per
    call at the decode1 layer shape;
  * "mxfp4" and "q4k" time the decode1 shape and the 2048-token prefill with
    MXFP4 and with Q4K routed experts;
  * "hc" times the hyper-connection mixer (4 streams of 4096, 20 Sinkhorn
    iterations) around the layer at T = 1 and T = 2048;
  * "stack43" times 43 decode1-shaped layers resident at once, one token at a
    time through all of them, first all CB2/Q2K, then as the q2-q4 mix (the
    last six layers' experts Q4K);
  * "cpu_baseline" times the CPU oracle on a bounded sample of decode tokens,
    on all host threads and on one.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor peak
WEIGHT_SIGMA = 0.02
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, vendor peak

METRIC = "routed-MoE layer decode tok/s + % HBM peak; 2048-tok prefill tok/s + % MFMA"

# HBM bytes per launch of the decode kernels, from rocprofv3 counter passes:
# the L2's read requests to memory by size (the terms of FETCH_SIZE, each
# 128-byte request at 128 bytes) and WRITE_SIZE, both checked against a
# 256 MiB device copy (factor 1.000); valid for the kernel sources with this
# hash only (profiles/decode_hbm_traffic.md holds the commands and counts).
TRAFFIC_SOURCE_HASH = "2f97323b2e9606f4"
TRAFFIC_BYTES = {"k_dec_stage1": 2.26e6, "k_dec_stage2": 60.09e6, "k_dec_stage3": 33.60e6}


def kernel_source_hash(csrc=None):
    """sha256 over the library's sources (name + code, sorted by name), with
    comments and whitespace removed, so that only a change to the code itself
    invalidates counters taken earlier."""
    import glob
    import hashlib
    import re
    csrc = csrc or os.path.join(ROOT, "bit_quantized_routed_router_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(csrc, "*"))):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(f, encoding="utf-8") as fh:
                code = fh.read()
            code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
            code = re.sub(r"//[^\n]*", " ", code)
            h.update(os.path.basename(f).encode())
            h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def expert_formats(efmt):
    """(gate/up format, down format, layer expert_fmt, label) of a routed-expert
    recipe: "cb2q2k" (CB2 gate/up, Q2K down), "mxfp4" or "q4k" (all three)."""
    from bit_quantized_routed_router_amd import ds4moe as D
    return {"cb2q2k": (D.FMT_CB2, D.FMT_Q2K, D.EXPERTS_CB2_Q2K, "CB2/Q2K"),
            "mxfp4": (D.FMT_MXFP4, D.FMT_MXFP4, D.EXPERTS_MXFP4, "MXFP4"),
            "q4k": (D.FMT_Q4K, D.FMT_Q4K, D.EXPERTS_Q4K, "Q4K")}[efmt]


def decode_bytes(cfg, n_distinct, T=1, efmt="cb2q2k"):
    """Algorithmic HBM bytes of one decode step and of each of its kernels:
    every weight byte the step needs read once, activations read/written once.
    stage 1: router; stage 2: routed gate/up + shared gate and up; stage 3:
    routed down + shared down."""
    from bit_quantized_routed_router_amd import ds4moe as D
    d, f, fs, E, k = cfg.d, cfg.f, cfg.fs, cfg.E, cfg.k
    fgu, fdn = expert_formats(efmt)[:2]
    cb = D.packed_bytes(fgu, f, d)
    qb = D.packed_bytes(fdn, d, f)
    x_bytes = T * d * 2
    s1 = E * d * 2 + x_bytes
    s2 = n_distinct * 2 * cb + 2 * fs * d * 2 + T * d * 2 + T * k * f * 2 + T * fs * 2
    s3 = n_distinct * qb + d * fs * 2 + T * fs * 2 + T * k * f * 2 + T * d * 4
    total = E * d * 2 + 3 * fs * d * 2 + n_distinct * (2 * cb + qb) + x_bytes + T * d * 4
    return dict(total=total, k_dec_stage1=s1, k_dec_stage2=s2, k_dec_stage3=s3)


def make_layer(cfg, copies=1, cfg_seed=None, efmt="cb2q2k"):
    import torch
    from bit_quantized_routed_router_amd import ds4moe as D
    from bit_quantized_routed_router_amd import synthetic as S

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).cuda()

    c = cfg
    fgu, fdn, ecode, label = expert_formats(efmt)
    cb = D.packed_bytes(fgu, c.f, c.d)
    qb = D.packed_bytes(fdn, c.d, c.f)
    gate = torch.empty(c.E * cb, dtype=torch.uint8, device="cuda")
    up = torch.empty(c.E * cb, dtype=torch.uint8, device="cuda")
    down = torch.empty(c.E * qb, dtype=torch.uint8, device="cuda")
    t0 = time.time()
    for e0 in range(0, c.E, 16):
        es = list(range(e0, min(c.E, e0 + 16)))
        for e, (g, u, dn) in zip(es, S.gen_experts(c, es, threads=16, cfg_seed=cfg_seed)):
            D.quantize(fgu, dev(g), c.f, c.d, gate[e * cb:(e + 1) * cb])
            D.quantize(fgu, dev(u), c.f, c.d, up[e * cb:(e + 1) * cb])
            D.quantize(fdn, dev(dn), c.d, c.f, down[e * qb:(e + 1) * qb])
        torch.cuda.synchronize()
    log(f"[bench] {c.name}: generated and quantized {c.E} {label} experts in {time.time() - t0:.1f}s")
    router = dev(S.gen_router(c, cfg_seed=cfg_seed))
    bias = S.gen_bias(c)
    bias = None if bias is None else dev(bias)
    sh = [dev(a) for a in S.gen_shared(c, cfg_seed=cfg_seed)]
    layers = [D.Layer(c.d, c.E, c.k, c.f, c.fs, router, bias, sh[0], sh[1], sh[2], gate, up, down, ecode)]
    for _ in range(1, copies):
        layers.append(D.Layer(c.d, c.E, c.k, c.f, c.fs, router.clone(), None if bias is None else bias.clone(),
                              sh[0].clone(), sh[1].clone(), sh[2].clone(), gate.clone(), up.clone(), down.clone(),
                              ecode))
    torch.cuda.synchronize()
    return layers


def bench_decode(args):
    import torch
    from bit_quantized_routed_router_amd import ds4moe as D
    from bit_quantized_routed_router_amd import synthetic as S

    cfg = S.CONFIGS["decode1"]
    layers = make_layer(cfg, copies=args.copies)
    nsteps = args.warmup + args.steps
    xs = np.concatenate([S.gen_x(cfg, variant=1000 + n) for n in range(nsteps)])
    x = torch.from_numpy(xs.view(np.int16)).cuda()
    y = torch.empty((nsteps, cfg.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((nsteps, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((nsteps, cfg.k), dtype=torch.float32, device="cuda")
    ws, wsn = layers[0].workspace(1, D.MODE_DECODE)

    def step(n, stream):
        L = layers[n % len(layers)]
        D.forward_decode(L.desc, x[n], D.DT_BF16, 1, y[n], idx[n], w[n], ws, wsn, stream=stream)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for n in range(args.warmup):
            step(n, s)
    torch.cuda.synchronize()

    def timed(run):
        """ms of one pass over the K timed steps, events on the launch stream,
        synchronized before and after."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            e0.record(s)
            run()
            e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def eager():
        for n in range(args.warmup, nsteps):
            step(n, s)

    # eager passes over the timed steps (host-launched)
    eager_runs = [timed(eager) / args.steps for _ in range(args.repeats)]
    eager_ms = float(np.median(eager_runs))
    y_eager = y.clone()

    # traced eager pass: per-kernel durations from the start/stop events the
    # library attaches to each kernel's dispatch (hipExtLaunchKernel)
    D.trace_read(reset=True)
    D.trace_enable(True)
    eager()
    torch.cuda.synchronize()
    D.trace_enable(False)
    kern = D.trace_read(reset=True)

    # graph: the timed steps captured once, replayed; the first replay is
    # untimed and checked against the eager results, then the median of
    # `repeats` timed replays
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for n in range(args.warmup, nsteps):
            step(n, torch.cuda.current_stream())
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    if not torch.equal(y[args.warmup:], y_eager[args.warmup:]):
        raise RuntimeError("graph replay differs from the eager run")
    graph_runs = [timed(g.replay) / args.steps for _ in range(args.repeats)]
    graph_ms = float(np.median(graph_runs))
    if not torch.equal(y[args.warmup:], y_eager[args.warmup:]):
        raise RuntimeError("graph replay differs from the eager run")

    # distinct experts per step (1 token: k distinct) -> algorithmic bytes;
    # the dominant kernel is the one with the largest share of the step time
    nb = decode_bytes(cfg, cfg.k, T=1)
    per = {}
    for name in ("k_dec_stage1", "k_dec_stage2", "k_dec_stage3"):
        # a stage's kernel is named for it, with template arguments or a
        # variant suffix (k_dec_stage3_one: the one-token form)
        hits = [v for k2, v in kern.items() if k2.split("<")[0] in (name, name + "_one")]
        ms = sum(v[0] for v in hits)
        cnt = sum(v[1] for v in hits)
        if cnt:
            us = ms / cnt * 1e3
            per[name] = dict(mean_us=us, bytes_per_launch=nb[name], gbs=nb[name] / (us * 1e-6) / 1e9)
    if not per:
        raise RuntimeError(f"no decode kernel in the trace: {sorted(kern)}")
    dom = max(per, key=lambda n: per[n]["mean_us"])
    achieved = per[dom]["gbs"]
    res = dict(ms_per_step=graph_ms, eager_ms_per_step=eager_ms, graph_runs_ms=graph_runs, eager_runs_ms=eager_runs,
               kernels={k: dict(mean_us=v[0] / max(v[1], 1) * 1e3,
               launches=v[1]) for k, v in kern.items()}, decode_kernels=per,
               roofline=dict(bound="hbm", kernel=dom, achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                             frac=achieved / HBM_PEAK_GBS,
                             timing="mean kernel duration over the K timed steps of one eager pass, from start/stop "
                                    "HIP events attached to each dispatch by hipExtLaunchKernel on the launch stream",
                             traffic=(TRAFFIC_BYTES[dom] if kernel_source_hash() == TRAFFIC_SOURCE_HASH
                                      else None),
                             traffic_unit="HBM bytes per launch",
                             bytes_per_launch=nb[dom], mean_launch_us=per[dom]["mean_us"]),
               layer_bytes=nb["total"], layer_gbs=nb["total"] / (graph_ms * 1e-3) / 1e9)
    res["layer_hbm_frac"] = res["layer_gbs"] / HBM_PEAK_GBS
    del layers, g
    torch.cuda.empty_cache()
    return res


def decode_batch(cfg, layers, T, steps, warmup, xvar0, efmt="cb2q2k"):
    """K graph-replayed T-token decode steps over the given layer copies (round
    robin) with fresh tokens per step.  Returns us/step, tok/s, the mean
    distinct-expert count and the whole-layer HBM fraction from the
    algorithmic bytes of the experts each step actually selected."""
    import torch
    from bit_quantized_routed_router_amd import ds4moe as D
    from bit_quantized_routed_router_amd import synthetic as S

    nsteps = warmup + steps
    xs = np.stack([S.gen_x(cfg, variant=xvar0 + n, T=T) for n in range(nsteps)])
    x = torch.from_numpy(xs.view(np.int16)).cuda()
    y = torch.empty((nsteps, T, cfg.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((nsteps, T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((nsteps, T, cfg.k), dtype=torch.float32, device="cuda")
    ws, wsn = layers[0].workspace(T, D.MODE_DECODE)

    def step(n, stream):
        L = layers[n % len(layers)]
        D.forward_decode(L.desc, x[n], D.DT_BF16, T, y[n], idx[n], w[n], ws, wsn, stream=stream)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for n in range(warmup):
            step(n, s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for n in range(warmup, nsteps):
            step(n, torch.cuda.current_stream())
    torch.cuda.synchronize()
    g.replay()  # first replay, untimed
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    with torch.cuda.stream(s):
        g.replay()
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    sel = idx[warmup:].cpu().numpy()
    distinct = [len(np.unique(sel[n])) for n in range(steps)]
    nbytes = float(np.mean([decode_bytes(cfg, nd, T=T, efmt=efmt)["total"] for nd in distinct]))
    del g
    # one eager pass with the library's dispatch-attached timer: per-kernel means
    D.trace_read(reset=True)
    D.trace_enable(True)
    with torch.cuda.stream(s):
        for n in range(warmup, nsteps):
            step(n, s)
    torch.cuda.synchronize()
    D.trace_enable(False)
    kern = D.trace_read(reset=True)
    return dict(tok_s=T / (ms * 1e-3), us_per_step=ms * 1e3, distinct_mean=float(np.mean(distinct)),
                bytes_per_step=nbytes, hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                kernels_us={k: round(v[0] / v[1] * 1e3, 2) for k, v in kern.items() if v[1] > 0})


def bench_decode16(copies=4, steps=64, warmup=8):
    """Side report: the 16-token batched decode (hot-pool router bias, about 60
    distinct experts per step)."""
    import torch
    from bit_quantized_routed_router_amd import synthetic as S

    cfg = S.CONFIGS["decode16"]
    layers = make_layer(cfg, copies=copies)
    r = decode_batch(cfg, layers, cfg.T, steps, warmup, 2000)
    del layers
    torch.cuda.empty_cache()
    return dict(workload=f"decode16: T={cfg.T}, hot-pool router bias, {copies} layer copies round-robin, "
                         "graph replay", **r)


def bench_decode_small(copies=4, steps=64, warmup=8, Ts=(2, 4, 8)):
    """Side report: speculative-verify and small-batch shapes, T = 2, 4, 8
    tokens per decode call at the decode1 layer shape (no router bias, so the
    T * 6 slots mostly select distinct experts)."""
    import torch
    from bit_quantized_routed_router_amd import synthetic as S

    cfg = S.CONFIGS["decode1"]
    layers = make_layer(cfg, copies=copies)
    out = {}
    for T in Ts:
        r = decode_batch(cfg, layers, T, steps, warmup, 3000 + 100 * T)
        out[f"T{T}"] = r
    del layers
    torch.cuda.empty_cache()
    return dict(workload=f"decode at T = {', '.join(map(str, Ts))}: decode1 layer shape, {copies} layer copies "
                         "round-robin, graph replay", **out)


def bench_wide(efmt, steps=64, warmup=8, copies=4):
    """Side report: a layer whose routed experts are MXFP4 (the model's native
    expert format) or Q4K (the Q4 layers of the q2-q4 mix), decode at T = 1
    over layer copies with graph replay."""
    import torch
    from bit_quantized_routed_router_amd import synthetic as S

    cfg = S.CONFIGS["decode1"]
    layers = make_layer(cfg, copies=copies, efmt=efmt)
    r = decode_batch(cfg, layers, 1, steps, warmup, 4000, efmt=efmt)
    del layers
    torch.cuda.empty_cache()
    return dict(workload=f"decode1 shape with {expert_formats(efmt)[3]} routed experts (gate, up, down), T=1, "
                         f"{copies} layer copies round-robin, graph replay", **r)


def bench_prefill(args, efmt="cb2q2k"):
    import torch
    from bit_quantized_routed_router_amd import ds4moe as D
    from bit_quantized_routed_router_amd import synthetic as S

    cfg = S.CONFIGS["prefill"]
    L = make_layer(cfg, efmt=efmt)[0]
    x = torch.from_numpy(S.gen_x(cfg).view(np.int16)).cuda()
    T = cfg.T
    y = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")
    ws, wsn = L.workspace(T, D.MODE_PREFILL)
    for _ in range(5):  # warm-up: the first calls after packing run slower (clocks, caches)
        D.forward_prefill(L.desc, x, D.DT_BF16, T, y, None, None, None, ws, wsn)
    torch.cuda.synchronize()
    runs = []
    for _ in range(args.repeats):  # median of `repeats` calls, each bracketed by events
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        D.forward_prefill(L.desc, x, D.DT_BF16, T, y, None, None, None, ws, wsn)
        e1.record()
        torch.cuda.synchronize()
        runs.append(e0.elapsed_time(e1))
    ms = float(np.median(runs))
    D.trace_read(reset=True)
    D.trace_enable(True)
    D.forward_prefill(L.desc, x, D.DT_BF16, T, y, None, None, None, ws, wsn)
    torch.cuda.synchronize()
    D.trace_enable(False)
    kern = D.trace_read(reset=True)
    flop = 2 * T * cfg.k * 3 * cfg.d * cfg.f + 2 * T * 3 * cfg.d * cfg.fs + 2 * T * cfg.E * cfg.d
    tflops = flop / (ms * 1e-3) / 1e12
    del L
    torch.cuda.empty_cache()
    return dict(workload=f"prefill T={T}, Zipf(1.1)-shaped expert loads, {expert_formats(efmt)[3]} routed experts",
                tok_s=T / (ms * 1e-3), ms=ms, runs_ms=runs,
                flop=flop, tflops=tflops, mfma_frac=tflops / MFMA_F16_PEAK_TFLOPS,
                kernels={k: dict(mean_us=v[0] / v[1] * 1e3, launches=v[1]) for k, v in kern.items() if v[1] > 0})


def bench_stack43(nlayers=43, tokens=256, warmup=16, repeats=3, n_q4=6):
    """The 43-layer stack of decode1-shaped layers, every layer's packed
    experts resident in HBM at once (about 80 GB), one token at a time
    through all layers (T = 1 per call).  Timed twice: all layers CB2/Q2K,
    then as the q2-q4 mix, the last `n_q4` layers' experts re-packed as Q4K
    from the same fp32 draws.

    Weights: layer l draws its fp32 weights N(0, 0.02) on the device from
    torch's generator seeded 1000 + l and packs them with ds4moe_quantize
    (untimed); router and shared expert are drawn likewise and rounded to
    binary16.  Inputs: each (layer, token) gets its own pre-drawn bf16
    N(0, 1) row (teacher forcing, as in the stack's parity test), so the
    timed region holds library calls only; the residual and normalisation
    between layers are outside the layer and not timed."""
    import torch
    from bit_quantized_routed_router_amd import ds4moe as D
    from bit_quantized_routed_router_amd import synthetic as S

    c = S.CONFIGS["stack43"]
    gen = torch.Generator(device="cuda")

    def pack_layer(l, efmt):
        fgu, fdn, ecode, _ = expert_formats(efmt)
        gen.manual_seed(1000 + l)
        packed = []
        for fmt, rows, cols in ((fgu, c.f, c.d), (fgu, c.f, c.d), (fdn, c.d, c.f)):
            nb = D.packed_bytes(fmt, rows, cols)
            w = torch.randn((c.E, rows * cols), generator=gen, device="cuda", dtype=torch.float32).mul_(WEIGHT_SIGMA)
            buf = torch.empty(c.E * nb, dtype=torch.uint8, device="cuda")
            for e in range(c.E):
                D.quantize(fmt, w[e], rows, cols, buf[e * nb:(e + 1) * nb])
            del w
            packed.append(buf)
        f16 = [torch.randn(n, generator=gen, device="cuda").mul_(WEIGHT_SIGMA).half()
               for n in (c.E * c.d, c.fs * c.d, c.fs * c.d, c.d * c.fs)]
        L = D.Layer(c.d, c.E, c.k, c.f, c.fs, f16[0], None, f16[1], f16[2], f16[3], *packed, ecode)
        return L, sum(t.numel() * t.element_size() for t in packed + f16)

    t0 = time.time()
    layers, sizes, recipe = [], [], ["cb2q2k"] * nlayers
    for l in range(nlayers):
        L, nbytes = pack_layer(l, "cb2q2k")
        layers.append(L)
        sizes.append(nbytes)
        if l % 8 == 7:
            torch.cuda.synchronize()
            log(f"[bench] stack43: {l + 1} layers packed, {time.time() - t0:.1f}s")
    torch.cuda.synchronize()
    pack_s = time.time() - t0
    nsteps = warmup + tokens
    gen.manual_seed(5000)
    x = torch.randn((nlayers, nsteps, c.d), generator=gen, device="cuda").to(torch.bfloat16)
    y = torch.empty((nlayers, nsteps, c.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((nlayers, nsteps, c.k), dtype=torch.int32, device="cuda")
    ws, wsn = layers[0].workspace(1, D.MODE_DECODE)
    s = torch.cuda.Stream()

    def run(n0, n1, stream):
        for n in range(n0, n1):
            for l in range(nlayers):
                D.forward_decode(layers[l].desc, x[l, n], D.DT_BF16, 1, y[l, n], idx[l, n], None, ws, wsn,
                                 stream=stream)

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            e0.record(s)
            fn()
            e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def measure(name):
        with torch.cuda.stream(s):
            run(0, warmup, s)
        eager_runs = [timed(lambda: run(warmup, nsteps, s)) for _ in range(repeats)]
        y_eager = y.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            run(warmup, nsteps, torch.cuda.current_stream())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(y, y_eager):
            raise RuntimeError(f"stack43 {name}: graph replay differs from the eager run")
        graph_runs = [timed(g.replay) for _ in range(repeats)]
        del g, y_eager
        ms = float(np.median(graph_runs)) / tokens
        eager_ms = float(np.median(eager_runs)) / tokens
        sel = idx[:, warmup:].cpu().numpy()
        distinct = float(np.mean([len(np.unique(sel[l, n])) for l in range(nlayers) for n in range(tokens)]))
        per_token = sum(decode_bytes(c, c.k, T=1, efmt=r)["total"] for r in recipe)
        return dict(recipe=name, tok_s=1.0 / (ms * 1e-3), us_per_token=ms * 1e3, eager_us_per_token=eager_ms * 1e3,
                    bytes_per_token=per_token, hbm_frac=per_token / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    resident_bytes=sum(sizes), distinct_per_layer=distinct)

    q2 = measure("q2 (all layers CB2/Q2K)")
    for l in range(nlayers - n_q4, nlayers):  # the q2-q4 mix: the last layers' experts at Q4K
        layers[l] = None
        torch.cuda.empty_cache()
        layers[l], sizes[l] = pack_layer(l, "q4k")
        recipe[l] = "q4k"
    torch.cuda.synchronize()
    mix = measure(f"q2-q4 (last {n_q4} layers Q4K)")
    del layers, x, y
    torch.cuda.empty_cache()
    return dict(q2, workload=f"stack43: {nlayers} decode1-shaped layers resident, {tokens} tokens x {nlayers} "
                             f"layers, T=1 per call, teacher-forced seeded inputs, graph replay (median of "
                             f"{repeats})", pack_s=pack_s, q2q4=mix)


def hc_bytes(d, T, n=4):
    """Bytes each mixer kernel moves by design, and the step's algorithmic
    bytes (streams read once): pre reads the projection and the streams,
    writes the coefficients, the fp32 and the bf16 reduced rows; post reads
    the streams, y and the coefficients and writes the streams."""
    no, nd = 2 * n + n * n, n * d
    ks = 1024 if T > 64 else 256
    part = (nd // ks) * T * 32 * 4
    x = T * nd * 4
    outs = T * (no * 4 + d * 4 + d * 2)
    if T <= 2:  # one launch: the partial kernel's last block also finishes the tokens
        partial = no * nd * 4 + 2 * x + 2 * part + outs
    else:
        partial = no * nd * 4 + x + part
    return dict(k_hc_partial=partial, k_hc_reduce=x + part + outs,
                k_hc_post=2 * x + T * (d * 4 + no * 4),
                pre_algorithmic=no * nd * 4 + x + outs, post_algorithmic=2 * x + T * (d * 4 + no * 4))


def bench_hc(repeats=5, copies=192, steps=192):
    """Side report: the hyper-connection mixer around the layer (4 streams of
    4096, 20 Sinkhorn iterations).  Decode: T = 1, `copies` mixers (distinct
    projections, 1.5 MB each, more than the 256 MB Infinity Cache holds)
    round-robin with fresh streams per step, pre + post captured in one graph;
    prefill: T = 2048, pre and post timed by events (median of `repeats`).
    Per-kernel times come from the library's dispatch-attached events."""
    import torch
    from bit_quantized_routed_router_amd import ds4moe as D
    from bit_quantized_routed_router_amd import synthetic as S

    d = 4096
    out = {}
    # decode
    X, phi, bias, alpha, y = S.gen_hc(d, steps)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    phis = torch.randn((copies, 24, 4 * d), generator=gen, device="cuda").mul_(1.0 / 128.0)
    bias_d = torch.from_numpy(bias).cuda()
    mixers = [D.Hc(d, phis[i], bias_d, alpha, S.HC_EPS, S.HC_SINKHORN_ITERS) for i in range(copies)]
    Xd = torch.from_numpy(X).cuda()
    yd = torch.from_numpy(y).cuda()
    Xo = torch.empty_like(Xd)
    coef = torch.empty((steps, 24), dtype=torch.float32, device="cuda")
    xo = torch.empty((steps, d), dtype=torch.float32, device="cuda")
    xb = torch.empty((steps, d), dtype=torch.int16, device="cuda")
    ws, wsn = mixers[0].workspace(1)

    def step(i, stream):
        H = mixers[i % copies].desc
        D.hc_pre(H, Xd[i], 1, coef[i], xo[i], xb[i], ws, wsn, stream=stream)
        D.hc_post(H, Xd[i], yd[i], coef[i], 1, Xo[i], stream=stream)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for i in range(steps):
            step(i, s)
    torch.cuda.synchronize()
    D.trace_read(reset=True)
    D.trace_enable(True)
    with torch.cuda.stream(s):
        for i in range(steps):
            step(i, s)
    torch.cuda.synchronize()
    D.trace_enable(False)
    kern = D.trace_read(reset=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(steps):
            step(i, torch.cuda.current_stream())
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    runs = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        with torch.cuda.stream(s):
            g.replay()
        e1.record(s)
        torch.cuda.synchronize()
        runs.append(e0.elapsed_time(e1) / steps)
    del g
    b = hc_bytes(d, 1)
    ku = {k: v[0] / v[1] * 1e3 for k, v in kern.items() if v[1] > 0}
    out["decode"] = dict(workload=f"T=1, {copies} mixers round-robin, pre + post per step, graph replay (median of "
                                  f"{repeats})", us_per_step=float(np.median(runs)) * 1e3,
                         kernels_us={k: round(v, 2) for k, v in ku.items()},
                         kernel_gbs={k: round(b[k.split("<")[0]] / (ku[k] * 1e-6) / 1e9, 1) for k in ku
                                     if k.split("<")[0] in b})
    del phis, mixers, Xd, yd, Xo, coef, xo, xb
    torch.cuda.empty_cache()
    # prefill
    T = 2048
    X, phi, bias, alpha, y = S.gen_hc(d, T)
    H = D.Hc(d, torch.from_numpy(phi).cuda(), torch.from_numpy(bias).cuda(), alpha, S.HC_EPS, S.HC_SINKHORN_ITERS)
    Xd = torch.from_numpy(X).cuda()
    yd = torch.from_numpy(y).cuda()
    Xo = torch.empty_like(Xd)
    coef = torch.empty((T, 24), dtype=torch.float32, device="cuda")
    xo = torch.empty((T, d), dtype=torch.float32, device="cuda")
    xb = torch.empty((T, d), dtype=torch.int16, device="cuda")
    ws, wsn = H.workspace(T)

    def pre():
        D.hc_pre(H.desc, Xd, T, coef, xo, xb, ws, wsn)

    def post():
        D.hc_post(H.desc, Xd, yd, coef, T, Xo)

    res = {}
    for name, fn in (("pre", pre), ("post", post)):
        fn()
        torch.cuda.synchronize()
        r = []
        for _ in range(repeats):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            r.append(e0.elapsed_time(e1))
        res[name] = float(np.median(r))
    D.trace_read(reset=True)
    D.trace_enable(True)
    pre()
    post()
    torch.cuda.synchronize()
    D.trace_enable(False)
    kern = D.trace_read(reset=True)
    b = hc_bytes(d, T)
    ku = {k: v[0] / v[1] * 1e3 for k, v in kern.items() if v[1] > 0}
    out["prefill"] = dict(workload=f"T={T}, one mixer, pre and post timed by events (median of {repeats})",
                          pre_us=res["pre"] * 1e3, post_us=res["post"] * 1e3,
                          pre_hbm_frac=b["pre_algorithmic"] / (res["pre"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          post_hbm_frac=b["post_algorithmic"] / (res["post"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          kernels_us={k: round(v, 2) for k, v in ku.items()},
                          kernel_gbs={k: round(b[k.split("<")[0]] / (ku[k] * 1e-6) / 1e9, 1) for k in ku
                                      if k.split("<")[0] in b})
    out["bytes_T1"] = hc_bytes(d, 1)
    out["bytes_T2048"] = b
    del Xd, yd, Xo, coef, xo, xb, H
    torch.cuda.empty_cache()
    return out


def measure_copy_gbs(nbytes=1 << 30, reps=5):
    """Device-to-device copy rate of a plain torch copy (bytes read + written
    per second), median of reps: the HBM figure measured beside the vendor
    peak."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


def measure_gemm_tflops(n=8192, reps=5):
    """fp16 GEMM (n x n x n) through torch's library matmul, median of reps:
    the dense-MFMA figure measured beside the vendor peak."""
    import torch
    a = torch.randn((n, n), dtype=torch.float16, device="cuda")
    b = torch.randn((n, n), dtype=torch.float16, device="cuda")
    c = a @ b
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    del a, b, c
    torch.cuda.empty_cache()
    return 2 * n ** 3 / (ms * 1e-3) / 1e12


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bench_cpu_oracle(seconds: float):
    """The CPU oracle on a bounded sample of decode1 tokens (experts the sample
    needs are packed by the oracle beforehand, untimed)."""
    from oracle import oracle as O
    from bit_quantized_routed_router_amd import synthetic as S

    cfg = S.CONFIGS["decode1"]
    router = S.gen_router(cfg)
    sh = S.gen_shared(cfg)
    cache = {}

    def expert(e):
        if e not in cache:
            g, u, dn = S.gen_expert(cfg, e)
            cache[e] = (O.cb2_quantize(g), O.cb2_quantize(u), O.q2k_quantize(dn))
        return cache[e]

    L = O.Layer(cfg.d, cfg.E, cfg.k, cfg.f, cfg.fs, router, None, sh[0], sh[1], sh[2], expert)
    ntok = 4
    xs = [S.gen_x(cfg, variant=1000 + n) for n in range(ntok)]
    for x in xs:  # pack the sample's experts (untimed)
        for e in np.unique(L.route(x, "bf16")["idx"]):
            L.expert(int(e))

    def rate(budget):
        done, t0 = 0, time.time()
        while True:
            for x in xs:
                L.forward(x, "bf16")
                done += 1
            if time.time() - t0 >= budget:
                break
        return done, time.time() - t0

    threads = len(os.sched_getaffinity(0))
    O.set_threads(threads)
    done, dt = rate(seconds)
    O.set_threads(1)
    done1, dt1 = rate(seconds)
    O.set_threads(threads)
    return dict(value=done / dt, unit="tok/s", cores=threads, kind="oracle",
                value_1thread=done1 / dt1, cpu_model=cpu_model(),
                sample=f"{done} decode1 tokens on {threads} threads in {dt:.1f}s and {done1} on 1 thread in "
                       f"{dt1:.1f}s (T=1 layer calls over {ntok} distinct seeded tokens, experts packed beforehand), "
                       "fp64")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--repeats", type=int, default=5, help="timed passes (eager) and graph replays; median reported")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-decode16", action="store_true")
    ap.add_argument("--no-decode-small", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stack", action="store_true", help="skip the 43-layer stack leg (about 80 GB resident)")
    ap.add_argument("--no-wide", action="store_true", help="skip the MXFP4- and Q4K-expert side reports")
    ap.add_argument("--no-hc", action="store_true", help="skip the hyper-connection mixer side report")
    ap.add_argument("--stack-tokens", type=int, default=256)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the layer on one GPU only; the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    dec = bench_decode(args)
    log(f"[bench] decode: graph {dec['ms_per_step'] * 1e3:.1f} us/step, eager {dec['eager_ms_per_step'] * 1e3:.1f} us/step")
    d16 = None if args.no_decode16 else bench_decode16()
    dsm = None if args.no_decode_small else bench_decode_small()
    if dsm:
        for key, r in dsm.items():
            if key.startswith("T"):
                log(f"[bench] decode {key}: {r['us_per_step']:.1f} us/step, {r['tok_s']:.0f} tok/s, "
                    f"{r['distinct_mean']:.1f} distinct experts, {100 * r['hbm_frac']:.1f} % of HBM peak")
    if d16:
        log(f"[bench] decode16: {d16['us_per_step']:.1f} us/step, {d16['tok_s']:.0f} tok/s, "
            f"{d16['distinct_mean']:.1f} distinct experts, {100 * d16['hbm_frac']:.1f} % of HBM peak")
    pre = None if args.no_prefill else bench_prefill(args)
    if pre:
        log(f"[bench] prefill: {pre['ms']:.3f} ms, {pre['tok_s']:.0f} tok/s, {pre['tflops']:.1f} TFLOP/s")
    wide = {}
    for efmt in () if args.no_wide else ("mxfp4", "q4k"):
        wd = bench_wide(efmt)
        log(f"[bench] {efmt} decode: {wd['us_per_step']:.1f} us/step, {wd['tok_s']:.0f} tok/s, "
            f"{100 * wd['hbm_frac']:.1f} % of HBM peak, kernels {wd['kernels_us']}")
        wp = None if args.no_prefill else bench_prefill(args, efmt=efmt)
        if wp:
            log(f"[bench] {efmt} prefill: {wp['ms']:.3f} ms, {wp['tok_s']:.0f} tok/s, {wp['tflops']:.1f} TFLOP/s")
        wide[efmt] = dict(decode=wd, prefill=None if wp is None else dict(
            {k: wp[k] for k in ("workload", "tok_s", "ms", "tflops", "mfma_frac")},
            kernels_us={k: round(v["mean_us"], 2) for k, v in wp["kernels"].items()}))
    hc = None if args.no_hc else bench_hc()
    if hc:
        log(f"[bench] hc decode: {hc['decode']['us_per_step']:.1f} us/step (pre + post), kernels "
            f"{hc['decode']['kernels_us']}; prefill pre {hc['prefill']['pre_us']:.1f} us "
            f"({100 * hc['prefill']['pre_hbm_frac']:.1f} % HBM), post {hc['prefill']['post_us']:.1f} us "
            f"({100 * hc['prefill']['post_hbm_frac']:.1f} % HBM), kernels {hc['prefill']['kernel_gbs']} GB/s")
    stk = None if args.no_stack else bench_stack43(tokens=args.stack_tokens)
    if stk:
        for r in (stk, stk["q2q4"]):
            log(f"[bench] stack43 {r['recipe']}: {r['us_per_token']:.1f} us/token, {r['tok_s']:.0f} tok/s, "
                f"{100 * r['hbm_frac']:.1f} % of HBM peak, {r['resident_bytes'] / 1e9:.1f} GB resident")
    copy_gbs = measure_copy_gbs()
    gemm_tflops = measure_gemm_tflops()
    log(f"[bench] measured: device copy {copy_gbs:.0f} GB/s, fp16 library GEMM {gemm_tflops:.0f} TFLOP/s")
    cpu = None if args.no_cpu_baseline else bench_cpu_oracle(args.cpu_seconds)
    ms = dec["ms_per_step"]
    out = {
        "metric": METRIC,
        "value": 1.0 / (ms * 1e-3),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "decode1: one MoE layer, T=1, d_model 4096, 256 experts top-6 + 1 shared, f=fs=2048, "
                        "CB2 gate/up + Q2K down, F16 router/shared, bf16 x; "
                        f"{args.copies} layer copies round-robin, HIP-graph replay",
            "global_batch": 1,
            "layer_copies": args.copies,
        },
        "roofline": dict(dec["roofline"], measured_copy_gbs=copy_gbs,
                         frac_of_measured_copy=dec["roofline"]["achieved"] / copy_gbs),
        "measured_peaks": {"hbm_copy_gbs": copy_gbs, "fp16_gemm_tflops": gemm_tflops,
                           "how": "median of 5: torch device copy of 1 GiB (read + write bytes); torch fp16 matmul "
                                  "8192^3"},
        "graph_runs_us": [round(v * 1e3, 2) for v in dec["graph_runs_ms"]],
        "layer_hbm": {"bytes_per_step": dec["layer_bytes"], "achieved_gbs": dec["layer_gbs"],
                      "frac": dec["layer_hbm_frac"]},
        "eager_ms_per_step": dec["eager_ms_per_step"],
        "kernels_us": {k: round(v["mean_us"], 2) for k, v in dec["kernels"].items()},
        "decode16": d16,
        "decode_small": dsm,
        "prefill": None if pre is None else dict(
            {k: pre[k] for k in ("workload", "tok_s", "ms", "runs_ms", "tflops", "mfma_frac")},
            frac_of_measured_gemm=pre["tflops"] / gemm_tflops,
            kernels_us={k: round(v["mean_us"], 2) for k, v in pre["kernels"].items()}),
        "stack43": stk,
        "mxfp4": wide.get("mxfp4"),
        "q4k": wide.get("q4k"),
        "hc": hc,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
