#!/usr/bin/env python3
"""Benchmark of the HQQ solve on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --op linear [--steps K] [--warmup W]
    python bench.py --op streamed [--steps K] [--warmup W]
    python bench.py --op meta [--steps K] [--warmup W]

A step quantizes every tensor of the workload once, with all fp16 inputs
already resident in HBM: consecutive tensors of one format go to
hqq_quantize_batch in even chunks of up to 48 (one kernel launch per chunk).  The default
workload is the 7B-shaped stack: 32 decoder layers of q/k/v/o [4096,4096],
gate/up [11008,4096], down [4096,11008] -- 6,476,005,376 fp16 weights
(12.95 GB) -- at nbits=4, group_size=64, axis=1, 20 iterations, p=0.7,
beta0=10, kappa=1.01.  Inputs are seeded synthetic weights generated on the
GPU (synth/), standing in for the trained checkpoints the pages quantize.

Prints one JSON line: the metric (GB/s of fp16 weights quantized), the
roofline of the solve kernel (measured with HIP events around each launch
inside the timed region, on the launch stream), and the CPU oracle timed on
this host on a bounded sample.

--op linear measures the consumer of the codes instead: one decode token of
the same 7B shape through the quantized layers (HQQ guide, sections 3.2 and
4.1: the layer's forward dequantizes and multiplies in fp16), i.e. the 224
linear layers of 32 decoder layers at batch 1, each an hqq_linear call on
4-bit g64 axis=1 codes.  The 224 calls are captured in one HIP graph and
replayed, so the timing is the GPU's; the same 224 products with fp16
weights (torch.matmul, hipBLASLt) are timed the same way beside it.  Codes
are seeded random, meta from a synthetic min/max distribution, activations
N(0, 1).

--op streamed measures the solve over weights held in host memory (models
larger than HBM): the workload (default the 7B stack; the 70B mixed stack
with --workload llama70b_stack80_mixed) in pinned host memory, quantized
layer by layer: one hqq_quantize_streamed call per layer and format,
copying double-buffered chunks of 512 MiB over PCIe while the solve runs.
Its bound is the host-to-device link, reported beside a plain pinned copy
of the same bytes.

--op meta measures the 8-bit quantization of the metadata (quant_scale /
quant_zero): the scale and zero arrays the solve produced for the 7B stack
(2 x 101 M fp32 values), quantized in groups of 128 by hqq_quantize_meta.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GB/s of fp16 weights quantized (HQQ 4b g64, 20 it), 7B-shaped; % roofline"

# MI355X (gfx950) peaks.  VALU: the 157.3 TFLOP/s fp32 vector figure is
# 256 CUs x 2.4 GHz x 128 FMA lanes per clock per CU (an FMA counts as 2
# flops), i.e. 78.6 T lane-ops/s; plain (non-packed) VALU instructions issue at
# that rate too.  HBM3E: 8 TB/s.
VALU_PEAK_TOPS = 256 * 128 * 2.4e9 / 1e12
HBM_PEAK_GBS = 8000.0


# The solve's binding roofline is HBM.  Its algorithmic traffic is the fp16
# weights read once plus codes and fp32 scale/zero written once.  The VALU
# work it needs per weight on gfx950 is far below the HBM time: 2.5 lane-ops
# per weight and iteration (fma, round-saturate-pack v_cvt_pk_u8_f32, and two
# v_sad_u8 per four weights) over the iterations a group runs before its zero
# is a fixed point (about 4 on these weights, iterations after it repeat the
# same zero exactly), plus about 10 once (widen, min, max, exact sum, final
# codes): ~20 lane-ops = 0.25 ps per weight at 78.6 T lane-ops/s, against
# 2.625 B / 8 TB/s = 0.33 ps.  The VALU figures actually issued, from the
# committed counter summary, are reported beside the roofline.
def hbm_bytes_per_weight(nbits: int, group_size: int) -> float:
    C = {8: 4, 4: 8, 3: 10, 2: 16, 1: 32}[nbits]
    return 2.0 + 4.0 / C + 8.0 / group_size


# HBM traffic of the solve kernel per launch, from the committed rocprofv3
# FETCH_SIZE / WRITE_SIZE summary; used only while the kernel's sources are
# byte-identical to the ones the counters were taken with.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "solve_4b_g64_llama7b_stack32.traffic.json")
KERNEL_SOURCES = ["weight_quantization_group_amd/csrc/hqq_solve_impl.h",
                  "weight_quantization_group_amd/csrc/hqq_solve_seg.h",
                  "weight_quantization_group_amd/csrc/hqq_solve_b4.hip",
                  "weight_quantization_group_amd/csrc/hqq_internal.h"]


def kernel_source_sha() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_summary(workload: str, wdtype: str):
    """Counter-measured figures of the dominant solve kernel (HBM bytes and
    issued VALU lane-ops per weight), or None if stale, absent, or taken on
    another workload or weight type (they were taken on fp16 weights)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("kernel_source_sha256") != kernel_source_sha():
        return None
    if t.get("workload") != workload or wdtype != "f16":
        return None
    return t


def work_items(t, nbits, group_size, axis):
    """Work items of one tensor in a solve launch: lcm(gs, codes per word)
    elements of a line each."""
    C = {8: 4, 4: 8, 3: 10, 2: 16, 1: 32}[nbits]
    lb = group_size * C // math.gcd(group_size, C)
    L, lines = (t["cols"], t["rows"]) if axis == 1 else (t["rows"], t["cols"])
    return -(-L // lb) * lines


def solve_kernel_name(hq, fmt, wdtype, items):
    nb, gs, ax = fmt
    m = hq.hqq_solve_mapping(nb, gs, ax, wdtype, items)
    if m != hq.MAPPING_LANE:
        return f"solve_seg_kernel<{nb},{gs},{2 if m == hq.MAPPING_SEG16 else 1}>"
    return f"solve_kernel<{nb},{gs},{ax},{'true' if wdtype == hq.DTYPE_BF16 else 'false'}>"


def host_cpu():
    """(CPU model, cores this process may run on)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return model, n


# The host share of a one-GPU machine is 16 cores; the oracle runs on at most
# this many processes whatever the machine reports.
CPU_BASELINE_MAX_PROCS = 16


def cpu_baseline(workload: str, iters: int, p: float = 0.7, beta0: float = 10.0,
                 max_procs: int = CPU_BASELINE_MAX_PROCS):
    """Time the oracle (single-threaded C, as it stands) on decoder layer 0 of
    the workload, in P independent processes over row slices."""
    import multiprocessing as mp

    import synth

    tensors = [t for t in synth.workload(workload) if t["layer"] == 0]
    model, avail = host_cpu()
    P = max(1, min(max_procs, avail))
    jobs = []
    for t in tensors:
        step = max(1, t["rows"] // P)
        for r0 in range(0, t["rows"], step):
            jobs.append((t, r0, min(step, t["rows"] - r0), iters, p, beta0))
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with ctx.Pool(P) as pool:
        res = pool.map(_cpu_job, jobs, chunksize=1)
    wall = time.perf_counter() - t0
    n = sum(r[0] for r in res)
    busy = sum(r[1] for r in res)
    # throughput over the oracle's own time (generation excluded): total
    # weights over the busy time spread across the P processes
    eff_wall = busy / P
    return dict(value=round(2.0 * n / eff_wall / 1e9, 6), unit="GB/s", cores=P, kind="oracle",
                sample=f"decoder layer 0 of {workload} ({n:,} weights), oracle in {P} "
                       f"single-threaded processes over row slices; {busy:.1f} core-s, "
                       f"{wall:.1f} s wall incl. host generation",
                cpu_model=model, cores_available=avail,
                cores_note=f"{P} processes: all available cores up to the {max_procs}-core host "
                           f"share of one GPU",
                weights_per_s=round(n / eff_wall, 1))


def _cpu_job(job):
    import oracle
    import synth

    t, r0, nr, iters, p, beta0 = job
    W = synth.generate_np(t["seed"], t["layer"], t["tensor_id"], t["rows"], t["cols"], row0=r0,
                          nrows=nr)
    t0 = time.perf_counter()
    oracle.quantize(W, t["nbits"], t["group_size"], t["axis"], iters=iters, p=p, beta0=beta0)
    return W.size, time.perf_counter() - t0


LINEAR_METRIC = "tokens/s, 7B decode (batch 1) through all 224 HQQ 4b g64 linear layers"
PREFILL_METRIC = "tokens/s, 7B prefill ({m} rows per step) through all 224 HQQ 4b g64 linear layers"
MFMA_PEAK_TFLOPS = 2500.0     # MI355X dense fp16 / bf16 MFMA
# HBM traffic of the linear kernel per step, from the committed rocprofv3
# summary; used only while the kernel's sources are the ones it was taken with
LINEAR_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "linear_4b_g64_llama7b_decode.traffic.json")
LINEAR_KERNEL_SOURCES = ["weight_quantization_group_amd/csrc/hqq_linear.hip",
                         "weight_quantization_group_amd/csrc/hqq_internal.h"]


def linear_counter_summary():
    try:
        with open(LINEAR_TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        return None
    import hashlib

    h = hashlib.sha256()
    for f in LINEAR_KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return t if t.get("kernel_source_sha256") == h.hexdigest() else None


def linear_cpu_baseline(nbits: int, gs: int, seconds: float = 15.0):
    """The oracle's linear layer (fp64, single thread) on 4096 x 4096 decode
    products, repeated for about `seconds`; scaled to tokens/s of the 224-layer
    7B step by weight count."""
    import numpy as np

    import oracle

    rng = np.random.RandomState(0)
    N = K = 4096
    qmax = (1 << nbits) - 1
    codes = rng.randint(0, qmax + 1, size=(N, K)).astype(np.uint8)
    packed = oracle.pack(codes, nbits, 1)
    scale = np.full((N, K // gs), qmax / 0.06, np.float32)
    zero = np.full((N, K // gs), qmax / 2, np.float32)
    X = (rng.standard_normal((1, K)).astype(np.float16)).view(np.uint16)
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        oracle.linear(X, packed, scale, zero, N, nbits, gs)
        n += 1
    dt = time.perf_counter() - t0
    w_per_s = n * N * K / dt
    return dict(value=round(w_per_s / LLAMA7B_WEIGHTS, 6), unit="tokens/s", cores=1, kind="oracle",
                sample=f"{n} oracle linear products of 1 x 4096 by a 4096 x 4096 4-bit g{gs} weight "
                       f"({dt:.1f} s, one thread), scaled by weight count to the 224-layer step",
                weights_per_s=round(w_per_s, 1))


# the 7B decoder's linear shapes (N, K) per layer: q, k, v, o, gate, up, down
LLAMA7B_LINEARS = [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]
LLAMA7B_LAYERS = 32
LLAMA7B_WEIGHTS = LLAMA7B_LAYERS * sum(n * k for n, k in LLAMA7B_LINEARS)


def bench_linear(args):
    import torch

    import weight_quantization_group_amd as hq

    hq.load_library()
    dev = torch.device("cuda:0")
    nbits, gs = 4, 64
    qmax = (1 << nbits) - 1
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    layers = []
    for li in range(LLAMA7B_LAYERS):
        for (N, K) in LLAMA7B_LINEARS:
            packed = torch.randint(-2 ** 31, 2 ** 31 - 1, (N, K * nbits // 32), dtype=torch.int32,
                                   device=dev, generator=gen)
            lo = -(0.03 + 0.01 * torch.rand((N, K // gs), device=dev, generator=gen)).abs()
            hi = (0.03 + 0.01 * torch.rand((N, K // gs), device=dev, generator=gen)).abs() + 1e-3
            scale = (qmax / (hi - lo)).float()
            zero = (-lo * scale).float()
            layers.append((N, K, packed, scale, zero))
    cdt = torch.bfloat16 if args.cdtype == "bf16" else torch.float16     # compute dtype
    M = args.rows                                                          # rows of X per step
    if M < 1:
        raise SystemExit("--rows must be at least 1")
    X = {K: torch.randn((M, K), device=dev, generator=gen).to(cdt) for K in (4096, 11008)}
    Y = {N: torch.empty((M, N), dtype=cdt, device=dev) for N in (4096, 11008)}
    # per layer, the projections that read the same activations share one
    # hqq_linear_batch call: (q, k, v), (o), (gate, up), (down)
    # (the outputs of one projection are shared by the 32 layers)
    nl = len(LLAMA7B_LINEARS)
    outs = [torch.empty((M, N), dtype=cdt, device=dev) for (N, K) in LLAMA7B_LINEARS]
    calls = []
    # one workspace for every call (they run in order on one stream): the
    # tiled kernel may split K for many rows, and from 256 rows the library
    # dequantizes each weight into it and runs a GEMM (hqq_linear_batch_ws);
    # the largest W_hat is 11008 x 4096 (gate, up; down is 4096 x 11008)
    groups = ((0, 1, 2), (3,), (4, 5), (6,))
    work = None
    if M > 1 and not args.no_split:
        nmax = max(sum(LLAMA7B_LINEARS[i][0] for i in idx) for idx in groups)
        wbytes = max(hq.linear_workspace_bytes(M, [nmax]), hq.linear_workspace_bytes(M, [11008], 4096))
        work = torch.empty(wbytes // 4, dtype=torch.float32, device=dev)
    for li in range(LLAMA7B_LAYERS):
        ly = layers[li * nl:(li + 1) * nl]
        for idx in groups:
            K = ly[idx[0]][1]
            items = [(ly[i][2], ly[i][3], ly[i][4], ly[i][0], outs[i]) for i in idx]
            calls.append((K, hq.LinearBatch(items, nbits, gs, dtype=cdt, workspace=work)))
    torch.cuda.synchronize()

    def token():
        for (K, b) in calls:
            b.run(X[K])

    def token_per_layer():
        for (N, K, p, s, z) in layers:
            hq.hqq_linear(X[K], p, s, z, N, nbits, gs, out=Y[N])

    def graph_of(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def timed(g, steps, warmup):
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall * 1e3 / steps

    if args.calib_copy:
        a = torch.empty(1 << 29, dtype=torch.float16, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    class Eager:
        def __init__(self, fn):
            self.replay = fn

    # --eager: plain launches (for profilers that count per dispatch); the
    # timing then includes the host's launch cost
    g = Eager(token) if args.eager else graph_of(token)
    ms_ev, ms_wall = timed(g, args.steps, args.warmup)
    del g
    # context: one call per product (skipped for profiler runs, whose
    # per-dispatch counters must see the batched calls only)
    ms_per_layer = None
    if not args.no_per_layer:
        g = Eager(token_per_layer) if args.eager else graph_of(token_per_layer)
        ms_per_layer, _ = timed(g, args.steps, args.warmup)
        del g

    # the dense reference: the same 224 products with distinct weights in the
    # compute dtype (12.95 GB) through torch.matmul (hipBLASLt), with the same
    # sharing of the inputs: q, k, v and gate, up as concatenated weights
    Wf = []
    for li in range(LLAMA7B_LAYERS):
        for idx in ((0, 1, 2), (3,), (4, 5), (6,)):
            N = sum(LLAMA7B_LINEARS[i][0] for i in idx)
            K = LLAMA7B_LINEARS[idx[0]][1]
            w = torch.empty((N, K), dtype=cdt, device=dev)
            w.normal_(0.0, 0.02, generator=gen)
            Wf.append((K, w, torch.empty((M, N), dtype=cdt, device=dev),
                       [LLAMA7B_LINEARS[i][0] for i in idx]))

    def token_fp16():
        for (K, w, y, _) in Wf:
            torch.matmul(X[K], w.t(), out=y)

    def token_fp16_per_layer():
        for (K, w, _, Ns) in Wf:
            n0 = 0
            for N in Ns:
                torch.matmul(X[K], w[n0:n0 + N].t(), out=Yf[N])
                n0 += N

    Yf = {N: torch.empty((M, N), dtype=cdt, device=dev) for N in (4096, 11008)}
    gf = Eager(token_fp16) if args.eager else graph_of(token_fp16)
    ms_fp16, _ = timed(gf, args.steps, args.warmup)
    del gf
    ms_fp16_per_layer = None
    if not args.no_per_layer:
        gf = Eager(token_fp16_per_layer) if args.eager else graph_of(token_fp16_per_layer)
        ms_fp16_per_layer, _ = timed(gf, args.steps, args.warmup)
        del gf
    del Wf

    bytes_per_token = sum(N * K * nbits / 8 + N * (K // gs) * 8 + K * 2 + N * 2
                          for (N, K) in LLAMA7B_LINEARS) * LLAMA7B_LAYERS
    gbs = bytes_per_token / (ms_ev * 1e-3) / 1e9
    metric = LINEAR_METRIC if M == 1 else PREFILL_METRIC.format(m=M)
    if M == 1:
        # decode: the codes and meta cross HBM once per token
        roofline = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4),
                    "traffic": (lambda c: c["hbm_bytes_per_step"] if c else None)(linear_counter_summary()),
                    "kernel": "linear_skinny_kernel (4-bit, g64)",
                    "bytes_per_step": int(bytes_per_token),
                    "bytes_per_weight": round(bytes_per_token / LLAMA7B_WEIGHTS, 4)}
    else:
        # many rows: 2 M N K flops per product on the MFMA units (fp16 or
        # bf16 inputs, fp32 accumulation)
        flops = 2.0 * M * LLAMA7B_WEIGHTS
        tfs = flops / (ms_ev * 1e-3) / 1e12
        # the route the library takes for the largest call (gate and up)
        wb = work.numel() * work.element_size() if work is not None else 0
        gemm = hq.hqq_linear_route(M, 4096, 2, 11008, wb) == hq.ROUTE_GEMM
        roofline = {"bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tfs / MFMA_PEAK_TFLOPS, 4), "traffic": None,
                    "kernel": ("dequant_kernel + hipBLASLt GEMM (4-bit, g64)" if gemm else
                               "linear_tiled_kernel (4-bit, g64)" if M > 32 else "linear_skinny_kernel (4-bit, g64)"),
                    "flops_per_step": flops}
    out = {
        "metric": metric if args.cdtype == "f16" else metric + ", compute dtype bf16",
        "value": round(M * 1e3 / ms_ev, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_ev, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.cdtype,
        "data": "synthetic",
        "config": {"workload": "llama7b_decode_b1_4b_g64" if M == 1 else f"llama7b_prefill_m{M}_4b_g64",
                   "linears": len(layers), "M": M,
                   "weights": LLAMA7B_WEIGHTS, "nbits": nbits, "group_size": gs, "axis": 1},
        "roofline": roofline,
        "dense_matmul": {"dtype": args.cdtype, "ms_per_step": round(ms_fp16, 4),
                         "tokens_per_s": round(M * 1e3 / ms_fp16, 3),
                         "speedup": round(ms_fp16 / ms_ev, 3),
                         "per_layer_calls_ms_per_step":
                             round(ms_fp16_per_layer, 4) if ms_fp16_per_layer else None},
        "per_layer_calls": {"ms_per_step": round(ms_per_layer, 4),
                            "tokens_per_s": round(M * 1e3 / ms_per_layer, 3)} if ms_per_layer else None,
        "wall_ms_per_step": round(ms_wall, 4),
        "launch": ("eager" if args.eager else "hip graph") +
                  " of 128 calls: hqq_linear_batch of (q, k, v), (o), (gate, up), (down) per layer" +
                  (", with a split-K workspace" if work is not None else ""),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = linear_cpu_baseline(nbits, gs)
    print(json.dumps(out), flush=True)


def bench_meta(args):
    import torch

    import synth
    import weight_quantization_group_amd as hq

    hq.load_library()
    dev = torch.device("cuda:0")
    tensors = synth.workload(args.workload)
    metas = []
    for t in tensors:
        W = torch.empty((t["rows"], t["cols"]), dtype=torch.float16, device=dev)
        synth.generate_gpu(W, t["seed"], t["layer"], t["tensor_id"])
        p, sc, ze = hq.hqq_quantize(W, t["nbits"], t["group_size"], t["axis"], iters=args.iters)
        del W, p
        metas += [sc, ze]
    gsm = 128
    outs = [(torch.empty(m.numel(), dtype=torch.uint8, device=dev),
             torch.empty(-(-m.numel() // gsm), dtype=torch.float32, device=dev),
             torch.empty(-(-m.numel() // gsm), dtype=torch.float32, device=dev)) for m in metas]
    batch = hq.MetaBatch([(m, *o) for m, o in zip(metas, outs)], gsm)
    n_vals = sum(m.numel() for m in metas)
    torch.cuda.synchronize()
    import ctypes

    # one C-ABI call quantizes all 448 arrays, 32 per kernel launch; the call
    # is captured in a HIP graph so that the step is the kernels alone
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        batch.quantize(ctypes.c_void_p(side.cuda_stream))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        batch.quantize(ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    bytes_per_val = 4 + 1 + 8.0 / gsm
    gbs = bytes_per_val * n_vals / (ms * 1e-3) / 1e9
    out = {
        "metric": "G meta values/s quantized to 8 bits (quant_scale / quant_zero), 7B stack's scale and zero",
        "value": round(n_vals / (ms * 1e-3) / 1e9, 3),
        "unit": "Gvalues/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload + "_meta", "values": n_vals, "arrays": len(metas),
                   "meta_group_size": gsm, "launches": -(-len(metas) // hq.META_BATCH)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "bytes_per_value": bytes_per_val,
                     "kernel": "meta_quant_kernel"},
    }
    print(json.dumps(out), flush=True)


# PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes x 128/130 / 8
PCIE_PEAK_GBS = 63.0


def bench_streamed(args):
    import torch

    import synth
    import weight_quantization_group_amd as hq

    hq.load_library()
    dev = torch.device("cuda:0")
    tensors = synth.workload(args.workload)
    n_weights = sum(t["rows"] * t["cols"] for t in tensors)
    # Host weights (generated on the device, copied out), one tensor each.
    # Up to 48 GiB they are all page-locked.  A larger model (the 70B stack,
    # 137 GB) stays in ordinary host memory, as a checkpoint loaded into RAM
    # would, and each layer passes through one of two page-locked layer
    # buffers: the host copies layer L + 1 into one while the device streams
    # layer L out of the other.
    pool_mode = 2 * n_weights > (48 << 30)
    items, hosts = [], []
    for t in tensors:
        nb, gs, ax = t["nbits"], t["group_size"], t["axis"]
        W = torch.empty((t["rows"], t["cols"]), dtype=torch.float16, device=dev)
        synth.generate_gpu(W, t["seed"], t["layer"], t["tensor_id"])
        h = torch.empty((t["rows"], t["cols"]), dtype=torch.int16, pin_memory=not pool_mode)
        h.copy_(W.view(torch.int16))
        hosts.append(h)
        del W
        items.append((h, torch.empty(hq.packed_shape(t["rows"], t["cols"], nb, ax), dtype=torch.int32, device=dev),
                      torch.empty(hq.meta_shape(t["rows"], t["cols"], gs, ax), dtype=torch.float32, device=dev),
                      torch.empty(hq.meta_shape(t["rows"], t["cols"], gs, ax), dtype=torch.float32, device=dev)))
    # layer by layer: one streamed call per run of consecutive tensors of one
    # layer and one format (a 70B layer: attention 4b g64, then MLP 2b g16)
    calls = []
    for i, t in enumerate(tensors):
        key = (t["layer"], t["nbits"], t["group_size"], t["axis"])
        if calls and calls[-1][0] == key:
            calls[-1][1].append(i)
        else:
            calls.append((key, [i]))
    staging = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cs, ks = torch.cuda.Stream(), torch.cuda.Stream()
    layers = []
    for key, idx in calls:
        if layers and layers[-1][0] == key[0]:
            layers[-1][1].append((key, idx))
        else:
            layers.append((key[0], [(key, idx)]))
    pool, freed = [], [None, None]
    if pool_mode:
        biggest = max(sum(hosts[i].numel() for _, idx in ls for i in idx) for _, ls in layers)
        pool = [torch.empty(biggest, dtype=torch.int16, pin_memory=True) for _ in range(2)]
    torch.cuda.synchronize()

    def step():
        if not pool_mode:
            for (_, nb, gs, ax), idx in calls:
                hq.hqq_quantize_streamed([items[i] for i in idx], nb, gs, ax, staging, copy_stream=cs,
                                         compute_stream=ks, iters=args.iters)
            return
        for li, (_, ls) in enumerate(layers):
            b = li % 2
            if freed[b] is not None:
                freed[b].synchronize()     # the copies out of this buffer are done
            off = 0
            for (_, nb, gs, ax), idx in ls:
                its = []
                for i in idx:
                    n = hosts[i].numel()
                    v = pool[b][off:off + n].view(hosts[i].shape)
                    v.copy_(hosts[i])
                    off += n
                    its.append((v, *items[i][1:]))
                hq.hqq_quantize_streamed(its, nb, gs, ax, staging, copy_stream=cs, compute_stream=ks,
                                         iters=args.iters)
            ev = torch.cuda.Event()
            ev.record(cs)
            freed[b] = ev

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # the link alone: the same bytes, pinned host -> device, in pieces of at
    # most 512 MiB (from the layer buffers in the pooled mode, without the
    # host-side copies)
    dst = staging.view(torch.int16)
    half = dst.numel() // 2
    srcs = [h.view(-1) for h in hosts] if not pool_mode else \
        [pool[0][:h.numel()] for h in hosts]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for flat in srcs:
        for i in range(0, flat.numel(), half):
            n = min(half, flat.numel() - i)
            dst[:n].copy_(flat[i:i + n], non_blocking=True)
    torch.cuda.synchronize()
    copy_ms = (time.perf_counter() - t0) * 1e3
    gbs = 2.0 * n_weights / (ms * 1e-3) / 1e9
    copy_gbs = 2.0 * n_weights / (copy_ms * 1e-3) / 1e9
    fmts = sorted({(t["nbits"], t["group_size"], t["axis"]) for t in tensors})
    fmt_s = ", ".join(f"{b}b g{g}" + (" axis 0" if a == 0 else "") for b, g, a in fmts)
    out = {
        "metric": f"GB/s of fp16 weights quantized from host memory, layer by layer (HQQ {fmt_s}, "
                  f"{args.iters} it), "
                  f"workload {args.workload}",
        "value": round(gbs, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "weights": n_weights, "tensors": len(tensors),
                   "streamed_calls_per_step": len(calls), "staging_bytes": staging.numel(),
                   "host_weights": ("ordinary host memory through two page-locked layer buffers"
                                    if pool_mode else "page-locked host memory"),
                   "formats": [list(f) for f in fmts], "iters": args.iters},
        "roofline": {"bound": "pcie", "achieved": round(gbs, 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / PCIE_PEAK_GBS, 4), "traffic": None,
                     "pinned_copy_GBs": round(copy_gbs, 2), "frac_of_copy": round(gbs / copy_gbs, 4)},
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama7b_stack32_4b_g64")
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--p", type=float, default=0.7,
                    help="solve: the lp norm's p (p > 1 or a large beta0 keeps the shrink active, "
                         "so the exact W_e = 0 shortcut never applies)")
    ap.add_argument("--beta0", type=float, default=10.0, help="solve: the initial beta")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--cdtype", choices=("f16", "bf16"), default="f16",
                    help="linear: compute dtype of the activations and outputs")
    ap.add_argument("--rows", type=int, default=1,
                    help="linear: rows of X per step (1: decode; e.g. 2048: a prefill chunk)")
    ap.add_argument("--no-per-layer", action="store_true",
                    help="linear: skip the one-call-per-product context timings (profiler runs)")
    ap.add_argument("--wdtype", choices=("f16", "bf16"), default="f16",
                    help="solve: element type of the weights (bf16: the synthetic fp16 weights rounded to bf16)")
    ap.add_argument("--eager", action="store_true",
                    help="--op linear: plain launches instead of a captured HIP graph")
    ap.add_argument("--no-split", action="store_true",
                    help="--op linear: no workspace: the fused kernels only, without K splits")
    ap.add_argument("--op", choices=("solve", "linear", "streamed", "meta"), default="solve",
                    help="solve: quantize the 7B stack (default); linear: one decode token "
                         "through the quantized layers; streamed: the solve from pinned host memory")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the solve shards by whole tensors or row blocks with no communication, so N GPUs "
              "would give N times the one-GPU rate)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import weight_quantization_group_amd as hq

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.op == "linear":
        bench_linear(args)
        return
    if args.op == "streamed":
        bench_streamed(args)
        return
    if args.op == "meta":
        bench_meta(args)
        return
    hq.load_library()
    dev = torch.device("cuda:0")
    tensors = synth.workload(args.workload)

    # resident inputs and outputs
    ins, outs = [], []
    for t in tensors:
        W = torch.empty((t["rows"], t["cols"]), dtype=torch.float16, device=dev)
        synth.generate_gpu(W, t["seed"], t["layer"], t["tensor_id"])
        if args.wdtype == "bf16":
            W = W.to(torch.bfloat16)
        ins.append(W)
        outs.append((torch.empty(hq.packed_shape(t["rows"], t["cols"], t["nbits"], t["axis"]),
                                 dtype=torch.int32, device=dev),
                     torch.empty(hq.meta_shape(t["rows"], t["cols"], t["group_size"], t["axis"]),
                                 dtype=torch.float32, device=dev),
                     torch.empty(hq.meta_shape(t["rows"], t["cols"], t["group_size"], t["axis"]),
                                 dtype=torch.float32, device=dev)))
    torch.cuda.synchronize()
    n_weights = sum(t["rows"] * t["cols"] for t in tensors)

    if args.calib_copy:
        a = torch.empty(1 << 29, dtype=torch.float16, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # launches: runs of consecutive tensors of one format, each cut into as
    # even pieces of at most MAX_BATCH as it allows (one hqq_quantize_batch
    # call, one kernel launch each)
    runs = []
    for i, t in enumerate(tensors):
        fmt = (t["nbits"], t["group_size"], t["axis"])
        if runs and runs[-1][0] == fmt:
            runs[-1][1].append(i)
        else:
            runs.append((fmt, [i]))
    chunks = []
    for fmt, idx in runs:
        parts = -(-len(idx) // hq.MAX_BATCH)
        per = -(-len(idx) // parts)
        for k in range(0, len(idx), per):
            chunks.append((fmt, idx[k:k + per]))
    # the descriptor arrays are marshalled once (host metadata only); a step
    # is then one C-ABI call per launch
    calls = [(fmt, hq.QuantizeBatch([(ins[i], *outs[i]) for i in idx], *fmt, iters=args.iters,
                                    p=args.p, beta0=args.beta0),
              sum(tensors[i]["rows"] * tensors[i]["cols"] for i in idx))
             for fmt, idx in chunks]
    # the kernel each launch runs (the library picks the mapping by launch size)
    wdt = hq.DTYPE_BF16 if args.wdtype == "bf16" else hq.DTYPE_FP16
    kernels = [solve_kernel_name(hq, fmt, wdt, sum(work_items(tensors[i], *fmt) for i in idx))
               for fmt, idx in chunks]

    def step(events=None):
        for j, (_, batch, _) in enumerate(calls):
            if events is not None:
                events[j][0].record()
            batch.run()
            if events is not None:
                events[j][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in calls] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # per-launch kernel durations (HIP events on the launch stream)
    by_fmt = {}
    for j, (fmt, items, w) in enumerate(calls):
        d = by_fmt.setdefault(fmt, dict(w=0, ms=0.0, launches=0))
        d["w"] += w * args.steps
        d["ms"] += sum(evs[k][j][0].elapsed_time(evs[k][j][1]) for k in range(args.steps))
        d["launches"] += args.steps
    # dominant kernel: the format with the most weights
    (nb, gs, ax), dom = max(by_fmt.items(), key=lambda kv: kv[1]["w"])
    dom_kernel = max(((kernels[j], w) for j, (fmt, _, w) in enumerate(calls) if fmt == (nb, gs, ax)),
                     key=lambda kw: kw[1])[0]
    w_per_launch = dom["w"] / dom["launches"]
    avg_ms = dom["ms"] / dom["launches"]
    bpw = hbm_bytes_per_weight(nb, gs)
    hbm_gbs = bpw * w_per_launch / (avg_ms * 1e-3) / 1e9
    default_params = args.p == 0.7 and args.beta0 == 10.0 and args.iters == 20
    cs = counter_summary(args.workload, args.wdtype) if default_params else None
    traffic = round(cs["hbm_bytes_per_weight"] * w_per_launch) if cs else None
    valu = {"peak_TOPs": round(VALU_PEAK_TOPS, 3)}
    if cs:
        lops = cs["valu_lane_ops_per_weight"]
        valu.update(issued_lane_ops_per_weight=lops,
                    issued_TOPs=round(lops * w_per_launch / (avg_ms * 1e-3) / 1e12, 3),
                    frac=round(lops * w_per_launch / (avg_ms * 1e-3) / 1e12 / VALU_PEAK_TOPS, 4))

    gbs = 2.0 * n_weights / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": METRIC if (args.workload == "llama7b_stack32_4b_g64" and args.wdtype == "f16"
                             and default_params) else
                  f"GB/s of {'fp16' if args.wdtype == 'f16' else 'bf16'} weights quantized "
                  f"(HQQ {nb}b g{gs}, {args.iters} it, p={args.p:g}, beta0={args.beta0:g}), "
                  f"workload {args.workload}",
        "value": round(gbs, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "weights": n_weights, "tensors": len(tensors),
                   "launches_per_step": len(calls),
                   "nbits": nb, "group_size": gs, "axis": ax, "iters": args.iters,
                   "p": args.p, "beta0": args.beta0, "kappa": 1.01},
        "weights_per_s": round(n_weights / (ms_per_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(hbm_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(hbm_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": dom_kernel, "avg_launch_ms": round(avg_ms, 5),
                     "weights_per_launch": round(w_per_launch), "bytes_per_weight": bpw,
                     "valu": valu},
        "context": {"pages_hqq_llama7b_quantize_minutes": 8.2, "hardware": "not stated on the pages"},
    }
    # the CPU baseline runs after the timed GPU region (a 16-core burst just
    # before it slows the GPU's launches measurably), in spawned processes
    # that never touch the GPU
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, args.iters, args.p, args.beta0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
