#!/usr/bin/env python3
"""Benchmark of the NVFP4 W4A4 prefill linear layer on one MI355X.

Workload: the Qwen3-8B-shaped attention projections at prefill, M = 8192
tokens, hidden 4096: Q 4096->4096, K and V 4096->1024, O 4096->4096.  One
step is one pass of the whole hot path over one batch:

    alpha + NVFP4 quantisation of X_qkv   (amax, prepare, quantize kernels)
    Q, K, V W4A4 GEMMs as one launch over the stacked weights (each keeps
        its own tensor scale; BF16 output [8192, 6144])
    alpha + NVFP4 quantisation of X_o
    O W4A4 GEMM

Weights are quantised once before timing (offline, as in the layer).  The
inputs of consecutive steps rotate over several copies whose total exceeds the
256 MB last-level cache, so every step reads its activations from HBM.

The same step with the BF16 comparison GEMM (no quantisation) and with
torch.matmul (hipBLASLt), both also over the stacked Q|K|V weights, gives the
speedups.  The oracle is timed on a
bounded sample on the host cores.  One JSON line goes to stdout.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_F16_PEAK_TFLOPS = 2500.0          # dense f16/bf16 MFMA, MI355X
MFMA_FP4_PEAK_TFLOPS = 10100.0         # dense fp4/fp6 MFMA, MI355X (context only: the
                                       # per-16 E4M3 scales rule out the block-scaled fp4 MFMA)
HBM_PEAK_GBPS = 8000.0
QUANT_BYTES_PER_ELEM = 2.0 + 0.5 + 1.0 / 16.0   # read BF16, write codes + scales
AMAX_BYTES_PER_ELEM = 2.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w4a4_gemm_qkv_8192x6144x4096_traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "nvfp4_w4a4_gemm_amd", "csrc", "gemm_w4a4.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(path):
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def stored_traffic(traffic_file=None, source=None):
    """HBM bytes per Q|K|V launch from the committed counter record, or None
    when there is none or the GEMM source has changed since it was taken."""
    traffic_file = traffic_file or TRAFFIC_FILE
    source = source or GEMM_SOURCE
    if not os.path.exists(traffic_file):
        return None
    with open(traffic_file) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != source_hash(source):
        return None
    return rec.get("bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the chip takes on the order of 100 ms of sustained load to settle its
    # clocks; 200 layer steps (about 0.12 s) reach that steady state
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--rotate", type=int, default=4, help="input copies cycled over steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=8192,
                    help="activation rows in the oracle's timed sample")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the layer step: time every GEMM and quantiser of the five "
                         "layer configurations (one JSON line per configuration)")
    ap.add_argument("--configs", default="1,2,3,4,5", help="configurations for --sweep")
    return ap.parse_args()


class Timer:
    """HIP events around launches on torch's current stream (the library's).

    The events are created, and recorded once, before the timed region
    (`prepare`), so that the timed loop only records existing events: event
    creation inside the loop stalls the host now and then."""

    def __init__(self, torch):
        self.torch = torch
        self.pool = {}
        self.used = {}

    def prepare(self, name, count):
        torch = self.torch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(count)]
        for s, e in evs:
            s.record()
            e.record()
        self.pool[name] = evs
        self.used[name] = 0

    def __call__(self, name):
        timer = self

        class _Ctx:
            def __enter__(self_):
                i = timer.used[name]
                self_.s, self_.e = timer.pool[name][i]
                timer.used[name] = i + 1
                self_.s.record()

            def __exit__(self_, *a):
                self_.e.record()
        return _Ctx()

    def total_ms(self, name):
        return sum(s.elapsed_time(e) for s, e in self.pool[name][:self.used[name]])

    def count(self, name):
        return self.used[name]

    def times_ms(self, name):
        return [s.elapsed_time(e) for s, e in self.pool[name][:self.used[name]]]

    def reset(self):
        for name in self.used:
            self.used[name] = 0


def time_ms(torch, fn, reps, warmup):
    """Mean milliseconds of fn(i) over reps calls (HIP events on the current stream)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(reps):
        fn(warmup + i)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this layer is measured on one GPU; a multi-GPU run "
                                   "(data-parallel over token rows) is not implemented",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.sweep:
        sweep(args)
        return

    import numpy as np
    import torch

    from nvfp4_w4a4_gemm_amd import binding as nv
    from nvfp4_w4a4_gemm_amd.workloads import workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workload(2)
    m, h = 8192, 4096
    log(f"workload: {wl.title}; generating inputs")
    t0 = time.time()
    x_host = {"X_qkv": wl.tensors["X_qkv"].full(), "X_o": wl.tensors["X_o"].full()}
    w_host = {n: wl.tensors[n].full() for n in ("W_q", "W_k", "W_v", "W_o")}
    log(f"inputs generated in {time.time() - t0:.1f} s")

    # rotated activation copies (copy r of a tensor is the seeded tensor with
    # its rows rolled by r, so every copy is a distinct HBM buffer)
    xs = []
    for r in range(args.rotate):
        xs.append({k: nv.to_device_bf16(np.roll(v, r, axis=0), dev) for k, v in x_host.items()})
    ws = {k: nv.to_device_bf16(v, dev) for k, v in w_host.items()}
    workspace = nv.new_workspace(dev)
    wq = {k: nv.nvfp4_quantize_weights(v, workspace=workspace) for k, v in ws.items()}
    qkv = nv.stack_tensors([wq["W_q"], wq["W_k"], wq["W_v"]])
    w_qkv = torch.cat([ws["W_q"], ws["W_k"], ws["W_v"]], dim=0).contiguous()
    n_qkv = qkv.rows
    qbuf = {k: nv.nvfp4_quantize_act(xs[0][k], workspace=workspace) for k in x_host}
    outs = {"qkv": torch.empty(m, n_qkv, dtype=torch.bfloat16, device=dev),
            "o": torch.empty(m, h, dtype=torch.bfloat16, device=dev)}
    torch.cuda.synchronize()

    flops_qkv = 2.0 * m * n_qkv * h
    flops_o = 2.0 * m * h * h
    flops_step = flops_qkv + flops_o
    timer = Timer(torch)

    class _Null:
        def __enter__(self):
            return None

        def __exit__(self, *a):
            return False

    def w4a4_step(i, timed, every=False):
        # timed: HIP events around the Q|K|V GEMM (the roofline kernel);
        # every: around every launch (a separate pass: many live events make
        # the runtime stall the host, so the timed region keeps them few)
        x = xs[i % args.rotate]
        null = lambda name: _Null()
        ctx_main = timer if timed else null
        ctx_rest = timer if every else null
        with ctx_rest("quantize"):
            nv.nvfp4_quantize_act(x["X_qkv"], out=qbuf["X_qkv"], workspace=workspace)
        with ctx_main("gemm_qkv"):
            nv.w4a4_gemm_multi(qbuf["X_qkv"], qkv, f32=False, y_bf16=outs["qkv"])
        with ctx_rest("quantize"):
            nv.nvfp4_quantize_act(x["X_o"], out=qbuf["X_o"], workspace=workspace)
        with ctx_rest("gemm_o"):
            nv.w4a4_gemm(qbuf["X_o"], wq["W_o"], f32=False, y_bf16=outs["o"])

    def bf16_step(i):
        x = xs[i % args.rotate]
        nv.bf16_gemm_baseline(x["X_qkv"], w_qkv, f32=False)
        nv.bf16_gemm_baseline(x["X_o"], ws["W_o"], f32=False)

    def blas_step(i):
        x = xs[i % args.rotate]
        torch.matmul(x["X_qkv"], w_qkv.t())
        torch.matmul(x["X_o"], ws["W_o"].t())

    def time_steps(fn, steps, warmup):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3 / steps

    # --- the timed region: K steps of the W4A4 layer -----------------------
    # Python's full garbage collections walk every object torch created at
    # import (tens of ms); frozen, those objects are skipped, so a long run
    # does not stall the host mid-loop
    gc.collect()
    gc.freeze()
    log(f"timing W4A4 layer: {args.warmup} warmup + {args.steps} steps")
    for i in range(args.warmup):
        w4a4_step(i, timed=False)
    timer.prepare("gemm_qkv", args.steps)
    torch.cuda.synchronize()
    timer.reset()
    t = time.perf_counter()
    for i in range(args.steps):
        w4a4_step(i, timed=True)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t) * 1e3 / args.steps
    qkv_ms = timer.total_ms("gemm_qkv") / timer.count("gemm_qkv")
    qkv_sorted = sorted(timer.times_ms("gemm_qkv"))
    qkv_stats = {"mean": round(qkv_ms * 1e3, 1), "median": round(qkv_sorted[len(qkv_sorted) // 2] * 1e3, 1),
                 "min": round(qkv_sorted[0] * 1e3, 1), "max": round(qkv_sorted[-1] * 1e3, 1),
                 "launches": len(qkv_sorted)}

    # the other launches' durations, from a second pass of the same steps
    passes = min(args.steps, 20)
    for name, per_step in (("quantize", 2), ("gemm_o", 1)):
        timer.prepare(name, per_step * passes)
    torch.cuda.synchronize()
    for i in range(passes):
        w4a4_step(i, timed=False, every=True)
    torch.cuda.synchronize()
    o_ms = timer.total_ms("gemm_o") / timer.count("gemm_o")
    quant_ms = timer.total_ms("quantize") / timer.count("quantize")
    gemm_ms_step = qkv_ms + o_ms
    qkv_tflops = flops_qkv / (qkv_ms * 1e-3) / 1e12
    o_tflops = flops_o / (o_ms * 1e-3) / 1e12
    quant_bytes = m * h * (QUANT_BYTES_PER_ELEM + AMAX_BYTES_PER_ELEM)
    quant_gbps = quant_bytes / (quant_ms * 1e-3) / 1e9
    log(f"W4A4 step {ms_step:.3f} ms; GEMM Q|K|V {m}x{n_qkv}x{h} {qkv_ms:.3f} ms "
        f"({qkv_tflops:.0f} TFLOP/s); GEMM O {m}x{h}x{h} {o_ms:.3f} ms ({o_tflops:.0f} TFLOP/s); "
        f"quantize {quant_ms:.3f} ms ({quant_gbps:.0f} GB/s incl. amax)")

    # --- quantiser passes on their own, and the attainable copy rate ----------
    xq = [x["X_qkv"] for x in xs]
    alpha_dev = qbuf["X_qkv"].alpha.clone()
    n_el = m * h
    t_alpha = time_ms(torch, lambda i: nv.nvfp4_tensor_alpha(xq[i % len(xq)], workspace=workspace),
                      args.steps, args.warmup)
    t_given = time_ms(torch, lambda i: nv.nvfp4_quantize_act(xq[i % len(xq)], alpha_in=alpha_dev,
                                                             out=qbuf["X_qkv"],
                                                             workspace=workspace),
                      args.steps, args.warmup)
    cpy = torch.empty_like(xq[0])
    t_copy = time_ms(torch, lambda i: cpy.copy_(xq[i % len(xq)]), args.steps, args.warmup)
    log(f"quantiser passes: amax+alpha {t_alpha * 1e3:.1f} us, quantize (alpha given) "
        f"{t_given * 1e3:.1f} us; device copy of X {t_copy * 1e3:.1f} us")

    # --- comparisons ---------------------------------------------------------
    log("timing BF16 baseline step (same skeleton) and torch.matmul (hipBLASLt)")
    bf16_ms = time_steps(bf16_step, args.steps, args.warmup)
    blas_ms = time_steps(blas_step, args.steps, args.warmup)
    log(f"BF16 baseline step {bf16_ms:.3f} ms; hipBLASLt step {blas_ms:.3f} ms")

    log("timing RMSNorm with the quantiser fused in, against RMSNorm then quantise")
    fused_norm = rmsnorm_block(nv, torch, [x["X_qkv"] for x in xs], workspace, args.steps,
                               args.warmup)

    log("timing the gate|up GEMM with SiLU(gate)*up and its quantiser fused in")
    fused_silu = silu_block(nv, torch, qbuf["X_qkv"], dev, workspace, args.steps, args.warmup)

    log("timing decode-shaped W4A4 GEMMs (w4a4_gemm_decode) against hipBLASLt BF16")
    decode = decode_block(nv, torch, dev, workspace, args.steps, args.warmup)

    traffic = stored_traffic()

    result = {
        "metric": "NVFP4 W4A4 GEMM TFLOP/s (% MFMA peak), quantize GB/s, speedup vs BF16",
        "value": round(flops_step / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "Qwen3-8B-shaped attention projections at prefill: M=8192, hidden 4096, "
                        "Q 4096->4096, K/V 4096->1024 (one launch over the stacked Q|K|V "
                        "weights), O 4096->4096; NVFP4 W4A4, BF16 out",
            "global_batch": m,
            "flops_per_step": flops_step,
            "parallelism": "single GPU",
            "input_rotation": args.rotate,
        },
        "roofline": {
            "kernel": f"w4a4_gemm_kernel<256,256> (stacked Q|K|V projection, {m}x{n_qkv}x{h})",
            "bound": "mfma",
            "achieved": round(qkv_tflops, 2),
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(qkv_tflops / MFMA_F16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "launch_us": qkv_stats,
        },
        "quantize": {
            "gbps": round(quant_gbps, 1),
            "frac_of_hbm_peak": round(quant_gbps / HBM_PEAK_GBPS, 4),
            "ms_per_tensor": round(quant_ms, 4),
            "bytes_per_elem": QUANT_BYTES_PER_ELEM + AMAX_BYTES_PER_ELEM,
            "amax_pass_gbps": round(n_el * AMAX_BYTES_PER_ELEM / (t_alpha * 1e-3) / 1e9, 1),
            "quantize_pass_gbps": round(n_el * QUANT_BYTES_PER_ELEM / (t_given * 1e-3) / 1e9, 1),
            "device_copy_gbps": round(2 * n_el * 2 / (t_copy * 1e-3) / 1e9, 1),
        },
        "gemm": {"ms_per_step": round(gemm_ms_step, 4),
                 "tflops": round(flops_step / (gemm_ms_step * 1e-3) / 1e12, 2),
                 "frac_of_f16_mfma_peak": round(
                     flops_step / (gemm_ms_step * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                 "frac_of_fp4_mfma_peak": round(
                     flops_step / (gemm_ms_step * 1e-3) / 1e12 / MFMA_FP4_PEAK_TFLOPS, 4),
                 "qkv_ms": round(qkv_ms, 4), "o_ms": round(o_ms, 4),
                 "o_tflops": round(o_tflops, 2)},
        "rmsnorm_quantize": fused_norm,
        "gate_up_silu_quantize": fused_silu,
        "decode": decode,
        "bf16_baseline": {"ms_per_step": round(bf16_ms, 4),
                          "speedup_layer": round(bf16_ms / ms_step, 3),
                          "speedup_gemm_only": round(bf16_ms / gemm_ms_step, 3),
                          "hipblaslt_ms_per_step": round(blas_ms, 4),
                          "speedup_vs_hipblaslt": round(blas_ms / ms_step, 3)},
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, x_host, w_host, args.cpu_rows, flops_step, m)
    print(json.dumps(result), flush=True)


def rmsnorm_block(nv, torch, xs, workspace, steps, warmup):
    """RMSNorm of the layer's activation (8192 x 4096, rotated copies) with
    the quantiser fused in, against the unfused pair torch RMSNorm (BF16 out)
    then nvfp4_quantize_act.  Algorithmic bytes: 2 + 2 + 0.5625 an element
    fused (x read twice, codes and scales written), 2 + 2 + 2 + 2.5625
    unfused."""
    m, k = xs[0].shape
    gen = torch.Generator(device=xs[0].device)
    gen.manual_seed(99)
    g = (1.0 + 0.1 * torch.randn(k, device=xs[0].device, generator=gen)).to(torch.bfloat16)
    out = nv.nvfp4_rmsnorm_quantize_act(xs[0], g, 1e-6, workspace=workspace)
    out2 = nv.nvfp4_quantize_act(xs[0], workspace=workspace)

    def fused(i):
        nv.nvfp4_rmsnorm_quantize_act(xs[i % len(xs)], g, 1e-6, out=out, workspace=workspace)

    def unfused(i):
        yn = torch.nn.functional.rms_norm(xs[i % len(xs)], (k,), g, 1e-6)
        nv.nvfp4_quantize_act(yn, out=out2, workspace=workspace)

    tf = time_ms(torch, fused, max(steps, 20), warmup) * 1e3
    tu = time_ms(torch, unfused, max(steps, 20), warmup) * 1e3
    gbps = m * k * 4.5625 / (tf * 1e-6) / 1e9
    log(f"RMSNorm+quantise fused {tf:.1f} us ({gbps:.0f} GB/s); torch RMSNorm then quantise "
        f"{tu:.1f} us; x{tu / tf:.2f}")
    return {"kernel": "rmsnorm_amax_kernel + prepare_kernel + rmsnorm_quantize_kernel",
            "shape": [m, k], "us": round(tf, 2), "gbps": round(gbps, 1),
            "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "bytes_per_elem": 4.5625,
            "unfused_us": round(tu, 2), "speedup_vs_unfused": round(tu / tf, 3)}


def silu_block(nv, torch, qa, dev, workspace, steps, warmup):
    """The MLP's gate|up projection of the same model at prefill (Qwen3-8B:
    8192 tokens, 4096 -> 2 x 12288) with SiLU(gate) * up and H's quantiser
    fused into the GEMM (w4a4_gemm_silu_mul_quantize), against the unfused
    chain: the same GEMM writing BF16 gate|up, torch silu and multiply, then
    nvfp4_quantize_act of H.  Weights are seeded N(0, 0.02) draws made on
    the device."""
    m, k = qa.rows, qa.k
    hidden = 12288
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    qg, qu = [nv.nvfp4_quantize_weights(
        (torch.randn(hidden, k, device=dev, generator=gen) * 0.02).to(torch.bfloat16),
        workspace=workspace) for _ in range(2)]
    stack = nv.interleave_gate_up(qg, qu)
    n = 2 * hidden
    ws = nv.silu_mul_workspace(m, n, dev)
    qh, h = nv.w4a4_gemm_silu_mul_quantize(qa, stack, workspace=ws)
    y = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    qh2 = nv.NVFP4Tensor(torch.empty_like(qh.alpha), torch.empty_like(qh.scales),
                         torch.empty_like(qh.codes))

    def fused(i):
        nv.w4a4_gemm_silu_mul_quantize(qa, stack, h=h, out=qh, workspace=ws)

    def unfused(i):
        nv.w4a4_gemm_multi(qa, stack, f32=False, y_bf16=y)
        v = y.view(m, n // 64, 2, 32)
        hu = (torch.nn.functional.silu(v[:, :, 0]) * v[:, :, 1]).reshape(m, hidden)
        nv.nvfp4_quantize_act(hu, out=qh2, workspace=workspace)

    tf = time_ms(torch, fused, max(steps, 10), warmup)
    tu = time_ms(torch, unfused, max(steps, 10), warmup)
    flops = 2.0 * m * n * k
    log(f"gate|up GEMM + SiLU*up + quantise fused {tf * 1e3:.1f} us "
        f"({flops / (tf * 1e-3) / 1e12:.0f} TFLOP/s); unfused {tu * 1e3:.1f} us; x{tu / tf:.2f}")
    return {"kernel": "w4a4_gemm_kernel<silu> + prepare_kernel + quantize_kernel",
            "shape": [m, n, k], "ms": round(tf, 4),
            "tflops": round(flops / (tf * 1e-3) / 1e12, 2),
            "unfused_ms": round(tu, 4), "speedup_vs_unfused": round(tu / tf, 3)}


def graph_ms(torch, fn, n, reps, check=None):
    """fn(0) .. fn(n - 1) captured once in a HIP graph and replayed reps
    times: ms per fn call with no host launch cost between the kernels.
    check(), if given, returns a tensor the calls write; every replay must
    reproduce the eager result bit for bit."""
    for i in range(n):
        fn(i)
    torch.cuda.synchronize()
    ref = check().clone() if check is not None else None
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        if check is not None and not torch.equal(check(), ref):
            raise RuntimeError("graph replay differs from the eager launches")
        fn(0)                                   # eager work between replays
        torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / (reps * n)


def decode_block(nv, torch, dev, workspace, steps, warmup):
    """Decode-shaped W4A4 GEMMs of the same model (Qwen3-8B): the attention
    projections (Q|K|V stacked 6144x4096, then O 4096x4096) and the MLP
    (gate|up stacked 24576x4096, then down 4096x12288) at 1 and 16 tokens,
    each pair of launches timed with HIP events around replays of a HIP
    graph of the launches over all weight copies (a decode step's kernels
    are a few microseconds each, less than the host's cost to launch them
    one by one from Python; the eagerly launched time is reported beside
    it as us_eager).  The kernel streams the
    NVFP4 weight (0.5625 bytes a weight), so the rate is weight bytes over
    time against HBM.  Weights are seeded N(0, 0.02) draws made on the
    device (the timing does not depend on their values), with enough copies
    rotated (> 512 MB) that they come from HBM, not from the 256 MB MALL;
    hipBLASLt (torch.matmul) on BF16 copies of the same weights is timed
    beside it."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(2024)
    parts = {"attention": [(6144, 4096), (4096, 4096)], "mlp": [(24576, 4096), (4096, 12288)]}
    rows = []
    for part, shapes in parts.items():
        wbytes = sum(n * k * 9 // 16 for n, k in shapes)
        copies = max(2, (576 << 20) // wbytes)
        bf_copies = max(2, (576 << 20) // sum(n * k * 2 for n, k in shapes))
        bf = [[(torch.randn(n, k, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
               for n, k in shapes] for _ in range(bf_copies)]
        q0 = [nv.nvfp4_quantize_weights(w, workspace=workspace) for w in bf[0]]
        qs = [[nv.NVFP4Tensor(q.alpha.clone(), q.scales.clone(), q.codes.clone()) for q in q0]
              for _ in range(copies)]
        for tokens in (1, 16):
            acts = [(torch.randn(tokens, k, device=dev, generator=gen)).to(torch.bfloat16)
                    for _, k in shapes]
            qa = [nv.nvfp4_quantize_act(a, workspace=workspace) for a in acts]
            ys = [torch.empty(tokens, n, dtype=torch.bfloat16, device=dev) for n, _ in shapes]

            def w4a4(i):
                w = qs[i % copies]
                for j in range(len(shapes)):
                    nv.w4a4_gemm_decode(qa[j], w[j], f32=False, y_bf16=ys[j])

            def blas(i):
                w = bf[i % bf_copies]
                for j in range(len(shapes)):
                    torch.matmul(acts[j], w[j].t())

            t_eager = time_ms(torch, w4a4, max(steps, 20), warmup) * 1e3
            reps = max(3, max(steps, 20) // copies)
            t = graph_ms(torch, w4a4, copies, reps, check=lambda: ys[-1]) * 1e3
            tb = graph_ms(torch, blas, bf_copies, max(3, max(steps, 20) // bf_copies)) * 1e3
            gbps = wbytes / (t * 1e-6) / 1e9
            rows.append({"part": part, "tokens": tokens,
                         "shapes_nk": [list(x) for x in shapes],
                         "us": round(t, 2), "weight_gbps": round(gbps, 1),
                         "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                         "us_eager": round(t_eager, 2),
                         "hipblaslt_bf16_us": round(tb, 2), "speedup_vs_hipblaslt": round(tb / t, 3)})
            log(f"decode {part} x{tokens}: {t:.1f} us ({gbps:.0f} GB/s of NVFP4 weight; "
                f"{t_eager:.1f} us launched one by one); hipBLASLt BF16 {tb:.1f} us; x{tb / t:.2f}")
        del bf, qs, q0
        torch.cuda.empty_cache()
    return {"kernel": "w4a4_gemm_decode", "bytes_per_weight": 0.5625, "rows": rows}


def sweep(args):
    """Every GEMM and activation quantiser of configurations 1-5 on one GPU.

    Per GEMM: the W4A4 kernel (BF16 out), the BF16 comparison kernel and
    torch.matmul (hipBLASLt) on the same shapes; per activation tensor: the
    whole quantiser (amax, alpha, tables, quantize).  Before each timing the
    GPU runs 0.15 s of BF16 matmuls, so that the timings start from loaded
    steady-state clocks, not from the idle left by host-side input
    generation.  Inputs rotate over
    copies totalling at least 512 MB where a tensor is smaller, so reads come
    from HBM.  Configuration 4 also times the quantise-on-load GEMM;
    configuration 5 the grouped GEMMs (hipBLASLt as one matmul per expert).
    """
    import numpy as np
    import torch

    from nvfp4_w4a4_gemm_amd import binding as nv
    from nvfp4_w4a4_gemm_amd.workloads import workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ws = nv.new_workspace(dev)
    reps, warm = max(5, args.steps // 2), max(2, args.warmup)

    def copies(bits):
        n = max(1, min(8, -(-(512 << 20) // bits.nbytes)))
        return [nv.to_device_bf16(np.roll(bits, r, axis=0) if r else bits, dev) for r in range(n)]

    def settle():
        # the host-side input generation leaves the GPU idle; about 0.15 s of
        # sustained load brings its clocks back to their loaded steady state
        a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
        t = time.perf_counter()
        while time.perf_counter() - t < 0.15:
            for _ in range(10):
                a @ a
            torch.cuda.synchronize()
        del a

    for cfg in [int(c) for c in args.configs.split(",")]:
        wl = workload(cfg)
        log(f"sweep: configuration {cfg}: {wl.title}")
        out = {"config": cfg, "workload": wl.title, "gemms": [], "quantize": []}
        if cfg == 5:
            out.update(sweep_grouped(wl, nv, torch, dev, ws, copies, reps, warm, settle))
            print(json.dumps(out), flush=True)
            continue
        acts, qacts = {}, {}
        for g in wl.gemms:
            if g.act in acts:
                continue
            xs = copies(wl.tensors[g.act].full())
            acts[g.act] = xs
            q = nv.nvfp4_quantize_act(xs[0], workspace=ws)
            qacts[g.act] = q
            settle()
            t = time_ms(torch, lambda i: nv.nvfp4_quantize_act(xs[i % len(xs)], out=q,
                                                               workspace=ws), reps, warm)
            el = xs[0].numel()
            gbps = el * (QUANT_BYTES_PER_ELEM + AMAX_BYTES_PER_ELEM) / (t * 1e-3) / 1e9
            out["quantize"].append({"tensor": g.act, "shape": list(xs[0].shape),
                                    "ms": round(t, 4), "gbps": round(gbps, 1),
                                    "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)})
        layer = {"w4a4_ms": sum(q["ms"] for q in out["quantize"]), "bf16_ms": 0.0,
                 "hipblaslt_ms": 0.0}
        for g in wl.gemms:
            w = nv.to_device_bf16(wl.tensors[g.weight].full(), dev)
            qw = nv.nvfp4_quantize_weights(w, workspace=ws)
            xs, qa = acts[g.act], qacts[g.act]
            mm, kk, nn = xs[0].shape[0], xs[0].shape[1], w.shape[0]
            y = torch.empty(mm, nn, dtype=torch.bfloat16, device=dev)
            fl = 2.0 * mm * nn * kk
            settle()
            t4 = time_ms(torch, lambda i: nv.w4a4_gemm(qa, qw, f32=False, y_bf16=y), reps, warm)
            tb = time_ms(torch, lambda i: nv.bf16_gemm_baseline(xs[i % len(xs)], w, f32=False),
                         reps, warm)
            th = time_ms(torch, lambda i: torch.matmul(xs[i % len(xs)], w.t()), reps, warm)
            rec = {"gemm": g.name, "m": mm, "n": nn, "k": kk, "w4a4_ms": round(t4, 4),
                   "tflops": round(fl / (t4 * 1e-3) / 1e12, 1),
                   "frac_of_f16_mfma_peak": round(fl / (t4 * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                   "bf16_ms": round(tb, 4), "hipblaslt_ms": round(th, 4),
                   "speedup_vs_bf16": round(tb / t4, 3), "speedup_vs_hipblaslt": round(th / t4, 3)}
            if cfg == 4:
                tf = time_ms(torch, lambda i: nv.w4a4_gemm_fused_act(
                    xs[i % len(xs)], qa.alpha, qw, f32=False, y_bf16=y, workspace=ws), reps, warm)
                rec["fused_quantize_gemm_ms"] = round(tf, 4)
            out["gemms"].append(rec)
            layer["w4a4_ms"] += t4
            layer["bf16_ms"] += tb
            layer["hipblaslt_ms"] += th
            log(f"  {g.name} {mm}x{nn}x{kk}: w4a4 {t4:.3f} ms ({rec['tflops']} TFLOP/s), "
                f"bf16 {tb:.3f} ms, hipBLASLt {th:.3f} ms")
            del w, qw, y
            torch.cuda.empty_cache()
        layer["speedup_vs_bf16"] = round(layer["bf16_ms"] / layer["w4a4_ms"], 3)
        layer["speedup_vs_hipblaslt"] = round(layer["hipblaslt_ms"] / layer["w4a4_ms"], 3)
        out["layer"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in layer.items()}
        print(json.dumps(out), flush=True)
        del acts, qacts
        torch.cuda.empty_cache()


def sweep_grouped(wl, nv, torch, dev, ws, copies, reps, warm, settle):
    """Configuration 5: quantise X once, gather by routing, grouped GEMMs."""
    token_of_row, offsets = wl.routing()
    off_t = torch.from_numpy(offsets).to(dev)
    tok_t = torch.from_numpy(token_of_row).to(dev)
    res = {"gemms": [], "quantize": []}
    xs = copies(wl.tensors["X"].full())
    hs = copies(wl.tensors["H"].full())
    layer = {"w4a4_ms": 0.0, "bf16_ms": 0.0, "hipblaslt_ms": 0.0}
    for name, act, wname, gather in (("gate_up_proj", xs, "W_gu", tok_t),
                                     ("down_proj", hs, "W_down", None)):
        q = nv.nvfp4_quantize_act(act[0], workspace=ws)
        settle()
        t = time_ms(torch, lambda i: nv.nvfp4_quantize_act(act[i % len(act)], out=q, workspace=ws),
                    reps, warm)
        el = act[0].numel()
        gbps = el * (QUANT_BYTES_PER_ELEM + AMAX_BYTES_PER_ELEM) / (t * 1e-3) / 1e9
        res["quantize"].append({"tensor": "X" if gather is not None else "H",
                                "shape": list(act[0].shape), "ms": round(t, 4),
                                "gbps": round(gbps, 1),
                                "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)})
        layer["w4a4_ms"] += t
        wbits = [wl.tensors[f"{wname}[{e}]"].full() for e in range(wl.experts)]
        w = torch.stack([nv.to_device_bf16(b, dev) for b in wbits])
        qws = [nv.nvfp4_quantize_weights(w[e], workspace=ws) for e in range(wl.experts)]
        b_codes = torch.stack([qq.codes for qq in qws])
        b_scales = torch.stack([qq.scales for qq in qws])
        b_alpha = torch.cat([qq.alpha for qq in qws])
        mm = int(offsets[-1])
        nn, kk = w.shape[1], w.shape[2]
        y = torch.empty(mm, nn, dtype=torch.bfloat16, device=dev)
        fl = 2.0 * mm * nn * kk
        settle()
        t4 = time_ms(torch, lambda i: nv.w4a4_gemm_grouped(q, b_codes, b_scales, b_alpha, off_t,
                                                           a_row_index=gather, f32=False,
                                                           y_bf16=y), reps, warm)
        xg = act[0].index_select(0, tok_t.long()) if gather is not None else act[0]
        tb = time_ms(torch, lambda i: nv.bf16_gemm_baseline(xg, w, group_offsets=off_t,
                                                            f32=False), reps, warm)
        bounds = offsets.tolist()

        def blas(i):
            for e in range(wl.experts):
                torch.matmul(xg[bounds[e]:bounds[e + 1]], w[e].t())
        th = time_ms(torch, blas, max(3, reps // 2), 1)
        res["gemms"].append({"gemm": name, "m": mm, "n": nn, "k": kk, "groups": wl.experts,
                             "w4a4_ms": round(t4, 4),
                             "tflops": round(fl / (t4 * 1e-3) / 1e12, 1),
                             "frac_of_f16_mfma_peak": round(fl / (t4 * 1e-3) / 1e12 /
                                                            MFMA_F16_PEAK_TFLOPS, 4),
                             "bf16_ms": round(tb, 4), "hipblaslt_per_expert_ms": round(th, 4),
                             "speedup_vs_bf16": round(tb / t4, 3),
                             "speedup_vs_hipblaslt": round(th / t4, 3)})
        layer["w4a4_ms"] += t4
        layer["bf16_ms"] += tb
        layer["hipblaslt_ms"] += th
        log(f"  {name} grouped {mm}x{nn}x{kk}: w4a4 {t4:.3f} ms, bf16 {tb:.3f} ms, "
            f"hipBLASLt per expert {th:.3f} ms")
        del w, qws, b_codes, b_scales, y, xg
        torch.cuda.empty_cache()
    layer["speedup_vs_bf16"] = round(layer["bf16_ms"] / layer["w4a4_ms"], 3)
    layer["speedup_vs_hipblaslt"] = round(layer["hipblaslt_ms"] / layer["w4a4_ms"], 3)
    res["layer"] = {k: round(v, 4) for k, v in layer.items()}
    return res


def cpu_baseline(wl, x_host, w_host, rows, flops_step, m):
    """The oracle on a bounded sample: `rows` rows of both activations.

    Timed: alpha of each full activation, quantisation of the sample rows and
    the exact W4A4 reference of those rows against all four projections.
    The weights are quantised by the oracle first (offline, untimed).
    """
    import numpy as np
    from oracle import nvfp4_oracle as orc

    log(f"cpu baseline: oracle on {rows} rows of X_qkv and X_o")
    wq = {k: orc.quantize(v) for k, v in w_host.items()}
    t = time.perf_counter()
    flops = 0.0
    for key, ws in (("X_qkv", ("W_q", "W_k", "W_v")), ("X_o", ("W_o",))):
        full = x_host[key]
        alpha = orc.tensor_scale(orc.bf16_to_f64(full))
        qa = orc.quantize(full[:rows], alpha=alpha)
        for w in ws:
            orc.w4a4_reference(qa, wq[w])
            flops += 2.0 * rows * wq[w][2].shape[0] * full.shape[1]
    dt = time.perf_counter() - t
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    log(f"cpu baseline: {dt:.1f} s for {flops / 1e9:.1f} GFLOP")
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{rows} of {m} rows of X_qkv and X_o: full-tensor alpha, quantisation of "
                      f"the rows, exact W4A4 reference against W_q, W_k, W_v, W_o "
                      f"({flops / 1e9:.1f} GFLOP in {dt:.1f} s)"}


if __name__ == "__main__":
    main()
