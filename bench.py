#!/usr/bin/env python3
"""Benchmark of the NVFP4 W4A4 prefill linear layer on one MI355X.

Workload: the Qwen3-8B-shaped attention projections at prefill, M = 8192
tokens, hidden 4096: Q 4096->4096, K and V 4096->1024, O 4096->4096.  One
step is one pass of the whole hot path over one batch:

    alpha + NVFP4 quantisation of X_qkv   (amax, prepare, quantize kernels)
    Q, K, V W4A4 GEMMs (BF16 outputs)
    alpha + NVFP4 quantisation of X_o
    O W4A4 GEMM

Weights are quantised once before timing (offline, as in the layer).  The
inputs of consecutive steps rotate over several copies whose total exceeds the
256 MB last-level cache, so every step reads its activations from HBM.

The same step with the BF16 comparison GEMM (no quantisation) and with
torch.matmul (hipBLASLt) gives the speedups.  The oracle is timed on a
bounded sample on the host cores.  One JSON line goes to stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_F16_PEAK_TFLOPS = 2500.0          # dense f16/bf16 MFMA, MI355X
HBM_PEAK_GBPS = 8000.0
QUANT_BYTES_PER_ELEM = 2.0 + 0.5 + 1.0 / 16.0   # read BF16, write codes + scales
AMAX_BYTES_PER_ELEM = 2.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w4a4_gemm_256x256_qwen3_8b_attn_m8192_traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "nvfp4_w4a4_gemm_amd", "csrc", "gemm_w4a4.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(path):
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotate", type=int, default=4, help="input copies cycled over steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2048,
                    help="activation rows in the oracle's timed sample")
    return ap.parse_args()


class Timer:
    """HIP events around launches on torch's current stream (the library's)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def __call__(self, name):
        torch = self.torch
        timer = self

        class _Ctx:
            def __enter__(self_):
                self_.s = torch.cuda.Event(enable_timing=True)
                self_.e = torch.cuda.Event(enable_timing=True)
                self_.s.record()

            def __exit__(self_, *a):
                self_.e.record()
                timer.pairs.setdefault(name, []).append((self_.s, self_.e))
        return _Ctx()

    def total_ms(self, name):
        return sum(s.elapsed_time(e) for s, e in self.pairs.get(name, []))

    def count(self, name):
        return len(self.pairs.get(name, []))

    def reset(self):
        self.pairs = {}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this layer is measured on one GPU; multi-GPU sharding is "
                                   "described in DESIGN.md but not run", "n_gpus": args.gpus}))
        sys.exit(2)

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
    qbuf = {k: nv.nvfp4_quantize_act(xs[0][k], workspace=workspace) for k in x_host}
    outs = {g: torch.empty(m, wq[w].rows, dtype=torch.bfloat16, device=dev)
            for g, w in (("q", "W_q"), ("k", "W_k"), ("v", "W_v"), ("o", "W_o"))}
    torch.cuda.synchronize()

    proj = (("q", "W_q"), ("k", "W_k"), ("v", "W_v"))
    flops_step = sum(2.0 * m * wq[w].rows * h for _, w in proj) + 2.0 * m * h * h
    timer = Timer(torch)

    def w4a4_step(i, timed):
        x = xs[i % args.rotate]
        ctx = timer if timed else None
        for name, key in (("quant_qkv", "X_qkv"),):
            if ctx:
                with ctx("quantize"):
                    nv.nvfp4_quantize_act(x[key], out=qbuf[key], workspace=workspace)
            else:
                nv.nvfp4_quantize_act(x[key], out=qbuf[key], workspace=workspace)
        for g, w in proj:
            kname = "gemm_big" if g == "q" else "gemm_small"
            if ctx:
                with ctx(kname):
                    nv.w4a4_gemm(qbuf["X_qkv"], wq[w], f32=False, y_bf16=outs[g])
            else:
                nv.w4a4_gemm(qbuf["X_qkv"], wq[w], f32=False, y_bf16=outs[g])
        if ctx:
            with ctx("quantize"):
                nv.nvfp4_quantize_act(x["X_o"], out=qbuf["X_o"], workspace=workspace)
            with ctx("gemm_big"):
                nv.w4a4_gemm(qbuf["X_o"], wq["W_o"], f32=False, y_bf16=outs["o"])
        else:
            nv.nvfp4_quantize_act(x["X_o"], out=qbuf["X_o"], workspace=workspace)
            nv.w4a4_gemm(qbuf["X_o"], wq["W_o"], f32=False, y_bf16=outs["o"])

    def bf16_step(i):
        x = xs[i % args.rotate]
        for g, w in proj:
            nv.bf16_gemm_baseline(x["X_qkv"], ws[w], f32=False)
        nv.bf16_gemm_baseline(x["X_o"], ws["W_o"], f32=False)

    def blas_step(i):
        x = xs[i % args.rotate]
        for g, w in proj:
            torch.matmul(x["X_qkv"], ws[w].t())
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
    log(f"timing W4A4 layer: {args.warmup} warmup + {args.steps} steps")
    for i in range(args.warmup):
        w4a4_step(i, timed=False)
    torch.cuda.synchronize()
    timer.reset()
    t = time.perf_counter()
    for i in range(args.steps):
        w4a4_step(i, timed=True)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t) * 1e3 / args.steps

    n_big = timer.count("gemm_big")
    big_ms = timer.total_ms("gemm_big") / n_big
    small_ms = timer.total_ms("gemm_small") / max(1, timer.count("gemm_small"))
    quant_ms = timer.total_ms("quantize") / timer.count("quantize")
    gemm_ms_step = (timer.total_ms("gemm_big") + timer.total_ms("gemm_small")) / args.steps
    big_flops = 2.0 * m * h * h
    big_tflops = big_flops / (big_ms * 1e-3) / 1e12
    quant_bytes = m * h * (QUANT_BYTES_PER_ELEM + AMAX_BYTES_PER_ELEM)
    quant_gbps = quant_bytes / (quant_ms * 1e-3) / 1e9
    log(f"W4A4 step {ms_step:.3f} ms; GEMM 8192x4096x4096 {big_ms:.3f} ms "
        f"({big_tflops:.0f} TFLOP/s); K/V GEMM {small_ms:.3f} ms; "
        f"quantize {quant_ms:.3f} ms ({quant_gbps:.0f} GB/s incl. amax)")

    # --- comparisons ---------------------------------------------------------
    log("timing BF16 baseline step (same skeleton) and torch.matmul (hipBLASLt)")
    bf16_ms = time_steps(bf16_step, args.steps, args.warmup)
    blas_ms = time_steps(blas_step, args.steps, args.warmup)
    log(f"BF16 baseline step {bf16_ms:.3f} ms; hipBLASLt step {blas_ms:.3f} ms")

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE))
        if rec.get("source_sha256") == source_hash(GEMM_SOURCE):
            traffic = rec.get("bytes_per_launch")

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
                        "Q 4096->4096, K/V 4096->1024, O 4096->4096; NVFP4 W4A4, BF16 out",
            "global_batch": m,
            "flops_per_step": flops_step,
            "parallelism": "single GPU",
            "input_rotation": args.rotate,
        },
        "roofline": {
            "kernel": "w4a4_gemm_kernel<256,256> (Q and O projections, 8192x4096x4096)",
            "bound": "mfma",
            "achieved": round(big_tflops, 2),
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(big_tflops / MFMA_F16_PEAK_TFLOPS, 4),
            "traffic": traffic,
        },
        "quantize": {
            "gbps": round(quant_gbps, 1),
            "frac_of_hbm_peak": round(quant_gbps / HBM_PEAK_GBPS, 4),
            "ms_per_tensor": round(quant_ms, 4),
            "bytes_per_elem": QUANT_BYTES_PER_ELEM + AMAX_BYTES_PER_ELEM,
        },
        "gemm": {"ms_per_step": round(gemm_ms_step, 4),
                 "tflops": round(flops_step / (gemm_ms_step * 1e-3) / 1e12, 2),
                 "kv_gemm_ms": round(small_ms, 4)},
        "bf16_baseline": {"ms_per_step": round(bf16_ms, 4),
                          "speedup_layer": round(bf16_ms / ms_step, 3),
                          "speedup_gemm_only": round(bf16_ms / gemm_ms_step, 3),
                          "hipblaslt_ms_per_step": round(blas_ms, 4),
                          "speedup_vs_hipblaslt": round(blas_ms / ms_step, 3)},
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, x_host, w_host, args.cpu_rows, flops_step, m)
    print(json.dumps(result), flush=True)


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
