#!/usr/bin/env python3
"""Benchmark of the NVFP4 W4A4 prefill linear layer on one MI355X.

Workload (the largest single-GPU configuration): a large dense-model linear
stack at prefill, M = 16384 tokens, hidden 5120.  One step is one pass of the
whole hot path over one batch:

    alpha + NVFP4 quantisation of X_qkv, then QKV      W4A4 GEMM 16384 x  7168 x  5120
    alpha + NVFP4 quantisation of X_o,   then O        W4A4 GEMM 16384 x  5120 x  5120
    alpha + NVFP4 quantisation of X_gu,  then gate+up  W4A4 GEMM 16384 x 51200 x  5120
    alpha + NVFP4 quantisation of H,     then down     W4A4 GEMM 16384 x  5120 x 25600

(14 946.5 GFLOP a step, BF16 outputs).  Activations are Student-t (nu = 4)
BF16, weights N(0, 0.015), drawn by the seeded generator of
nvfp4_w4a4_gemm_amd.workloads.  Weights are quantised once before timing
(offline, as in the layer).  A step reads 1.3 GB of activations, five times
the 256 MB last-level cache, so every step reads them from HBM.

Before the warm-up steps the GPU runs layer steps for --settle-ms (untimed):
under sustained load the chip takes on the order of 100 ms to settle its
clocks.  The same step with the BF16 comparison GEMM (no quantisation) and
with torch.matmul (hipBLASLt) gives the speedups, stated against the faster
of the two.  The oracle is timed on a bounded sample on the host cores.  One
JSON line goes to stdout.

--sweep times every GEMM and quantiser of the five configurations instead;
--counter-pass runs the fixed launch sequence the hardware-counter summaries
under profiles/ are taken on (rocprofv3 --pmc ... -- python3 bench.py
--counter-pass).
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w4a4_gemm_gate_up_16384x51200x5120_traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "nvfp4_w4a4_gemm_amd", "csrc", "gemm_w4a4.hip")

# the layer step: (activation, weight, output) in launch order
LAYER = (("X_qkv", "W_qkv", "qkv"), ("X_o", "W_o", "o"), ("X_gu", "W_gu", "gate_up"),
         ("H", "W_down", "down"))
ROOFLINE_GEMM = "gate_up"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(path):
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def stored_traffic(traffic_file=None, source=None):
    """HBM bytes per gate+up launch from the committed counter record, or
    None when there is none or the GEMM source has changed since it was
    taken."""
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
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="untimed layer steps before the warm-up, so the clocks settle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the extra fields (smaller configuration, fused producers, decode)")
    ap.add_argument("--cpu-rows", type=int, default=1024,
                    help="activation rows of each GEMM in the oracle's timed sample")
    ap.add_argument("--cpu-cols", type=int, default=2048,
                    help="weight rows (output columns) of each GEMM in the oracle's sample")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the layer step: time every GEMM and quantiser of the five "
                         "layer configurations (one JSON line per configuration)")
    ap.add_argument("--configs", default="1,2,3,4,5", help="configurations for --sweep")
    ap.add_argument("--counter-pass", action="store_true",
                    help="run the fixed launch sequence of the hardware-counter summaries")
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


class _Null:
    def __enter__(self):
        return None

    def __exit__(self, *a):
        return False


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


def settle_with(torch, fn, ms):
    """Run fn(i) repeatedly for at least `ms` milliseconds of wall time
    (untimed), so that the clocks reach their loaded steady state."""
    t = time.perf_counter()
    i = 0
    while (time.perf_counter() - t) * 1e3 < ms:
        fn(i)
        i += 1
        if i % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def threads_used():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count()


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
    if args.counter_pass:
        counter_pass()
        return

    import torch

    from nvfp4_w4a4_gemm_amd import binding as nv
    from nvfp4_w4a4_gemm_amd.workloads import workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workload(4)
    log(f"workload: {wl.title}; generating inputs")
    t0 = time.time()
    x_dev, w_dev = {}, {}
    for xname, wname, _ in LAYER:
        x_dev[xname] = nv.to_device_bf16(wl.tensors[xname].full(), dev)
        w_dev[wname] = nv.to_device_bf16(wl.tensors[wname].full(), dev)
    log(f"inputs generated and uploaded in {time.time() - t0:.1f} s")

    workspace = nv.new_workspace(dev)
    wq = {k: nv.nvfp4_quantize_weights(v, workspace=workspace) for k, v in w_dev.items()}
    qbuf = {k: nv.nvfp4_quantize_act(v, workspace=workspace) for k, v in x_dev.items()}
    m = x_dev["X_qkv"].shape[0]
    outs = {name: torch.empty(m, w_dev[wname].shape[0], dtype=torch.bfloat16, device=dev)
            for _, wname, name in LAYER}
    flops = {name: 2.0 * m * w_dev[wname].shape[0] * w_dev[wname].shape[1]
             for _, wname, name in LAYER}
    flops_step = sum(flops.values())
    torch.cuda.synchronize()
    timer = Timer(torch)
    null = lambda name: _Null()

    def w4a4_step(i, timed=False, every=False):
        # timed: HIP events around the gate+up GEMM (the roofline kernel);
        # every: around every launch (a separate pass: many live events make
        # the runtime stall the host, so the timed region keeps them few)
        for xname, wname, name in LAYER:
            with (timer if every else null)("q_" + xname):
                nv.nvfp4_quantize_act(x_dev[xname], out=qbuf[xname], workspace=workspace)
            ctx = timer if (every or (timed and name == ROOFLINE_GEMM)) else null
            with ctx("g_" + name):
                nv.w4a4_gemm(qbuf[xname], wq[wname], f32=False, y_bf16=outs[name])

    def bf16_step(i):
        for xname, wname, name in LAYER:
            nv.bf16_gemm_baseline(x_dev[xname], w_dev[wname], f32=False)

    def blas_step(i):
        for xname, wname, name in LAYER:
            torch.matmul(x_dev[xname], w_dev[wname].t())

    def time_steps(fn, steps, warmup, settle_ms):
        settle_with(torch, fn, settle_ms)
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
    log(f"timing W4A4 layer: {args.settle_ms:.0f} ms settle, {args.warmup} warmup + "
        f"{args.steps} steps")
    settle_with(torch, w4a4_step, args.settle_ms)
    for i in range(args.warmup):
        w4a4_step(i)
    timer.prepare("g_" + ROOFLINE_GEMM, args.steps)
    torch.cuda.synchronize()
    timer.reset()
    t = time.perf_counter()
    for i in range(args.steps):
        w4a4_step(i, timed=True)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t) * 1e3 / args.steps
    roof_times = sorted(timer.times_ms("g_" + ROOFLINE_GEMM))
    roof_ms = sum(roof_times) / len(roof_times)
    roof_stats = {"mean": round(roof_ms * 1e3, 1),
                  "median": round(roof_times[len(roof_times) // 2] * 1e3, 1),
                  "min": round(roof_times[0] * 1e3, 1), "max": round(roof_times[-1] * 1e3, 1),
                  "launches": len(roof_times)}

    # every launch's duration, from a second pass of the same steps
    passes = min(args.steps, 10)
    for xname, wname, name in LAYER:
        timer.prepare("q_" + xname, passes)
        timer.prepare("g_" + name, passes)
    torch.cuda.synchronize()
    for i in range(passes):
        w4a4_step(i, every=True)
    torch.cuda.synchronize()
    per = {}
    for xname, wname, name in LAYER:
        per["q_" + xname] = timer.total_ms("q_" + xname) / timer.count("q_" + xname)
        per["g_" + name] = timer.total_ms("g_" + name) / timer.count("g_" + name)
    gemm_ms_step = sum(per["g_" + name] for _, _, name in LAYER)
    quant_ms_step = sum(per["q_" + xname] for xname, _, _ in LAYER)
    roof_tflops = flops[ROOFLINE_GEMM] / (roof_ms * 1e-3) / 1e12
    log(f"W4A4 step {ms_step:.3f} ms ({flops_step / (ms_step * 1e-3) / 1e12:.0f} TFLOP/s); "
        f"gate+up GEMM {roof_ms:.3f} ms ({roof_tflops:.0f} TFLOP/s, "
        f"{roof_tflops / MFMA_F16_PEAK_TFLOPS:.3f} of the f16 MFMA peak)")
    log("per launch: " + ", ".join(f"{k} {v * 1e3:.1f} us" for k, v in per.items()))

    # --- quantiser passes on their own, and the attainable copy rate ----------
    quant = {}
    for xname in ("X_gu", "H"):
        x = x_dev[xname]
        n_el = x.numel()
        alpha_dev = qbuf[xname].alpha.clone()
        t_all = per["q_" + xname]
        t_alpha = time_ms(torch, lambda i: nv.nvfp4_tensor_alpha(x, workspace=workspace),
                          args.steps, 3)
        t_given = time_ms(torch, lambda i: nv.nvfp4_quantize_act(x, alpha_in=alpha_dev,
                                                                 out=qbuf[xname],
                                                                 workspace=workspace),
                          args.steps, 3)
        cpy = torch.empty_like(x)
        t_copy = time_ms(torch, lambda i: cpy.copy_(x), args.steps, 3)
        del cpy
        gbps = n_el * (QUANT_BYTES_PER_ELEM + AMAX_BYTES_PER_ELEM) / (t_all * 1e-3) / 1e9
        copy_gbps = 2 * n_el * 2 / (t_copy * 1e-3) / 1e9
        quant[xname] = {
            "shape": list(x.shape), "ms": round(t_all, 4), "gbps": round(gbps, 1),
            "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "bytes_per_elem": QUANT_BYTES_PER_ELEM + AMAX_BYTES_PER_ELEM,
            "amax_pass_gbps": round(n_el * AMAX_BYTES_PER_ELEM / (t_alpha * 1e-3) / 1e9, 1),
            "quantize_pass_gbps": round(n_el * QUANT_BYTES_PER_ELEM / (t_given * 1e-3) / 1e9, 1),
            "device_copy_gbps": round(copy_gbps, 1),
            "frac_of_device_copy": round(gbps / copy_gbps, 4)}
        log(f"quantiser {xname} {list(x.shape)}: {t_all * 1e3:.1f} us in the step "
            f"({gbps:.0f} GB/s incl. amax); amax+alpha {t_alpha * 1e3:.1f} us, quantize "
            f"(alpha given) {t_given * 1e3:.1f} us; device copy {t_copy * 1e3:.1f} us")
    quant_bytes_step = sum(x_dev[xname].numel() for xname, _, _ in LAYER) * (
        QUANT_BYTES_PER_ELEM + AMAX_BYTES_PER_ELEM)

    # --- comparisons ---------------------------------------------------------
    log("timing the BF16 comparison kernel and torch.matmul (hipBLASLt) steps")
    bf16_ms = time_steps(bf16_step, args.steps, args.warmup, args.settle_ms)
    blas_ms = time_steps(blas_step, args.steps, args.warmup, args.settle_ms)
    faster = "hipblaslt" if blas_ms <= bf16_ms else "same_skeleton_kernel"
    ref_ms = min(blas_ms, bf16_ms)
    log(f"BF16 comparison kernel step {bf16_ms:.3f} ms; hipBLASLt step {blas_ms:.3f} ms; "
        f"W4A4 x{ref_ms / ms_step:.3f} against the faster ({faster})")

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
            "workload": "large dense-model linear stack at prefill: M=16384 tokens, hidden 5120; "
                        "QKV 5120->7168, O 5120->5120, gate+up 5120->51200, down 25600->5120; "
                        "each activation quantised to NVFP4 in the step; Student-t(4) "
                        "activations, N(0, 0.015) weights; BF16 out",
            "global_batch": m,
            "flops_per_step": flops_step,
            "parallelism": "single GPU",
            "settle_ms": args.settle_ms,
        },
        "roofline": {
            "kernel": f"w4a4_gemm_kernel<256,256> (gate+up projection, {m}x"
                      f"{w_dev['W_gu'].shape[0]}x{w_dev['W_gu'].shape[1]}, persistent tile walk)",
            "bound": "mfma",
            "achieved": round(roof_tflops, 2),
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(roof_tflops / MFMA_F16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "launch_us": roof_stats,
        },
        "gemm": {"ms_per_step": round(gemm_ms_step, 4),
                 "tflops": round(flops_step / (gemm_ms_step * 1e-3) / 1e12, 2),
                 "frac_of_f16_mfma_peak": round(
                     flops_step / (gemm_ms_step * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                 "frac_of_fp4_mfma_peak": round(
                     flops_step / (gemm_ms_step * 1e-3) / 1e12 / MFMA_FP4_PEAK_TFLOPS, 4),
                 "per_gemm_ms": {name: round(per["g_" + name], 4) for _, _, name in LAYER},
                 "per_gemm_tflops": {name: round(flops[name] / (per["g_" + name] * 1e-3) / 1e12, 1)
                                     for _, _, name in LAYER}},
        "quantize": {"ms_per_step": round(quant_ms_step, 4),
                     "gbps": round(quant_bytes_step / (quant_ms_step * 1e-3) / 1e9, 1),
                     "frac_of_hbm_peak": round(
                         quant_bytes_step / (quant_ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "per_tensor_ms": {xname: round(per["q_" + xname], 4)
                                       for xname, _, _ in LAYER},
                     "tensors": quant},
        "bf16_baseline": {"same_skeleton_kernel_ms_per_step": round(bf16_ms, 4),
                          "hipblaslt_ms_per_step": round(blas_ms, 4),
                          "faster": faster,
                          "speedup_layer": round(ref_ms / ms_step, 3),
                          "speedup_gemm_only": round(ref_ms / gemm_ms_step, 3),
                          "speedup_layer_vs_same_skeleton_kernel": round(bf16_ms / ms_step, 3),
                          "speedup_layer_vs_hipblaslt": round(blas_ms / ms_step, 3)},
    }

    if not args.no_extras:
        # the same steps replayed from HIP graphs (two steps a graph, every
        # replay checked against the eager result): no host launch cost or
        # launch gaps between the 16 W4A4 launches or the 4 hipBLASLt ones
        log("timing the layer step replayed from HIP graphs, W4A4 and hipBLASLt")
        bl_out = {name: torch.empty(m, w_dev[wname].shape[0], dtype=torch.bfloat16, device=dev)
                  for _, wname, name in LAYER}

        def blas_step_out(i):
            for xname, wname, name in LAYER:
                torch.matmul(x_dev[xname], w_dev[wname].t(), out=bl_out[name])
        reps_g = max(5, args.steps // 2)
        settle_with(torch, w4a4_step, args.settle_ms)
        g_w4 = graph_ms(torch, w4a4_step, 2, reps_g, check=lambda: outs["down"])
        settle_with(torch, blas_step_out, args.settle_ms)
        g_bl = graph_ms(torch, blas_step_out, 2, reps_g, check=lambda: bl_out["down"])
        result["graph_step"] = {"w4a4_ms_per_step": round(g_w4, 4),
                                "hipblaslt_ms_per_step": round(g_bl, 4),
                                "speedup_vs_hipblaslt": round(g_bl / g_w4, 3),
                                "steps_per_graph": 2, "replays": reps_g}
        log(f"graph-replayed step: W4A4 {g_w4:.3f} ms, hipBLASLt {g_bl:.3f} ms")
        del outs, bl_out
        torch.cuda.empty_cache()
        result["attention_qwen3_8b_m8192"] = attention_block(nv, torch, dev, workspace, args)
        log("timing RMSNorm with the quantiser fused in, against RMSNorm then quantise")
        result["rmsnorm_quantize"] = rmsnorm_block(nv, torch, [x_dev["X_qkv"]], workspace,
                                                   args.steps, 3)
        log("timing the gate|up GEMM with SiLU(gate)*up and its quantiser fused in")
        result["gate_up_silu_quantize"] = silu_block(nv, torch, qbuf["X_gu"], dev, workspace,
                                                     args.steps, 3, hidden=25600, std=0.015)
        log("timing decode-shaped W4A4 GEMMs (w4a4_gemm_decode) against hipBLASLt BF16")
        result["decode"] = decode_block(nv, torch, dev, workspace, args.steps, 3)
        log("timing the layer with its producers (RMSNorm, SiLU*up) on both sides")
        result["layer_with_producers"] = producers_block(nv, torch, dev, x_dev, w_dev, wq,
                                                         qbuf, workspace, args)
        # the other layer configurations, so that every configuration has a
        # figure from this run: each GEMM beside hipBLASLt, each quantiser
        log("timing configurations 1, 2, 3 and 5: each GEMM beside hipBLASLt, each quantiser")
        result["other_configs"] = {}
        for cfg in (1, 2, 3, 5):
            try:
                result["other_configs"][str(cfg)] = sweep_config(cfg, nv, torch, dev, workspace,
                                                                  5, 2, bf16_kernel=False)
            except Exception as exc:      # the headline line is printed regardless
                torch.cuda.synchronize()
                result["other_configs"][str(cfg)] = {"error": f"{type(exc).__name__}: {exc}"}
                log(f"configuration {cfg} not timed: {exc}")
            torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_rows, args.cpu_cols, m)
    print(json.dumps(result), flush=True)


def producers_block(nv, torch, dev, x_dev, w_dev, wq, qbuf, workspace, args):
    """The same four projections with the operations that produce their
    inputs in a transformer block, on both sides: RMSNorm before Q|K|V and
    before gate|up, and H = SiLU(gate) * up between gate|up and down (the
    attention that produces O's input is not part of either side; X_o is
    given).  W4A4: nvfp4_rmsnorm_quantize_act for the two normalised inputs,
    the gate|up GEMM with SiLU*up and H's quantiser fused in
    (w4a4_gemm_silu_mul_quantize, gate and up rows interleaved), the
    quantiser for X_o, and the W4A4 GEMMs.  BF16: torch rms_norm, torch.matmul
    (hipBLASLt) and torch silu and multiply.  The GEMM FLOPs are the same on
    both sides."""
    m, hid = x_dev["X_qkv"].shape
    inter = w_dev["W_down"].shape[1]
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    g1, g2 = [(1.0 + 0.1 * torch.randn(hid, device=dev, generator=gen)).to(torch.bfloat16)
              for _ in range(2)]
    wgu = w_dev["W_gu"]
    qg = nv.nvfp4_quantize_weights(wgu[:inter].contiguous(), workspace=workspace)
    qu = nv.nvfp4_quantize_weights(wgu[inter:].contiguous(), workspace=workspace)
    stack = nv.interleave_gate_up(qg, qu)
    del qg, qu
    ws_silu = nv.silu_mul_workspace(m, 2 * inter, dev)
    ws_norm = nv.rmsnorm_workspace(m, dev)
    qn1 = nv.nvfp4_rmsnorm_quantize_act(x_dev["X_qkv"], g1, 1e-6, workspace=ws_norm)
    qn2 = nv.nvfp4_rmsnorm_quantize_act(x_dev["X_gu"], g2, 1e-6, workspace=ws_norm)
    qh, h = nv.w4a4_gemm_silu_mul_quantize(qn2, stack, workspace=ws_silu)
    y = {name: torch.empty(m, w_dev[wname].shape[0], dtype=torch.bfloat16, device=dev)
         for _, wname, name in LAYER if name != "gate_up"}
    torch.cuda.synchronize()

    def w4a4(i):
        nv.nvfp4_rmsnorm_quantize_act(x_dev["X_qkv"], g1, 1e-6, out=qn1, workspace=ws_norm)
        nv.w4a4_gemm(qn1, wq["W_qkv"], f32=False, y_bf16=y["qkv"])
        nv.nvfp4_quantize_act(x_dev["X_o"], out=qbuf["X_o"], workspace=workspace)
        nv.w4a4_gemm(qbuf["X_o"], wq["W_o"], f32=False, y_bf16=y["o"])
        nv.nvfp4_rmsnorm_quantize_act(x_dev["X_gu"], g2, 1e-6, out=qn2, workspace=ws_norm)
        nv.w4a4_gemm_silu_mul_quantize(qn2, stack, h=h, out=qh, workspace=ws_silu)
        nv.w4a4_gemm(qh, wq["W_down"], f32=False, y_bf16=y["down"])

    def bf16(i):
        a = torch.nn.functional.rms_norm(x_dev["X_qkv"], (hid,), g1, 1e-6)
        torch.matmul(a, w_dev["W_qkv"].t())
        torch.matmul(x_dev["X_o"], w_dev["W_o"].t())
        b = torch.nn.functional.rms_norm(x_dev["X_gu"], (hid,), g2, 1e-6)
        gu = torch.matmul(b, wgu.t())
        hb = torch.nn.functional.silu(gu[:, :inter]) * gu[:, inter:]
        del gu
        torch.matmul(hb, w_dev["W_down"].t())

    def run(fn):
        settle_with(torch, fn, args.settle_ms)
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(args.steps):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3 / args.steps

    tw = run(w4a4)
    tb = run(bf16)
    flops = sum(2.0 * m * w_dev[wname].shape[0] * w_dev[wname].shape[1] for _, wname, _ in LAYER)
    log(f"layer with producers: W4A4 {tw:.3f} ms ({flops / (tw * 1e-3) / 1e12:.0f} TFLOP/s), "
        f"BF16 hipBLASLt + torch {tb:.3f} ms; x{tb / tw:.3f}")
    return {"w4a4_ms_per_step": round(tw, 4), "bf16_hipblaslt_torch_ms_per_step": round(tb, 4),
            "gemm_tflops_w4a4": round(flops / (tw * 1e-3) / 1e12, 1),
            "speedup_vs_bf16": round(tb / tw, 3),
            "w4a4_ops": "rmsnorm+quantise, QKV GEMM, quantise X_o, O GEMM, rmsnorm+quantise, "
                        "gate|up GEMM with SiLU*up and H's quantiser, down GEMM",
            "bf16_ops": "torch rms_norm, matmul, matmul, rms_norm, matmul, silu*mul, matmul"}


def attention_block(nv, torch, dev, workspace, args):
    """The smaller attention configuration (Qwen3-8B-shaped, M = 8192): the
    quantisers and the stacked Q|K|V and O GEMMs, as a layer step, over four
    rotated input copies (512 MiB, so the activations come from HBM)."""
    import numpy as np
    from nvfp4_w4a4_gemm_amd.workloads import workload
    wl = workload(2)
    log(f"extra: {wl.title}")
    xh = {k: wl.tensors[k].full() for k in ("X_qkv", "X_o")}
    xs = [{k: nv.to_device_bf16(np.roll(v, r, axis=0), dev) for k, v in xh.items()}
          for r in range(4)]
    wq = {n: nv.nvfp4_quantize_weights(nv.to_device_bf16(wl.tensors[n].full(), dev),
                                       workspace=workspace) for n in ("W_q", "W_k", "W_v", "W_o")}
    qkv = nv.stack_tensors([wq["W_q"], wq["W_k"], wq["W_v"]])
    qb = {k: nv.nvfp4_quantize_act(xs[0][k], workspace=workspace) for k in xh}
    m, h = 8192, 4096
    y_qkv = torch.empty(m, qkv.rows, dtype=torch.bfloat16, device=dev)
    y_o = torch.empty(m, h, dtype=torch.bfloat16, device=dev)

    def step(i):
        x = xs[i % 4]
        nv.nvfp4_quantize_act(x["X_qkv"], out=qb["X_qkv"], workspace=workspace)
        nv.w4a4_gemm_multi(qb["X_qkv"], qkv, f32=False, y_bf16=y_qkv)
        nv.nvfp4_quantize_act(x["X_o"], out=qb["X_o"], workspace=workspace)
        nv.w4a4_gemm(qb["X_o"], wq["W_o"], f32=False, y_bf16=y_o)

    settle_with(torch, step, args.settle_ms)
    ms = time_ms(torch, step, max(args.steps, 20), args.warmup)
    t_qkv = time_ms(torch, lambda i: nv.w4a4_gemm_multi(qb["X_qkv"], qkv, f32=False,
                                                        y_bf16=y_qkv), 20, 3)
    fl = 2.0 * m * (qkv.rows + h) * h
    fq = 2.0 * m * qkv.rows * h
    log(f"attention M=8192: step {ms:.3f} ms ({fl / (ms * 1e-3) / 1e12:.0f} TFLOP/s), "
        f"Q|K|V GEMM {t_qkv * 1e3:.1f} us ({fq / (t_qkv * 1e-3) / 1e12:.0f} TFLOP/s)")
    return {"shape": "M=8192, hidden 4096, Q|K|V 4096->6144 stacked, O 4096->4096",
            "ms_per_step": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
            "qkv_gemm_us": round(t_qkv * 1e3, 1),
            "qkv_gemm_frac_of_f16_mfma_peak": round(
                fq / (t_qkv * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}


def rmsnorm_block(nv, torch, xs, workspace, steps, warmup):
    """RMSNorm of the layer's QKV activation (16384 x 5120, read from HBM)
    with the quantiser fused in, against the unfused pair torch RMSNorm (BF16
    out) then nvfp4_quantize_act.  Algorithmic bytes: 2 + 2 + 0.5625 an
    element fused (x read twice, codes and scales written), 2 + 2 + 2 +
    2.5625 unfused."""
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


def silu_block(nv, torch, qa, dev, workspace, steps, warmup, hidden, std):
    """The layer's gate|up projection (16384 tokens, 5120 -> 2 x 25600) with
    SiLU(gate) * up and H's quantiser fused into the GEMM
    (w4a4_gemm_silu_mul_quantize), against the unfused chain: the same GEMM
    writing BF16 gate|up, torch silu and multiply, then nvfp4_quantize_act of
    H.  Weights are seeded N(0, std) draws made on the device."""
    m, k = qa.rows, qa.k
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    qg, qu = [nv.nvfp4_quantize_weights(
        (torch.randn(hidden, k, device=dev, generator=gen) * std).to(torch.bfloat16),
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
    """Decode-shaped W4A4 GEMMs of the same layer: the attention projections
    (QKV 7168x5120, then O 5120x5120) and the MLP (gate+up 51200x5120, then
    down 5120x25600), and a Qwen3-8B-shaped gate+up weight 24576x4096, at 1
    and 16 tokens,
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
    parts = {"attention": [(7168, 5120), (5120, 5120)], "mlp": [(51200, 5120), (5120, 25600)],
             "qwen3_8b_gate_up": [(24576, 4096)]}
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
    """Every GEMM and activation quantiser of configurations 1-5 on one GPU,
    one JSON line per configuration (sweep_config)."""
    import torch

    from nvfp4_w4a4_gemm_amd import binding as nv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ws = nv.new_workspace(dev)
    reps, warm = max(5, args.steps // 2), max(2, args.warmup)
    for cfg in [int(c) for c in args.configs.split(",")]:
        print(json.dumps(sweep_config(cfg, nv, torch, dev, ws, reps, warm)), flush=True)
        torch.cuda.empty_cache()


def sweep_config(cfg, nv, torch, dev, ws, reps, warm, bf16_kernel=True):
    """Every GEMM and activation quantiser of one layer configuration.

    Per GEMM: the W4A4 kernel (BF16 out), the BF16 comparison kernel (unless
    bf16_kernel is false) and torch.matmul (hipBLASLt) on the same shapes;
    per activation tensor: the whole quantiser (amax, alpha, tables,
    quantize).  Before each timing the GPU runs 0.15 s of BF16 matmuls, so
    that the timings start from loaded steady-state clocks, not from the idle
    left by host-side input generation.  Inputs rotate over copies totalling
    at least 512 MB where a tensor is smaller, so reads come from HBM.
    Configuration 4 also times the quantise-on-load GEMM; configuration 5
    the grouped GEMMs (hipBLASLt as one matmul per expert).
    """
    import numpy as np

    from nvfp4_w4a4_gemm_amd.workloads import workload

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

    wl = workload(cfg)
    log(f"sweep: configuration {cfg}: {wl.title}")
    out = {"config": cfg, "workload": wl.title, "gemms": [], "quantize": []}
    if cfg == 5:
        out.update(sweep_grouped(wl, nv, torch, dev, ws, copies, reps, warm, settle, bf16_kernel))
        return out
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
    layer = {"w4a4_ms": sum(q["ms"] for q in out["quantize"]), "hipblaslt_ms": 0.0}
    if bf16_kernel:
        layer["bf16_ms"] = 0.0
    for g in wl.gemms:
        w = nv.to_device_bf16(wl.tensors[g.weight].full(), dev)
        qw = nv.nvfp4_quantize_weights(w, workspace=ws)
        xs, qa = acts[g.act], qacts[g.act]
        mm, kk, nn = xs[0].shape[0], xs[0].shape[1], w.shape[0]
        y = torch.empty(mm, nn, dtype=torch.bfloat16, device=dev)
        fl = 2.0 * mm * nn * kk
        settle()
        t4 = time_ms(torch, lambda i: nv.w4a4_gemm(qa, qw, f32=False, y_bf16=y), reps, warm)
        th = time_ms(torch, lambda i: torch.matmul(xs[i % len(xs)], w.t()), reps, warm)
        rec = {"gemm": g.name, "m": mm, "n": nn, "k": kk, "w4a4_ms": round(t4, 4),
               "tflops": round(fl / (t4 * 1e-3) / 1e12, 1),
               "frac_of_f16_mfma_peak": round(fl / (t4 * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
               "hipblaslt_ms": round(th, 4), "speedup_vs_hipblaslt": round(th / t4, 3)}
        if bf16_kernel:
            tb = time_ms(torch, lambda i: nv.bf16_gemm_baseline(xs[i % len(xs)], w, f32=False),
                         reps, warm)
            rec["bf16_ms"] = round(tb, 4)
            rec["speedup_vs_bf16"] = round(tb / t4, 3)
            layer["bf16_ms"] += tb
        if cfg == 4 and bf16_kernel:
            tf = time_ms(torch, lambda i: nv.w4a4_gemm_fused_act(
                xs[i % len(xs)], qa.alpha, qw, f32=False, y_bf16=y, workspace=ws), reps, warm)
            rec["fused_quantize_gemm_ms"] = round(tf, 4)
        out["gemms"].append(rec)
        layer["w4a4_ms"] += t4
        layer["hipblaslt_ms"] += th
        log(f"  {g.name} {mm}x{nn}x{kk}: w4a4 {t4:.3f} ms ({rec['tflops']} TFLOP/s), "
            f"hipBLASLt {th:.3f} ms")
        del w, qw, y
        torch.cuda.empty_cache()
    if bf16_kernel:
        layer["speedup_vs_bf16"] = round(layer["bf16_ms"] / layer["w4a4_ms"], 3)
    layer["speedup_vs_hipblaslt"] = round(layer["hipblaslt_ms"] / layer["w4a4_ms"], 3)
    out["layer"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in layer.items()}
    del acts, qacts
    return out


def sweep_grouped(wl, nv, torch, dev, ws, copies, reps, warm, settle, bf16_kernel=True):
    """Configuration 5: quantise X once, gather by routing, grouped GEMMs."""
    token_of_row, offsets = wl.routing()
    off_t = torch.from_numpy(offsets).to(dev)
    tok_t = torch.from_numpy(token_of_row).to(dev)
    res = {"gemms": [], "quantize": []}
    xs = copies(wl.tensors["X"].full())
    hs = copies(wl.tensors["H"].full())
    layer = {"w4a4_ms": 0.0, "hipblaslt_ms": 0.0}
    if bf16_kernel:
        layer["bf16_ms"] = 0.0
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
        tb = (time_ms(torch, lambda i: nv.bf16_gemm_baseline(xg, w, group_offsets=off_t,
                                                             f32=False), reps, warm)
              if bf16_kernel else None)
        bounds = offsets.tolist()

        def blas(i):
            for e in range(wl.experts):
                torch.matmul(xg[bounds[e]:bounds[e + 1]], w[e].t())
        th = time_ms(torch, blas, max(3, reps // 2), 1)
        rec = {"gemm": name, "m": mm, "n": nn, "k": kk, "groups": wl.experts,
               "w4a4_ms": round(t4, 4),
               "tflops": round(fl / (t4 * 1e-3) / 1e12, 1),
               "frac_of_f16_mfma_peak": round(fl / (t4 * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
               "hipblaslt_per_expert_ms": round(th, 4),
               "speedup_vs_hipblaslt": round(th / t4, 3)}
        if bf16_kernel:
            rec["bf16_ms"] = round(tb, 4)
            rec["speedup_vs_bf16"] = round(tb / t4, 3)
            layer["bf16_ms"] += tb
        res["gemms"].append(rec)
        layer["w4a4_ms"] += t4
        layer["hipblaslt_ms"] += th
        log(f"  {name} grouped {mm}x{nn}x{kk}: w4a4 {t4:.3f} ms, "
            f"hipBLASLt per expert {th:.3f} ms")
        del w, qws, b_codes, b_scales, y, xg
        torch.cuda.empty_cache()
    if bf16_kernel:
        layer["speedup_vs_bf16"] = round(layer["bf16_ms"] / layer["w4a4_ms"], 3)
    layer["speedup_vs_hipblaslt"] = round(layer["hipblaslt_ms"] / layer["w4a4_ms"], 3)
    res["layer"] = {k: round(v, 4) for k, v in layer.items()}
    return res


def cpu_baseline(wl, rows, cols, m):
    """The oracle on a bounded sample of the layer step, extrapolated
    linearly to the whole step.

    For each of the four GEMMs: the first `rows` rows of the activation and
    the first `cols` rows of the weight.  Timed per GEMM: the oracle's
    quantisation of the activation rows (alpha from those rows, then scales
    and codes: work proportional to rows x K) and its exact W4A4 reference of
    those rows against the weight rows (work proportional to rows x cols x
    K).  The weight rows are quantised first (offline, untimed).  The whole
    step's oracle time is estimated as sum over GEMMs of
    t_quant * M / rows + t_gemm * (M N) / (rows cols); the oracle's matrix
    products run faster on larger blocks, so the estimate is an upper bound
    on its time.
    """
    from oracle import nvfp4_oracle as orc

    log(f"cpu baseline: oracle on {rows} activation rows x {cols} weight rows of each GEMM")
    t_est = 0.0
    t_meas = 0.0
    flops_full = 0.0
    flops_sample = 0.0
    for xname, wname, name in LAYER:
        xt, wt = wl.tensors[xname], wl.tensors[wname]
        xb = xt.rows_of(range(rows))
        wb = wt.rows_of(range(cols))
        qw = orc.quantize(wb)
        t = time.perf_counter()
        qa = orc.quantize(xb)
        t_q = time.perf_counter() - t
        t = time.perf_counter()
        orc.w4a4_reference(qa, qw)
        t_g = time.perf_counter() - t
        n, k = wt.rows, wt.cols
        t_meas += t_q + t_g
        t_est += t_q * (m / rows) + t_g * (m * n) / (rows * cols)
        flops_full += 2.0 * m * n * k
        flops_sample += 2.0 * rows * cols * k
        log(f"cpu baseline: {name}: quantise {rows}x{k} {t_q:.2f} s, exact GEMM "
            f"{rows}x{cols}x{k} {t_g:.2f} s")
    log(f"cpu baseline: {t_meas:.1f} s measured, whole step estimated at {t_est:.0f} s")
    return {"value": round(flops_full / t_est / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads_used(), "kind": "oracle",
            "sample": f"first {rows} activation rows x first {cols} weight rows of each of the "
                      f"four GEMMs ({flops_sample / 1e9:.1f} GFLOP): oracle quantisation of the "
                      f"rows and its exact W4A4 reference, {t_meas:.1f} s measured; value = "
                      f"step FLOPs over the step time extrapolated linearly from the sample "
                      f"({t_est:.0f} s)"}


def counter_pass():
    """Fixed launch sequence for hardware-counter passes (rocprofv3 --pmc),
    on cuda:0 with nothing else in between:
      1. a plain device copy of 256 MiB (torch copy_), three times: the
         calibration of FETCH_SIZE / WRITE_SIZE against known bytes;
      2. the quantiser (amax, prepare, quantize) on the layer's X_gu
         16384 x 5120, three times;
      3. the gate+up W4A4 GEMM 16384 x 51200 x 5120 (BF16 out), three times;
      4. the BF16 comparison GEMM and torch.matmul of the same shape, once each;
      5. the decode-shaped W4A4 GEMM of one token against a seeded
         N(0, 0.02) 24576 x 4096 weight made on the device, three times;
      6. the quantiser and the fused RMSNorm + quantiser on a seeded N(0, 1)
         8192 x 4096 activation, three times each;
      7. the down W4A4 GEMM 16384 x 5120 x 25600 (BF16 out) three times, then
         torch.matmul of that shape once.
    """
    import torch
    from nvfp4_w4a4_gemm_amd import binding as nv
    from nvfp4_w4a4_gemm_amd.workloads import workload

    dev = torch.device("cuda:0")
    wl = workload(4)
    x = nv.to_device_bf16(wl.tensors["X_gu"].full(), dev)
    w = nv.to_device_bf16(wl.tensors["W_gu"].full(), dev)
    ws = nv.new_workspace(dev)
    qw = nv.nvfp4_quantize_weights(w, workspace=ws)
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    y = torch.empty(x.shape[0], w.shape[0], dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    print("copy 256 MiB x3", flush=True)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    print("quantize X_gu 16384x5120 x3", flush=True)
    for _ in range(3):
        qa = nv.nvfp4_quantize_act(x, workspace=ws)
    torch.cuda.synchronize()
    print("w4a4 gemm gate+up 16384x51200x5120 x3", flush=True)
    for _ in range(3):
        nv.w4a4_gemm(qa, qw, f32=False, y_bf16=y)
    torch.cuda.synchronize()
    del y
    print("bf16 comparison gemm and torch.matmul 16384x51200x5120", flush=True)
    nv.bf16_gemm_baseline(x, w, f32=False)
    torch.matmul(x, w.t())
    torch.cuda.synchronize()
    del w
    torch.cuda.empty_cache()
    print("w4a4 decode gemm 1x24576x4096 x3", flush=True)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    wgu = (torch.randn(24576, 4096, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    qgu = nv.nvfp4_quantize_weights(wgu, workspace=ws)
    del wgu
    xt = (torch.randn(1, 4096, device=dev, generator=gen)).to(torch.bfloat16)
    qt = nv.nvfp4_quantize_act(xt, workspace=ws)
    yd = torch.empty(1, 24576, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    for _ in range(3):
        nv.w4a4_gemm_decode(qt, qgu, f32=False, y_bf16=yd)
    torch.cuda.synchronize()
    del qgu
    print("quantize and rmsnorm+quantize 8192x4096 x3", flush=True)
    xa = torch.randn(8192, 4096, device=dev, generator=gen).to(torch.bfloat16)
    ga = (1.0 + 0.1 * torch.randn(4096, device=dev, generator=gen)).to(torch.bfloat16)
    torch.cuda.synchronize()
    for _ in range(3):
        nv.nvfp4_quantize_act(xa, workspace=ws)
    torch.cuda.synchronize()
    for _ in range(3):
        nv.nvfp4_rmsnorm_quantize_act(xa, ga, 1e-6, workspace=ws)
    torch.cuda.synchronize()
    del xa, ga
    print("w4a4 gemm down 16384x5120x25600 x3", flush=True)
    hd = nv.to_device_bf16(wl.tensors["H"].full(), dev)
    wd = nv.to_device_bf16(wl.tensors["W_down"].full(), dev)
    qh = nv.nvfp4_quantize_act(hd, workspace=ws)
    qwd = nv.nvfp4_quantize_weights(wd, workspace=ws)
    yd = torch.empty(hd.shape[0], wd.shape[0], dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    for _ in range(3):
        nv.w4a4_gemm(qh, qwd, f32=False, y_bf16=yd)
    torch.cuda.synchronize()
    torch.matmul(hd, wd.t())
    torch.cuda.synchronize()
    print("done", flush=True)


if __name__ == "__main__":
    main()
