"""Fixed launch sequence for hardware-counter passes (rocprofv3 --pmc).

Runs, on cuda:0, with nothing else in between:
  1. a plain device copy of 256 MiB (torch copy_), three times - the
     calibration of FETCH_SIZE / WRITE_SIZE against known bytes;
  2. the quantiser (amax, prepare, quantize) on X_qkv 8192 x 4096, three times;
  3. the stacked Q|K|V W4A4 GEMM 8192 x 6144 x 4096 (BF16 out), three times;
  4. the BF16 comparison GEMM of the same shape, three times;
  5. the decode-shaped W4A4 GEMM (w4a4_gemm_decode) of one token against the
     stacked gate|up weight 24576 x 4096 (seeded N(0, 0.02) made on the
     device), three times.
Usage: rocprofv3 --pmc FETCH_SIZE -d OUT -o NAME -- python3 nvfp4_w4a4_gemm_amd/prof_driver.py
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main():
    import torch
    from nvfp4_w4a4_gemm_amd import binding as nv
    from nvfp4_w4a4_gemm_amd.workloads import workload

    dev = torch.device("cuda:0")
    wl = workload(2)
    x = nv.to_device_bf16(wl.tensors["X_qkv"].full(), dev)
    ws = nv.new_workspace(dev)
    wb = [nv.to_device_bf16(wl.tensors[n].full(), dev) for n in ("W_q", "W_k", "W_v")]
    qkv = nv.stack_tensors([nv.nvfp4_quantize_weights(w, workspace=ws) for w in wb])
    w = torch.cat(wb, dim=0).contiguous()
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    y = torch.empty(8192, qkv.rows, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    print("copy 256 MiB x3", flush=True)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("quantize X 8192x4096 x3", flush=True)
    for _ in range(3):
        qa = nv.nvfp4_quantize_act(x, workspace=ws)
    torch.cuda.synchronize()
    print("w4a4 gemm 8192x6144x4096 (stacked Q|K|V) x3", flush=True)
    for _ in range(3):
        nv.w4a4_gemm_multi(qa, qkv, f32=False, y_bf16=y)
    torch.cuda.synchronize()
    print("bf16 gemm 8192x6144x4096 x3", flush=True)
    for _ in range(3):
        nv.bf16_gemm_baseline(x, w, f32=False)
    torch.cuda.synchronize()
    print("w4a4 decode gemm 1x24576x4096 x3", flush=True)
    del w
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
    print("done", flush=True)


if __name__ == "__main__":
    main()
