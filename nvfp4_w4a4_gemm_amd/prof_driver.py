"""Fixed launch sequence for hardware-counter passes (rocprofv3 --pmc).

Runs, on cuda:0, with nothing else in between:
  1. a plain device copy of 256 MiB (torch copy_), three times - the
     calibration of FETCH_SIZE / WRITE_SIZE against known bytes;
  2. the quantiser (amax, prepare, quantize) on X_qkv 8192 x 4096, three times;
  3. the stacked Q|K|V W4A4 GEMM 8192 x 6144 x 4096 (BF16 out), three times;
  4. the BF16 comparison GEMM of the same shape, three times.
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
    print("done", flush=True)


if __name__ == "__main__":
    main()
