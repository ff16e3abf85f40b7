"""The allocation-free quantiser entry point, nvfp4_quantize_act_noalloc,
against nvfp4_quantize_act with a caller workspace (and the oracle on the
smaller tensor).  Two calls in a row share the library's per-device scratch:
the second is smaller, has a smaller amax (so a stale partial maximum of the
first call would raise its alpha) and fewer amax workgroups.  Codes, scale
bytes and alpha must be identical, bit for bit.
"""
import numpy as np
import pytest
import torch

from nvfp4_w4a4_gemm_amd import binding as nv
from oracle import nvfp4_oracle as orc

pytestmark = pytest.mark.gpu


def bf16_bits(m, k, seed, outlier_scale):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k), dtype=np.float32)
    cols = rng.choice(k, size=max(1, round(0.005 * k)), replace=False)
    x[:, cols] *= outlier_scale
    u = x.view(np.uint32)
    # float32 -> BF16 bits, round to nearest even (finite inputs)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def same(a: nv.NVFP4Tensor, b: nv.NVFP4Tensor):
    assert torch.equal(a.alpha, b.alpha)
    assert torch.equal(a.scales, b.scales)
    assert torch.equal(a.codes, b.codes)


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    dev = torch.device("cuda:0")
    ws = nv.new_workspace(dev)
    big = nv.to_device_bf16(bf16_bits(2048, 8192, 11, 50.0), dev)      # 1024 amax workgroups
    small_bits = bf16_bits(192, 1040, 12, 1.0)                         # ragged K, smaller amax
    small = nv.to_device_bf16(small_bits, dev)

    print("noalloc: call 1, 2048 x 8192", flush=True)
    got1 = nv.nvfp4_quantize_act_noalloc(big)
    print("noalloc: call 2, 192 x 1040", flush=True)
    got2 = nv.nvfp4_quantize_act_noalloc(small)
    want1 = nv.nvfp4_quantize_act(big, workspace=ws)
    want2 = nv.nvfp4_quantize_act(small, workspace=ws)
    torch.cuda.synchronize()
    same(got1, want1)
    same(got2, want2)
    assert got2.alpha.item() < got1.alpha.item()

    alpha, scales, codes = orc.quantize(small_bits)
    assert got2.alpha.item() == float(alpha)
    assert np.array_equal(got2.scales.cpu().numpy(), scales)
    assert np.array_equal(got2.codes.cpu().numpy(), codes)


def test_noalloc_with_given_alpha_and_empty_input():
    dev = torch.device("cuda:0")
    ws = nv.new_workspace(dev)
    x = nv.to_device_bf16(bf16_bits(300, 4096, 13, 50.0), dev)
    alpha = torch.tensor([0.0123], dtype=torch.float32, device=dev)
    print("noalloc: given alpha, 300 x 4096", flush=True)
    got = nv.nvfp4_quantize_act_noalloc(x, alpha_in=alpha)
    want = nv.nvfp4_quantize_act(x, alpha_in=alpha, workspace=ws)
    print("noalloc: M = 0", flush=True)
    empty = nv.nvfp4_quantize_act_noalloc(x[:0])
    torch.cuda.synchronize()
    same(got, want)
    assert got.alpha.item() == alpha.item()
    assert empty.alpha.item() == 0.0
