"""The binding's argument checks: the library sees raw pointers only, so
shapes, dtypes, layouts and devices are checked in Python before any call.
The CPU tests reach the checks that come before the device check; the GPU
test covers the rest with device tensors."""
import pytest
import torch

from nvfp4_w4a4_gemm_amd import binding as nv


def quantized(rows, k, device="cpu"):
    return nv.NVFP4Tensor(torch.ones(1, dtype=torch.float32, device=device),
                          torch.zeros(rows, k // 16, dtype=torch.uint8, device=device),
                          torch.zeros(rows, k // 2, dtype=torch.uint8, device=device))


def test_operand_layout_is_checked_before_any_call():
    a, b = quantized(8, 64), quantized(16, 64)
    wide = torch.zeros(8, 64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="contiguous"):
        nv.w4a4_gemm(nv.NVFP4Tensor(a.alpha, a.scales, wide[:, :32]), b)
    with pytest.raises(ValueError, match="scales"):
        nv.w4a4_gemm(nv.NVFP4Tensor(a.alpha, torch.zeros(8, 3, dtype=torch.uint8), a.codes), b)
    with pytest.raises(ValueError, match="disagree on K"):
        nv.w4a4_gemm(a, quantized(16, 128))
    with pytest.raises(ValueError, match="CUDA"):
        nv.w4a4_gemm(a, b)                     # well formed, but host memory


def test_output_pair_must_share_a_row_stride():
    y32 = torch.zeros(8, 16, dtype=torch.float32)
    y16 = torch.zeros(8, 24, dtype=torch.bfloat16)[:, :16]
    with pytest.raises(ValueError, match="share one row stride"):
        nv._check_outputs(y32, y16, 8, 16, torch.device("cpu"))
    with pytest.raises(ValueError, match="y_bf16 must be"):
        nv._check_outputs(None, torch.zeros(8, 16, dtype=torch.float32), 8, 16, None)


def test_grouped_and_stacked_shapes():
    a = quantized(8, 64)
    with pytest.raises(ValueError, match="b_codes"):
        nv.w4a4_gemm_grouped(a, torch.zeros(32, 32, dtype=torch.uint8),
                             torch.zeros(32, 4, dtype=torch.uint8),
                             torch.ones(2), torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError, match="disagree on K"):
        nv.w4a4_gemm_grouped(a, torch.zeros(2, 16, 64, dtype=torch.uint8),
                             torch.zeros(2, 16, 8, dtype=torch.uint8),
                             torch.ones(2), torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError, match="NVFP4Stack"):
        nv.w4a4_gemm_multi(a, quantized(16, 64))


@pytest.mark.gpu
def test_device_arguments_are_checked():
    dev = "cuda:0"
    a, b = quantized(8, 64, dev), quantized(16, 64, dev)
    x = torch.zeros(8, 128, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="disagree on K"):
        nv.w4a4_gemm_fused_act(x, a.alpha, b)
    y32 = torch.zeros(8, 16, dtype=torch.float32, device=dev)
    y16 = torch.zeros(8, 24, dtype=torch.bfloat16, device=dev)[:, :16]
    with pytest.raises(ValueError, match="share one row stride"):
        nv.w4a4_gemm(a, b, y_f32=y32, y_bf16=y16)
    with pytest.raises(ValueError, match="y_f32 must be"):
        nv.w4a4_gemm(a, b, y_f32=torch.zeros(8, 17, device=dev), bf16=False)
    with pytest.raises(ValueError, match="CUDA tensor on"):
        nv.w4a4_gemm(a, quantized(16, 64))
    y32, y16 = nv.w4a4_gemm(a, b)              # well formed: runs
    torch.cuda.synchronize()
    assert torch.all(y32 == 0) and torch.all(y16 == 0)


def test_bf16_baseline_rejects_row_strided_activations():
    # the library's BF16 GEMM takes no row stride: a column slice of a wider
    # tensor would be read with the wrong pitch
    big = torch.zeros(8, 96, dtype=torch.bfloat16)
    w = torch.zeros(16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="row-contiguous"):
        nv.bf16_gemm_baseline(big[:, :64], w)
