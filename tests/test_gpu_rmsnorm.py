"""RMSNorm with the quantiser fused in (nvfp4_rmsnorm_quantize_act) against
the oracle.

The kernel's normalised values y are compared with the oracle's RMSNorm
(reading R16, exact up to float64 roundings, one BF16 rounding): equal or
adjacent BF16 values (the kernel's float32 sum and reciprocal square root
can put a value on the other side of a BF16 midpoint).  The quantisation of
those y is then compared bit for bit: alpha, scale bytes and codes equal the
oracle's quantisation of the kernel's own y.
"""
import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as orc
from nvfp4_w4a4_gemm_amd import binding as nv
from nvfp4_w4a4_gemm_amd.workloads import workload

from test_gpu_parity import bf16_ordered, dev_bf16, host_bits, normal_bits
from oracle_pool import new_pool, quantize_all_rows, rmsnorm_all_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def gamma_bits(k, seed):
    g = (1.0 + 0.1 * np.random.default_rng(seed).standard_normal(k)).astype(np.float32)
    return orc.f64_to_bf16_bits(g)


def check(xb, gb, eps, alpha_in=None, pool=None):
    m, k = xb.shape
    x = dev_bf16(xb)
    g = torch.from_numpy(gb.view(np.int16)).to(DEV).view(torch.bfloat16)
    y = torch.empty(m, k, dtype=torch.bfloat16, device=DEV)
    a_in = None if alpha_in is None else torch.tensor([alpha_in], dtype=torch.float32, device=DEV)
    q = nv.nvfp4_rmsnorm_quantize_act(x, g, eps, alpha_in=a_in, y_out=y)
    q2 = nv.nvfp4_rmsnorm_quantize_act(x, g, eps, alpha_in=a_in)     # without y
    # the quantiser's workspace alone: the quantise pass sums each row again
    # instead of reading the r the amax pass stored; the same bits
    y3 = torch.empty_like(y)
    q3 = nv.nvfp4_rmsnorm_quantize_act(x, g, eps, alpha_in=a_in, y_out=y3,
                                       workspace=nv.new_workspace(DEV))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y3.view(torch.int16))
    assert torch.equal(q.codes, q3.codes) and torch.equal(q.scales, q3.scales)
    assert torch.equal(q.alpha, q3.alpha)
    yk = host_bits(y)
    yref = orc.rmsnorm(xb, gb, eps)[1] if pool is None else rmsnorm_all_rows(pool, xb, gb, eps)
    assert yref.shape == yk.shape
    d = np.abs(bf16_ordered(yk) - bf16_ordered(yref))
    assert d.max() <= 1, f"normalised values differ by {d.max()} BF16 ulp"
    # quantisation of the kernel's own y: bit-exact (alpha from the whole y)
    alpha = np.float32(alpha_in) if alpha_in is not None else orc.tensor_scale(orc.bf16_to_f64(yk))
    assert q.alpha.item() == float(alpha)
    ref = (alpha,) + (orc.quantize(yk, alpha=alpha)[1:] if pool is None
                      else quantize_all_rows(pool, yk, alpha))
    s = q.scales.cpu().numpy()
    c = q.codes.cpu().numpy()
    assert s.shape == ref[1].shape and c.shape == ref[2].shape
    assert np.array_equal(s, ref[1]), np.argwhere(s != ref[1])[:4]
    assert np.array_equal(c, ref[2]), np.argwhere(c != ref[2])[:4]
    assert torch.equal(q.codes, q2.codes) and torch.equal(q.scales, q2.scales)
    assert torch.equal(q.alpha, q2.alpha)
    return int((d == 1).sum())


@pytest.mark.parametrize("m,k", [(64, 4096), (37, 2816), (5, 16), (300, 5120), (1, 8192),
                                 (200, 1040), (130, 48), (9, 6144)])
def test_rmsnorm_quantize_matches_oracle(m, k):
    xb = normal_bits(m, k, seed=m * 7 + k)
    off = check(xb, gamma_bits(k, k), 1e-6)
    print(f"[{m}x{k}] {off} of {m * k} normalised values one BF16 ulp from the oracle")


def test_rmsnorm_quantize_zero_rows_tiny_eps_and_given_alpha():
    m, k = 48, 1024
    xb = normal_bits(m, k, seed=5)
    xb[3] = 0                      # a zero row: y = 0 (eps > 0)
    xb[7] = 0x8000                 # -0.0 everywhere: y = -0.0, code 0x8
    check(xb, gamma_bits(k, 6), 1e-5)
    check(xb, gamma_bits(k, 6), 0.25)                  # eps that matters
    check(xb, gamma_bits(k, 6), 1e-5, alpha_in=2.0 ** -9)


@pytest.mark.parametrize("m,k", [(37, 2816), (9, 6144), (5, 16), (64, 5120)])
@pytest.mark.parametrize("alpha_in", [2.0 ** -120, 2.0 ** 110])
def test_rmsnorm_quantize_extreme_given_alpha(m, k, alpha_in):
    """alpha's exponent beyond +-100 (the rescaling block path) for rows held
    in registers (K <= 5120) and streamed (K = 6144)."""
    xb = normal_bits(m, k, seed=m + k)
    check(xb, gamma_bits(k, 3), 1e-6, alpha_in=alpha_in)


@pytest.mark.parametrize("k", [4096, 2816])
def test_rmsnorm_quantize_zero_row_without_eps(k):
    """eps = 0 and a row of zeros: r = 1/sqrt(0) is infinite and that row's y
    is 0 * inf = NaN by the definition, so alpha is NaN (the amax pass takes
    such rows through BF16 bit patterns, in which NaN is the largest); the
    other rows' y are unaffected."""
    m = 12
    xb = normal_bits(m, k, seed=k)
    xb[5] = 0
    g = torch.from_numpy(gamma_bits(k, 2).view(np.int16)).to(DEV).view(torch.bfloat16)
    y = torch.empty(m, k, dtype=torch.bfloat16, device=DEV)
    q = nv.nvfp4_rmsnorm_quantize_act(dev_bf16(xb), g, 0.0, y_out=y)
    torch.cuda.synchronize()
    assert torch.isnan(q.alpha).all()
    assert torch.isnan(y[5].float()).all()
    yk = host_bits(y)
    yref = orc.rmsnorm(np.delete(xb, 5, axis=0), gamma_bits(k, 2), 0.0)[1]
    d = np.abs(bf16_ordered(np.delete(yk, 5, axis=0)) - bf16_ordered(yref))
    assert d.max() <= 1


@pytest.mark.parametrize("m,k", [(37, 2816), (70, 5120), (9, 4096)])
def test_rmsnorm_quantize_strided_rows(m, k):
    """x and y with row strides beyond K (views into wider rows): the same
    codes, scales and y as the dense call, with and without the stored r."""
    xb = normal_bits(m, k, seed=11 * m + k)
    g = torch.from_numpy(gamma_bits(k, 4).view(np.int16)).to(DEV).view(torch.bfloat16)
    x = dev_bf16(xb)
    wide = torch.full((m, k + 72), 3.0, dtype=torch.bfloat16, device=DEV)
    wide[:, :k] = x
    y = torch.empty(m, k, dtype=torch.bfloat16, device=DEV)
    q = nv.nvfp4_rmsnorm_quantize_act(x, g, 1e-6, y_out=y)
    for ws in (None, nv.new_workspace(DEV)):
        yw = torch.full((m, k + 24), 5.0, dtype=torch.bfloat16, device=DEV)
        qs = nv.nvfp4_rmsnorm_quantize_act(wide[:, :k], g, 1e-6, y_out=yw[:, :k], workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(qs.codes, q.codes) and torch.equal(qs.scales, q.scales)
        assert torch.equal(qs.alpha, q.alpha)
        assert torch.equal(yw[:, :k].view(torch.int16), y.view(torch.int16))
        assert torch.all(yw[:, k:] == 5.0)


def test_rmsnorm_quantize_full_size():
    """The layer's X_qkv (8192 x 4096, outlier channels) at full size: every
    normalised value within one BF16 ulp of the oracle, alpha and every code
    and scale byte exact (the oracle runs in row slices in worker processes)."""
    xb = workload(2).tensors["X_qkv"].full()
    with new_pool() as pool:
        off = check(xb, gamma_bits(xb.shape[1], 10), 1e-6, pool=pool)
    print(f"[8192x4096] {off} of {xb.size} normalised values one BF16 ulp from the oracle")
