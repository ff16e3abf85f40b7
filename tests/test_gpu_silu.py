"""The gate|up W4A4 GEMM with SiLU(gate) * up and the next quantiser fused in
(w4a4_gemm_silu_mul_quantize) against the oracle.

Two checks of H, one of which assumes nothing about the fused kernel's
internals:
  - end to end: H against SiLU(g) u of the exact oracle gate and up, within
    the GEMM tolerance carried through SiLU (|d SiLU/dg| <= 1.1 everywhere)
    plus one BF16 ulp for H's own rounding;
  - tighter: the fused kernel shares the GEMM's main loop with
    w4a4_gemm_multi, so H is within one BF16 ulp of the oracle's gated
    activation (reading R17, float64, one BF16 rounding) of the float32 gate
    and up that w4a4_gemm_multi writes for the same interleaved weight.
The quantisation of H is compared bit for bit: alpha (from the kernel's
per-tile maxima), scale bytes and codes equal the oracle's quantisation of
the kernel's own H.
"""
import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as orc
from nvfp4_w4a4_gemm_amd import binding as nv

from test_gpu_parity import (assert_gemm_close, assert_quant_equal, bf16_ordered, dev_bf16,
                             host_bits, normal_bits)
from oracle_pool import new_pool, quantize_all_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


SILU_SLOPE = 1.1   # max over g of |d SiLU(g) / dg| (about 1.0998, near g = 2.40)


def assert_h_near_exact(hb, g_ref, u_ref, tol_g, tol_u):
    """H (BF16 bits) against SiLU(g) u of the exact gate and up values, where
    the kernel's own g and u may differ from them by up to tol_g and tol_u
    (the GEMM tolerance): |dH| <= (|u| + tol_u) 1.1 tol_g + (|SiLU(g)| +
    1.1 tol_g) tol_u, plus one BF16 ulp of H (its rounding and the float32
    arithmetic of SiLU, about 2^-17 relative)."""
    g = np.asarray(g_ref, dtype=np.float64)
    u = np.asarray(u_ref, dtype=np.float64)
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    exact = silu * u
    h = orc.bf16_to_f64(hb)
    bound = ((np.abs(u) + tol_u) * SILU_SLOPE * tol_g + (np.abs(silu) + SILU_SLOPE * tol_g) * tol_u
             + 2.0 ** -7 * np.maximum(np.abs(h), np.abs(exact)) + 1e-30)
    err = np.abs(h - exact)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{bad.shape[0]} H values outside the propagated bound, e.g. " \
        f"{bad[0].tolist()}: {h[tuple(bad[0])]} vs {exact[tuple(bad[0])]}"


def gate_up_columns(hidden):
    """Columns of the interleaved output that hold gate and up of each unit."""
    u = np.arange(hidden)
    gate = (u // 32) * 64 + u % 32
    return gate, gate + 32


def run_case(m, hidden, k, seed, gate_std=0.02, up_std=0.02, check_gemm=False):
    xb = normal_bits(m, k, seed=seed)
    gb = normal_bits(hidden, k, seed=seed + 1, std=gate_std, outliers=False)
    ub = normal_bits(hidden, k, seed=seed + 2, std=up_std, outliers=False)
    qa = nv.nvfp4_quantize_act(dev_bf16(xb))
    qg = nv.nvfp4_quantize_weights(dev_bf16(gb))
    qu = nv.nvfp4_quantize_weights(dev_bf16(ub))
    stack = nv.interleave_gate_up(qg, qu)
    qh, h = nv.w4a4_gemm_silu_mul_quantize(qa, stack)
    y32, _ = nv.w4a4_gemm_multi(qa, stack, bf16=False)
    torch.cuda.synchronize()
    gcol, ucol = gate_up_columns(hidden)
    y = y32.cpu().numpy()
    g, u = y[:, gcol], y[:, ucol]
    hb = host_bits(h)
    if check_gemm:
        ra = orc.quantize(xb)
        exact = []
        for w, part in ((gb, g), (ub, u)):
            ref, bound, ref16 = orc.w4a4_reference(ra, orc.quantize(w))
            assert_gemm_close(torch.from_numpy(part), None, ref, bound, ref16)
            exact.append((ref, 1e-4 * bound + 1e-6))
        (g_ref, tol_g), (u_ref, tol_u) = exact
        assert_h_near_exact(hb, g_ref, u_ref, tol_g, tol_u)
    _, h_ref = orc.silu_mul(g, u)
    diff = np.abs(bf16_ordered(hb) - bf16_ordered(h_ref))
    assert diff.max(initial=0) <= 1, f"H off by {diff.max()} BF16 ulps at " \
        f"{np.unravel_index(diff.argmax(), diff.shape)}"
    assert (diff == 0).mean() > 0.99
    assert_quant_equal(qh, orc.quantize(hb))
    return g, hb


@pytest.mark.parametrize("m,hidden,k", [(256, 1024, 1024), (300, 320, 512), (37, 96, 48),
                                        (1, 32, 16), (129, 160, 1408)])
def test_silu_mul_quantize_matches_oracle(m, hidden, k):
    run_case(m, hidden, k, seed=m + hidden + k, check_gemm=(m * hidden * k <= 300 * 320 * 512))


def test_silu_mul_large_tile_path():
    # 256 x 256 tiles (>= 256 workgroups): H is checked on every row
    run_case(2048, 4096, 256, seed=5)


def test_silu_mul_saturating_gate():
    """Gate values far into both tails of SiLU (exp(-g) overflows float32
    for g < -88.7) and up values of both signs."""
    g, hb = run_case(200, 256, 512, seed=9, gate_std=2.0, up_std=0.5, check_gemm=True)
    assert g.min() < -90 and g.max() > 90
    h = orc.bf16_to_f64(hb)
    assert np.all(h[g < -120] == 0)


def test_silu_mul_h_row_pitch():
    m, hidden, k = 70, 96, 256
    xb = normal_bits(m, k, seed=13)
    qa = nv.nvfp4_quantize_act(dev_bf16(xb))
    qg = nv.nvfp4_quantize_weights(dev_bf16(normal_bits(hidden, k, seed=14, std=0.05)))
    qu = nv.nvfp4_quantize_weights(dev_bf16(normal_bits(hidden, k, seed=15, std=0.05)))
    stack = nv.interleave_gate_up(qg, qu)
    q1, h1 = nv.w4a4_gemm_silu_mul_quantize(qa, stack)
    wide = torch.full((m, hidden + 40), -7.0, dtype=torch.bfloat16, device=DEV)
    q2, h2 = nv.w4a4_gemm_silu_mul_quantize(qa, stack, h=wide[:, :hidden])
    torch.cuda.synchronize()
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))
    assert torch.all(wide[:, hidden:] == -7.0)
    assert torch.equal(q1.codes, q2.codes) and torch.equal(q1.scales, q2.scales)
    assert q1.alpha.item() == q2.alpha.item()


def test_silu_mul_empty_rows():
    k, hidden = 256, 64
    qg = nv.nvfp4_quantize_weights(dev_bf16(normal_bits(hidden, k, seed=3)))
    stack = nv.interleave_gate_up(qg, qg)
    qa = nv.NVFP4Tensor(torch.zeros(1, dtype=torch.float32, device=DEV),
                        torch.empty(0, k // 16, dtype=torch.uint8, device=DEV),
                        torch.empty(0, k // 2, dtype=torch.uint8, device=DEV))
    qh, h = nv.w4a4_gemm_silu_mul_quantize(qa, stack)
    torch.cuda.synchronize()
    assert h.shape == (0, hidden) and qh.alpha.item() == 0.0


def test_silu_mul_persistent_equals_grid():
    """4096 tokens, hidden 4096: 512 tiles of 256 x 256, so the persistent
    tile walk runs; H, alpha, codes and scales equal the one-workgroup-per-
    tile launch bit for bit."""
    m, hidden, k = 4096, 4096, 512
    qa = nv.nvfp4_quantize_act(dev_bf16(normal_bits(m, k, seed=41)))
    qg = nv.nvfp4_quantize_weights(dev_bf16(normal_bits(hidden, k, seed=42, std=0.05)))
    qu = nv.nvfp4_quantize_weights(dev_bf16(normal_bits(hidden, k, seed=43, std=0.05)))
    stack = nv.interleave_gate_up(qg, qu)
    res = []
    for on in (True, False):
        with nv.path_flags(0 if on else nv.PATH_GEMM_GRID):
            q, h = nv.w4a4_gemm_silu_mul_quantize(qa, stack)
            torch.cuda.synchronize()
        res.append((q, h))
    (q1, h1), (q2, h2) = res
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))
    assert q1.alpha.item() == q2.alpha.item()
    assert torch.equal(q1.codes, q2.codes) and torch.equal(q1.scales, q2.scales)
    rows = np.array([0, 255, 256, 2049, m - 1])
    y32, _ = nv.w4a4_gemm_multi(qa, stack, bf16=False)
    torch.cuda.synchronize()
    gcol, ucol = gate_up_columns(hidden)
    y = y32.cpu().numpy()[rows]
    _, h_ref = orc.silu_mul(y[:, gcol], y[:, ucol])
    d = np.abs(bf16_ordered(host_bits(h1)[rows]) - bf16_ordered(h_ref))
    assert d.max() <= 1


def test_silu_mul_full_size_mlp_config():
    """The gate|up projection of the Qwen3-8B-shaped MLP configuration at
    full size (X 32768x4096 with outlier channels, gate and up 12288x4096 ~
    N(0, 0.02)), in the launch configuration the benchmark times: alpha of H
    exact against the oracle's amax of the kernel's whole H, every code and
    scale byte of H equal to the oracle's quantisation of the kernel's H, and
    sampled rows of H within one BF16 ulp of the oracle's SiLU*up of the
    kernel's float32 gate/up."""
    from nvfp4_w4a4_gemm_amd.workloads import workload
    from test_gpu_configs import oracle_alpha, sample
    wl = workload(3)
    x = nv.to_device_bf16(wl.tensors["X"].full(), DEV)
    qa = nv.nvfp4_quantize_act(x)
    qg = nv.nvfp4_quantize_weights(nv.to_device_bf16(wl.tensors["W_gate"].full(), DEV))
    qu = nv.nvfp4_quantize_weights(nv.to_device_bf16(wl.tensors["W_up"].full(), DEV))
    del x
    stack = nv.interleave_gate_up(qg, qu)
    del qg, qu
    qh, h = nv.w4a4_gemm_silu_mul_quantize(qa, stack)
    torch.cuda.synchronize()
    m, hidden = h.shape
    hb_all = host_bits(h)
    alpha = oracle_alpha(hb_all)
    assert qh.alpha.item() == float(alpha)
    rows = sample(m, 64, 777, must=(int(np.argmax((hb_all & np.uint16(0x7FFF)).max(axis=1))),))
    y32, _ = nv.w4a4_gemm_multi(qa, stack, bf16=False)
    torch.cuda.synchronize()
    y = y32.index_select(0, torch.from_numpy(rows).to(DEV)).cpu().numpy()
    del y32
    torch.cuda.empty_cache()
    gcol, ucol = gate_up_columns(hidden)
    _, h_ref = orc.silu_mul(y[:, gcol], y[:, ucol])
    hb = hb_all[rows]
    d = np.abs(bf16_ordered(hb) - bf16_ordered(h_ref))
    assert d.max() <= 1
    with new_pool() as pool:
        # end to end on 16 of the sampled rows: the exact oracle gate and up
        ra = orc.quantize(wl.tensors["X"].rows_of(rows[:16]),
                          alpha=oracle_alpha(wl.tensors["X"].full()))
        exact = []
        for name in ("W_gate", "W_up"):
            wb = wl.tensors[name].full()
            aw = oracle_alpha(wb)
            ws, wc = quantize_all_rows(pool, wb, aw)
            ref, bound, _ = orc.w4a4_reference(ra, (aw, ws, wc))
            exact.append((ref, 1e-4 * bound + 1e-6))
        (g_ref, tol_g), (u_ref, tol_u) = exact
        assert_h_near_exact(hb[:16], g_ref, u_ref, tol_g, tol_u)
        ref_s, ref_c = quantize_all_rows(pool, hb_all, alpha)
    got_s, got_c = qh.scales.cpu().numpy(), qh.codes.cpu().numpy()
    assert got_s.shape == ref_s.shape and got_c.shape == ref_c.shape
    assert np.array_equal(got_s, ref_s) and np.array_equal(got_c, ref_c)
    print(f"[mlp gate|up] {m}x{2 * hidden}x{qa.k}: alpha of H exact, every code and scale "
          f"byte of H bit-exact, {len(rows)} rows of H within one ulp "
          f"({int((d > 0).sum())} off by one)")
