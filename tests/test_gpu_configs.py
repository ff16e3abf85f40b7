"""Parity at the full sizes of the five layer configurations.

Each configuration's tensors are drawn by ``workloads`` (the same bytes the
benchmark uses) and pushed through the C ABI in the launch configuration the
benchmark times (BF16 output; the float32 output is requested in a second
launch of the same kernel).  The oracle cannot quantise or multiply the
largest tensors whole in test time, so:

* alpha of every tensor is compared exactly (the oracle takes the amax of
  the full BF16 tensor);
* codes and scale bytes are compared bit-exactly on every element of every
  activation and weight tensor (the oracle runs in row slices in parallel
  worker processes);
* GEMM outputs are compared on 2048 rows (the first and last, the row of
  the activation's largest magnitude and seeded random rows) by every
  column, against the exact oracle GEMM of those rows.

The grouped (MoE) configuration gathers the quantised token rows by the
seeded routing and checks rows of several experts, and the dense stack of
configuration 4 checks that the quantise-on-load GEMM is bit-identical to
quantise-then-GEMM at full size.
"""
import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as orc
from nvfp4_w4a4_gemm_amd import binding as nv
from nvfp4_w4a4_gemm_amd.workloads import workload

from test_gpu_parity import assert_gemm_close, host_bits
from oracle_pool import new_pool, quantize_all_rows, quantize_many

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ROWS = 192          # sampled rows per tensor (beyond first / last / amax row)
GEMM_ROWS = 2048    # output rows per GEMM (all columns)


@pytest.fixture(scope="module")
def pool():
    with new_pool() as p:
        yield p


def sample(n, count, seed, must=()):
    rng = np.random.default_rng(seed)
    if n <= count + len(must):
        return np.arange(n)
    picks = set(int(i) for i in must) | {0, n - 1}
    picks |= set(int(i) for i in rng.choice(n, count, replace=False))
    return np.array(sorted(picks))


def oracle_alpha(bits):
    amax = np.array([int((bits & np.uint16(0x7FFF)).max())], dtype=np.uint16)
    return orc.tensor_scale(orc.bf16_to_f64(amax))


def amax_row(bits):
    return int(np.argmax((bits & np.uint16(0x7FFF)).max(axis=1)))


class Quantized:
    """A tensor quantised on the GPU, with the oracle's view of sampled rows."""

    def __init__(self, name, bits, weights, seed):
        self.name = name
        self.bits = bits
        self.alpha = oracle_alpha(bits)
        x = nv.to_device_bf16(bits, DEV)
        self.q = nv.nvfp4_quantize_weights(x) if weights else nv.nvfp4_quantize_act(x)
        self.dev = x
        torch.cuda.synchronize()
        self.rows = sample(bits.shape[0], ROWS, seed, must=(amax_row(bits),))

    def check(self, pool):
        """alpha exact; every scale byte and code byte equal to the oracle's."""
        assert self.q.alpha.item() == float(self.alpha), (self.name, self.q.alpha.item(), self.alpha)
        ref_s, ref_c = quantize_all_rows(pool, self.bits, self.alpha)
        self.ref = (self.alpha, ref_s, ref_c)
        s = self.q.scales.cpu().numpy()
        c = self.q.codes.cpu().numpy()
        assert s.shape == ref_s.shape and c.shape == ref_c.shape, self.name
        bad = np.argwhere(s != ref_s)
        assert bad.size == 0, f"{self.name}: scale bytes differ at {bad[:4].tolist()}"
        bad = np.argwhere(c != ref_c)
        assert bad.size == 0, f"{self.name}: code bytes differ at {bad[:4].tolist()}"

    def oracle_rows(self, rows=None):
        """The oracle's quantisation of some rows (all rows by default)."""
        if rows is None:
            return self.ref
        return (self.alpha, self.ref[1][rows], self.ref[2][rows])


def check_gemm(name, a, w, seed, a_rows_of_output=None, out_rows=None):
    """Full-size W4A4 GEMM on the GPU vs the oracle on a sampled grid."""
    m = a.bits.shape[0] if a_rows_of_output is None else len(a_rows_of_output)
    n = w.bits.shape[0]
    y16 = torch.empty(m, n, dtype=torch.bfloat16, device=DEV)
    nv.w4a4_gemm(a.q, w.q, f32=False, y_bf16=y16)
    y32, _ = nv.w4a4_gemm(a.q, w.q, bf16=False)
    torch.cuda.synchronize()
    rows = out_rows if out_rows is not None else sample(m, GEMM_ROWS, seed,
                                                          must=(amax_row(a.bits),))
    src = rows if a_rows_of_output is None else a_rows_of_output[rows]
    y, bound, y16_ref = orc.w4a4_reference(a.oracle_rows(src), w.oracle_rows())
    r_t = torch.from_numpy(rows).to(DEV)
    assert_gemm_close(y32.index_select(0, r_t), y16.index_select(0, r_t), y, bound, y16_ref)
    print(f"[{name}] {m}x{n}x{a.bits.shape[1]}: {len(rows)} rows x all {n} columns match")
    return y16


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_dense_config(cfg, pool):
    wl = workload(cfg)
    print(f"\n[cfg {cfg}] {wl.title}: generating", flush=True)
    acts, wts, keep = {}, {}, {}
    for i, g in enumerate(wl.gemms):
        if g.act not in acts:
            acts[g.act] = Quantized(g.act, wl.tensors[g.act].full(), False, 100 * cfg + i)
            acts[g.act].check(pool)
            print(f"[cfg {cfg}] {g.act} {acts[g.act].bits.shape}: alpha and every "
                  f"code/scale byte bit-exact", flush=True)
        wts[g.weight] = Quantized(g.weight, wl.tensors[g.weight].full(), True, 200 * cfg + i)
        wts[g.weight].check(pool)
        y16 = check_gemm(f"cfg {cfg} {g.name}", acts[g.act], wts[g.weight], 300 * cfg + i)
        if cfg == 4:
            # quantise-on-load: bit-identical to quantise-then-GEMM at full size
            _, f16 = nv.w4a4_gemm_fused_act(acts[g.act].dev, acts[g.act].q.alpha,
                                            wts[g.weight].q, f32=False)
            torch.cuda.synchronize()
            assert torch.equal(f16.view(torch.int16), y16.view(torch.int16)), g.name
            print(f"[cfg 4 {g.name}] fused quantise-on-load GEMM bit-identical", flush=True)
        if cfg == 2 and g.name != "o_proj":
            keep[g.weight] = (wts[g.weight].q, y16)
        del wts[g.weight]
        torch.cuda.empty_cache()
    if cfg == 2:
        # Q, K and V as one launch over the stacked weights: bit-identical
        stack = nv.stack_tensors([keep[w][0] for w in ("W_q", "W_k", "W_v")])
        _, y16 = nv.w4a4_gemm_multi(acts["X_qkv"].q, stack, f32=False)
        torch.cuda.synchronize()
        for w, lo, hi in zip(("W_q", "W_k", "W_v"), stack.offsets[:-1], stack.offsets[1:]):
            assert torch.equal(y16[:, lo:hi].contiguous().view(torch.int16),
                               keep[w][1].view(torch.int16)), w
        print("[cfg 2] Q|K|V stacked GEMM bit-identical to the three GEMMs", flush=True)


def test_grouped_moe_config(pool):
    wl = workload(5)
    e_count, topk = wl.experts, wl.topk
    token_of_row, offsets = wl.routing()
    print(f"\n[cfg 5] {wl.title}: generating", flush=True)
    x = Quantized("X", wl.tensors["X"].full(), False, 501)
    x.check(pool)
    h = Quantized("H", wl.tensors["H"].full(), False, 502)
    h.check(pool)
    w_gu = [wl.tensors[f"W_gu[{e}]"].full() for e in range(e_count)]
    w_dn = [wl.tensors[f"W_down[{e}]"].full() for e in range(e_count)]
    off_t = torch.from_numpy(offsets).to(DEV)
    tok_t = torch.from_numpy(token_of_row).to(DEV)
    rng = np.random.default_rng(503)
    experts = sorted(set(int(e) for e in rng.choice(e_count, 2, replace=False)) | {0, e_count - 1})

    for name, act, wbits, gather in (("gate_up", x, w_gu, tok_t), ("down", h, w_dn, None)):
        qws = [nv.nvfp4_quantize_weights(nv.to_device_bf16(b, DEV)) for b in wbits]
        b_codes = torch.stack([q.codes for q in qws])
        b_scales = torch.stack([q.scales for q in qws])
        b_alpha = torch.cat([q.alpha for q in qws])
        del qws
        # every expert's weight: alpha exact, every code and scale byte
        alphas = [oracle_alpha(b) for b in wbits]
        assert np.array_equal(b_alpha.cpu().numpy(), np.array(alphas, dtype=np.float32)), name
        refs = quantize_many(pool, list(zip(wbits, alphas)))
        got_s, got_c = b_scales.cpu().numpy(), b_codes.cpu().numpy()
        for e, (rs, rc) in enumerate(refs):
            assert rs.shape == got_s[e].shape and rc.shape == got_c[e].shape, (name, e)
            assert np.array_equal(got_s[e], rs) and np.array_equal(got_c[e], rc), (name, e)
        print(f"[cfg 5 {name}] all {e_count} expert weights: alpha and every code/scale byte "
              f"bit-exact", flush=True)
        m = int(offsets[-1])
        n = wbits[0].shape[0]
        y16 = torch.empty(m, n, dtype=torch.bfloat16, device=DEV)
        nv.w4a4_gemm_grouped(act.q, b_codes, b_scales, b_alpha, off_t, a_row_index=gather,
                             f32=False, y_bf16=y16)
        y32, _ = nv.w4a4_gemm_grouped(act.q, b_codes, b_scales, b_alpha, off_t,
                                      a_row_index=gather, bf16=False)
        torch.cuda.synchronize()
        checked = 0
        for e in experts:
            # every row the expert received, by every column
            lo, hi = int(offsets[e]), int(offsets[e + 1])
            rows = np.arange(lo, hi)
            src = token_of_row[rows] if gather is not None else rows
            y, bound, y16_ref = orc.w4a4_reference(act.oracle_rows(src),
                                                   (alphas[e],) + refs[e])
            r_t = torch.from_numpy(rows).to(DEV)
            assert_gemm_close(y32.index_select(0, r_t), y16.index_select(0, r_t), y, bound,
                              y16_ref)
            checked += len(rows)
        print(f"[cfg 5 {name}] {m}x{n}x{wbits[0].shape[1]} grouped over {e_count} experts: "
              f"all {checked} rows of experts {experts} by all {n} columns match", flush=True)
        del b_codes, b_scales, y16, y32
        torch.cuda.empty_cache()
