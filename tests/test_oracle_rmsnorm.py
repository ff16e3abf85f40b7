"""Pins of the oracle's RMSNorm (reading R16), which produces the input that
the fused RMSNorm -> NVFP4 quantiser quantises.

* hand-worked rows (tests/golden/rmsnorm_rows.json);
* torch's own RMSNorm (torch.nn.functional.rms_norm) in float64;
* invariants of the definition: power-of-two scaling of a row (eps = 0)
  leaves y unchanged, doubling gamma doubles y, a row permutation permutes
  y when gamma is permuted with it;
* planted mistakes in a copy of the function must fail one of them.
"""
import contextlib
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rmsnorm_rows.json")


def _bits(vals):
    return orc.f64_to_bf16_bits(np.array([float(Fraction(v)) for v in vals]))


def check_golden():
    for case in json.load(open(GOLDEN))["cases"]:
        x = np.zeros(16, np.uint16)
        x[:len(case["x"])] = _bits(case["x"])
        g = np.full(16, 0x3F80, np.uint16)
        g[:len(case["gamma"])] = _bits(case["gamma"])
        _, yb = orc.rmsnorm(x[None, :], g, float(Fraction(case["eps"])))
        want = [int(b, 16) for b in case["y_bits"]]
        assert [int(v) for v in yb[0, :len(want)]] == want, (case["id"], yb[0, :len(want)])


def _random_rows(rows, k, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k)).astype(np.float32)
    x[:, rng.choice(k, max(1, k // 200), replace=False)] *= 50.0
    g = (1.0 + 0.1 * rng.standard_normal(k)).astype(np.float32)
    return orc.f64_to_bf16_bits(x), orc.f64_to_bf16_bits(g)


def check_torch():
    xb, gb = _random_rows(24, 4096, 11)
    for eps in (1e-6, 0.5):
        y, _ = orc.rmsnorm(xb, gb, eps)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(orc.bf16_to_f64(xb)), (4096,),
                                           torch.from_numpy(orc.bf16_to_f64(gb)), eps).numpy()
        assert np.allclose(y, ref, rtol=1e-12, atol=0), (eps, np.abs(y - ref).max())


def check_invariants():
    xb, gb = _random_rows(8, 512, 12)
    _, y0 = orc.rmsnorm(xb, gb, 0.0)
    x = orc.bf16_to_f64(xb)
    for k in (-7, 3):
        _, yk = orc.rmsnorm(orc.f64_to_bf16_bits(np.ldexp(x, k)), gb, 0.0)
        assert np.array_equal(yk, y0), k
    y, _ = orc.rmsnorm(xb, gb, 1e-5)
    y2, _ = orc.rmsnorm(xb, orc.f64_to_bf16_bits(2.0 * orc.bf16_to_f64(gb)), 1e-5)
    assert np.array_equal(y2, 2.0 * y)
    perm = np.random.default_rng(13).permutation(512)
    yp, _ = orc.rmsnorm(xb[:, perm], gb[perm], 1e-5)
    assert np.allclose(yp, y[:, perm], rtol=1e-14, atol=0)


def pins_pass():
    for c in (check_golden, check_torch, check_invariants):
        try:
            c()
        except AssertionError:
            return False
    return True


def test_golden_rows():
    check_golden()


def test_matches_torch_rms_norm_float64():
    check_torch()


def test_invariants():
    check_invariants()


def _variant(sum_fn=None, k_off=0, eps_on=True, gamma_on=True, root=True):
    def f(x_bits, gamma_bits, eps):
        x = orc.bf16_to_f64(x_bits)
        g = orc.bf16_to_f64(gamma_bits) if gamma_on else np.ones(x.shape[1])
        ss = (sum_fn or (lambda r: np.sum(r * r)))
        s = np.array([ss(row) for row in x])
        d = s / (x.shape[1] + k_off) + (eps if eps_on else 0.0)
        inv = 1.0 / (np.sqrt(d) if root else d)
        y = x * inv[:, None] * g[None, :]
        return y, orc.f64_to_bf16_bits(y)
    return f


MUTANTS = {
    "eps_dropped": _variant(eps_on=False),
    "mean_over_k_minus_1": _variant(k_off=-1),
    "gamma_dropped": _variant(gamma_on=False),
    "no_square_root": _variant(root=False),
    "float32_sum_of_squares": _variant(sum_fn=lambda r: float(np.sum((r * r).astype(np.float32),
                                                                      dtype=np.float32))),
}


@contextlib.contextmanager
def mutated(name):
    old = orc.rmsnorm
    orc.rmsnorm = MUTANTS[name]
    try:
        yield
    finally:
        orc.rmsnorm = old


def test_pins_pass_on_the_oracle():
    assert pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    with mutated(name):
        assert not pins_pass(), f"pins did not catch mutant {name}"
