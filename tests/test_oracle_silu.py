"""Pins of the oracle's gated activation H = SiLU(g) * u (reading R17).

* torch's SiLU (torch.nn.functional.silu) in float64, times u;
* closed forms: SiLU(0) = 0; SiLU(g) - SiLU(-g) = g; SiLU(g) -> g for large
  g and -> 0 for very negative g; SiLU(ln 3) = (3/4) ln 3 exactly in reals;
* the BF16 rounding is the oracle's pinned single rounding;
* planted mistakes must fail one of them.
"""
import contextlib
import math

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as orc


def check_torch():
    rng = np.random.default_rng(21)
    g = (rng.standard_normal(4096) * 4).astype(np.float32)
    u = (rng.standard_normal(4096) * 2).astype(np.float32)
    h, hb = orc.silu_mul(g, u)
    ref = (torch.nn.functional.silu(torch.from_numpy(g.astype(np.float64))) *
           torch.from_numpy(u.astype(np.float64))).numpy()
    assert np.allclose(h, ref, rtol=1e-13, atol=1e-300)
    assert np.array_equal(hb, orc.f64_to_bf16_bits(ref))


def check_closed_forms():
    one = np.ones(5)
    h, _ = orc.silu_mul(np.array([0.0, 50.0, -60.0, math.log(3.0), -math.log(3.0)]), one)
    assert h[0] == 0.0
    assert abs(h[1] - 50.0) < 1e-15 * 50 and abs(h[2]) < 1e-20
    assert abs(h[3] - 0.75 * math.log(3.0)) < 1e-15
    assert abs((h[3] - h[4]) - math.log(3.0)) < 1e-15        # SiLU(g) - SiLU(-g) = g
    h2, _ = orc.silu_mul(np.array([1.5, -2.25]), np.array([-2.0, 0.5]))
    h1, _ = orc.silu_mul(np.array([1.5, -2.25]), np.array([1.0, 1.0]))
    assert np.array_equal(h2, h1 * np.array([-2.0, 0.5]))    # linear in u


def pins_pass():
    for c in (check_torch, check_closed_forms):
        try:
            c()
        except AssertionError:
            return False
    return True


def test_matches_torch_silu_float64():
    check_torch()


def test_closed_forms():
    check_closed_forms()


def _variant(kind):
    def f(g, u):
        g = np.asarray(g, dtype=np.float64)
        u = np.asarray(u, dtype=np.float64)
        if kind == "sigmoid_only":
            h = u / (1.0 + np.exp(-g))
        elif kind == "sign_flipped":
            h = g * u / (1.0 + np.exp(g))
        elif kind == "gate_up_swapped":
            h = u * g / (1.0 + np.exp(-u))
        else:                       # float32 evaluation
            g32, u32 = g.astype(np.float32), u.astype(np.float32)
            h = (g32 * u32 / (np.float32(1) + np.exp(-g32))).astype(np.float64)
        return h, orc.f64_to_bf16_bits(h)
    return f


MUTANTS = {k: _variant(k) for k in ("sigmoid_only", "sign_flipped", "gate_up_swapped",
                                     "float32_evaluation")}


@contextlib.contextmanager
def mutated(name):
    old = orc.silu_mul
    orc.silu_mul = MUTANTS[name]
    try:
        yield
    finally:
        orc.silu_mul = old


def test_pins_pass_on_the_oracle():
    assert pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    with mutated(name):
        assert not pins_pass(), f"pins did not catch mutant {name}"
