"""Pins of the CPU oracle against facts that do not come from the oracle.

* hand-worked blocks (tests/golden/hand_blocks.json), derived by hand from
  the quantisation formulas of the Mix-Quant digests (paper.rainbus.top,
  section 方法步骤详情, step (3); r9-hu.github.io, section Method, item 1);
* an exhaustive sweep against an exact rational (fractions.Fraction)
  nearest-grid-point rounding written independently below;
* library casts (torch float32 -> float8_e4m3fn, float32 -> bfloat16) on
  inputs where a single rounding is guaranteed;
* invariants of the definition (error bound, idempotence, power-of-two
  equivariance, sign symmetry, row permutation) and exact brute-force dot
  products for the GEMM;
* planted mistakes: each plausible bug in a copy of the oracle must make at
  least one of the pins fail.
"""
import contextlib
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import nvfp4_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")

E2M1_GRID = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]


def _e4m3_grid():
    out = []
    for b in range(127):            # 0x00..0x7E: every finite non-negative
        e, m = b >> 3, b & 7
        if e == 0:
            out.append(Fraction(m, 512))
        else:
            out.append(Fraction(8 + m, 8) * Fraction(2) ** (e - 7))
    return out


E4M3_GRID = _e4m3_grid()


def nearest_even(value: Fraction, grid):
    """Index of the grid point nearest to value; ties -> even index.

    Grid index parity equals mantissa-bit parity for both the E2M1 codes and
    the E4M3 bytes, so "even index" is ties-to-even.  Values beyond the top
    of the grid go to its largest point (saturation).
    """
    best = None
    for i, g in enumerate(grid):
        d = abs(value - g)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def parse_value(s: str) -> float:
    if s == "-0":
        return -0.0
    return float(Fraction(s))


def parse_alpha(s: str) -> np.float32:
    if s.startswith("fp32("):
        num, den = s[5:-1].split("/")
        return np.float32(np.float32(int(num)) / np.float32(int(den)))
    return np.float32(Fraction(s))


def to_bf16_bits(vals) -> np.ndarray:
    f = np.asarray(vals, dtype=np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back.view(np.uint32), f.view(np.uint32)), \
        "golden value is not exactly a BF16 number"
    return bits


def load_golden():
    with open(GOLDEN, encoding="utf-8") as fh:
        return json.load(fh)


def golden_tensor(case):
    vals = [parse_value(v) for v in case["block"]]
    row = vals + [0.0] * (16 - len(vals))
    row += [parse_value(case["anchor"]) if case["anchor"] else 0.0] + [0.0] * 15
    return to_bf16_bits(np.array([row]))


# ---------------------------------------------------------------------------
# hand-worked blocks
# ---------------------------------------------------------------------------

def check_golden_blocks():
    g = load_golden()
    for case in g["cases"]:
        x = golden_tensor(case)
        alpha, scales, codes = orc.quantize(x)
        assert alpha == parse_alpha(case["alpha"]), case["id"]
        assert int(scales[0, 0]) == case["scale_byte"], case["id"]
        assert orc.unpack_codes(codes)[0, :16].tolist() == case["codes"], case["id"]
        assert codes[0, :8].tolist() == case["packed"], case["id"]
        if case["xhat"] is not None:
            want = [parse_value(v) for v in case["xhat"]]
            got = orc.dequantize(alpha, scales, codes)[0, :len(want)]
            assert got.tolist() == want, case["id"]


def test_golden_blocks():
    check_golden_blocks()


def check_golden_gemm():
    g = load_golden()
    w6 = next(c for c in g["cases"] if c["id"].startswith("W6"))
    x = golden_tensor(w6)
    alpha, scales, codes = orc.quantize(x)
    q = (alpha, scales[:, :1], codes[:, :8])      # the W6 block alone
    y, bound, ybf = orc.w4a4_reference(q, q)
    assert y[0, 0] == float(Fraction(g["gemm"]["y"]))
    got = (ybf.astype(np.uint32) << 16).view(np.float32)
    assert float(got[0, 0]) == float(Fraction(g["gemm"]["y_bf16"]))


def test_golden_gemm():
    check_golden_gemm()


# ---------------------------------------------------------------------------
# exhaustive sweeps against exact rational rounding
# ---------------------------------------------------------------------------

SWEEP_ALPHAS = [np.float32(1.0),
                np.float32(np.float32(3) / np.float32(2688)),
                np.float32(np.float32(7) / np.float32(2688)),
                np.float32(np.float32(37.25) / np.float32(2688)),
                np.float32(1.0 + 2.0 ** -23),
                np.float32(1.0 - 2.0 ** -24)]


def bf16_range(lo: float, hi: float) -> np.ndarray:
    """Every positive finite BF16 bit pattern with lo <= value <= hi."""
    allbits = np.arange(1, 0x7F80, dtype=np.uint16)
    vals = orc.bf16_to_f64(allbits)
    return allbits[(vals >= lo) & (vals <= hi)]


def sweep_e2m1(alphas, sigmas_bytes):
    for alpha in alphas:
        for sbyte in sigmas_bytes:
            sig = float(E4M3_GRID[sbyte])
            d = float(alpha) * sig
            bits = bf16_range(0.2 * d, 6.4 * d)
            bits = np.concatenate([bits, bits | np.uint16(0x8000)])
            pad = (-len(bits)) % 16
            x = orc.bf16_to_f64(np.concatenate([bits, np.zeros(pad, np.uint16)]))
            x = x.reshape(-1, 16)
            sigma = np.full((x.shape[0], 1), sig)
            codes = orc.element_codes(x, alpha, sigma).reshape(-1)[:len(bits)]
            den = Fraction(float(alpha)) * E4M3_GRID[sbyte]
            for b, c in zip(bits.tolist(), codes.tolist()):
                xv = Fraction(float(orc.bf16_to_f64(np.uint16(b))))
                want = nearest_even(abs(xv) / den, E2M1_GRID)
                want |= 8 if b & 0x8000 else 0
                assert c == want, (float(alpha), sbyte, hex(b))


def test_e2m1_exhaustive_all_scales():
    """Every BF16 input around the grid, every nonzero E4M3 scale, 2 alphas."""
    sweep_e2m1(SWEEP_ALPHAS[:2], range(1, 127))


def test_e2m1_exhaustive_other_alphas():
    sweep_e2m1(SWEEP_ALPHAS[2:], range(1, 127, 5))


def sweep_e4m3(alphas):
    for alpha in alphas:
        six_a = 6.0 * float(alpha)
        bits = bf16_range(six_a * 2.0 ** -12, six_a * 600.0)
        x = np.zeros((len(bits), 16))
        x[:, 0] = orc.bf16_to_f64(bits)
        x[:, 5] = -0.0
        _, sbytes = orc.block_scales(x, alpha)
        den = 6 * Fraction(float(alpha))
        for b, s in zip(bits.tolist(), sbytes[:, 0].tolist()):
            v = Fraction(float(orc.bf16_to_f64(np.uint16(b)))) / den
            assert s == nearest_even(v, E4M3_GRID), (float(alpha), hex(b))


def test_e4m3_exhaustive():
    sweep_e4m3(SWEEP_ALPHAS)


def test_e4m3_matches_torch_cast_on_float32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    v = np.exp(rng.uniform(np.log(2.0 ** -11), np.log(448.0), 200000))
    v = v.astype(np.float32)
    # include exact midpoints of the grid (single rounding in both paths)
    mids = np.array([(float(E4M3_GRID[i]) + float(E4M3_GRID[i + 1])) / 2
                     for i in range(126)], dtype=np.float32)
    v = np.concatenate([v, mids])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.e4m3_encode(orc.e4m3_round(v.astype(np.float64)))
    assert np.array_equal(got, ref)


def test_bf16_rounding_matches_torch_on_float32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    v = (rng.standard_normal(300000) * 10.0 ** rng.uniform(-30, 30, 300000))
    v = v.astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy()
    got = orc.f64_to_bf16_bits(v.astype(np.float64))
    assert np.array_equal(got.view(np.int16), ref)


def test_bf16_rounding_is_single_rounding_from_float64():
    # 1 + 2^-8 + 2^-30 rounds up in one step; via float32 it would first
    # become 1 + 2^-8 (a BF16 tie) and then go to even (1.0).
    y = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30, -(1.0 + 2.0 ** -8 + 2.0 ** -30)])
    got = (orc.f64_to_bf16_bits(y).astype(np.uint32) << 16).view(np.float32)
    assert got.tolist() == [1.0 + 2.0 ** -7, -(1.0 + 2.0 ** -7)]


# ---------------------------------------------------------------------------
# invariants on random tensors
# ---------------------------------------------------------------------------

def random_tensor(rows=64, k=256, seed=0, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k)).astype(np.float32)
    if outliers:
        ch = rng.choice(k, max(1, k // 50), replace=False)
        x[:, ch] *= 50.0
    x[1, :] *= 1e-3                      # small-magnitude row
    x[2, 16:32] = 0.0                    # an all-zero block
    x[3, :16] = 2.0 ** -20               # a block whose scale underflows
    x[4, 5] = -0.0
    bits = x.view(np.uint32)
    bits = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    return bits


def check_error_bound(seed=0):
    xb = random_tensor(seed=seed)
    x = orc.bf16_to_f64(xb)
    alpha, scales, codes = orc.quantize(xb)
    xh = orc.dequantize(alpha, scales, codes)
    sig = np.repeat(orc.e4m3_decode(scales), 16, axis=1)
    d = float(alpha) * sig
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.where(d > 0, np.abs(x) / d, 0.0)
    step = np.where(s <= 2, 0.5, np.where(s <= 4, 1.0, 2.0))
    normal = sig >= 2.0 ** -6
    allowed = np.where(normal, 0.5 * step, np.maximum(0.5 * step, s - 6.0)) * d
    allowed *= 1.0 + 2.0 ** -40          # s - 6 is itself rounded
    # a zero scale means every element of the block is below half the
    # smallest subnormal scale's first step
    zero_blk = sig == 0
    assert np.all(np.abs(x - xh)[~zero_blk] <= allowed[~zero_blk])
    assert np.all(np.abs(x[zero_blk]) <= 6.0 * float(alpha) * 2.0 ** -10)
    assert np.all(xh[zero_blk] == 0)
    return True


def test_error_bound():
    for seed in range(3):
        check_error_bound(seed)


def test_idempotent_when_scales_are_normal():
    """Requantising xhat at the same alpha returns the same scales and codes.

    Holds when every scale is a normal E4M3 value: the block maximum then
    always gets code 7, so max|xhat_b| = 6 alpha sigma_b and sigma_b is
    reproduced.  xhat is not a BF16 tensor, so the float64 block functions
    are called directly.
    """
    xb = random_tensor(seed=5)
    xb[1:5] = xb[10:14]                  # drop the special rows
    alpha, scales, codes = orc.quantize(xb)
    assert np.all(orc.e4m3_decode(scales) >= 2.0 ** -6)
    xh = orc.dequantize(alpha, scales, codes)
    sig2, s2 = orc.block_scales(xh, alpha)
    c2 = orc.element_codes(xh, alpha, sig2)
    assert np.array_equal(s2, scales)
    assert np.array_equal(c2, orc.unpack_codes(codes))


def test_power_of_two_scaling():
    xb = random_tensor(seed=6)
    alpha, scales, codes = orc.quantize(xb)
    for k in (-20, -3, 1, 7, 40):
        xs = orc.bf16_to_f64(xb) * 2.0 ** k
        xs_bits = orc.f64_to_bf16_bits(xs)
        assert np.array_equal(orc.bf16_to_f64(xs_bits), xs)
        a2, s2, c2 = orc.quantize(xs_bits)
        assert float(a2) == float(alpha) * 2.0 ** k
        assert np.array_equal(s2, scales) and np.array_equal(c2, codes)


def test_sign_symmetry():
    xb = random_tensor(seed=7)
    alpha, scales, codes = orc.quantize(xb)
    a2, s2, c2 = orc.quantize(xb ^ np.uint16(0x8000))
    assert a2 == alpha and np.array_equal(s2, scales)
    assert np.array_equal(orc.unpack_codes(c2), orc.unpack_codes(codes) ^ 8)


def test_rows_permute_and_duplicate_at_fixed_alpha():
    xb = random_tensor(seed=8)
    alpha, scales, codes = orc.quantize(xb)
    rng = np.random.default_rng(3)
    idx = rng.integers(0, xb.shape[0], 100)
    a2, s2, c2 = orc.quantize(xb[idx], alpha=alpha)
    assert a2 == alpha
    assert np.array_equal(s2, scales[idx]) and np.array_equal(c2, codes[idx])


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------

def check_gemm_bruteforce(seed=0):
    rng = np.random.default_rng(seed)
    for (m, n, k) in [(1, 1, 16), (3, 2, 32), (4, 3, 64), (2, 4, 48)]:
        xb = random_tensor(rows=m + 5, k=k, seed=seed + m)[5:]
        wb = random_tensor(rows=n + 5, k=k, seed=seed + 100 + n)[5:]
        qa, qw = orc.quantize(xb), orc.quantize(wb)
        y, bound, _ = orc.w4a4_reference(qa, qw)
        ah, wh = orc.dequantize(*qa), orc.dequantize(*qw)
        for i in range(m):
            for j in range(n):
                exact = sum(Fraction(float(ah[i, t])) * Fraction(float(wh[j, t]))
                            for t in range(k))
                babs = sum(abs(Fraction(float(ah[i, t])) * Fraction(float(wh[j, t])))
                           for t in range(k))
                assert abs(Fraction(float(y[i, j])) - exact) <= abs(exact) * Fraction(1, 2 ** 51)
                assert abs(Fraction(float(bound[i, j])) - babs) <= babs * Fraction(1, 2 ** 48)
    return True


def test_gemm_bruteforce_tiny():
    check_gemm_bruteforce()


def check_gemm_exact_cancellation():
    """Dot products that are exactly zero or tiny must come out exactly."""
    rng = np.random.default_rng(17)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    x[:, 32:] = x[:, :32]                      # second half repeats the first
    xb = bf16_bits_of(x)
    w = np.ones((3, 64), dtype=np.float32)
    w[0, 32:] = -1.0                           # exact cancellation
    w[1, 32:] = -1.0
    w[1, 0] = 2.0 ** -6                        # plus one tiny term
    wb = bf16_bits_of(w)
    qa, qw = orc.quantize(xb), orc.quantize(wb)
    y, bound, _ = orc.w4a4_reference(qa, qw)
    ah, wh = orc.dequantize(*qa), orc.dequantize(*qw)
    assert np.all(y[:, 0] == 0.0)
    for i in range(8):
        exact = sum(Fraction(float(ah[i, t])) * Fraction(float(wh[1, t])) for t in range(64))
        assert abs(Fraction(float(y[i, 1])) - exact) <= abs(exact) * Fraction(1, 2 ** 52)
    return True


def bf16_bits_of(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_gemm_exact_cancellation():
    check_gemm_exact_cancellation()


def test_gemm_one_hot():
    a = np.zeros((3, 32))
    w = np.zeros((5, 32))
    a[0, 7], a[1, 20], a[2, 31] = 1.5, -6.0, 0.25
    w[:, 7] = [2, 0, 0, 0, -1]
    w[:, 20] = [0, 3, 0, 0, 0]
    w[:, 31] = [0, 0, 0, 4, 0]
    y, bound = orc.gemm_ref(a, w)
    want = np.zeros((3, 5))
    want[0, 0], want[0, 4] = 3.0, -1.5
    want[1, 1] = -18.0
    want[2, 3] = 1.0
    assert np.array_equal(y, want) and np.array_equal(bound, np.abs(want))


def test_bf16_gemm_reference_is_float64_product():
    xb = random_tensor(rows=6, k=48, seed=9)
    wb = random_tensor(rows=7, k=48, seed=10)
    y, bound, _ = orc.bf16_gemm_reference(xb, wb)
    x, w = orc.bf16_to_f64(xb), orc.bf16_to_f64(wb)
    for i in range(6):
        for j in range(7):
            exact = sum(Fraction(float(x[i, t])) * Fraction(float(w[j, t])) for t in range(48))
            assert abs(Fraction(float(y[i, j])) - exact) <= Fraction(float(bound[i, j])) / 2 ** 48


# ---------------------------------------------------------------------------
# planted mistakes: each must break at least one pin
# ---------------------------------------------------------------------------

def pins_pass() -> bool:
    checks = [check_golden_blocks, check_golden_gemm,
              lambda: sweep_e2m1(SWEEP_ALPHAS[:2], range(40, 127, 29)),
              lambda: sweep_e4m3(SWEEP_ALPHAS[:2]),
              check_error_bound, check_gemm_bruteforce, check_gemm_exact_cancellation]
    for c in checks:
        try:
            c()
        except (AssertionError, IndexError, ValueError):
            return False
    return True


def _ties_away(v, mant_bits, min_exp, max_val):
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    q = np.ldexp(1.0, np.maximum(e - 1, min_exp) - mant_bits)
    return np.minimum(np.floor(v / q + 0.5) * q, max_val)


def _fp32_codes(x, alpha, sigma):
    sig = np.repeat(sigma, 16, axis=1).astype(np.float32)
    d = (np.float32(alpha) * sig)
    s = (np.abs(x).astype(np.float32) / np.where(d > 0, d, 1)).astype(np.float64)
    mag = np.where(d > 0, orc.e2m1_round(s), 0.0)
    return orc.e2m1_encode(mag) | (np.signbit(x).astype(np.uint8) << 3)


def _fp32_scales(x, alpha):
    rows, k = x.shape
    amax_b = np.abs(x).reshape(rows, k // 16, 16).max(axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (amax_b.astype(np.float32)
             / (np.float32(alpha) * np.float32(6))).astype(np.float64)
    sig = orc.e4m3_round(v) if alpha != 0 else np.zeros_like(v)
    return sig, orc.e4m3_encode(sig)


MUTANTS = {
    "ties_away_from_zero": ("round_to_minifloat", _ties_away),
    "nibbles_swapped": ("pack_codes",
                        lambda c: (c[:, 1::2] | (c[:, 0::2] << 4)).astype(np.uint8)),
    "float32_element_quotient": ("element_codes", _fp32_codes),
    "float32_scale_quotient": ("block_scales", _fp32_scales),
    "no_negative_zero": ("element_codes",
                         lambda x, a, s, f=orc.element_codes:
                         np.where(x == 0, f(x, a, s) & 7, f(x, a, s))),
    "float64_alpha": ("tensor_scale",
                      lambda x: np.float64(np.max(np.abs(x))) / 2688.0),
    "e4m3_bias_8": ("e4m3_decode",
                    lambda b, f=orc.e4m3_decode: f(b) / 2.0),
    "e2m1_no_saturation": ("e2m1_round",
                           lambda s: orc.round_to_minifloat(s, 1, 0, np.inf)),
    "dequant_drops_alpha": ("dequantize",
                            lambda a, s, p, f=orc.dequantize: f(1.0, s, p)),
    "gemm_drops_last_k": ("exact_dot",
                          lambda a, b, f=orc.exact_dot: f(a[:, :-1], b[:, :-1])),
    "gemm_low_half_dropped": ("exact_dot",
                              lambda a, b, f=orc.exact_dot: f(a & ~2047, b & ~2047)),
    "gemm_float64_blas": ("exact_dot",
                          lambda a, b: np.rint(a.astype(np.float64) @ b.astype(np.float64).T
                                               * (1 + 2.0 ** -30)).astype(np.int64)),
}


@contextlib.contextmanager
def mutated(name):
    attr, fn = MUTANTS[name]
    old = getattr(orc, attr)
    setattr(orc, attr, fn)
    try:
        yield
    finally:
        setattr(orc, attr, old)


def test_pins_pass_on_the_oracle():
    assert pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    with mutated(name):
        assert not pins_pass(), f"pins did not catch mutant {name}"
