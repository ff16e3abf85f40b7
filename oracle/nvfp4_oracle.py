"""CPU oracle for the NVFP4 W4A4 prefill linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
constants with the HIP library and imports nothing from it.

What it computes (plain numpy, float64 unless stated):

* NVFP4 quantisation of a tensor x, as written in
  "Mix-Quant：面向智能体LLM的量化预填充与精确解码" (paper.rainbus.top digest),
  section 方法步骤详情, step (3), and in
  "Mix-Quant: Quantized Prefilling, Precise Decoding for Agentic LLMs"
  (r9-hu.github.io paper digest), section Method, item 1:

      sigma_b = Pi_E4M3( max_{i in b} |x_i| / (alpha_x * q_max) )
      q_i     = Pi_FP4 ( x_i / (alpha_x * sigma_b(i)) )
      xhat_i  = alpha_x * sigma_b(i) * q_i

  over groups b of 16 consecutive elements, with round-to-nearest and no
  rotation.  The format (E2M1 values, one FP8 E4M3 scale per 16 elements,
  plus one tensor-level scale) is the one described in the same digest,
  section 前置知识, "NVFP4 微缩放量化".

* The W4A4 linear layer Y = Xhat . What^T.  Every dequantised value is
  alpha * T * 2**-10 with a small integer T, so the sum over K is taken
  exactly in integers and rounded once; also the bound
  B = |Xhat| . |What|^T used for the tolerance of a float32 result.

Readings where the pages are silent (each one is also listed in the design
notes of the repository):

  R1  alpha_x = RNE_fp32(amax / (6 * 448)); amax = 0 gives alpha_x = 0.
  R2  q_max = 6, the largest E2M1 magnitude.
  R3  every division is taken in exact real arithmetic; float64 reproduces
      it exactly here (see ``_why_float64_is_exact``).
  R4  Pi_FP4 is round-to-nearest, ties to the even code, saturating at 6.
  R5  Pi_E4M3 is round-to-nearest, ties to even mantissa, onto the OCP
      E4M3FN grid (bias 7, largest finite 448, NaN byte 0x7F never produced),
      saturating at 448.
  R6  a block whose scale rounds to 0 (or alpha_x = 0) gets magnitude code 0.
  R7  the code's sign bit is the sign bit of x, so -0.0 gives code 0x8.
  R8  two codes per byte, element 2j in the low nibble; rows are stored
      K-contiguous; scales are bytes, row-major [rows][K/16].

* The normalisation whose output feeds a quantised projection, for the
  quantiser fused into its producer.  The pages' models (Qwen3-8B,
  Qwen3.5-9B, Gemma-4; paper.rainbus.top digest, 实验结果) normalise the input
  of each attention and MLP block with RMSNorm; the pages do not define it.

  R16 y_i = x_i * gamma_i / sqrt(mean_j(x_j^2) + eps) over each row, in
      exact real arithmetic rounded once to BF16 (RNE); here: the sum of
      the (exact) squares correctly rounded (math.fsum), then float64, a
      few roundings of 2**-53 before the single BF16 rounding.

* The gated MLP activation H = SiLU(G) * U of the gate and up projections'
  outputs, which the down projection's quantiser takes as its input (the
  pages' models' MLPs; the configuration of the layer names the down input
  "SiLU(gate) * up").

  R17 H = RNE_bf16( g * u / (1 + exp(-g)) ) element by element, from the
      projections' float32 outputs g and u, in float64 before the single
      BF16 rounding.

Parity pins: every function here is checked by ``tests/test_oracle.py``
against hand-worked blocks (``tests/golden/``), an exact rational
brute force, closed forms and invariants.  No function is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

GROUP = 16            # elements per block scale
Q_MAX = 6.0           # largest E2M1 magnitude (reading R2)
E4M3_MAX = 448.0      # largest finite OCP E4M3FN value (reading R5)

# E2M1 magnitudes indexed by the 3-bit code (sign in bit 3).
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


# ---------------------------------------------------------------------------
# bfloat16 helpers (inputs and the BF16 output reference)
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_to_minifloat(v: np.ndarray, mant_bits: int, min_exp: int,
                       max_val: float) -> np.ndarray:
    """Round non-negative float64 values to a binary floating-point grid.

    The grid has ``mant_bits`` stored mantissa bits, smallest normal exponent
    ``min_exp`` (below it the spacing stays 2**(min_exp - mant_bits), i.e.
    subnormals), round-to-nearest with ties to the even last mantissa bit,
    and saturation at ``max_val``.  Inputs must be finite and >= 0.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                    # v = f * 2**e, f in [0.5, 1)
    exp = np.maximum(e - 1, min_exp)      # binade of v, clamped to subnormal
    quantum = np.ldexp(1.0, exp - mant_bits)
    r = np.rint(v / quantum) * quantum    # np.rint: ties to even integer
    return np.minimum(r, max_val)


def f64_to_bf16_bits(y: np.ndarray) -> np.ndarray:
    """Round float64 directly to BF16 (RNE, one rounding) -> uint16 bits.

    BF16 has 7 stored mantissa bits and the float32 exponent range; results
    beyond the largest finite BF16 are out of scope here.
    """
    y = np.asarray(y, dtype=np.float64)
    mag = round_to_minifloat(np.abs(y), 7, -126, 3.3895313892515355e38)
    val = np.where(np.signbit(y), -mag, mag).astype(np.float32)
    return (val.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# E4M3 and E2M1 encodings
# ---------------------------------------------------------------------------

def e4m3_round(v: np.ndarray) -> np.ndarray:
    """Pi_E4M3 on non-negative values (reading R5): value on the grid."""
    return round_to_minifloat(v, 3, -6, E4M3_MAX)


def e4m3_encode(val: np.ndarray) -> np.ndarray:
    """Non-negative E4M3 grid values -> OCP E4M3FN bytes (sign bit 0)."""
    val = np.asarray(val, dtype=np.float64)
    _, e = np.frexp(val)
    exp = e - 1
    sub = val < 2.0 ** -6
    mant_sub = np.rint(val / 2.0 ** -9)
    mant_norm = np.rint((val / np.ldexp(1.0, exp) - 1.0) * 8.0)
    byte = np.where(sub, mant_sub, (exp + 7) * 8 + mant_norm)
    byte = np.where(val == 0, 0, byte)
    return byte.astype(np.uint8)


def e4m3_decode(byte: np.ndarray) -> np.ndarray:
    """OCP E4M3FN bytes (finite, sign 0) -> float64 values."""
    b = np.asarray(byte).astype(np.int64)
    e = (b >> 3) & 15
    m = b & 7
    return np.where(e == 0, m * 2.0 ** -9,
                    (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))


def e2m1_round(s: np.ndarray) -> np.ndarray:
    """Pi_FP4 on non-negative values (reading R4): value on the E2M1 grid."""
    return round_to_minifloat(s, 1, 0, Q_MAX)


def e2m1_encode(mag: np.ndarray) -> np.ndarray:
    """E2M1 grid magnitudes -> 3-bit codes 0..7."""
    idx = np.searchsorted(E2M1_VALUES, np.asarray(mag, dtype=np.float64))
    return idx.astype(np.uint8)


# ---------------------------------------------------------------------------
# Quantise / dequantise
# ---------------------------------------------------------------------------

def tensor_scale(x: np.ndarray) -> np.float32:
    """alpha_x = RNE_fp32(amax / 2688) (readings R1, R2).

    numpy's float32 division is the IEEE correctly rounded one; amax is a
    BF16 value and 2688 = 6 * 448 is exact in float32, so the quotient is
    rounded once.
    """
    amax = np.float32(np.max(np.abs(x))) if np.size(x) else np.float32(0)
    return np.float32(amax / np.float32(Q_MAX * E4M3_MAX))


def block_scales(x: np.ndarray, alpha: np.float32):
    """sigma_b for every 16-element block of the rows of x (float64 [R, K]).

    Returns (sigma values float64 [R, K/16], bytes uint8 [R, K/16]).
    """
    rows, k = x.shape
    blocks = np.abs(x).reshape(rows, k // GROUP, GROUP)
    amax_b = blocks.max(axis=2)
    a = np.float64(alpha)
    if a == 0.0:
        sigma = np.zeros_like(amax_b)
    else:
        sigma = e4m3_round(amax_b / (a * Q_MAX))
    return sigma, e4m3_encode(sigma)


def element_codes(x: np.ndarray, alpha: np.float32,
                  sigma: np.ndarray) -> np.ndarray:
    """4-bit codes (sign in bit 3) of every element; x float64 [R, K]."""
    rows, k = x.shape
    sig = np.repeat(sigma, GROUP, axis=1)
    denom = np.float64(alpha) * sig            # exact: <= 28 significant bits
    safe = np.where(denom > 0, denom, 1.0)
    s = np.abs(x) / safe
    mag = np.where(denom > 0, e2m1_round(s), 0.0)   # reading R6
    code = e2m1_encode(mag)
    return code | (np.signbit(x).astype(np.uint8) << 3)   # reading R7


def pack_codes(code: np.ndarray) -> np.ndarray:
    """[R, K] 4-bit codes -> [R, K/2] bytes, element 2j in the low nibble."""
    c = code.astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[R, K/2] bytes -> [R, K] 4-bit codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 15
    out[:, 1::2] = p >> 4
    return out


def quantize(x_bits: np.ndarray, alpha=None):
    """NVFP4-quantise a BF16 tensor [R, K] (K % 16 == 0).

    ``alpha`` None means the tensor's own alpha_x (reading R1); otherwise the
    given float32 value is used for every row (rows of one tensor quantised
    in slices share the tensor's alpha).

    Returns (alpha float32, scales uint8 [R, K/16], codes uint8 [R, K/2]).
    """
    x = bf16_to_f64(x_bits)
    if x.ndim != 2 or x.shape[1] % GROUP:
        raise ValueError("quantize expects [rows, K] with K % 16 == 0")
    a = tensor_scale(x) if alpha is None else np.float32(alpha)
    sigma, sbytes = block_scales(x, a)
    codes = element_codes(x, a, sigma)
    return a, sbytes, pack_codes(codes)


def dequantize(alpha, scales: np.ndarray, packed: np.ndarray) -> np.ndarray:
    """xhat = alpha * sigma_b * q (exact in float64: <= 30 significant bits)."""
    code = unpack_codes(packed)
    mag = E2M1_VALUES[code & 7]
    q = np.where(code & 8, -mag, mag)
    sig = np.repeat(e4m3_decode(scales), GROUP, axis=1)
    return np.float64(np.float32(alpha)) * sig * q


# ---------------------------------------------------------------------------
# GEMMs
# ---------------------------------------------------------------------------

def gemm_ref(a_hat: np.ndarray, w_hat: np.ndarray):
    """Y = Ahat . What^T and B = |Ahat| . |What|^T in float64.

    a_hat: [M, K], w_hat: [N, K] (both float64).  The float32 output of a
    W4A4 GEMM must satisfy |y - Y| <= 1e-4 * B + 1e-6.
    """
    y = a_hat @ w_hat.T
    bound = np.abs(a_hat) @ np.abs(w_hat).T
    return y, bound


def integer_operand(q):
    """(alpha, scales, codes) -> int64 T with xhat = alpha * T * 2**-10 exactly.

    T = (2 q) * (sigma * 2**9): 2q is an integer in [-12, 12] and every E4M3
    value is an integer multiple of 2**-9 (at most 448 * 512 = 229376), so
    |T| < 2**22.
    """
    _, scales, packed = q
    code = unpack_codes(packed)
    two_q = np.array([0, 1, 2, 3, 4, 6, 8, 12], dtype=np.int64)[code & 7]
    two_q = np.where(code & 8, -two_q, two_q)
    sig512 = np.rint(e4m3_decode(scales) * 512.0).astype(np.int64)
    return two_q * np.repeat(sig512, GROUP, axis=1)


def exact_dot(ta: np.ndarray, tb: np.ndarray) -> np.ndarray:
    """Exact int64 S = ta . tb^T for |entries| < 2**22 and K <= 2**16.

    Each operand is split into signed 11-bit halves; every float64 product of
    halves is an integer below 2**22 and every partial sum of K of them is an
    integer below 2**38, so the four float64 matrix products are exact in
    any summation order.  S < 2**60 fits int64.
    """
    if ta.shape[1] > 1 << 16:
        raise ValueError("K too large for the exact split")

    def halves(t):
        mag = np.abs(t)
        sgn = np.sign(t)
        return (sgn * (mag >> 11)).astype(np.float64), (sgn * (mag & 2047)).astype(np.float64)

    a1, a0 = halves(ta)
    b1, b0 = halves(tb)
    p11 = (a1 @ b1.T).astype(np.int64)
    p10 = (a1 @ b0.T).astype(np.int64) + (a0 @ b1.T).astype(np.int64)
    p00 = (a0 @ b0.T).astype(np.int64)
    return (p11 << 22) + (p10 << 11) + p00


def w4a4_reference(a_q, w_q):
    """Reference of the W4A4 layer from two quantised operands.

    a_q, w_q: (alpha, scales, codes) triples as returned by ``quantize``.
    Y = sum_k xhat_a xhat_w = alpha_a alpha_w 2**-20 sum_k T_a T_w, with the
    integer sum taken exactly (``exact_dot``) and then rounded once to
    float64 (relative error <= 2**-52).
    Returns (Y float64 [M, N], B = |Ahat| . |What|^T float64, Y rounded to
    BF16 bits).
    """
    ta, tw = integer_operand(a_q), integer_operand(w_q)
    s = exact_dot(ta, tw)
    babs = exact_dot(np.abs(ta), np.abs(tw))
    scale = float(np.float64(np.float32(a_q[0])) * np.float64(np.float32(w_q[0])))  # exact
    y = s.astype(np.float64) * scale * 2.0 ** -20
    bound = babs.astype(np.float64) * abs(scale) * 2.0 ** -20
    return y, bound, f64_to_bf16_bits(y)


def bf16_gemm_reference(x_bits: np.ndarray, w_bits: np.ndarray):
    """Reference of the BF16 comparison GEMM: Y = X . W^T in float64."""
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    y, bound = gemm_ref(x, w)
    return y, bound, f64_to_bf16_bits(y)


# ---------------------------------------------------------------------------
# RMSNorm producing the quantised activation (reading R16)
# ---------------------------------------------------------------------------

def rmsnorm(x_bits: np.ndarray, gamma_bits: np.ndarray, eps: float):
    """Row-wise RMSNorm of BF16 x [rows][K] with BF16 weights gamma [K].

    Returns (y, y_bits): the float64 values x*gamma/sqrt(mean(x^2)+eps) and
    their BF16 rounding (RNE, one rounding).  Each row's sum of squares is
    the correctly rounded sum of the exact squares (math.fsum)."""
    x = bf16_to_f64(x_bits)
    g = bf16_to_f64(gamma_bits)
    k = x.shape[1]
    ss = np.array([math.fsum(row * row) for row in x], dtype=np.float64)
    inv = 1.0 / np.sqrt(ss / k + np.float64(eps))
    y = x * inv[:, None] * g[None, :]
    return y, f64_to_bf16_bits(y)


def silu_mul(g: np.ndarray, u: np.ndarray):
    """H = SiLU(g) * u (reading R17) from float32 (or float64) g and u:
    returns (h, h_bits), the float64 values and their BF16 rounding."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    with np.errstate(over="ignore"):
        h = g * u / (1.0 + np.exp(-g))
    return h, f64_to_bf16_bits(h)


def _why_float64_is_exact():
    """Why float64 division reproduces exact real rounding decisions.

    x is a BF16 value (<= 8 significant bits), alpha a float32 (24 bits),
    6*alpha and alpha*sigma have <= 28 bits, and every rounding midpoint of
    the E4M3 and E2M1 grids has <= 5 bits.  If an exact quotient p/d differs
    from a midpoint m, then |p - m d| is at least one unit of the coarser of
    the two binary grids, which puts p/d at relative distance >= 2**-33 from
    m; float64 division is correctly rounded (relative error <= 2**-53), so
    it lands on the same side of m, and equals m only when p/d == m.
    """
    return None
