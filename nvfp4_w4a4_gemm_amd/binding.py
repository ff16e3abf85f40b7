"""ctypes binding of libnvfp4_w4a4.so with the C ABI's names.

Argument marshalling only: torch tensors in (device memory, current HIP
stream), raw pointers and sizes to the library, status codes back as
exceptions.  Every step of the layer runs in the library's HIP kernels; if
the library is missing the binding raises instead of computing anything.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4_w4a4.so")

_c_void = ctypes.c_void_p
_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_c_size = ctypes.c_size_t

# name -> argument types (all return nvfp4_status_t, an int)
_SIGNATURES = {
    "nvfp4_quantize_act": [_c_void, _c_i64, _c_i64, _c_i64, _c_void, _c_void, _c_void,
                           _c_void, _c_void, _c_size, _c_void],
    "nvfp4_quantize_act_noalloc": [_c_void, _c_i64, _c_i64, _c_i64, _c_void, _c_void, _c_void,
                                   _c_void, _c_void],
    "nvfp4_quantize_weights": [_c_void, _c_i64, _c_i64, _c_i64, _c_i64, _c_void, _c_void,
                               _c_void, _c_void, _c_size, _c_void],
    "nvfp4_rmsnorm_quantize_act": [_c_void, _c_void, _c_i64, _c_i64, _c_i64, ctypes.c_float,
                                   _c_void, _c_void, _c_void, _c_void, _c_void, _c_i64,
                                   _c_void, _c_size, _c_void],
    "nvfp4_tensor_alpha": [_c_void, _c_i64, _c_i64, _c_i64, _c_void, _c_void, _c_size,
                           _c_void],
    "w4a4_gemm": [_c_void, _c_void, _c_void, _c_void, _c_void, _c_void, _c_i64, _c_i64,
                  _c_i64, _c_void, _c_void, _c_i64, _c_void],
    "w4a4_gemm_multi": [_c_void, _c_void, _c_void, _c_void, _c_void, _c_void, _c_i64, _c_i64,
                        _c_i64, _c_void, _c_void, _c_i64, _c_void],
    "w4a4_gemm_silu_mul_quantize": [_c_void, _c_void, _c_void, _c_void, _c_void, _c_void,
                                    _c_i64, _c_i64, _c_i64, _c_void, _c_i64, _c_void, _c_void,
                                    _c_void, _c_void, _c_size, _c_void],
    "w4a4_gemm_decode": [_c_void, _c_void, _c_void, _c_void, _c_void, _c_void, _c_void,
                         _c_i64, _c_i64, _c_i64, _c_void, _c_void, _c_i64, _c_void],
    "w4a4_gemm_grouped": [_c_void, _c_void, _c_void, _c_i64, _c_void, _c_void, _c_void,
                          _c_void, _c_i64, _c_i64, _c_i64, _c_i32, _c_void, _c_void,
                          _c_void, _c_i64, _c_void],
    "w4a4_gemm_fused_act": [_c_void, _c_i64, _c_void, _c_void, _c_void, _c_void, _c_i64,
                            _c_i64, _c_i64, _c_void, _c_void, _c_i64, _c_void, _c_size,
                            _c_void],
    "bf16_gemm_baseline": [_c_void, _c_void, _c_i64, _c_i64, _c_i64, _c_i32, _c_void,
                           _c_void, _c_void, _c_i64, _c_void],
}

EXPORTS = sorted(list(_SIGNATURES) + ["nvfp4_status_string", "nvfp4_workspace_bytes",
                                      "w4a4_gemm_silu_mul_workspace_bytes",
                                      "nvfp4_rmsnorm_workspace_bytes",
                                      "nvfp4_set_path_flags", "nvfp4_path_flags"])

# kernel-path flags (nvfp4_set_path_flags), for tests and benchmarks
PATH_GEMM_GRID = 1
PATH_DECODE_DIRECT = 2
PATH_REJECT_DEVICE = 4

STATUS = {0: "NVFP4_OK", 1: "NVFP4_ERR_NULL", 2: "NVFP4_ERR_SHAPE", 3: "NVFP4_ERR_ALIGN",
          4: "NVFP4_ERR_UNSUPPORTED", 5: "NVFP4_ERR_LAUNCH", 6: "NVFP4_ERR_WORKSPACE"}

_lib = None


class NvFP4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)} "
                         f"({lib().nvfp4_status_string(status).decode()})")


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m nvfp4_w4a4_gemm_amd.build` (no fallback exists)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        handle.nvfp4_status_string.argtypes = [ctypes.c_int]
        handle.nvfp4_status_string.restype = ctypes.c_char_p
        handle.nvfp4_workspace_bytes.argtypes = []
        handle.nvfp4_workspace_bytes.restype = ctypes.c_size_t
        handle.w4a4_gemm_silu_mul_workspace_bytes.argtypes = [_c_i64, _c_i64]
        handle.w4a4_gemm_silu_mul_workspace_bytes.restype = ctypes.c_size_t
        handle.nvfp4_rmsnorm_workspace_bytes.argtypes = [_c_i64]
        handle.nvfp4_rmsnorm_workspace_bytes.restype = ctypes.c_size_t
        handle.nvfp4_set_path_flags.argtypes = [ctypes.c_int]
        handle.nvfp4_set_path_flags.restype = None
        handle.nvfp4_path_flags.argtypes = []
        handle.nvfp4_path_flags.restype = ctypes.c_int
        _lib = handle
    return _lib


def _call(name: str, *args) -> None:
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise NvFP4Error(name, st)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class path_flags:
    """Context manager: run a block with the library's kernel-path flags set
    (NVFP4_PATH_* of the C header), restoring the previous flags after."""

    def __init__(self, flags: int):
        self.flags = flags

    def __enter__(self):
        self.prev = lib().nvfp4_path_flags()
        lib().nvfp4_set_path_flags(self.flags)
        return self

    def __exit__(self, *exc):
        lib().nvfp4_set_path_flags(self.prev)
        return False


def workspace_bytes() -> int:
    return int(lib().nvfp4_workspace_bytes())


def new_workspace(device) -> torch.Tensor:
    return torch.empty(workspace_bytes(), dtype=torch.uint8, device=device)


def rmsnorm_workspace(m: int, device) -> torch.Tensor:
    """Workspace with which nvfp4_rmsnorm_quantize_act keeps each of m rows'
    r between its two passes (the faster quantise pass)."""
    return torch.empty(int(lib().nvfp4_rmsnorm_workspace_bytes(m)), dtype=torch.uint8,
                       device=device)


@dataclass
class NVFP4Tensor:
    """A quantised operand: alpha (float32 [1]), scales [rows, K/16], codes [rows, K/2]."""
    alpha: torch.Tensor
    scales: torch.Tensor
    codes: torch.Tensor

    @property
    def rows(self) -> int:
        return self.codes.shape[-2]

    @property
    def k(self) -> int:
        return self.codes.shape[-1] * 2


def _check_bf16_2d(x: torch.Tensor, name: str):
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
        raise ValueError(f"{name} must be a 2-D bfloat16 CUDA tensor")
    if x.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along K")


# The library sees raw pointers only: shapes, dtypes, layouts and devices of
# everything it reads or writes are checked here, before any call.

def _check_device(t: torch.Tensor, dev, name: str):
    if not t.is_cuda or t.device != dev:
        raise ValueError(f"{name} must be a CUDA tensor on {dev}")


def _check_dense(t: torch.Tensor, dtype, shape, name: str):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")


def _check_quantized(codes: torch.Tensor, scales: torch.Tensor, rows: int, k: int, dev,
                     name: str):
    if k % 16 != 0:
        raise ValueError(f"{name}: K = {k} is not a multiple of 16")
    _check_dense(codes, torch.uint8, (rows, k // 2), name + ".codes")
    _check_dense(scales, torch.uint8, (rows, k // 16), name + ".scales")
    _check_device(codes, dev, name + ".codes")
    _check_device(scales, dev, name + ".scales")


def _check_alpha(alpha: torch.Tensor, n: int, dev, name: str):
    if alpha.dtype != torch.float32 or alpha.numel() != n or not alpha.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor of {n} element(s)")
    _check_device(alpha, dev, name)


def _check_tensor(q: "NVFP4Tensor", dev, name: str):
    if q.codes.dim() != 2:
        raise ValueError(f"{name}.codes must be 2-D")
    _check_quantized(q.codes, q.scales, q.rows, q.k, dev, name)
    _check_alpha(q.alpha, 1, dev, name + ".alpha")


def _check_weight(b, dev, name: str):
    """An NVFP4Tensor, or an NVFP4Stack with one tensor scale per row."""
    if isinstance(b, NVFP4Stack):
        if b.codes.dim() != 2:
            raise ValueError(f"{name}.codes must be 2-D")
        _check_quantized(b.codes, b.scales, b.rows, b.k, dev, name)
        _check_alpha(b.alpha_rows, b.rows, dev, name + ".alpha_rows")
    else:
        _check_tensor(b, dev, name)


def _check_outputs(y_f32, y_bf16, m: int, n: int, dev):
    outs = [(y, dtype, name) for y, dtype, name in
            ((y_f32, torch.float32, "y_f32"), (y_bf16, torch.bfloat16, "y_bf16")) if y is not None]
    for y, dtype, name in outs:
        if y.dtype != dtype or y.dim() != 2 or tuple(y.shape) != (m, n) or y.stride(1) != 1:
            raise ValueError(f"{name} must be a {dtype} [{m}, {n}] tensor with unit column stride")
    # one leading dimension is passed for both
    if len(outs) == 2 and y_f32.stride(0) != y_bf16.stride(0):
        raise ValueError("y_f32 and y_bf16 must share one row stride")
    for y, _, name in outs:
        _check_device(y, dev, name)


def nvfp4_quantize_act(x: torch.Tensor, alpha_in: torch.Tensor | None = None,
                       out: NVFP4Tensor | None = None,
                       workspace: torch.Tensor | None = None) -> NVFP4Tensor:
    """Quantise a BF16 activation [M, K] (alpha from the tensor unless given)."""
    _check_bf16_2d(x, "x")
    m, k = x.shape
    dev = x.device
    if out is None:
        out = NVFP4Tensor(torch.empty(1, dtype=torch.float32, device=dev),
                          torch.empty(m, k // 16, dtype=torch.uint8, device=dev),
                          torch.empty(m, k // 2, dtype=torch.uint8, device=dev))
    _check_quantized(out.codes, out.scales, m, k, dev, "out")
    _check_alpha(out.alpha, 1, dev, "out.alpha")
    if alpha_in is not None:
        _check_alpha(alpha_in, 1, dev, "alpha_in")
    ws = workspace if workspace is not None else new_workspace(dev)
    _call("nvfp4_quantize_act", _ptr(x), m, k, x.stride(0), _ptr(alpha_in), _ptr(out.alpha),
          _ptr(out.codes), _ptr(out.scales), _ptr(ws), ws.numel(), _stream(dev))
    return out


def nvfp4_quantize_act_noalloc(x: torch.Tensor, alpha_in: torch.Tensor | None = None,
                               out: NVFP4Tensor | None = None) -> NVFP4Tensor:
    """nvfp4_quantize_act with the library's own per-device scratch instead of a
    workspace (the library allocates nothing; calls on one device must not
    overlap in time)."""
    _check_bf16_2d(x, "x")
    m, k = x.shape
    dev = x.device
    if out is None:
        out = NVFP4Tensor(torch.empty(1, dtype=torch.float32, device=dev),
                          torch.empty(m, k // 16, dtype=torch.uint8, device=dev),
                          torch.empty(m, k // 2, dtype=torch.uint8, device=dev))
    _check_quantized(out.codes, out.scales, m, k, dev, "out")
    _check_alpha(out.alpha, 1, dev, "out.alpha")
    if alpha_in is not None:
        _check_alpha(alpha_in, 1, dev, "alpha_in")
    _call("nvfp4_quantize_act_noalloc", _ptr(x), m, k, x.stride(0), _ptr(alpha_in),
          _ptr(out.alpha), _ptr(out.codes), _ptr(out.scales), _stream(dev))
    return out


def nvfp4_rmsnorm_quantize_act(x: torch.Tensor, gamma: torch.Tensor, eps: float,
                               alpha_in: torch.Tensor | None = None,
                               out: NVFP4Tensor | None = None, y_out: torch.Tensor | None = None,
                               workspace: torch.Tensor | None = None) -> NVFP4Tensor:
    """RMSNorm of a BF16 activation [M, K] with weights gamma [K], produced
    directly as NVFP4 (alpha from the normalised tensor unless given); y_out
    (BF16 [M, K] view) also receives the normalised values when given.
    Without a workspace one of rmsnorm_workspace(M) is made; a smaller one
    (at least new_workspace's) selects the pass that sums each row again."""
    _check_bf16_2d(x, "x")
    m, k = x.shape
    if gamma.dtype != torch.bfloat16 or gamma.shape != (k,) or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous bfloat16 vector of length K")
    if y_out is not None:
        _check_bf16_2d(y_out, "y_out")
        if tuple(y_out.shape) != (m, k):
            raise ValueError("y_out must be [M, K]")
    dev = x.device
    _check_device(gamma, dev, "gamma")
    if y_out is not None:
        _check_device(y_out, dev, "y_out")
    if out is None:
        out = NVFP4Tensor(torch.empty(1, dtype=torch.float32, device=dev),
                          torch.empty(m, k // 16, dtype=torch.uint8, device=dev),
                          torch.empty(m, k // 2, dtype=torch.uint8, device=dev))
    _check_quantized(out.codes, out.scales, m, k, dev, "out")
    _check_alpha(out.alpha, 1, dev, "out.alpha")
    if alpha_in is not None:
        _check_alpha(alpha_in, 1, dev, "alpha_in")
    ws = workspace if workspace is not None else rmsnorm_workspace(m, dev)
    _call("nvfp4_rmsnorm_quantize_act", _ptr(x), _ptr(gamma), m, k, x.stride(0),
          ctypes.c_float(eps), _ptr(alpha_in), _ptr(out.alpha), _ptr(out.codes),
          _ptr(out.scales), _ptr(y_out), y_out.stride(0) if y_out is not None else 0,
          _ptr(ws), ws.numel(), _stream(dev))
    return out


def nvfp4_quantize_weights(w: torch.Tensor, layout: str = "nk",
                           workspace: torch.Tensor | None = None) -> NVFP4Tensor:
    """Quantise a BF16 weight: layout "nk" for [N, K], "kn" for [K, N]."""
    if w.dtype != torch.bfloat16 or w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous 2-D bfloat16 tensor")
    if layout == "nk":
        n, k = w.shape
        sn, sk = k, 1
    elif layout == "kn":
        k, n = w.shape
        sn, sk = 1, n
    else:
        raise ValueError("layout must be 'nk' or 'kn'")
    dev = w.device
    out = NVFP4Tensor(torch.empty(1, dtype=torch.float32, device=dev),
                      torch.empty(n, k // 16, dtype=torch.uint8, device=dev),
                      torch.empty(n, k // 2, dtype=torch.uint8, device=dev))
    ws = workspace if workspace is not None else new_workspace(dev)
    _call("nvfp4_quantize_weights", _ptr(w), n, k, sn, sk, _ptr(out.alpha), _ptr(out.codes),
          _ptr(out.scales), _ptr(ws), ws.numel(), _stream(dev))
    return out


def nvfp4_tensor_alpha(x: torch.Tensor, workspace: torch.Tensor | None = None) -> torch.Tensor:
    _check_bf16_2d(x, "x")
    alpha = torch.empty(1, dtype=torch.float32, device=x.device)
    ws = workspace if workspace is not None else new_workspace(x.device)
    _call("nvfp4_tensor_alpha", _ptr(x), x.shape[0], x.shape[1], x.stride(0), _ptr(alpha),
          _ptr(ws), ws.numel(), _stream(x.device))
    return alpha


def _outputs(m, n, dev, want_f32, want_bf16, y_f32, y_bf16):
    if want_f32 and y_f32 is None:
        y_f32 = torch.empty(m, n, dtype=torch.float32, device=dev)
    if want_bf16 and y_bf16 is None:
        y_bf16 = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    return y_f32, y_bf16


def w4a4_gemm(a: NVFP4Tensor, b: NVFP4Tensor, f32: bool = True, bf16: bool = True,
              y_f32: torch.Tensor | None = None, y_bf16: torch.Tensor | None = None):
    """Y = (alpha_a alpha_b) sum (sigma q)_a (sigma q)_b -> (y_f32, y_bf16)."""
    m, k = a.rows, a.k
    n = b.rows
    if b.k != k:
        raise ValueError("operands disagree on K")
    dev = a.codes.device
    _check_tensor(a, dev, "a")
    _check_tensor(b, dev, "b")
    y_f32, y_bf16 = _outputs(m, n, dev, f32, bf16, y_f32, y_bf16)
    _check_outputs(y_f32, y_bf16, m, n, dev)
    ld = (y_f32 if y_f32 is not None else y_bf16).stride(0)
    _call("w4a4_gemm", _ptr(a.codes), _ptr(a.scales), _ptr(a.alpha), _ptr(b.codes),
          _ptr(b.scales), _ptr(b.alpha), m, n, k, _ptr(y_f32), _ptr(y_bf16), ld,
          _stream(a.codes.device))
    return y_f32, y_bf16


@dataclass
class NVFP4Stack:
    """Several NVFP4 tensors of the same K stacked along rows (e.g. Q, K, V
    weights): codes [N, K/2], scales [N, K/16], alpha_rows [N] (float32)."""
    codes: torch.Tensor
    scales: torch.Tensor
    alpha_rows: torch.Tensor
    offsets: list

    @property
    def rows(self) -> int:
        return self.codes.shape[0]

    @property
    def k(self) -> int:
        return self.codes.shape[1] * 2


def stack_tensors(parts) -> NVFP4Stack:
    """Concatenate quantised tensors along rows, each keeping its own alpha."""
    codes = torch.cat([t.codes for t in parts], dim=0)
    scales = torch.cat([t.scales for t in parts], dim=0)
    alpha_rows = torch.cat([t.alpha.expand(t.rows) for t in parts]).contiguous()
    offsets = [0]
    for t in parts:
        offsets.append(offsets[-1] + t.rows)
    return NVFP4Stack(codes, scales, alpha_rows, offsets)


def w4a4_gemm_multi(a: NVFP4Tensor, b: NVFP4Stack, f32: bool = True, bf16: bool = True,
                    y_f32: torch.Tensor | None = None, y_bf16: torch.Tensor | None = None):
    """W4A4 GEMM against stacked weights; column n is scaled by b.alpha_rows[n]."""
    m, k = a.rows, a.k
    n = b.rows
    if b.k != k:
        raise ValueError("operands disagree on K")
    if not isinstance(b, NVFP4Stack):
        raise ValueError("b must be an NVFP4Stack")
    dev = a.codes.device
    _check_tensor(a, dev, "a")
    _check_weight(b, dev, "b")
    y_f32, y_bf16 = _outputs(m, n, dev, f32, bf16, y_f32, y_bf16)
    _check_outputs(y_f32, y_bf16, m, n, dev)
    ld = (y_f32 if y_f32 is not None else y_bf16).stride(0)
    _call("w4a4_gemm_multi", _ptr(a.codes), _ptr(a.scales), _ptr(a.alpha), _ptr(b.codes),
          _ptr(b.scales), _ptr(b.alpha_rows), m, n, k, _ptr(y_f32), _ptr(y_bf16), ld,
          _stream(a.codes.device))
    return y_f32, y_bf16


def interleave_gate_up(gate: NVFP4Tensor, up: NVFP4Tensor) -> NVFP4Stack:
    """The gate and up weights (each [hidden, K], hidden a multiple of 32) as
    one B operand for w4a4_gemm_silu_mul_quantize: 32-row blocks alternate,
    gate rows 32j..32j+31 then up rows 32j..32j+31, with each row's tensor
    scale in alpha_rows.  A row permutation of the quantised weights (offline
    layout, no arithmetic)."""
    hidden = gate.rows
    if up.rows != hidden or up.k != gate.k or hidden % 32 != 0:
        raise ValueError("gate and up must have the same shape, rows a multiple of 32")
    nb = hidden // 32

    def mix(a, b):
        return torch.stack([a.view(nb, 32, -1), b.view(nb, 32, -1)], dim=1).reshape(2 * hidden, -1)

    dev = gate.codes.device
    ar = torch.stack([gate.alpha.expand(hidden).reshape(nb, 32),
                      up.alpha.expand(hidden).reshape(nb, 32)], dim=1).reshape(2 * hidden)
    return NVFP4Stack(mix(gate.codes, up.codes).contiguous(),
                      mix(gate.scales, up.scales).contiguous(),
                      ar.to(torch.float32).contiguous().to(dev), [0, 2 * hidden])


def silu_mul_workspace(m: int, n: int, device) -> torch.Tensor:
    return torch.empty(int(lib().w4a4_gemm_silu_mul_workspace_bytes(m, n)), dtype=torch.uint8,
                       device=device)


def w4a4_gemm_silu_mul_quantize(a: NVFP4Tensor, b: NVFP4Stack, h: torch.Tensor | None = None,
                                out: NVFP4Tensor | None = None,
                                workspace: torch.Tensor | None = None):
    """H = SiLU(gate) * up of the interleaved gate|up weight b, produced by
    the GEMM's epilogue, and H quantised to NVFP4 -> (NVFP4Tensor, H)."""
    m, k = a.rows, a.k
    n = b.rows
    if b.k != k:
        raise ValueError("operands disagree on K")
    if not isinstance(b, NVFP4Stack):
        raise ValueError("b must be the NVFP4Stack of interleave_gate_up")
    dev = a.codes.device
    _check_tensor(a, dev, "a")
    _check_weight(b, dev, "b")
    nh = n // 2
    if h is None:
        h = torch.empty(m, nh, dtype=torch.bfloat16, device=dev)
    _check_bf16_2d(h, "h")
    _check_device(h, dev, "h")
    if tuple(h.shape) != (m, nh):
        raise ValueError(f"h must be [{m}, {nh}]")
    if out is None:
        out = NVFP4Tensor(torch.empty(1, dtype=torch.float32, device=dev),
                          torch.empty(m, nh // 16, dtype=torch.uint8, device=dev),
                          torch.empty(m, nh // 2, dtype=torch.uint8, device=dev))
    _check_quantized(out.codes, out.scales, m, nh, dev, "out")
    _check_alpha(out.alpha, 1, dev, "out.alpha")
    ws = workspace if workspace is not None else silu_mul_workspace(m, n, dev)
    _call("w4a4_gemm_silu_mul_quantize", _ptr(a.codes), _ptr(a.scales), _ptr(a.alpha),
          _ptr(b.codes), _ptr(b.scales), _ptr(b.alpha_rows), m, n, k, _ptr(h), h.stride(0),
          _ptr(out.alpha), _ptr(out.codes), _ptr(out.scales), _ptr(ws), ws.numel(), _stream(dev))
    return out, h


DECODE_MAX_ROWS = 64


def w4a4_gemm_decode(a: NVFP4Tensor, b, f32: bool = True, bf16: bool = True,
                     y_f32: torch.Tensor | None = None, y_bf16: torch.Tensor | None = None):
    """Decode-shaped W4A4 GEMM (a.rows <= DECODE_MAX_ROWS) against an
    NVFP4Tensor weight or an NVFP4Stack (per-row tensor scales)."""
    m, k = a.rows, a.k
    n = b.rows
    if b.k != k:
        raise ValueError("operands disagree on K")
    dev = a.codes.device
    _check_tensor(a, dev, "a")
    _check_weight(b, dev, "b")
    y_f32, y_bf16 = _outputs(m, n, dev, f32, bf16, y_f32, y_bf16)
    _check_outputs(y_f32, y_bf16, m, n, dev)
    ld = (y_f32 if y_f32 is not None else y_bf16).stride(0)
    stacked = isinstance(b, NVFP4Stack)
    _call("w4a4_gemm_decode", _ptr(a.codes), _ptr(a.scales), _ptr(a.alpha), _ptr(b.codes),
          _ptr(b.scales), None if stacked else _ptr(b.alpha),
          _ptr(b.alpha_rows) if stacked else None, m, n, k, _ptr(y_f32), _ptr(y_bf16), ld,
          _stream(a.codes.device))
    return y_f32, y_bf16


def w4a4_gemm_grouped(a: NVFP4Tensor, b_codes: torch.Tensor, b_scales: torch.Tensor,
                      b_alpha: torch.Tensor, group_offsets: torch.Tensor,
                      a_row_index: torch.Tensor | None = None, m: int | None = None,
                      f32: bool = True, bf16: bool = True,
                      y_f32: torch.Tensor | None = None, y_bf16: torch.Tensor | None = None):
    """Grouped (MoE) GEMM: b_* are [G, N, K/2], [G, N, K/16], [G] tensors."""
    if b_codes.dim() != 3:
        raise ValueError("b_codes must be [G, N, K/2]")
    g, n, kc = b_codes.shape
    k = kc * 2
    if k != a.k:
        raise ValueError("operands disagree on K")
    dev = a.codes.device
    _check_tensor(a, dev, "a")
    _check_dense(b_codes, torch.uint8, (g, n, k // 2), "b_codes")
    _check_dense(b_scales, torch.uint8, (g, n, k // 16), "b_scales")
    _check_device(b_codes, dev, "b_codes")
    _check_device(b_scales, dev, "b_scales")
    _check_alpha(b_alpha, g, dev, "b_alpha")
    _check_dense(group_offsets, torch.int64, (g + 1,), "group_offsets")
    _check_device(group_offsets, dev, "group_offsets")
    if m is None:
        m = a_row_index.numel() if a_row_index is not None else a.rows
    if a_row_index is not None:
        _check_dense(a_row_index, torch.int32, (m,), "a_row_index")
        _check_device(a_row_index, dev, "a_row_index")
    y_f32, y_bf16 = _outputs(m, n, dev, f32, bf16, y_f32, y_bf16)
    _check_outputs(y_f32, y_bf16, m, n, dev)
    ld = (y_f32 if y_f32 is not None else y_bf16).stride(0)
    _call("w4a4_gemm_grouped", _ptr(a.codes), _ptr(a.scales), _ptr(a.alpha), a.rows,
          _ptr(a_row_index), _ptr(b_codes), _ptr(b_scales), _ptr(b_alpha), m, n, k, g,
          _ptr(group_offsets), _ptr(y_f32), _ptr(y_bf16), ld, _stream(a.codes.device))
    return y_f32, y_bf16


def w4a4_gemm_fused_act(x: torch.Tensor, alpha_a: torch.Tensor, b: NVFP4Tensor,
                        f32: bool = True, bf16: bool = True,
                        workspace: torch.Tensor | None = None,
                        y_f32: torch.Tensor | None = None,
                        y_bf16: torch.Tensor | None = None):
    """Quantise-on-load GEMM: BF16 activation x [M, K] under alpha_a."""
    _check_bf16_2d(x, "x")
    m, k = x.shape
    n = b.rows
    if b.k != k:
        raise ValueError("operands disagree on K")
    dev = x.device
    _check_alpha(alpha_a, 1, dev, "alpha_a")
    _check_tensor(b, dev, "b")
    y_f32, y_bf16 = _outputs(m, n, dev, f32, bf16, y_f32, y_bf16)
    _check_outputs(y_f32, y_bf16, m, n, dev)
    ld = (y_f32 if y_f32 is not None else y_bf16).stride(0)
    ws = workspace if workspace is not None else new_workspace(x.device)
    _call("w4a4_gemm_fused_act", _ptr(x), x.stride(0), _ptr(alpha_a), _ptr(b.codes),
          _ptr(b.scales), _ptr(b.alpha), m, n, k, _ptr(y_f32), _ptr(y_bf16), ld, _ptr(ws),
          ws.numel(), _stream(x.device))
    return y_f32, y_bf16


def bf16_gemm_baseline(x: torch.Tensor, w: torch.Tensor,
                       group_offsets: torch.Tensor | None = None,
                       f32: bool = True, bf16: bool = True):
    """BF16 comparison GEMM: Y = X W^T (w [N, K] or [G, N, K] with offsets)."""
    if x.dim() == 2 and x.shape[0] > 1 and x.stride(0) != x.shape[1]:
        raise ValueError("x must be row-contiguous (the BF16 GEMM takes no row stride)")
    _check_bf16_2d(x, "x")
    m, k = x.shape
    if w.dim() not in (2, 3):
        raise ValueError("w must be [N, K] or [G, N, K]")
    g = 1 if w.dim() == 2 else w.shape[0]
    n = w.shape[-2]
    _check_dense(w, torch.bfloat16, (n, k) if w.dim() == 2 else (g, n, k), "w")
    _check_device(w, x.device, "w")
    if group_offsets is not None:
        _check_dense(group_offsets, torch.int64, (g + 1,), "group_offsets")
        _check_device(group_offsets, x.device, "group_offsets")
    y_f32, y_bf16 = _outputs(m, n, x.device, f32, bf16, None, None)
    ld = (y_f32 if y_f32 is not None else y_bf16).stride(0)
    _call("bf16_gemm_baseline", _ptr(x), _ptr(w), m, n, k, g, _ptr(group_offsets),
          _ptr(y_f32), _ptr(y_bf16), ld, _stream(x.device))
    return y_f32, y_bf16


def to_device_bf16(bits, device) -> torch.Tensor:
    """uint16 BF16 bit patterns (numpy) -> bfloat16 tensor on device."""
    import numpy as np
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)
