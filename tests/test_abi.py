"""The C-ABI library: it loads, exports every function include/*.h declares,
and rejects bad arguments before launching anything.

These tests make no compute calls.  Calls with otherwise valid arguments run
under the NVFP4_PATH_REJECT_DEVICE path flag, so the library stops at the
device check (NVFP4_ERR_UNSUPPORTED) on any machine, GPU or not.
"""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "nvfp4_w4a4_gemm_amd", "libnvfp4_w4a4.so")

OK, NULL, SHAPE, ALIGN, UNSUPPORTED, LAUNCH, WORKSPACE = range(7)

needs_lib = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")


def header_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, re.M):
            names.add(m.group(1))
    return names


def test_header_declares_the_four_entry_points():
    names = header_functions()
    for n in ("nvfp4_quantize_weights", "nvfp4_quantize_act", "w4a4_gemm", "bf16_gemm_baseline",
              "w4a4_gemm_multi", "w4a4_gemm_grouped", "w4a4_gemm_fused_act",
              "w4a4_gemm_decode", "nvfp4_rmsnorm_quantize_act", "w4a4_gemm_silu_mul_quantize",
              "w4a4_gemm_silu_mul_workspace_bytes", "nvfp4_rmsnorm_workspace_bytes"):
        assert n in names


@needs_lib
def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(LIB)
    for n in header_functions():
        assert hasattr(lib, n), n


@needs_lib
def test_binding_signatures_cover_the_header():
    from nvfp4_w4a4_gemm_amd import binding
    assert set(binding.EXPORTS) == header_functions()


@pytest.fixture
def lib():
    from nvfp4_w4a4_gemm_amd import binding
    with binding.path_flags(binding.PATH_REJECT_DEVICE):
        yield binding.lib()


FAKE = 0x10000          # 64 KiB-aligned fake device address (never dereferenced)
WS = 1 << 16


def p(off=0):
    return ctypes.c_void_p(FAKE + off)


@needs_lib
def test_status_strings(lib):
    for s in range(7):
        assert lib.nvfp4_status_string(s)
    assert lib.nvfp4_workspace_bytes() > 0


@needs_lib
def test_quantize_act_validation(lib):
    f = lib.nvfp4_quantize_act
    # x, M, K, ld, alpha_in, alpha_out, codes, scales, ws, ws_bytes, stream
    assert f(p(), 4, 32, 32, None, p(), p(), p(), p(), WS, None) == UNSUPPORTED
    assert f(p(), 4, 33, 33, None, p(), p(), p(), p(), WS, None) == SHAPE   # K % 16
    assert f(p(), 4, 0, 32, None, p(), p(), p(), p(), WS, None) == SHAPE    # K = 0
    assert f(p(), -1, 32, 32, None, p(), p(), p(), p(), WS, None) == SHAPE  # M < 0
    assert f(p(), 4, 32, 16, None, p(), p(), p(), p(), WS, None) == SHAPE   # ld < K
    assert f(None, 4, 32, 32, None, p(), p(), p(), p(), WS, None) == NULL
    assert f(p(), 4, 32, 32, None, None, p(), p(), p(), WS, None) == NULL   # alpha_out
    assert f(p(), 4, 32, 32, None, p(), None, p(), p(), WS, None) == NULL
    assert f(p(2), 4, 32, 32, None, p(), p(), p(), p(), WS, None) == ALIGN  # x
    assert f(p(), 4, 32, 36, None, p(), p(), p(), p(), WS, None) == ALIGN   # ld * 2
    assert f(p(), 4, 32, 32, None, p(), p(4), p(), p(), WS, None) == ALIGN  # codes
    assert f(p(), 4, 32, 32, None, p(), p(), p(), None, WS, None) == WORKSPACE
    assert f(p(), 4, 32, 32, None, p(), p(), p(), p(), 64, None) == WORKSPACE


@needs_lib
def test_quantize_act_noalloc_validation(lib):
    f = lib.nvfp4_quantize_act_noalloc
    # x, M, K, ld, alpha_in, alpha_out, codes, scales, stream (no workspace)
    assert f(p(), 4, 32, 32, None, p(), p(), p(), None) == UNSUPPORTED
    assert f(p(), 4, 33, 33, None, p(), p(), p(), None) == SHAPE     # K % 16
    assert f(p(), -1, 32, 32, None, p(), p(), p(), None) == SHAPE    # M < 0
    assert f(p(), 4, 32, 16, None, p(), p(), p(), None) == SHAPE     # ld < K
    assert f(p(), 1 << 27, 1 << 8, 1 << 8, None, p(), p(), p(), None) == SHAPE  # blocks
    assert f(None, 4, 32, 32, None, p(), p(), p(), None) == NULL
    assert f(p(), 4, 32, 32, None, None, p(), p(), None) == NULL     # alpha_out
    assert f(p(2), 4, 32, 32, None, p(), p(), p(), None) == ALIGN    # x
    assert f(p(), 4, 32, 32, None, p(), p(4), p(), None) == ALIGN    # codes


@needs_lib
def test_fused_gemm_rejects_weights_beyond_32_bit_offsets(lib):
    f = lib.w4a4_gemm_fused_act
    # x, ld_x, alpha_a, b_codes, b_scales, alpha_b, M, N, K, y32, y16, ld_y, ws, ws_bytes, stream
    ok = [p(), 256, p(), p(), p(), p(), 16, 64, 256, None, p(), 1 << 20, p(), WS, None]
    assert f(*ok) == UNSUPPORTED
    big = list(ok); big[7] = 1 << 20; big[8] = 1 << 13       # N * K / 2 = 2^32 bytes
    big[1] = 1 << 13
    assert f(*big) == SHAPE


@needs_lib
def test_quantize_weights_validation(lib):
    f = lib.nvfp4_quantize_weights
    # w, N, K, stride_n, stride_k, alpha_out, codes, scales, ws, ws_bytes, stream
    assert f(p(), 8, 32, 32, 1, p(), p(), p(), p(), WS, None) == UNSUPPORTED
    assert f(p(), 8, 32, 1, 8, p(), p(), p(), p(), WS, None) == UNSUPPORTED   # K x N source
    assert f(p(), 8, 32, 2, 2, p(), p(), p(), p(), WS, None) == SHAPE         # neither unit
    assert f(p(), 8, 40, 40, 1, p(), p(), p(), p(), WS, None) == SHAPE


@needs_lib
def test_gemm_validation(lib):
    f = lib.w4a4_gemm
    # a_codes, a_scales, alpha_a, b_codes, b_scales, alpha_b, M, N, K, y32, y16, ld, stream
    args = [p(), p(), p(), p(), p(), p(), 64, 64, 256, p(), p(), 64, None]
    assert f(*args) == UNSUPPORTED
    bad = list(args); bad[8] = 40
    assert f(*bad) == SHAPE
    bad = list(args); bad[6] = -1
    assert f(*bad) == SHAPE
    bad = list(args); bad[9] = None; bad[10] = None
    assert f(*bad) == NULL
    bad = list(args); bad[11] = 32                           # ld_y < N
    assert f(*bad) == SHAPE
    bad = list(args); bad[0] = p(8)
    assert f(*bad) == ALIGN
    bad = list(args); bad[9] = p(2)                           # float output
    assert f(*bad) == ALIGN
    bad = list(args); bad[2] = None
    assert f(*bad) == NULL
    zero = list(args); zero[6] = 0                            # M = 0: nothing to do
    assert f(*zero) == OK


@needs_lib
def test_gemm_multi_validation(lib):
    f = lib.w4a4_gemm_multi
    # a_codes, a_scales, alpha_a, b_codes, b_scales, alpha_b_rows, M, N, K, y32, y16, ld, stream
    args = [p(), p(), p(), p(), p(), p(), 64, 96, 256, p(), p(), 96, None]
    assert f(*args) == UNSUPPORTED
    bad = list(args); bad[5] = None                           # per-row scales required
    assert f(*bad) == NULL
    bad = list(args); bad[8] = 24
    assert f(*bad) == SHAPE
    bad = list(args); bad[3] = p(4)
    assert f(*bad) == ALIGN


@needs_lib
def test_rmsnorm_quantize_validation(lib):
    f = lib.nvfp4_rmsnorm_quantize_act
    # x, gamma, M, K, ld_x, eps, alpha_in, alpha_out, codes, scales, y, ld_y, ws, ws_bytes, stream
    args = [p(), p(), 64, 4096, 4096, 1e-6, None, p(), p(), p(), None, 0, p(), WS, None]
    assert f(*args) == UNSUPPORTED
    with_y = list(args); with_y[10] = p(); with_y[11] = 4096
    assert f(*with_y) == UNSUPPORTED
    bad = list(args); bad[1] = None                           # gamma required
    assert f(*bad) == NULL
    bad = list(args); bad[3] = 8192 + 16                      # row beyond the register budget
    assert f(*bad) == SHAPE
    bad = list(args); bad[3] = 40
    assert f(*bad) == SHAPE
    bad = list(args); bad[5] = -1.0                           # eps must be >= 0
    assert f(*bad) == SHAPE
    bad = list(args); bad[5] = float("nan")
    assert f(*bad) == SHAPE
    bad = list(args); bad[1] = p(8)                           # gamma 16-byte aligned
    assert f(*bad) == ALIGN
    bad = list(with_y); bad[11] = 4000                        # ld_y < K
    assert f(*bad) == SHAPE
    bad = list(with_y); bad[10] = p(2)
    assert f(*bad) == ALIGN
    bad = list(args); bad[13] = 100
    assert f(*bad) == WORKSPACE
    zero = list(args); zero[2] = 0                            # M = 0: alpha of nothing
    assert f(*zero) == UNSUPPORTED


@needs_lib
def test_gemm_decode_validation(lib):
    f = lib.w4a4_gemm_decode
    # a_codes, a_scales, alpha_a, b_codes, b_scales, alpha_b, alpha_b_rows, M, N, K,
    # y32, y16, ld, stream
    args = [p(), p(), p(), p(), p(), p(), None, 16, 96, 256, p(), p(), 96, None]
    assert f(*args) == UNSUPPORTED
    rows = list(args); rows[5] = None; rows[6] = p()          # per-row scales instead
    assert f(*rows) == UNSUPPORTED
    bad = list(args); bad[5] = None                           # neither tensor scale
    assert f(*bad) == NULL
    bad = list(args); bad[7] = 65                             # more rows than decode takes
    assert f(*bad) == SHAPE
    ok64 = list(args); ok64[7] = 64
    assert f(*ok64) == UNSUPPORTED
    bad = list(args); bad[9] = 40
    assert f(*bad) == SHAPE
    bad = list(args); bad[4] = p(1)                           # scale pairs are 2-byte loads
    assert f(*bad) == ALIGN
    odd = list(args); odd[9] = 272; odd[4] = p(1)             # K % 32 != 0: byte loads
    assert f(*odd) == UNSUPPORTED
    bad = list(args); bad[3] = p(8)
    assert f(*bad) == ALIGN
    bad = list(args); bad[8] = 1 << 22; bad[9] = 1 << 11; bad[12] = 1 << 22  # > 4 GiB of B
    assert f(*bad) == SHAPE
    zero = list(args); zero[7] = 0
    assert f(*zero) == OK


@needs_lib
def test_rmsnorm_workspace_bytes(lib):
    """One float a row after the quantiser's workspace (256-byte aligned
    start), so the r of a row fits; nothing for a negative M."""
    base = lib.nvfp4_workspace_bytes()
    for m in (0, 1, 8192, 16384):
        need = lib.nvfp4_rmsnorm_workspace_bytes(m)
        assert need >= base + 4 * m and (need - 4 * m) % 256 == 0
        assert need - 4 * m - base < 512
    assert lib.nvfp4_rmsnorm_workspace_bytes(-1) == 0


@needs_lib
def test_gemm_silu_mul_validation(lib):
    f = lib.w4a4_gemm_silu_mul_quantize
    ws_need = lib.w4a4_gemm_silu_mul_workspace_bytes(300, 640)
    assert ws_need == lib.nvfp4_workspace_bytes() + 4 * 3 * 5    # 128 x 128 tiles at most
    assert lib.w4a4_gemm_silu_mul_workspace_bytes(-1, 64) == 0
    # a_codes, a_scales, alpha_a, b_codes, b_scales, alpha_b_rows, M, N, K, h, ld_h,
    # alpha_h, h_codes, h_scales, ws, ws_bytes, stream
    args = [p(), p(), p(), p(), p(), p(), 300, 640, 512, p(), 320, p(), p(), p(), p(),
            ws_need, None]
    assert f(*args) == UNSUPPORTED
    bad = list(args); bad[7] = 608                            # N = 2 x hidden, 32-unit blocks
    assert f(*bad) == SHAPE
    bad = list(args); bad[8] = 40
    assert f(*bad) == SHAPE
    bad = list(args); bad[10] = 312                           # ld_h < N / 2
    assert f(*bad) == SHAPE
    bad = list(args); bad[10] = 324                           # 16-byte rows of H
    assert f(*bad) == ALIGN
    bad = list(args); bad[9] = p(2)
    assert f(*bad) == ALIGN
    bad = list(args); bad[5] = None                           # per-row tensor scales required
    assert f(*bad) == NULL
    bad = list(args); bad[11] = None
    assert f(*bad) == NULL
    bad = list(args); bad[15] = ws_need - 4
    assert f(*bad) == WORKSPACE
    bad = list(args); bad[14] = p(8)
    assert f(*bad) == ALIGN
    zero = list(args); zero[6] = 0                            # M = 0: alpha of nothing
    assert f(*zero) == UNSUPPORTED


@needs_lib
def test_grouped_and_fused_and_bf16_validation(lib):
    g = lib.w4a4_gemm_grouped
    # a_codes, a_scales, alpha_a, a_rows, a_row_index, b_codes, b_scales, alpha_b,
    # M, N, K, groups, offsets, y32, y16, ld, stream
    args = [p(), p(), p(), 100, None, p(), p(), p(), 100, 64, 128, 4, p(), p(), None, 64, None]
    assert g(*args) == UNSUPPORTED
    bad = list(args); bad[12] = None
    assert g(*bad) == NULL
    bad = list(args); bad[11] = 0
    assert g(*bad) == SHAPE
    bad = list(args); bad[3] = 10                             # fewer A rows than M
    assert g(*bad) == SHAPE
    fu = lib.w4a4_gemm_fused_act
    # x, ld_x, alpha_a, b_codes, b_scales, alpha_b, M, N, K, y32, y16, ld, ws, ws_bytes, st
    fargs = [p(), 128, p(), p(), p(), p(), 32, 64, 128, p(), None, 64, p(), WS, None]
    assert fu(*fargs) == UNSUPPORTED
    bad = list(fargs); bad[12] = None
    assert fu(*bad) == WORKSPACE
    bad = list(fargs); bad[1] = 100
    assert fu(*bad) == SHAPE
    b = lib.bf16_gemm_baseline
    # x, w, M, N, K, groups, offsets, y32, y16, ld, stream
    bargs = [p(), p(), 32, 64, 128, 1, None, p(), None, 64, None]
    assert b(*bargs) == UNSUPPORTED
    bad = list(bargs); bad[5] = 2
    assert b(*bad) == NULL
    bad = list(bargs); bad[4] = 24
    assert b(*bad) == SHAPE
    bad = list(bargs); bad[1] = p(2)
    assert b(*bad) == ALIGN
