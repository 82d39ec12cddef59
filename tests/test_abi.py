"""The C-ABI library: it loads, exports every symbol the header declares, and
its host-side argument validation returns the documented status codes before
anything is enqueued (CPU only: no call here reaches the GPU)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")
LIB = os.path.join(ROOT, "mixture_experts_routed_router_amd", "libmoe_mi355x.so")
DEBUG_LIB = os.path.join(ROOT, "mixture_experts_routed_router_amd", "libmoe_mi355x_debug.so")

OK, NULLP, SHAPE, ALIGN, OVERFLOW, MISALIGNED, WORKSPACE, HIP, VALUE, PRECONDITION = range(10)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from mixture_experts_routed_router_amd.build import build
        build()
    lib = ctypes.CDLL(LIB)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_last_error_message.restype = ctypes.c_char_p
    lib.moe_padded_rows_max.argtypes = [i64, i32, i32, i32]
    lib.moe_padded_rows_max.restype = i64
    lib.moe_permute_workspace_size.argtypes = [i64, i32, i32, ctypes.POINTER(sz)]
    lib.moe_route_topk.argtypes = [vp, i64, i32, i32, vp, vp, vp]
    lib.moe_permute.argtypes = [vp, vp, i64, i32, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_grouped_glu_gemm.argtypes = [vp, vp, vp, vp, i32, i32, i32, i64, vp, vp]
    lib.moe_grouped_down_gemm.argtypes = [vp, vp, vp, vp, i32, i32, i32, i64, vp, vp]
    lib.moe_grouped_glu_gemm_gather.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, i64, vp, vp]
    lib.moe_combine.argtypes = [vp, vp, vp, i64, i32, i32, i64, vp, vp]
    lib.moe_quantize_fp8.argtypes = [vp, i64, i32, i32, vp, vp, vp]
    lib.moe_grouped_glu_gemm_fp8w.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i64, vp, vp]
    lib.moe_grouped_down_gemm_fp8w.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i64, vp, vp]
    lib.moe_grouped_glu_gemm_gather_fp8w.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i64,
                                                     vp, vp]
    lib.moe_grouped_gemm.argtypes = [vp, vp, vp, vp, i32, i32, i32, i64, vp, vp]
    lib.moe_swiglu.argtypes = [vp, vp, i32, i32, i64, vp, vp]
    lib.moe_swiglu_backward.argtypes = [vp, vp, vp, i32, i32, i64, vp, vp]
    lib.moe_grouped_gemm_swiglu_backward.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i64, vp, vp]
    lib.moe_grouped_glu_gemm_clamped.argtypes = [vp, vp, vp, vp, i32, i32, i32, i64, ctypes.c_float, vp, vp]
    lib.moe_transpose_experts.argtypes = [vp, i64, i32, i32, vp, vp]
    lib.moe_combine_backward.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i64, vp, vp, vp]
    lib.moe_route_backward.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp]
    lib.moe_permute_backward.argtypes = [vp, vp, i64, i32, i32, i64, vp, vp]
    lib.moe_grouped_wgrad.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i64, vp, vp]
    lib.moe_router_prepare.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.moe_router_topk.argtypes = [vp, vp, vp, i64, i32, i32, i32, vp, vp, vp, vp]
    lib.moe_tile_rows.argtypes = [vp, i64, i32, vp, vp]
    lib.moe_untile_rows.argtypes = [vp, i64, i32, vp, vp]
    lib.moe_permute_tiled.argtypes = lib.moe_permute.argtypes
    lib.moe_grouped_glu_gemm_tiled.argtypes = lib.moe_grouped_glu_gemm.argtypes
    lib.moe_grouped_down_gemm_tiled.argtypes = lib.moe_grouped_down_gemm.argtypes
    lib.moe_grouped_glu_gemm_gather_tiled.argtypes = lib.moe_grouped_glu_gemm_gather.argtypes
    lib.moe_tile_fp8_rows.argtypes = [vp, i64, i32, vp, vp]
    lib.moe_untile_fp8_rows.argtypes = [vp, i64, i32, vp, vp]
    lib.moe_grouped_glu_gemm_fp8w_tiled.argtypes = lib.moe_grouped_glu_gemm_fp8w.argtypes
    lib.moe_grouped_down_gemm_fp8w_tiled.argtypes = lib.moe_grouped_down_gemm_fp8w.argtypes
    lib.moe_grouped_gemm_tiled.argtypes = lib.moe_grouped_gemm.argtypes
    lib.moe_swiglu_tiled.argtypes = lib.moe_swiglu.argtypes
    lib.moe_swiglu_backward_tiled.argtypes = lib.moe_swiglu_backward.argtypes
    lib.moe_grouped_wgrad_tiled.argtypes = [vp, i32, vp, i32, vp, vp, i32, i32, i32, i64, vp, vp]
    return lib


def test_header_declares_the_five_calls():
    fns = declared_functions()
    for name in ("moe_route_topk", "moe_permute", "moe_grouped_glu_gemm",
                 "moe_grouped_down_gemm", "moe_combine"):
        assert name in fns


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in the header but not exported"


@pytest.fixture(scope="module")
def debug_lib():
    if not os.path.exists(DEBUG_LIB):
        from mixture_experts_routed_router_amd.build import build
        build(debug=True)
    return ctypes.CDLL(DEBUG_LIB)


def test_debug_library_exports_the_same_calls(lib, debug_lib):
    for name in declared_functions():
        assert hasattr(debug_lib, name), f"{name} not exported by the debug library"
    assert debug_lib.moe_debug_build() == 1
    assert lib.moe_debug_build() == 0
    # host validation is the same in both
    assert debug_lib.moe_route_topk(FAKE, 4, 8, 9, FAKE, FAKE, None) == SHAPE
    assert debug_lib.moe_combine(FAKE, FAKE, FAKE, 4, 128, 2, 100, None, None) == NULLP


def test_route_hist_validation(lib):
    n = ctypes.c_size_t(0)
    assert lib.moe_route_hist_workspace_size(8192, 8, 128, ctypes.byref(n)) == OK
    assert n.value >= (8192 // 32) * 128 * 4 and n.value % 256 == 0
    assert lib.moe_route_hist_workspace_size(10, 9, 8, ctypes.byref(n)) == SHAPE      # k > E
    lib.moe_route_topk_hist.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]
    assert lib.moe_route_topk_hist(FAKE, 64, 8, 2, FAKE, FAKE, None, 1 << 20, None) == NULLP
    assert lib.moe_route_topk_hist(FAKE, 64, 8, 2, FAKE, FAKE, FAKE, 4, None) == WORKSPACE
    assert lib.moe_route_topk_hist(None, 0, 8, 2, None, None, None, 0, None) == OK     # no tokens
    lib.moe_permute_from_hist.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64] + \
        [ctypes.c_int32] * 4 + [ctypes.c_int64] + [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p]
    assert lib.moe_permute_from_hist(FAKE, FAKE, 64, 128, 8, 2, 32, 64 * 2 + 8 * 31, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, 4, None) == WORKSPACE
    assert lib.moe_permute_from_hist(FAKE, FAKE, 64, 100, 8, 2, 32, 64 * 2 + 8 * 31, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, FAKE, 1 << 20, None) == SHAPE               # H % 64


def test_fused_layer_validation(lib):
    n = ctypes.c_size_t(0)
    assert lib.moe_fused_layer_workspace_size(8192, 8, 128, ctypes.byref(n)) == OK
    assert n.value >= 256 + (8192 * 8 // 256) * 128 * 4
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.moe_fused_layer.argtypes = [vp] * 5 + [i64] + [i32] * 5 + [i64] + [vp] * 8 + [ctypes.c_size_t, vp]

    def call(T=64, H=128, E=8, k=2, I=128, align=32, ws=1 << 20, x=FAKE, out=FAKE):
        return lib.moe_fused_layer(x, FAKE, FAKE, FAKE, FAKE, T, H, E, k, I, align, T * k + E * (align - 1),
                                   FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, out, FAKE, ws, None)
    assert call(x=None) == NULLP
    assert call(out=None) == NULLP
    assert call(T=0) == SHAPE
    assert call(I=100) == SHAPE
    assert call(k=9) == SHAPE
    assert call(ws=16) == WORKSPACE
    assert call(T=1 << 20, H=4096) == OVERFLOW          # T * H * 2 reaches 2^32 (32-bit gather offsets)
    lib.moe_fused_layer_status.argtypes = [vp, vp]
    assert lib.moe_fused_layer_status(None, None) == NULLP


def test_probe_validation(lib):
    assert lib.moe_probe_copy(None, FAKE, 1024, None) == NULLP
    assert lib.moe_probe_copy(FAKE, FAKE, 1000, None) == SHAPE      # not a multiple of 16
    assert lib.moe_probe_copy(FAKE, FAKE, 0, None) == SHAPE
    fl = ctypes.c_double(0.0)
    lib.moe_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    assert lib.moe_probe_mfma_bf16(None, 1 << 20, 10, ctypes.byref(fl), None) == NULLP
    assert lib.moe_probe_mfma_bf16(FAKE, 1 << 20, 0, ctypes.byref(fl), None) == VALUE
    assert lib.moe_probe_mfma_bf16(FAKE, 1 << 20, 10, None, None) == NULLP
    lib.moe_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_void_p]
    assert lib.moe_probe_read(None, 1024, FAKE, 1 << 30, None) == NULLP
    assert lib.moe_probe_read(FAKE, 1000, FAKE, 1 << 30, None) == SHAPE          # not a multiple of 16
    assert lib.moe_probe_read(FAKE, 1024, FAKE + 4, 1 << 30, None) == MISALIGNED
    assert lib.moe_probe_read(FAKE, 1024, FAKE, 16, None) == WORKSPACE            # sink too small


def test_status_strings(lib):
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(OVERFLOW) == b"MOE_ERR_SIZE_OVERFLOW"
    assert lib.moe_status_string(99) == b"MOE_ERR_UNKNOWN"
    assert lib.moe_status_string(VALUE) == b"MOE_ERR_INVALID_VALUE"
    assert lib.moe_status_string(PRECONDITION) == b"MOE_ERR_PRECONDITION"


def test_padded_rows_and_workspace(lib):
    assert lib.moe_padded_rows_max(8192, 8, 128, 32) == 8192 * 8 + 128 * 31
    assert lib.moe_padded_rows_max(-1, 8, 128, 32) == -1
    n = ctypes.c_size_t(0)
    assert lib.moe_permute_workspace_size(8192, 8, 128, ctypes.byref(n)) == OK
    assert n.value >= (8192 * 8 // 1024) * 128 * 4 and n.value % 256 == 0
    assert lib.moe_permute_workspace_size(10, 3, 2, ctypes.byref(n)) == SHAPE  # k > E
    assert lib.moe_permute_workspace_size(10, 2, 2, None) == NULLP


FAKE = 0x10000  # a 16-byte-aligned non-null address; validation fails before any use


def test_route_topk_validation(lib):
    assert lib.moe_route_topk(None, 4, 8, 2, FAKE, FAKE, None) == NULLP
    assert b"logits" in lib.moe_last_error_message()
    assert lib.moe_route_topk(FAKE + 4, 4, 8, 2, FAKE, FAKE, None) == MISALIGNED
    assert lib.moe_route_topk(FAKE, 4, 8, 9, FAKE, FAKE, None) == SHAPE       # k > E
    assert lib.moe_route_topk(FAKE, 4, 8, 0, FAKE, FAKE, None) == SHAPE
    assert lib.moe_route_topk(FAKE, 4, 2048, 8, FAKE, FAKE, None) == SHAPE    # E > 1024
    assert lib.moe_route_topk(FAKE, 4, 64, 33, FAKE, FAKE, None) == SHAPE     # k > 32
    assert lib.moe_route_topk(FAKE, -1, 8, 2, FAKE, FAKE, None) == SHAPE
    # no tokens: T-sized buffers may be NULL, and nothing is launched
    assert lib.moe_route_topk(None, 0, 8, 2, None, None, None) == OK
    assert lib.moe_route_topk(FAKE + 4, 0, 8, 2, None, None, None) == MISALIGNED


def _permute(lib, T=4, H=128, E=8, k=2, align=32, P_max=None, ws=1 << 20, x=FAKE, x_perm=FAKE):
    if P_max is None:
        P_max = T * k + E * (align - 1)
    return lib.moe_permute(x, FAKE, T, H, E, k, align, P_max, FAKE, FAKE, FAKE, FAKE, x_perm, FAKE,
                           ws, None)


def test_permute_validation(lib):
    assert _permute(lib, x=None) == NULLP
    assert _permute(lib, H=96) == SHAPE
    assert _permute(lib, align=24) == ALIGN
    assert _permute(lib, align=512) == ALIGN
    assert _permute(lib, P_max=4 * 2 + 8 * 31 - 1) == OVERFLOW
    assert _permute(lib, P_max=1 << 31) == OVERFLOW
    assert _permute(lib, ws=0) == WORKSPACE
    assert b"workspace" in lib.moe_last_error_message()
    # x_perm NULL: the layout only, x is not needed (validation goes on to the shape check)
    assert _permute(lib, x=None, x_perm=None, H=96) == SHAPE
    assert _permute(lib, x=FAKE, x_perm=FAKE + 8) == MISALIGNED


def test_gemm_validation(lib):
    for fn in (lib.moe_grouped_glu_gemm, lib.moe_grouped_down_gemm):
        assert fn(FAKE, FAKE, FAKE, FAKE, 8, 128, 256, 1000, None, None) == NULLP
        assert fn(FAKE, FAKE, FAKE, FAKE, 8, 100, 256, 1000, FAKE, None) == SHAPE   # H % 64
        assert fn(FAKE, FAKE, FAKE, FAKE, 8, 128, 200, 1000, FAKE, None) == SHAPE   # I % 64
        assert fn(FAKE, FAKE, FAKE, FAKE, 0, 128, 256, 1000, FAKE, None) == SHAPE
        assert fn(FAKE, FAKE, FAKE, FAKE, 8, 128, 256, 0, FAKE, None) == OVERFLOW
        assert fn(FAKE, FAKE + 8, FAKE, FAKE, 8, 128, 256, 1000, FAKE, None) == MISALIGNED


def test_gemm_clamped_validation(lib):
    fn = lib.moe_grouped_glu_gemm_clamped
    assert fn(FAKE, FAKE, FAKE, FAKE, 8, 128, 256, 1000, 1.0, None, None) == NULLP
    assert fn(FAKE, FAKE, FAKE, FAKE, 8, 128, 200, 1000, 1.0, FAKE, None) == SHAPE     # I % 64
    assert fn(FAKE, FAKE, FAKE, FAKE, 8, 128, 256, 1000, -1.0, FAKE, None) == VALUE
    assert fn(FAKE, FAKE, FAKE, FAKE, 8, 128, 256, 1000, float("nan"), FAKE, None) == VALUE
    assert b"limit" in lib.moe_last_error_message()


def test_gemm_gather_validation(lib):
    fn = lib.moe_grouped_glu_gemm_gather
    assert fn(FAKE, None, FAKE, FAKE, FAKE, 100, 8, 128, 256, 1000, FAKE, None) == NULLP
    assert b"row_token" in lib.moe_last_error_message()
    assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 128, 256, 1000, FAKE, None) == SHAPE       # T < 1
    assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 100, 8, 100, 256, 1000, FAKE, None) == SHAPE     # H % 64
    # T * H * 2 bytes of x must stay below 2^32 (32-bit offsets)
    assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, 8, 2048, 256, 1000, FAKE, None) == OVERFLOW
    assert fn(FAKE + 8, FAKE, FAKE, FAKE, FAKE, 100, 8, 128, 256, 1000, FAKE, None) == MISALIGNED


def test_gemm_weight_size_limit(lib):
    """One expert's weights are addressed with 32-bit byte offsets: 4*H*I < 2^32."""
    for fn in (lib.moe_grouped_glu_gemm, lib.moe_grouped_down_gemm):
        assert fn(FAKE, FAKE, FAKE, FAKE, 8, 32768, 32768, 1000, FAKE, None) == OVERFLOW
        assert b"2^32" in lib.moe_last_error_message()


def test_quantize_fp8_validation(lib):
    fn = lib.moe_quantize_fp8
    assert fn(None, 4, 128, 256, FAKE, FAKE, None) == NULLP
    assert fn(FAKE, 4, 128, 256, FAKE, None, None) == NULLP
    assert b"scale" in lib.moe_last_error_message()
    assert fn(FAKE, 4, 96, 256, FAKE, FAKE, None) == SHAPE      # R % 64
    assert fn(FAKE, 4, 128, 200, FAKE, FAKE, None) == SHAPE     # K % 64
    assert fn(FAKE, 0, 128, 256, FAKE, FAKE, None) == SHAPE
    assert fn(FAKE, 4, 128, 256, FAKE + 4, FAKE, None) == MISALIGNED


def test_fp8_gemm_validation(lib):
    for fn in (lib.moe_grouped_glu_gemm_fp8w, lib.moe_grouped_down_gemm_fp8w):
        assert fn(FAKE, FAKE, None, FAKE, FAKE, 8, 128, 256, 1000, FAKE, None) == NULLP   # scale
        assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 128, 256, 1000, None, None) == NULLP
        assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 100, 256, 1000, FAKE, None) == SHAPE
        assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 128, 200, 1000, FAKE, None) == SHAPE
        assert fn(FAKE, FAKE, FAKE + 4, FAKE, FAKE, 8, 128, 256, 1000, FAKE, None) == MISALIGNED
    fn = lib.moe_grouped_glu_gemm_gather_fp8w
    assert fn(FAKE, None, FAKE, FAKE, FAKE, FAKE, 100, 8, 128, 256, 1000, FAKE, None) == NULLP
    assert fn(FAKE, FAKE, FAKE, None, FAKE, FAKE, 100, 8, 128, 256, 1000, FAKE, None) == NULLP
    assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 128, 256, 1000, FAKE, None) == SHAPE
    assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, 8, 2048, 256, 1000, FAKE, None) == OVERFLOW


def test_training_validation(lib):
    assert lib.moe_grouped_gemm(FAKE, FAKE, FAKE, FAKE, 8, 128, 256, 1000, None, None) == NULLP
    assert lib.moe_grouped_gemm(FAKE, FAKE, FAKE, FAKE, 8, 100, 256, 1000, FAKE, None) == SHAPE   # K % 64
    assert lib.moe_swiglu(FAKE, FAKE, 4, 96, 100, FAKE, None) == SHAPE                             # I % 64
    assert lib.moe_swiglu_backward(FAKE, None, FAKE, 4, 128, 100, FAKE, None) == NULLP
    fn = lib.moe_grouped_gemm_swiglu_backward
    assert fn(FAKE, FAKE, None, FAKE, FAKE, 8, 128, 256, 1000, FAKE, None) == NULLP          # gu
    assert fn(FAKE, FAKE, FAKE + 8, FAKE, FAKE, 8, 128, 256, 1000, FAKE, None) == MISALIGNED  # gu
    assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 128, 200, 1000, FAKE, None) == SHAPE           # I % 64
    assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 100, 256, 1000, FAKE, None) == SHAPE           # H % 64
    assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 128, 256, 1000, None, None) == NULLP           # dgu
    assert lib.moe_transpose_experts(FAKE, 2, 64, 100, FAKE, None) == SHAPE
    assert lib.moe_transpose_experts(FAKE + 8, 2, 64, 64, FAKE, None) == MISALIGNED
    assert lib.moe_combine_backward(FAKE, FAKE, FAKE, FAKE, None, FAKE, 4, 128, 8, 2, 100, FAKE, FAKE,
                                    None) == NULLP                                                  # row_token
    assert lib.moe_combine_backward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 128, 8, 9, 100, FAKE, FAKE,
                                    None) == SHAPE                                                  # k > E
    assert lib.moe_route_backward(FAKE, FAKE, FAKE, 4, 8, 0, FAKE, None) == SHAPE
    assert lib.moe_route_backward(None, None, None, 0, 8, 2, None, None) == OK                    # no tokens
    assert lib.moe_permute_backward(FAKE, FAKE, 4, 130, 2, 100, FAKE, None) == SHAPE
    assert lib.moe_grouped_wgrad(FAKE, FAKE, None, FAKE, FAKE, 8, 128, 96, 1000, FAKE, None) == SHAPE  # N % 64
    assert lib.moe_grouped_wgrad(FAKE, FAKE, FAKE + 4, FAKE, FAKE, 8, 128, 128, 1000, FAKE,
                                 None) == MISALIGNED
    assert lib.moe_grouped_wgrad(FAKE, FAKE, None, FAKE, FAKE, 8, 128, 128, 1000, None, None) == NULLP
    assert lib.moe_grouped_wgrad(FAKE, FAKE, None, FAKE, FAKE, 8, 128, 128, 1000, FAKE + 4, None) == MISALIGNED


def test_router_validation(lib):
    assert lib.moe_router_prepare(None, 128, 8, FAKE, FAKE, None) == NULLP
    assert lib.moe_router_prepare(FAKE, 100, 8, FAKE, FAKE, None) == SHAPE          # H % 64
    assert lib.moe_router_prepare(FAKE, 128, 2048, FAKE, FAKE, None) == SHAPE       # E > 1024
    assert lib.moe_router_topk(FAKE, FAKE, FAKE, 4, 128, 8, 9, None, FAKE, FAKE, None) == SHAPE  # k > E
    assert lib.moe_router_topk(FAKE, FAKE, FAKE, 4, 128, 8, 2, FAKE + 4, FAKE, FAKE, None) == MISALIGNED
    assert lib.moe_router_topk(FAKE, None, FAKE, 4, 128, 8, 2, None, FAKE, FAKE, None) == NULLP
    assert lib.moe_router_topk(None, FAKE, FAKE, 0, 128, 8, 2, None, None, None, None) == OK     # no tokens


def test_combine_validation(lib):
    assert lib.moe_combine(FAKE, FAKE, FAKE, 4, 128, 2, 100, None, None) == NULLP
    assert lib.moe_combine(FAKE, FAKE, FAKE, 4, 130, 2, 100, FAKE, None) == SHAPE
    assert lib.moe_combine(FAKE, FAKE, FAKE, 4, 128, 33, 100, FAKE, None) == SHAPE
    assert lib.moe_combine(FAKE, FAKE, FAKE, 4, 128, 2, 1 << 31, FAKE, None) == OVERFLOW


@pytest.mark.parametrize("path", [LIB, DEBUG_LIB], ids=["release", "debug"])
def test_library_is_gfx950_only(path):
    """The code object inside the library targets gfx950 and nothing else."""
    data = open(path, "rb").read()
    assert b"gfx950" in data
    for other in (b"gfx942", b"gfx90a", b"gfx1100", b"sm_"):
        assert b"amdgcn-amd-amdhsa--" + other not in data


def test_tiled_validation(lib):
    """The row-pair tiled calls: whole row pairs (even rows / P_max), 32-column
    blocks, distinct buffers; otherwise as their row-major counterparts."""
    for fn in (lib.moe_tile_rows, lib.moe_untile_rows):
        assert fn(None, 6, 64, FAKE, None) == NULLP
        assert fn(FAKE, 5, 64, FAKE + 4096, None) == SHAPE          # odd rows
        assert fn(FAKE, -2, 64, FAKE + 4096, None) == SHAPE
        assert fn(FAKE, 6, 48, FAKE + 4096, None) == SHAPE          # cols % 32
        assert fn(FAKE, 6, 0, FAKE + 4096, None) == SHAPE
        assert fn(FAKE, 6, 64, FAKE, None) == VALUE                 # in place
        assert fn(FAKE + 8, 6, 64, FAKE + 4096, None) == MISALIGNED
        assert fn(None, 0, 64, None, None) == OK                    # nothing to do
    P_max = 4 * 2 + 8 * 31
    perm = lambda pm, xp=FAKE: lib.moe_permute_tiled(FAKE, FAKE, 4, 128, 8, 2, 32, pm, FAKE, FAKE, FAKE, FAKE,  # noqa: E731
                                                      xp, FAKE, 1 << 20, None)
    assert perm(P_max + 1) == SHAPE                                  # odd P_max
    assert b"even" in lib.moe_last_error_message()
    assert perm(P_max - 2) == OVERFLOW                               # below T*k + E*(align-1)
    assert perm(P_max, xp=FAKE + 8) == MISALIGNED
    for fn in (lib.moe_grouped_glu_gemm_tiled, lib.moe_grouped_down_gemm_tiled):
        assert fn(FAKE, FAKE, FAKE, FAKE, 8, 128, 256, 1001, FAKE, None) == SHAPE   # odd P_max
        assert fn(FAKE, FAKE, FAKE, FAKE, 8, 100, 256, 1000, FAKE, None) == SHAPE   # H % 64
        assert fn(FAKE, FAKE, FAKE, FAKE, 8, 128, 256, 1000, None, None) == NULLP
        assert fn(FAKE, FAKE + 8, FAKE, FAKE, 8, 128, 256, 1000, FAKE, None) == MISALIGNED
    fn = lib.moe_grouped_glu_gemm_gather_tiled
    assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 100, 8, 128, 256, 1001, FAKE, None) == SHAPE
    assert fn(FAKE, None, FAKE, FAKE, FAKE, 100, 8, 128, 256, 1000, FAKE, None) == NULLP
    assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, 8, 2048, 256, 1000, FAKE, None) == OVERFLOW


def test_tiled_training_validation(lib):
    """The training steps on tiled operands: as their row-major counterparts, plus
    whole row pairs (even P_max) wherever an operand is tiled."""
    fn = lib.moe_grouped_gemm_tiled
    assert fn(FAKE, FAKE, FAKE, FAKE, 8, 128, 256, 1001, FAKE, None) == SHAPE        # odd P_max
    assert fn(FAKE, FAKE, FAKE, FAKE, 8, 100, 256, 1000, FAKE, None) == SHAPE        # K % 64
    assert fn(FAKE, FAKE, FAKE, FAKE, 8, 128, 256, 1000, None, None) == NULLP
    assert fn(FAKE, FAKE + 8, FAKE, FAKE, 8, 128, 256, 1000, FAKE, None) == MISALIGNED
    assert lib.moe_swiglu_tiled(FAKE, FAKE, 4, 128, 101, FAKE, None) == SHAPE        # odd P_max
    assert lib.moe_swiglu_tiled(FAKE, FAKE, 4, 96, 100, FAKE, None) == SHAPE         # I % 64
    assert lib.moe_swiglu_tiled(FAKE, FAKE, 4, 128, 100, None, None) == NULLP
    fn = lib.moe_swiglu_backward_tiled
    assert fn(FAKE, FAKE, FAKE, 4, 128, 101, FAKE, None) == SHAPE                     # odd P_max
    assert fn(FAKE, FAKE, FAKE, 4, 128, 100, None, None) == NULLP
    assert fn(None, FAKE, FAKE, 4, 128, 100, FAKE, None) == NULLP
    fn = lib.moe_grouped_wgrad_tiled
    assert fn(FAKE, 2, FAKE, 1, FAKE, FAKE, 8, 128, 128, 1000, FAKE, None) == SHAPE   # flag not 0 / 1
    assert fn(FAKE, 1, FAKE, -1, FAKE, FAKE, 8, 128, 128, 1000, FAKE, None) == SHAPE
    assert fn(FAKE, 1, FAKE, 0, FAKE, FAKE, 8, 128, 128, 1001, FAKE, None) == SHAPE   # odd P_max, a tiled
    assert fn(FAKE, 0, FAKE, 1, FAKE, FAKE, 8, 128, 128, 1001, FAKE, None) == SHAPE   # odd P_max, b tiled
    assert fn(FAKE, 1, FAKE, 1, FAKE, FAKE, 8, 128, 96, 1000, FAKE, None) == SHAPE    # N % 64
    assert fn(FAKE, 1, FAKE, 1, FAKE, FAKE, 8, 128, 128, 1000, None, None) == NULLP
    assert fn(FAKE, 1, FAKE, 1, FAKE, FAKE, 8, 128, 128, 1000, FAKE + 4, None) == MISALIGNED


def test_tiled_fp8_validation(lib):
    for fn in (lib.moe_tile_fp8_rows, lib.moe_untile_fp8_rows):
        assert fn(None, 8, 64, FAKE, None) == NULLP
        assert fn(FAKE, 6, 64, FAKE + 4096, None) == SHAPE        # rows % 4
        assert fn(FAKE, 8, 48, FAKE + 4096, None) == SHAPE        # cols % 32
        assert fn(FAKE, 8, 64, FAKE, None) == VALUE               # in place
        assert fn(None, 0, 64, None, None) == OK
    for fn in (lib.moe_grouped_glu_gemm_fp8w_tiled, lib.moe_grouped_down_gemm_fp8w_tiled):
        assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 128, 256, 1001, FAKE, None) == SHAPE   # odd P_max
        assert fn(FAKE, FAKE, None, FAKE, FAKE, 8, 128, 256, 1000, FAKE, None) == NULLP   # no scales
        assert fn(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 100, 256, 1000, FAKE, None) == SHAPE   # H % 64
