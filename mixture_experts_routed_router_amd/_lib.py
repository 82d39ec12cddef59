"""Python binding of the C ABI in ``include/moe_mi355x.h`` (argument marshalling only).

Every step of the layer runs in the HIP library ``libmoe_mi355x.so``; this
module only checks tensor dtypes/devices/shapes, allocates outputs with torch
(device memory) and passes raw pointers plus torch's current HIP stream.  There
is no CPU or torch fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch  # loads the HIP runtime that the library then shares

from .build import library_path

_LIB = None
_HANDLES = {}  # debug flag -> loaded library

_c_i32, _c_i64, _c_sz, _c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

MOE_MAX_K = 32
MOE_MAX_E = 1024


class MoEError(RuntimeError):
    """A nonzero moe_status returned by the library."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {status_string(status)}: {message}")
        self.status = status


def load():
    """The library every call goes to: the release library unless use_debug_library
    switched to the debug one. Built first only if nothing is built; a failed build
    or load raises: there is no fallback path."""
    global _LIB
    if _LIB is None:
        _LIB = _open(False)
    return _LIB


def use_debug_library(debug: bool = True):
    """Route every later call to the debug library (device-side precondition
    checks, moe_debug_status) or back to the release library."""
    global _LIB
    _LIB = _open(debug)
    return _LIB


def _open(debug: bool):
    if debug in _HANDLES:
        return _HANDLES[debug]
    path = library_path(debug)
    if not os.path.exists(path):
        from .build import build
        build(debug=debug)
    lib = ctypes.CDLL(path)
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_last_error_message.argtypes = []
    lib.moe_last_error_message.restype = ctypes.c_char_p
    lib.moe_padded_rows_max.argtypes = [_c_i64, _c_i32, _c_i32, _c_i32]
    lib.moe_padded_rows_max.restype = _c_i64
    lib.moe_permute_workspace_size.argtypes = [_c_i64, _c_i32, _c_i32, ctypes.POINTER(_c_sz)]
    lib.moe_route_topk.argtypes = [_c_vp, _c_i64, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp]
    lib.moe_permute.argtypes = [_c_vp, _c_vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64,
                                _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]
    lib.moe_grouped_glu_gemm.argtypes = [_c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32,
                                         _c_i64, _c_vp, _c_vp]
    lib.moe_grouped_glu_gemm_gather.argtypes = [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i32,
                                                _c_i32, _c_i32, _c_i64, _c_vp, _c_vp]
    lib.moe_tile_rows.argtypes = [_c_vp, _c_i64, _c_i32, _c_vp, _c_vp]
    lib.moe_untile_rows.argtypes = [_c_vp, _c_i64, _c_i32, _c_vp, _c_vp]
    lib.moe_permute_tiled.argtypes = lib.moe_permute.argtypes
    lib.moe_grouped_glu_gemm_tiled.argtypes = lib.moe_grouped_glu_gemm.argtypes
    lib.moe_grouped_glu_gemm_gather_tiled.argtypes = lib.moe_grouped_glu_gemm_gather.argtypes
    lib.moe_grouped_down_gemm.argtypes = [_c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32,
                                          _c_i64, _c_vp, _c_vp]
    lib.moe_grouped_down_gemm_tiled.argtypes = lib.moe_grouped_down_gemm.argtypes
    lib.moe_tile_fp8_rows.argtypes = [_c_vp, _c_i64, _c_i32, _c_vp, _c_vp]
    lib.moe_untile_fp8_rows.argtypes = [_c_vp, _c_i64, _c_i32, _c_vp, _c_vp]
    lib.moe_combine.argtypes = [_c_vp, _c_vp, _c_vp, _c_i64, _c_i32, _c_i32, _c_i64, _c_vp, _c_vp]
    lib.moe_quantize_fp8.argtypes = [_c_vp, _c_i64, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp]
    lib.moe_grouped_glu_gemm_fp8w.argtypes = [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32,
                                              _c_i32, _c_i64, _c_vp, _c_vp]
    lib.moe_grouped_glu_gemm_gather_fp8w.argtypes = [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64,
                                                     _c_i32, _c_i32, _c_i32, _c_i64, _c_vp, _c_vp]
    lib.moe_grouped_glu_gemm_fp8w_tiled.argtypes = [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32,
                                                     _c_i64, _c_vp, _c_vp]
    lib.moe_grouped_down_gemm_fp8w_tiled.argtypes = [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32,
                                                      _c_i64, _c_vp, _c_vp]
    lib.moe_grouped_down_gemm_fp8w.argtypes = [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32,
                                               _c_i32, _c_i64, _c_vp, _c_vp]
    lib.moe_grouped_gemm.argtypes = [_c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i64, _c_vp, _c_vp]
    lib.moe_grouped_glu_gemm_clamped.argtypes = [_c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i64,
                                                 ctypes.c_float, _c_vp, _c_vp]
    lib.moe_grouped_gemm_swiglu_backward.argtypes = [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32,
                                                     _c_i64, _c_vp, _c_vp]
    lib.moe_swiglu.argtypes = [_c_vp, _c_vp, _c_i32, _c_i32, _c_i64, _c_vp, _c_vp]
    lib.moe_swiglu_backward.argtypes = [_c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i64, _c_vp, _c_vp]
    lib.moe_transpose_experts.argtypes = [_c_vp, _c_i64, _c_i32, _c_i32, _c_vp, _c_vp]
    lib.moe_combine_backward.argtypes = [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i32, _c_i32,
                                         _c_i32, _c_i64, _c_vp, _c_vp, _c_vp]
    lib.moe_route_backward.argtypes = [_c_vp, _c_vp, _c_vp, _c_i64, _c_i32, _c_i32, _c_vp, _c_vp]
    lib.moe_permute_backward.argtypes = [_c_vp, _c_vp, _c_i64, _c_i32, _c_i32, _c_i64, _c_vp, _c_vp]
    lib.moe_grouped_wgrad.argtypes = [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32, _c_i64,
                                      _c_vp, _c_vp]
    lib.moe_grouped_wgrad_tiled.argtypes = [_c_vp, _c_i32, _c_vp, _c_i32, _c_vp, _c_vp, _c_i32, _c_i32, _c_i32,
                                            _c_i64, _c_vp, _c_vp]
    lib.moe_grouped_gemm_tiled.argtypes = lib.moe_grouped_gemm.argtypes
    lib.moe_swiglu_tiled.argtypes = lib.moe_swiglu.argtypes
    lib.moe_swiglu_backward_tiled.argtypes = lib.moe_swiglu_backward.argtypes
    lib.moe_router_prepare.argtypes = [_c_vp, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp]
    lib.moe_router_topk.argtypes = [_c_vp, _c_vp, _c_vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp,
                                    _c_vp]
    lib.moe_probe_copy.argtypes = [_c_vp, _c_vp, _c_sz, _c_vp]
    lib.moe_probe_mfma_bf16.argtypes = [_c_vp, _c_i64, _c_i32, ctypes.POINTER(ctypes.c_double), _c_vp]
    lib.moe_probe_read.argtypes = [_c_vp, _c_sz, _c_vp, _c_sz, _c_vp]
    lib.moe_probe_read.restype = ctypes.c_int
    lib.moe_probe_read_sink_bytes.argtypes = []
    lib.moe_probe_read_sink_bytes.restype = _c_sz
    lib.moe_probe_mfma_sink_floats.argtypes = []
    lib.moe_probe_mfma_sink_floats.restype = _c_i64
    lib.moe_route_hist_workspace_size.argtypes = [_c_i64, _c_i32, _c_i32, ctypes.POINTER(_c_sz)]
    lib.moe_route_hist_workspace_size.restype = ctypes.c_int
    lib.moe_route_topk_hist.argtypes = [_c_vp, _c_i64, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]
    lib.moe_route_topk_hist.restype = ctypes.c_int
    lib.moe_permute_from_hist.argtypes = [_c_vp, _c_vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64,
                                          _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]
    lib.moe_permute_from_hist.restype = ctypes.c_int
    lib.moe_fused_layer_workspace_size.argtypes = [_c_i64, _c_i32, _c_i32, ctypes.POINTER(_c_sz)]
    lib.moe_fused_layer_workspace_size.restype = ctypes.c_int
    lib.moe_fused_layer.argtypes = [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32,
                                    _c_i32, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz,
                                    _c_vp]
    lib.moe_fused_layer.restype = ctypes.c_int
    lib.moe_fused_layer_status.argtypes = [_c_vp, _c_vp]
    lib.moe_fused_layer_status.restype = ctypes.c_int
    lib.moe_permute_noalloc.argtypes = [_c_vp, _c_vp, _c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64,
                                        _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp]
    lib.moe_permute_noalloc.restype = ctypes.c_int
    lib.moe_permute_noalloc_max_workspace.argtypes = []
    lib.moe_permute_noalloc_max_workspace.restype = _c_sz
    lib.moe_debug_build.argtypes = []
    lib.moe_debug_build.restype = ctypes.c_int
    lib.moe_debug_status.argtypes = [_c_vp]
    lib.moe_debug_status.restype = ctypes.c_int
    lib.moe_debug_reset.argtypes = [_c_vp]
    lib.moe_debug_reset.restype = ctypes.c_int
    for fn in ("moe_permute_workspace_size", "moe_route_topk", "moe_permute", "moe_probe_copy",
               "moe_probe_mfma_bf16",
               "moe_grouped_glu_gemm", "moe_grouped_glu_gemm_gather", "moe_grouped_down_gemm",
               "moe_combine", "moe_quantize_fp8", "moe_grouped_glu_gemm_fp8w",
               "moe_grouped_glu_gemm_gather_fp8w", "moe_grouped_down_gemm_fp8w", "moe_grouped_gemm",
               "moe_swiglu", "moe_swiglu_backward", "moe_transpose_experts", "moe_combine_backward",
               "moe_route_backward", "moe_permute_backward", "moe_grouped_wgrad", "moe_router_prepare",
               "moe_router_topk", "moe_grouped_gemm_swiglu_backward", "moe_grouped_glu_gemm_clamped",
               "moe_grouped_gemm_tiled", "moe_swiglu_tiled", "moe_swiglu_backward_tiled",
               "moe_grouped_wgrad_tiled"):
        getattr(lib, fn).restype = ctypes.c_int
    _HANDLES[debug] = lib
    return lib


def status_string(status: int) -> str:
    return load().moe_status_string(status).decode()


def _call(fn: str, *args):
    lib = load()
    st = getattr(lib, fn)(*args)
    if st != 0:
        raise MoEError(fn, st, lib.moe_last_error_message().decode())


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t: torch.Tensor, dtype, name: str, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def padded_rows_max(T: int, k: int, E: int, align: int) -> int:
    return int(load().moe_padded_rows_max(T, k, E, align))


def permute_workspace_size(T: int, k: int, E: int) -> int:
    n = _c_sz(0)
    _call("moe_permute_workspace_size", T, k, E, ctypes.byref(n))
    return int(n.value)


# ---- the five calls -----------------------------------------------------------------

def route_topk(logits: torch.Tensor, k: int, topk_idx=None, topk_w=None, stream=None):
    T, E = logits.shape
    dev = logits.device
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _call("moe_route_topk", _ptr(logits, torch.float32, "logits"), T, E, k,
          _ptr(topk_idx, torch.int32, "topk_idx", (T, k)),
          _ptr(topk_w, torch.float32, "topk_w", (T, k)), _stream(stream))
    return topk_idx, topk_w


def router_prepare(w_router, stream=None):
    """(w_hi, w_lo) bf16 [E, H] from the fp32 router weight [H, E], once per weight update."""
    H, E = w_router.shape
    w_hi = torch.empty((E, H), dtype=torch.bfloat16, device=w_router.device)
    w_lo = torch.empty((E, H), dtype=torch.bfloat16, device=w_router.device)
    _call("moe_router_prepare", _ptr(w_router, torch.float32, "w_router"), H, E,
          _ptr(w_hi, torch.bfloat16, "w_hi"), _ptr(w_lo, torch.bfloat16, "w_lo"), _stream(stream))
    return w_hi, w_lo


def router_topk(x, w_hi, w_lo, k: int, topk_idx=None, topk_w=None, logits=None, stream=None):
    """Router projection and top-k in one kernel; logits [T, E] fp32 written only if given."""
    T, H = x.shape
    E = w_hi.shape[0]
    dev = x.device
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _call("moe_router_topk", _ptr(x, torch.bfloat16, "x"), _ptr(w_hi, torch.bfloat16, "w_hi", (E, H)),
          _ptr(w_lo, torch.bfloat16, "w_lo", (E, H)), T, H, E, k,
          _ptr(logits, torch.float32, "logits", (T, E)) if logits is not None else None,
          _ptr(topk_idx, torch.int32, "topk_idx", (T, k)), _ptr(topk_w, torch.float32, "topk_w", (T, k)),
          _stream(stream))
    return topk_idx, topk_w


@dataclass
class Layout:
    counts: torch.Tensor     # [E] int32
    offsets: torch.Tensor    # [E+1] int32
    route_row: torch.Tensor  # [T*k] int32
    row_token: torch.Tensor  # [P_max] int32
    x_perm: torch.Tensor | None  # [P_max, H] bf16 (None: the layout only)
    P_max: int


def alloc_layout(T: int, H: int, E: int, k: int, P_max: int, device, gather: bool = True) -> Layout:
    return Layout(torch.empty(E, dtype=torch.int32, device=device),
                  torch.empty(E + 1, dtype=torch.int32, device=device),
                  torch.empty(T * k, dtype=torch.int32, device=device),
                  torch.empty(P_max, dtype=torch.int32, device=device),
                  torch.empty((P_max, H), dtype=torch.bfloat16, device=device) if gather else None,
                  P_max)


def permute(x: torch.Tensor, topk_idx: torch.Tensor, E: int, align: int = 32, P_max=None,
            out: Layout | None = None, workspace: torch.Tensor | None = None, stream=None,
            gather: bool = True, tiled: bool = False) -> Layout:
    """The padded layout; with gather=False (or out.x_perm None) no x_perm is
    written, for grouped_glu_gemm_gather. tiled=True writes x_perm in the
    row-pair tiled order (moe_permute_tiled; P_max must be even)."""
    T, H = x.shape
    k = topk_idx.shape[1]
    if P_max is None:
        P_max = padded_rows_max(T, k, E, align)
    if out is None:
        out = alloc_layout(T, H, E, k, P_max, x.device, gather=gather)
    gather = gather and out.x_perm is not None
    ws_bytes = permute_workspace_size(T, k, E)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=x.device)
    _call("moe_permute_tiled" if tiled else "moe_permute", _ptr(x, torch.bfloat16, "x"),
          _ptr(topk_idx, torch.int32, "topk_idx", (T, k)), T, H, E, k, align, P_max,
          _ptr(out.counts, torch.int32, "counts", (E,)),
          _ptr(out.offsets, torch.int32, "offsets", (E + 1,)),
          _ptr(out.route_row, torch.int32, "route_row", (T * k,)),
          _ptr(out.row_token, torch.int32, "row_token", (P_max,)),
          _ptr(out.x_perm, torch.bfloat16, "x_perm", (P_max, H)) if gather else None,
          _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    return out


def route_hist_workspace_size(T: int, k: int, E: int) -> int:
    n = _c_sz(0)
    _call("moe_route_hist_workspace_size", T, k, E, ctypes.byref(n))
    return int(n.value)


def route_topk_hist(logits: torch.Tensor, k: int, workspace: torch.Tensor, topk_idx=None, topk_w=None,
                    stream=None):
    """route_topk, plus the permute's per-workgroup expert counts written into
    `workspace` (uint8, route_hist_workspace_size bytes) for permute_from_hist."""
    T, E = logits.shape
    dev = logits.device
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _call("moe_route_topk_hist", _ptr(logits, torch.float32, "logits"), T, E, k,
          _ptr(topk_idx, torch.int32, "topk_idx", (T, k)), _ptr(topk_w, torch.float32, "topk_w", (T, k)),
          _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    return topk_idx, topk_w


def permute_from_hist(x: torch.Tensor, topk_idx: torch.Tensor, E: int, align: int, workspace: torch.Tensor,
                      P_max=None, out: Layout | None = None, stream=None, gather: bool = True) -> Layout:
    """permute() starting from the histogram route_topk_hist wrote into `workspace`."""
    T, H = x.shape
    k = topk_idx.shape[1]
    if P_max is None:
        P_max = padded_rows_max(T, k, E, align)
    if out is None:
        out = alloc_layout(T, H, E, k, P_max, x.device, gather=gather)
    gather = gather and out.x_perm is not None
    _call("moe_permute_from_hist", _ptr(x, torch.bfloat16, "x"), _ptr(topk_idx, torch.int32, "topk_idx", (T, k)),
          T, H, E, k, align, P_max,
          _ptr(out.counts, torch.int32, "counts", (E,)),
          _ptr(out.offsets, torch.int32, "offsets", (E + 1,)),
          _ptr(out.route_row, torch.int32, "route_row", (T * k,)),
          _ptr(out.row_token, torch.int32, "row_token", (P_max,)),
          _ptr(out.x_perm, torch.bfloat16, "x_perm", (P_max, H)) if gather else None,
          _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    return out


class FusedLayer:
    """The layer after routing as one persistent kernel (moe_fused_layer): caller's
    route_topk outputs in, out [T, H] out; the layout, h and y are kept here."""

    def __init__(self, T: int, H: int, E: int, k: int, I: int, align: int = 32, device=None):
        dev = device or torch.device("cuda")
        self.T, self.H, self.E, self.k, self.I, self.align = T, H, E, k, I, align
        self.P_max = padded_rows_max(T, k, E, align)
        self.layout = alloc_layout(T, H, E, k, self.P_max, dev, gather=False)
        self.h = torch.empty((self.P_max, I), dtype=torch.bfloat16, device=dev)
        self.y = torch.empty((self.P_max, H), dtype=torch.bfloat16, device=dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        n = _c_sz(0)
        _call("moe_fused_layer_workspace_size", T, k, E, ctypes.byref(n))
        self.workspace = torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=dev)

    def __call__(self, x, topk_idx, topk_w, w_gate_up, w_down, stream=None):
        T, H, E, k, I = self.T, self.H, self.E, self.k, self.I
        L = self.layout
        _call("moe_fused_layer", _ptr(x, torch.bfloat16, "x", (T, H)),
              _ptr(topk_idx, torch.int32, "topk_idx", (T, k)), _ptr(topk_w, torch.float32, "topk_w", (T, k)),
              _ptr(w_gate_up, torch.bfloat16, "w_gate_up", (E, 2 * I, H)),
              _ptr(w_down, torch.bfloat16, "w_down", (E, H, I)), T, H, E, k, I, self.align, self.P_max,
              _ptr(L.counts, torch.int32, "counts", (E,)), _ptr(L.offsets, torch.int32, "offsets", (E + 1,)),
              _ptr(L.route_row, torch.int32, "route_row", (T * k,)),
              _ptr(L.row_token, torch.int32, "row_token", (self.P_max,)),
              _ptr(self.h, torch.bfloat16, "h"), _ptr(self.y, torch.bfloat16, "y"),
              _ptr(self.out, torch.bfloat16, "out"), _ptr(self.workspace, torch.uint8, "workspace"),
              self.workspace.numel(), _stream(stream))
        return self.out

    def status(self, stream=None):
        """Synchronises; raises MoEError if a grid barrier of the last call timed out."""
        _call("moe_fused_layer_status", _ptr(self.workspace, torch.uint8, "workspace"), _stream(stream))


def permute_noalloc(x: torch.Tensor, topk_idx: torch.Tensor, E: int, align: int, out: Layout, stream=None,
                    gather: bool = True) -> Layout:
    """permute() without a workspace: the library's fixed device scratch holds the
    per-chunk histogram (no allocation by the library or here; `out` is the
    caller's). Calls that overlap on one device race on that scratch."""
    T, H = x.shape
    k = topk_idx.shape[1]
    P_max = out.P_max
    gather = gather and out.x_perm is not None
    _call("moe_permute_noalloc", _ptr(x, torch.bfloat16, "x"), _ptr(topk_idx, torch.int32, "topk_idx", (T, k)),
          T, H, E, k, align, P_max,
          _ptr(out.counts, torch.int32, "counts", (E,)),
          _ptr(out.offsets, torch.int32, "offsets", (E + 1,)),
          _ptr(out.route_row, torch.int32, "route_row", (T * k,)),
          _ptr(out.row_token, torch.int32, "row_token", (P_max,)),
          _ptr(out.x_perm, torch.bfloat16, "x_perm", (P_max, H)) if gather else None, _stream(stream))
    return out


def permute_noalloc_max_workspace() -> int:
    """Bytes of the fixed scratch moe_permute_noalloc has (its size limit)."""
    return int(load().moe_permute_noalloc_max_workspace())


def grouped_glu_gemm(x_perm, w_gate_up, counts, offsets, h=None, stream=None):
    P_max, H = x_perm.shape
    E, two_i, H2 = w_gate_up.shape
    I = two_i // 2
    if H2 != H or two_i != 2 * I:
        raise ValueError("w_gate_up must be [E, 2I, H]")
    if h is None:
        h = torch.empty((P_max, I), dtype=torch.bfloat16, device=x_perm.device)
    _call("moe_grouped_glu_gemm", _ptr(x_perm, torch.bfloat16, "x_perm"),
          _ptr(w_gate_up, torch.bfloat16, "w_gate_up"), _ptr(counts, torch.int32, "counts", (E,)),
          _ptr(offsets, torch.int32, "offsets", (E + 1,)), E, H, I, P_max,
          _ptr(h, torch.bfloat16, "h", (P_max, I)), _stream(stream))
    return h


def grouped_glu_gemm_clamped(x_perm, w_gate_up, counts, offsets, limit: float, h=None, stream=None):
    """grouped_glu_gemm with a clamped SwiGLU: h = silu(min(g, limit)) * clip(u, -limit, limit)."""
    P_max, H = x_perm.shape
    E, two_i, H2 = w_gate_up.shape
    I = two_i // 2
    if H2 != H or two_i != 2 * I:
        raise ValueError("w_gate_up must be [E, 2I, H]")
    if h is None:
        h = torch.empty((P_max, I), dtype=torch.bfloat16, device=x_perm.device)
    _call("moe_grouped_glu_gemm_clamped", _ptr(x_perm, torch.bfloat16, "x_perm"),
          _ptr(w_gate_up, torch.bfloat16, "w_gate_up"), _ptr(counts, torch.int32, "counts", (E,)),
          _ptr(offsets, torch.int32, "offsets", (E + 1,)), E, H, I, P_max, float(limit),
          _ptr(h, torch.bfloat16, "h", (P_max, I)), _stream(stream))
    return h


def grouped_glu_gemm_gather(x, row_token, w_gate_up, counts, offsets, h=None, stream=None):
    """grouped_glu_gemm on the layout rows x[row_token[p]] read in place (no x_perm);
    h's pad rows are unspecified."""
    T, H = x.shape
    P_max = row_token.shape[0]
    E, two_i, H2 = w_gate_up.shape
    I = two_i // 2
    if H2 != H or two_i != 2 * I:
        raise ValueError("w_gate_up must be [E, 2I, H]")
    if h is None:
        h = torch.empty((P_max, I), dtype=torch.bfloat16, device=x.device)
    _call("moe_grouped_glu_gemm_gather", _ptr(x, torch.bfloat16, "x"),
          _ptr(row_token, torch.int32, "row_token", (P_max,)),
          _ptr(w_gate_up, torch.bfloat16, "w_gate_up"), _ptr(counts, torch.int32, "counts", (E,)),
          _ptr(offsets, torch.int32, "offsets", (E + 1,)), T, E, H, I, P_max,
          _ptr(h, torch.bfloat16, "h", (P_max, I)), _stream(stream))
    return h


def grouped_down_gemm(h, w_down, counts, offsets, y=None, stream=None):
    P_max, I = h.shape
    E, H, I2 = w_down.shape
    if I2 != I:
        raise ValueError("w_down must be [E, H, I]")
    if y is None:
        y = torch.empty((P_max, H), dtype=torch.bfloat16, device=h.device)
    _call("moe_grouped_down_gemm", _ptr(h, torch.bfloat16, "h"), _ptr(w_down, torch.bfloat16, "w_down"),
          _ptr(counts, torch.int32, "counts", (E,)), _ptr(offsets, torch.int32, "offsets", (E + 1,)),
          E, H, I, P_max, _ptr(y, torch.bfloat16, "y", (P_max, H)), _stream(stream))
    return y


def combine(y, route_row, topk_w, out=None, stream=None):
    P_max, H = y.shape
    T, k = topk_w.shape
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _call("moe_combine", _ptr(y, torch.bfloat16, "y"), _ptr(route_row, torch.int32, "route_row", (T * k,)),
          _ptr(topk_w, torch.float32, "topk_w", (T, k)), T, H, k, P_max,
          _ptr(out, torch.bfloat16, "out", (T, H)), _stream(stream))
    return out


# ---- row-pair tiled operands ------------------------------------------------------------

def even_rows(P_max: int) -> int:
    """P_max rounded up to whole row pairs (the tiled calls need it even)."""
    return P_max + (P_max & 1)


def tile_rows(src: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Row-major bf16 [R, C] -> the same shape holding the row-pair tiled order."""
    R, C = src.shape
    if out is None:
        out = torch.empty((R, C), dtype=torch.bfloat16, device=src.device)
    _call("moe_tile_rows", _ptr(src, torch.bfloat16, "src"), R, C, _ptr(out, torch.bfloat16, "dst", (R, C)),
          _stream(stream))
    return out


def untile_rows(src: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The inverse of tile_rows."""
    R, C = src.shape
    if out is None:
        out = torch.empty((R, C), dtype=torch.bfloat16, device=src.device)
    _call("moe_untile_rows", _ptr(src, torch.bfloat16, "src"), R, C, _ptr(out, torch.bfloat16, "dst", (R, C)),
          _stream(stream))
    return out


@dataclass
class TiledWeights:
    """bf16 expert weights [E, R, C] stored in the row-pair tiled order (each
    expert's R rows tiled on their own; tile_weights)."""
    data: torch.Tensor

    @property
    def shape(self):
        return tuple(self.data.shape)


def tile_weights(w: torch.Tensor, stream=None) -> TiledWeights:
    """Expert weights [E, R, C] (w_gate_up [E, 2I, H], w_down [E, H, I]) in tiled order,
    once per weight update."""
    E, R, C = w.shape
    out = torch.empty((E, R, C), dtype=torch.bfloat16, device=w.device)
    tile_rows(w.reshape(E * R, C), out=out.view(E * R, C), stream=stream)
    return TiledWeights(out)


def grouped_glu_gemm_tiled(x_perm, w_gate_up: TiledWeights, counts, offsets, h=None, stream=None):
    """grouped_glu_gemm with x_perm, the weights and h in tiled order."""
    P_max, H = x_perm.shape
    E, two_i, H2 = w_gate_up.shape
    I = two_i // 2
    if H2 != H or two_i != 2 * I:
        raise ValueError("w_gate_up must be [E, 2I, H]")
    if h is None:
        h = torch.empty((P_max, I), dtype=torch.bfloat16, device=x_perm.device)
    _call("moe_grouped_glu_gemm_tiled", _ptr(x_perm, torch.bfloat16, "x_perm"),
          _ptr(w_gate_up.data, torch.bfloat16, "w_gate_up"), _ptr(counts, torch.int32, "counts", (E,)),
          _ptr(offsets, torch.int32, "offsets", (E + 1,)), E, H, I, P_max,
          _ptr(h, torch.bfloat16, "h", (P_max, I)), _stream(stream))
    return h


def grouped_glu_gemm_gather_tiled(x, row_token, w_gate_up: TiledWeights, counts, offsets, h=None, stream=None):
    """grouped_glu_gemm_gather with the weights and h in tiled order (x row-major)."""
    T, H = x.shape
    P_max = row_token.shape[0]
    E, two_i, H2 = w_gate_up.shape
    I = two_i // 2
    if H2 != H or two_i != 2 * I:
        raise ValueError("w_gate_up must be [E, 2I, H]")
    if h is None:
        h = torch.empty((P_max, I), dtype=torch.bfloat16, device=x.device)
    _call("moe_grouped_glu_gemm_gather_tiled", _ptr(x, torch.bfloat16, "x"),
          _ptr(row_token, torch.int32, "row_token", (P_max,)),
          _ptr(w_gate_up.data, torch.bfloat16, "w_gate_up"), _ptr(counts, torch.int32, "counts", (E,)),
          _ptr(offsets, torch.int32, "offsets", (E + 1,)), T, E, H, I, P_max,
          _ptr(h, torch.bfloat16, "h", (P_max, I)), _stream(stream))
    return h


def grouped_down_gemm_tiled(h, w_down: TiledWeights, counts, offsets, y=None, stream=None):
    """grouped_down_gemm with h and the weights in tiled order; y row-major."""
    P_max, I = h.shape
    E, H, I2 = w_down.shape
    if I2 != I:
        raise ValueError("w_down must be [E, H, I]")
    if y is None:
        y = torch.empty((P_max, H), dtype=torch.bfloat16, device=h.device)
    _call("moe_grouped_down_gemm_tiled", _ptr(h, torch.bfloat16, "h"),
          _ptr(w_down.data, torch.bfloat16, "w_down"), _ptr(counts, torch.int32, "counts", (E,)),
          _ptr(offsets, torch.int32, "offsets", (E + 1,)), E, H, I, P_max,
          _ptr(y, torch.bfloat16, "y", (P_max, H)), _stream(stream))
    return y


# ---- FP8 expert weights ----------------------------------------------------------------

@dataclass
class FP8Weights:
    """Block-scaled E4M3 expert weights: codes [E, R, K] uint8, one fp32 scale per
    64 rows, scale [E, R // 64]. tiled: the codes in 4-row tiled order
    (tile_fp8_weights), for the *_fp8w_tiled GEMMs."""
    w8: torch.Tensor
    scale: torch.Tensor
    tiled: bool = False

    @property
    def shape(self):
        return tuple(self.w8.shape)


def quantize_fp8(w: torch.Tensor, out: FP8Weights | None = None, stream=None) -> FP8Weights:
    """Quantize bf16 expert weights [E, R, K] (w_gate_up as [E, 2I, H], w_down as [E, H, I])."""
    E, R, K = w.shape
    if out is None:
        out = FP8Weights(torch.empty((E, R, K), dtype=torch.uint8, device=w.device),
                         torch.empty((E, R // 64), dtype=torch.float32, device=w.device))
    _call("moe_quantize_fp8", _ptr(w, torch.bfloat16, "w"), E, R, K,
          _ptr(out.w8, torch.uint8, "w8", (E, R, K)),
          _ptr(out.scale, torch.float32, "scale", (E, R // 64)), _stream(stream))
    return out


def tile_fp8_weights(wq: FP8Weights, stream=None) -> FP8Weights:
    """The same weights with the codes in 4-row tiled order (once per weight update)."""
    if wq.tiled:
        raise ValueError("already tiled")
    E, R, K = wq.w8.shape
    out = torch.empty((E, R, K), dtype=torch.uint8, device=wq.w8.device)
    _call("moe_tile_fp8_rows", _ptr(wq.w8, torch.uint8, "w8"), E * R, K, _ptr(out, torch.uint8, "dst", (E, R, K)),
          _stream(stream))
    return FP8Weights(out, wq.scale, tiled=True)


def untile_fp8_rows(src: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Tiled FP8 codes [R, K] back to row-major."""
    R, K = src.shape
    if out is None:
        out = torch.empty((R, K), dtype=torch.uint8, device=src.device)
    _call("moe_untile_fp8_rows", _ptr(src, torch.uint8, "src"), R, K, _ptr(out, torch.uint8, "dst", (R, K)),
          _stream(stream))
    return out


def _fp8_args(wq: FP8Weights, name: str):
    E, R, K = wq.w8.shape
    return (_ptr(wq.w8, torch.uint8, f"{name}.w8"),
            _ptr(wq.scale, torch.float32, f"{name}.scale", (E, R // 64)))


def grouped_glu_gemm_fp8w(x_perm, w_gate_up: FP8Weights, counts, offsets, h=None, stream=None):
    """With tiled FP8 weights (tile_fp8_weights) x_perm and h are in row-pair tiled order."""
    P_max, H = x_perm.shape
    E, two_i, H2 = w_gate_up.shape
    I = two_i // 2
    if H2 != H or two_i != 2 * I:
        raise ValueError("w_gate_up must be [E, 2I, H]")
    if h is None:
        h = torch.empty((P_max, I), dtype=torch.bfloat16, device=x_perm.device)
    _call("moe_grouped_glu_gemm_fp8w" + ("_tiled" if w_gate_up.tiled else ""), _ptr(x_perm, torch.bfloat16, "x_perm"),
          *_fp8_args(w_gate_up, "w_gate_up"), _ptr(counts, torch.int32, "counts", (E,)),
          _ptr(offsets, torch.int32, "offsets", (E + 1,)), E, H, I, P_max,
          _ptr(h, torch.bfloat16, "h", (P_max, I)), _stream(stream))
    return h


def grouped_glu_gemm_gather_fp8w(x, row_token, w_gate_up: FP8Weights, counts, offsets, h=None,
                                 stream=None):
    T, H = x.shape
    if w_gate_up.tiled:
        raise ValueError("the gathering gate/up GEMM takes row-major FP8 weights (no tiled variant)")
    P_max = row_token.shape[0]
    E, two_i, H2 = w_gate_up.shape
    I = two_i // 2
    if H2 != H or two_i != 2 * I:
        raise ValueError("w_gate_up must be [E, 2I, H]")
    if h is None:
        h = torch.empty((P_max, I), dtype=torch.bfloat16, device=x.device)
    _call("moe_grouped_glu_gemm_gather_fp8w", _ptr(x, torch.bfloat16, "x"),
          _ptr(row_token, torch.int32, "row_token", (P_max,)), *_fp8_args(w_gate_up, "w_gate_up"),
          _ptr(counts, torch.int32, "counts", (E,)), _ptr(offsets, torch.int32, "offsets", (E + 1,)),
          T, E, H, I, P_max, _ptr(h, torch.bfloat16, "h", (P_max, I)), _stream(stream))
    return h


def grouped_down_gemm_fp8w(h, w_down: FP8Weights, counts, offsets, y=None, stream=None):
    """With tiled FP8 weights h is in row-pair tiled order (y row-major either way)."""
    P_max, I = h.shape
    E, H, I2 = w_down.shape
    if I2 != I:
        raise ValueError("w_down must be [E, H, I]")
    if y is None:
        y = torch.empty((P_max, H), dtype=torch.bfloat16, device=h.device)
    _call("moe_grouped_down_gemm_fp8w" + ("_tiled" if w_down.tiled else ""), _ptr(h, torch.bfloat16, "h"),
          *_fp8_args(w_down, "w_down"),
          _ptr(counts, torch.int32, "counts", (E,)), _ptr(offsets, torch.int32, "offsets", (E + 1,)),
          E, H, I, P_max, _ptr(y, torch.bfloat16, "y", (P_max, H)), _stream(stream))
    return y


# ---- the whole layer -----------------------------------------------------------------

class MoELayer:
    """Preallocated buffers for repeated layer calls of one shape; ``__call__``
    enqueues the five library calls on the current stream and allocates nothing.
    fused_gather=True runs the permute without its gather and the gate/up GEMM
    reading token rows in place (moe_grouped_glu_gemm_gather); no x_perm exists.
    Weights are bf16 tensors or FP8Weights (from quantize_fp8), which select the
    FP8-weight GEMMs. tiled=True runs the row-pair tiled calls: weights must be
    TiledWeights (tile_weights), x_perm and h are kept in tiled order, and P_max
    is rounded up to even."""

    def __init__(self, T: int, H: int, E: int, k: int, I: int, align: int = 32, device="cuda",
                 fused_gather: bool = False, tiled: bool = False):
        self.T, self.H, self.E, self.k, self.I, self.align = T, H, E, k, I, align
        self.fused_gather = fused_gather
        self.tiled = tiled
        self.P_max = padded_rows_max(T, k, E, align)
        if tiled:
            self.P_max = even_rows(self.P_max)
        dev = torch.device(device)
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.layout = alloc_layout(T, H, E, k, self.P_max, dev, gather=not fused_gather)
        self.workspace = torch.empty(max(permute_workspace_size(T, k, E), 256), dtype=torch.uint8,
                                     device=dev)
        self.h = torch.empty((self.P_max, I), dtype=torch.bfloat16, device=dev)
        self.y = torch.empty((self.P_max, H), dtype=torch.bfloat16, device=dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def __call__(self, x, logits, w_gate_up, w_down, stream=None):
        def is_tiled(w):
            return isinstance(w, TiledWeights) or (isinstance(w, FP8Weights) and w.tiled)
        if (is_tiled(w_gate_up), is_tiled(w_down)) != (self.tiled, self.tiled):
            raise ValueError("a tiled layer takes tiled weights (TiledWeights, or FP8Weights from "
                             "tile_fp8_weights) for both, a row-major one neither")
        route_topk(logits, self.k, self.topk_idx, self.topk_w, stream=stream)
        permute(x, self.topk_idx, self.E, self.align, self.P_max, out=self.layout,
                workspace=self.workspace, stream=stream, gather=not self.fused_gather, tiled=self.tiled)
        L = self.layout
        if self.tiled:
            f8_gu, f8_d = isinstance(w_gate_up, FP8Weights), isinstance(w_down, FP8Weights)
            if self.fused_gather:
                glu = grouped_glu_gemm_gather_fp8w if f8_gu else grouped_glu_gemm_gather_tiled
                glu(x, L.row_token, w_gate_up, L.counts, L.offsets, h=self.h, stream=stream)
            else:
                glu = grouped_glu_gemm_fp8w if f8_gu else grouped_glu_gemm_tiled
                glu(L.x_perm, w_gate_up, L.counts, L.offsets, h=self.h, stream=stream)
            down = grouped_down_gemm_fp8w if f8_d else grouped_down_gemm_tiled
            down(self.h, w_down, L.counts, L.offsets, y=self.y, stream=stream)
            combine(self.y, L.route_row, self.topk_w, out=self.out, stream=stream)
            return self.out
        fp8_gu, fp8_d = isinstance(w_gate_up, FP8Weights), isinstance(w_down, FP8Weights)
        if self.fused_gather:
            glu = grouped_glu_gemm_gather_fp8w if fp8_gu else grouped_glu_gemm_gather
            glu(x, L.row_token, w_gate_up, L.counts, L.offsets, h=self.h, stream=stream)
        else:
            glu = grouped_glu_gemm_fp8w if fp8_gu else grouped_glu_gemm
            glu(L.x_perm, w_gate_up, L.counts, L.offsets, h=self.h, stream=stream)
        down = grouped_down_gemm_fp8w if fp8_d else grouped_down_gemm
        down(self.h, w_down, L.counts, L.offsets, y=self.y, stream=stream)
        combine(self.y, L.route_row, self.topk_w, out=self.out, stream=stream)
        return self.out

    def graph(self, x, logits, w_gate_up, w_down):
        """Capture one layer call on these input and weight tensors as a HIP graph.
        ``replay()`` reruns the five kernels' launches as one submission, writing
        ``self.out``; to run on new inputs, copy them into ``x`` and ``logits``
        first. The library calls allocate and clear nothing, so the graph holds
        kernel nodes only. One eager call on a side stream (default priority)
        precedes the capture."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self(x, logits, w_gate_up, w_down)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self(x, logits, w_gate_up, w_down)
        return g


# ---- training: forward with saved gate/up output, and the backward -------------------

def grouped_gemm(a, w, counts, offsets, c=None, stream=None):
    """c[p] = a[p] w[e]^T on each expert's padded segment; w [E, N, K]."""
    P_max, K = a.shape
    E, N, K2 = w.shape
    if K2 != K:
        raise ValueError("w must be [E, N, K] with K = a.shape[1]")
    if c is None:
        c = torch.empty((P_max, N), dtype=torch.bfloat16, device=a.device)
    _call("moe_grouped_gemm", _ptr(a, torch.bfloat16, "a"), _ptr(w, torch.bfloat16, "w"),
          _ptr(counts, torch.int32, "counts", (E,)), _ptr(offsets, torch.int32, "offsets", (E + 1,)),
          E, K, N, P_max, _ptr(c, torch.bfloat16, "c", (P_max, N)), _stream(stream))
    return c


def grouped_gemm_swiglu_backward(dy, w_down_t, gu, counts, offsets, dgu=None, stream=None):
    """dgu [P_max, 2I] = SwiGLU backward of dh = dy w_down_t[e]^T (dh is never written);
    w_down_t [E, I, H] from transpose_experts, gu the forward's saved gate/up output."""
    P_max, H = dy.shape
    E, I, H2 = w_down_t.shape
    if H2 != H:
        raise ValueError("w_down_t must be [E, I, H] with H = dy.shape[1]")
    if dgu is None:
        dgu = torch.empty((P_max, 2 * I), dtype=torch.bfloat16, device=dy.device)
    _call("moe_grouped_gemm_swiglu_backward", _ptr(dy, torch.bfloat16, "dy"),
          _ptr(w_down_t, torch.bfloat16, "w_down_t"), _ptr(gu, torch.bfloat16, "gu", (P_max, 2 * I)),
          _ptr(counts, torch.int32, "counts", (E,)), _ptr(offsets, torch.int32, "offsets", (E + 1,)),
          E, H, I, P_max, _ptr(dgu, torch.bfloat16, "dgu", (P_max, 2 * I)), _stream(stream))
    return dgu


def swiglu(gu, offsets, h=None, stream=None):
    P_max, two_i = gu.shape
    E = offsets.shape[0] - 1
    if h is None:
        h = torch.empty((P_max, two_i // 2), dtype=torch.bfloat16, device=gu.device)
    _call("moe_swiglu", _ptr(gu, torch.bfloat16, "gu"), _ptr(offsets, torch.int32, "offsets", (E + 1,)), E,
          two_i // 2, P_max, _ptr(h, torch.bfloat16, "h", (P_max, two_i // 2)), _stream(stream))
    return h


def swiglu_backward(dh, gu, offsets, dgu=None, stream=None):
    P_max, I = dh.shape
    E = offsets.shape[0] - 1
    if dgu is None:
        dgu = torch.empty((P_max, 2 * I), dtype=torch.bfloat16, device=dh.device)
    _call("moe_swiglu_backward", _ptr(dh, torch.bfloat16, "dh"), _ptr(gu, torch.bfloat16, "gu", (P_max, 2 * I)),
          _ptr(offsets, torch.int32, "offsets", (E + 1,)), E, I, P_max,
          _ptr(dgu, torch.bfloat16, "dgu", (P_max, 2 * I)), _stream(stream))
    return dgu


def transpose_experts(w, wt=None, stream=None):
    """wt [E, C, R] = w [E, R, C] transposed per expert (once per weight update)."""
    E, R, C = w.shape
    if wt is None:
        wt = torch.empty((E, C, R), dtype=torch.bfloat16, device=w.device)
    _call("moe_transpose_experts", _ptr(w, torch.bfloat16, "w"), E, R, C,
          _ptr(wt, torch.bfloat16, "wt", (E, C, R)), _stream(stream))
    return wt


def combine_backward(dout, y, route_row, topk_w, row_token, offsets, dy=None, dw=None, stream=None):
    T, H = dout.shape
    P_max = y.shape[0]
    k = topk_w.shape[1]
    E = offsets.shape[0] - 1
    if dy is None:
        dy = torch.empty((P_max, H), dtype=torch.bfloat16, device=y.device)
    if dw is None:
        dw = torch.empty((T, k), dtype=torch.float32, device=y.device)
    _call("moe_combine_backward", _ptr(dout, torch.bfloat16, "dout"), _ptr(y, torch.bfloat16, "y", (P_max, H)),
          _ptr(route_row, torch.int32, "route_row", (T * k,)), _ptr(topk_w, torch.float32, "topk_w", (T, k)),
          _ptr(row_token, torch.int32, "row_token", (P_max,)), _ptr(offsets, torch.int32, "offsets", (E + 1,)),
          T, H, E, k, P_max, _ptr(dy, torch.bfloat16, "dy", (P_max, H)), _ptr(dw, torch.float32, "dw", (T, k)),
          _stream(stream))
    return dy, dw


def route_backward(topk_idx, topk_w, dw, E: int, dlogits=None, stream=None):
    T, k = topk_idx.shape
    if dlogits is None:
        dlogits = torch.empty((T, E), dtype=torch.float32, device=dw.device)
    _call("moe_route_backward", _ptr(topk_idx, torch.int32, "topk_idx"), _ptr(topk_w, torch.float32, "topk_w", (T, k)),
          _ptr(dw, torch.float32, "dw", (T, k)), T, E, k, _ptr(dlogits, torch.float32, "dlogits", (T, E)),
          _stream(stream))
    return dlogits


def permute_backward(dx_perm, route_row, T: int, k: int, dx=None, stream=None):
    P_max, H = dx_perm.shape
    if dx is None:
        dx = torch.empty((T, H), dtype=torch.bfloat16, device=dx_perm.device)
    _call("moe_permute_backward", _ptr(dx_perm, torch.bfloat16, "dx_perm"),
          _ptr(route_row, torch.int32, "route_row", (T * k,)), T, H, k, P_max,
          _ptr(dx, torch.bfloat16, "dx", (T, H)), _stream(stream))
    return dx


def grouped_wgrad(a, b, counts, offsets, row_token=None, dw=None, stream=None):
    """dw [E, M, N] fp32 = sum over each expert's padded segment of a[p]^T b[p]; with
    row_token, b is the token matrix read as b[p] = x[row_token[p]]."""
    P_max, M = a.shape
    N = b.shape[1]
    E = counts.shape[0]
    if dw is None:
        dw = torch.empty((E, M, N), dtype=torch.float32, device=a.device)
    _call("moe_grouped_wgrad", _ptr(a, torch.bfloat16, "a"), _ptr(b, torch.bfloat16, "b"),
          _ptr(row_token, torch.int32, "row_token", (P_max,)) if row_token is not None else None,
          _ptr(counts, torch.int32, "counts", (E,)), _ptr(offsets, torch.int32, "offsets", (E + 1,)),
          E, M, N, P_max, _ptr(dw, torch.float32, "dw", (E, M, N)), _stream(stream))
    return dw


# the training steps on row-pair tiled operands (each bit for bit its row-major
# counterpart once un-tiled)

def grouped_gemm_tiled(a, w: TiledWeights, counts, offsets, c=None, stream=None):
    """grouped_gemm with a [P_max, K] and the weights [E, N, K] tiled; c row-major."""
    P_max, K = a.shape
    E, N, K2 = w.shape
    if not isinstance(w, TiledWeights):
        raise TypeError("w must be TiledWeights (tile_weights)")
    if K2 != K:
        raise ValueError("w must be [E, N, K] with K = a.shape[1]")
    if c is None:
        c = torch.empty((P_max, N), dtype=torch.bfloat16, device=a.device)
    _call("moe_grouped_gemm_tiled", _ptr(a, torch.bfloat16, "a"), _ptr(w.data, torch.bfloat16, "w"),
          _ptr(counts, torch.int32, "counts", (E,)), _ptr(offsets, torch.int32, "offsets", (E + 1,)),
          E, K, N, P_max, _ptr(c, torch.bfloat16, "c", (P_max, N)), _stream(stream))
    return c


def swiglu_tiled(gu, offsets, h=None, stream=None):
    """swiglu with h written in tiled order."""
    P_max, two_i = gu.shape
    E = offsets.shape[0] - 1
    if h is None:
        h = torch.empty((P_max, two_i // 2), dtype=torch.bfloat16, device=gu.device)
    _call("moe_swiglu_tiled", _ptr(gu, torch.bfloat16, "gu"), _ptr(offsets, torch.int32, "offsets", (E + 1,)), E,
          two_i // 2, P_max, _ptr(h, torch.bfloat16, "h", (P_max, two_i // 2)), _stream(stream))
    return h


def swiglu_backward_tiled(dh, gu, offsets, dgu=None, stream=None):
    """swiglu_backward (dh, gu row-major) with dgu written in tiled order."""
    P_max, I = dh.shape
    E = offsets.shape[0] - 1
    if dgu is None:
        dgu = torch.empty((P_max, 2 * I), dtype=torch.bfloat16, device=dh.device)
    _call("moe_swiglu_backward_tiled", _ptr(dh, torch.bfloat16, "dh"),
          _ptr(gu, torch.bfloat16, "gu", (P_max, 2 * I)), _ptr(offsets, torch.int32, "offsets", (E + 1,)), E, I,
          P_max, _ptr(dgu, torch.bfloat16, "dgu", (P_max, 2 * I)), _stream(stream))
    return dgu


def grouped_wgrad_tiled(a, b, counts, offsets, a_tiled: bool, b_tiled: bool, dw=None, stream=None):
    """grouped_wgrad with a and / or b in tiled order (no row_token)."""
    P_max, M = a.shape
    N = b.shape[1]
    E = counts.shape[0]
    if dw is None:
        dw = torch.empty((E, M, N), dtype=torch.float32, device=a.device)
    _call("moe_grouped_wgrad_tiled", _ptr(a, torch.bfloat16, "a"), int(bool(a_tiled)),
          _ptr(b, torch.bfloat16, "b", (P_max, N)), int(bool(b_tiled)), _ptr(counts, torch.int32, "counts", (E,)),
          _ptr(offsets, torch.int32, "offsets", (E + 1,)), E, M, N, P_max,
          _ptr(dw, torch.float32, "dw", (E, M, N)), _stream(stream))
    return dw


def training_weights(w_gate_up, w_down, tiled: bool = False, stream=None):
    """The four weight operands of MoETrainingLayer, made once per weight update:
    (w_gate_up, w_down) for forward() and (w_gate_up^T, w_down^T) for backward().
    tiled: the forward's pair and w_gate_up^T as TiledWeights; w_down^T stays
    row-major (its GEMM reads dy, which the combine backward writes row-major)."""
    wgu_t = transpose_experts(w_gate_up, stream=stream)
    wd_t = transpose_experts(w_down, stream=stream)
    if not tiled:
        return w_gate_up, w_down, wgu_t, wd_t
    return (tile_weights(w_gate_up, stream=stream), tile_weights(w_down, stream=stream),
            tile_weights(wgu_t, stream=stream), wd_t)


class MoETrainingLayer:
    """Forward that keeps what the backward needs (x_perm, gu = [g | u], h, y), and
    the backward: dx, dlogits and fp32 weight gradients. All buffers are
    preallocated; forward() and backward() only enqueue library calls.
    The backward takes the weights transposed once per update (transpose_experts;
    training_weights makes all four).
    fuse_swiglu_backward: dh and its SwiGLU backward in one GEMM
    (grouped_gemm_swiglu_backward), or, by default, grouped_gemm + swiglu_backward
    with dh written to memory -- the two steps measured faster on MI355X (the fused
    epilogue's gu loads wait behind the next tile's prefetched stages).
    tiled=True: x_perm, h and dgu in row-pair tiled order and the GEMMs on tiled
    operands (training_weights(..., tiled=True)); P_max is rounded up to even. Every
    output is bit for bit the row-major layer's."""

    def __init__(self, T: int, H: int, E: int, k: int, I: int, align: int = 32, device="cuda",
                 fuse_swiglu_backward: bool = False, tiled: bool = False):
        self.T, self.H, self.E, self.k, self.I, self.align = T, H, E, k, I, align
        if tiled and fuse_swiglu_backward:
            raise ValueError("the fused dh GEMM has no tiled form: tiled layers run the two steps")
        self.fuse_swiglu_backward = fuse_swiglu_backward
        self.tiled = tiled
        self.P_max = padded_rows_max(T, k, E, align)
        if tiled:
            self.P_max = even_rows(self.P_max)
        dev = torch.device(device)
        bf = dict(dtype=torch.bfloat16, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, k), **f32)
        self.layout = alloc_layout(T, H, E, k, self.P_max, dev)
        self.workspace = torch.empty(max(permute_workspace_size(T, k, E), 256), dtype=torch.uint8, device=dev)
        P = self.P_max
        self.gu, self.h, self.y = torch.empty((P, 2 * I), **bf), torch.empty((P, I), **bf), torch.empty((P, H), **bf)
        self.out = torch.empty((T, H), **bf)
        self.dy = torch.empty((P, H), **bf)
        self.dh = None if fuse_swiglu_backward else torch.empty((P, I), **bf)
        self.dgu, self.dx_perm = torch.empty((P, 2 * I), **bf), torch.empty((P, H), **bf)
        self.dw, self.dlogits = torch.empty((T, k), **f32), torch.empty((T, E), **f32)
        self.dx = torch.empty((T, H), **bf)
        self.dw_gu, self.dw_d = torch.empty((E, 2 * I, H), **f32), torch.empty((E, H, I), **f32)

    def _check_weights(self, *ws, row_major_last=False):
        for i, w in enumerate(ws):
            want = self.tiled and not (row_major_last and i == len(ws) - 1)
            if isinstance(w, TiledWeights) != want:
                raise ValueError("a tiled training layer takes the weights of training_weights(..., tiled=True), "
                                 "a row-major one plain tensors")

    def forward(self, x, logits, w_gate_up, w_down, stream=None):
        self._check_weights(w_gate_up, w_down)
        route_topk(logits, self.k, self.topk_idx, self.topk_w, stream=stream)
        L = permute(x, self.topk_idx, self.E, self.align, self.P_max, out=self.layout, workspace=self.workspace,
                    stream=stream, tiled=self.tiled)
        if self.tiled:
            grouped_gemm_tiled(L.x_perm, w_gate_up, L.counts, L.offsets, c=self.gu, stream=stream)
            swiglu_tiled(self.gu, L.offsets, h=self.h, stream=stream)
            grouped_down_gemm_tiled(self.h, w_down, L.counts, L.offsets, y=self.y, stream=stream)
        else:
            grouped_gemm(L.x_perm, w_gate_up, L.counts, L.offsets, c=self.gu, stream=stream)
            swiglu(self.gu, L.offsets, h=self.h, stream=stream)
            grouped_down_gemm(self.h, w_down, L.counts, L.offsets, y=self.y, stream=stream)
        combine(self.y, L.route_row, self.topk_w, out=self.out, stream=stream)
        return self.out

    def backward(self, dout, w_gate_up_t, w_down_t, stream=None):
        """w_gate_up_t [E, H, 2I] and w_down_t [E, I, H] from transpose_experts
        (tiled layer: w_gate_up_t as TiledWeights, w_down_t row-major)."""
        self._check_weights(w_gate_up_t, w_down_t, row_major_last=True)
        L = self.layout
        combine_backward(dout, self.y, L.route_row, self.topk_w, L.row_token, L.offsets, dy=self.dy, dw=self.dw,
                         stream=stream)
        route_backward(self.topk_idx, self.topk_w, self.dw, self.E, dlogits=self.dlogits, stream=stream)
        if self.tiled:
            grouped_gemm(self.dy, w_down_t, L.counts, L.offsets, c=self.dh, stream=stream)
            swiglu_backward_tiled(self.dh, self.gu, L.offsets, dgu=self.dgu, stream=stream)
            grouped_gemm_tiled(self.dgu, w_gate_up_t, L.counts, L.offsets, c=self.dx_perm, stream=stream)
            permute_backward(self.dx_perm, L.route_row, self.T, self.k, dx=self.dx, stream=stream)
            grouped_wgrad_tiled(self.dy, self.h, L.counts, L.offsets, False, True, dw=self.dw_d, stream=stream)
            grouped_wgrad_tiled(self.dgu, L.x_perm, L.counts, L.offsets, True, True, dw=self.dw_gu, stream=stream)
            return self.dx, self.dlogits, self.dw_gu, self.dw_d
        if self.fuse_swiglu_backward:
            grouped_gemm_swiglu_backward(self.dy, w_down_t, self.gu, L.counts, L.offsets, dgu=self.dgu,
                                         stream=stream)
        else:
            grouped_gemm(self.dy, w_down_t, L.counts, L.offsets, c=self.dh, stream=stream)
            swiglu_backward(self.dh, self.gu, L.offsets, dgu=self.dgu, stream=stream)
        grouped_gemm(self.dgu, w_gate_up_t, L.counts, L.offsets, c=self.dx_perm, stream=stream)
        permute_backward(self.dx_perm, L.route_row, self.T, self.k, dx=self.dx, stream=stream)
        grouped_wgrad(self.dy, self.h, L.counts, L.offsets, dw=self.dw_d, stream=stream)
        grouped_wgrad(self.dgu, L.x_perm, L.counts, L.offsets, dw=self.dw_gu, stream=stream)
        return self.dx, self.dlogits, self.dw_gu, self.dw_d


def moe_forward(x, logits, w_gate_up, w_down, k: int, align: int = 32):
    """One layer call with fresh buffers: returns out [T, H] bf16."""
    T, H = x.shape
    E, two_i, _ = w_gate_up.shape
    layer = MoELayer(T, H, E, k, two_i // 2, align, device=x.device)
    return layer(x, logits, w_gate_up, w_down).clone()


# ---- measurement probes (not part of the layer) ----------------------------------------

def probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None):
    """dst = src bytewise through the library's streaming copy kernel."""
    if src.numel() * src.element_size() != dst.numel() * dst.element_size():
        raise ValueError("src and dst must hold the same number of bytes")
    nbytes = src.numel() * src.element_size()
    _call("moe_probe_copy", _ptr(src, src.dtype, "src"), _ptr(dst, dst.dtype, "dst"), nbytes,
          _stream(stream))


def probe_read_sink(device=None) -> torch.Tensor:
    return torch.empty(int(load().moe_probe_read_sink_bytes()), dtype=torch.uint8, device=device or "cuda")


def probe_read(src: torch.Tensor, sink: torch.Tensor, stream=None):
    """Reads every byte of src once through the library's read-only streaming kernel."""
    nbytes = src.numel() * src.element_size()
    _call("moe_probe_read", _ptr(src, src.dtype, "src"), nbytes, _ptr(sink, torch.uint8, "sink"),
          sink.numel(), _stream(stream))


def probe_mfma_sink(device=None) -> torch.Tensor:
    return torch.empty(int(load().moe_probe_mfma_sink_floats()), dtype=torch.float32, device=device or "cuda")


def probe_mfma_bf16(sink: torch.Tensor, iters: int, stream=None) -> float:
    """Launches the register-only bf16 MFMA loop; returns its flops per launch."""
    fl = ctypes.c_double(0.0)
    _call("moe_probe_mfma_bf16", _ptr(sink, torch.float32, "sink"), sink.numel(), iters, ctypes.byref(fl),
          _stream(stream))
    return float(fl.value)


# ---- debug build ------------------------------------------------------------------------

def debug_build() -> bool:
    return bool(load().moe_debug_build())


def debug_status(stream=None):
    """(status, message) of the device-side precondition checks; synchronises the
    stream. The release library always reports (0, "release build: ...")."""
    lib = load()
    st = int(lib.moe_debug_status(_stream(stream)))
    return st, lib.moe_last_error_message().decode()


def debug_reset(stream=None):
    _call("moe_debug_reset", _stream(stream))
