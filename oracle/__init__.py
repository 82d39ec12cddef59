"""CPU oracle for the routed-expert MoE forward path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never loads it, and the
two share no code: this is a plain C implementation (``moe_oracle.c``) built
with gcc, wrapped here with numpy arrays.

Every function follows the page passage cited in ``moe_oracle.c``:
routing [PocketLLM "Qwen4-Exp Heterogeneous TP4 Performance", Runtime
architecture], layout and combine [prime-rl PR 3885, Changes: single-pass local
layout], grouped experts [Halo "Performance", Levers that help], FP8 expert
weights [Halo "Performance", Levers that do not help here; prime-rl, Changes:
FP8 expert weights quantized once per optimizer step], and the backward of the
path [prime-rl, Changes: gathers in backward too; forward, dgrad and wgrad
grouped GEMMs].

All floating-point results are float64 and exact up to rounding order: bf16
inputs are widened exactly and nothing in the chain is rounded. The FP8
quantizer is the one step that rounds, by its definition: fp32 scale and
quotient, then the nearest E4M3 code.

Pins: each function is checked by ``tests/test_oracle_pins.py`` against brute
force, closed forms and invariants that do not reuse this code.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import build_oracle, build_variant, library_path

_LIB = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_u8p = ctypes.POINTER(ctypes.c_uint8)

_ERRORS = {-1: "invalid argument", -2: "non-finite logit", -3: "index out of range"}


class OracleError(RuntimeError):
    pass


def _load(path: str):
    lib = ctypes.CDLL(path)
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    lib.moe_oracle_route_topk.argtypes = [_f32p, i64, i32, i32, _i32p, _f64p]
    lib.moe_oracle_layout.argtypes = [_i32p, i64, i32, i32, i32, i64, _i32p, _i32p, _i32p, _i32p]
    lib.moe_oracle_gather.argtypes = [_u16p, _i32p, i64, i64, i32, _u16p]
    lib.moe_oracle_glu.argtypes = [_u16p, _u16p, _i32p, _i32p, i32, i32, i32, _f64p]
    lib.moe_oracle_down.argtypes = [_f64p, _u16p, _i32p, _i32p, i32, i32, i32, _f64p]
    lib.moe_oracle_combine.argtypes = [_f64p, _i32p, _f64p, i64, i32, i32, i64, _f64p]
    lib.moe_oracle_forward.argtypes = [_u16p, _f32p, _u16p, _u16p, i64, i32, i32, i32, i32,
                                       _i64p, i64, _f64p]
    lib.moe_oracle_fp8_encode.argtypes = [_f32p, i64, _u8p]
    lib.moe_oracle_fp8_decode.argtypes = [_u8p, i64, _f64p]
    lib.moe_oracle_quantize_fp8.argtypes = [_u16p, i64, i32, i32, _u8p, _f32p]
    lib.moe_oracle_dequantize_fp8.argtypes = [_u8p, _f32p, i64, i32, i32, _f64p]
    lib.moe_oracle_glu_w64.argtypes = [_u16p, _f64p, _i32p, _i32p, i32, i32, i32, _f64p]
    lib.moe_oracle_down_w64.argtypes = [_f64p, _f64p, _i32p, _i32p, i32, i32, i32, _f64p]
    lib.moe_oracle_combine_bwd.argtypes = [_f64p, _f64p, _i32p, _f64p, i64, i32, i32, i64, _f64p, _f64p]
    lib.moe_oracle_route_bwd.argtypes = [_i32p, _f64p, _f64p, i64, i32, i32, _f64p]
    lib.moe_oracle_swiglu.argtypes = [_f64p, i64, i32, _f64p]
    lib.moe_oracle_swiglu_bwd.argtypes = [_f64p, _f64p, i64, i32, _f64p]
    lib.moe_oracle_swiglu_clamped.argtypes = [_f64p, i64, i32, ctypes.c_double, _f64p]
    lib.moe_oracle_gemm_nn.argtypes = [_f64p, _u16p, _i32p, _i32p, i32, i32, i32, _f64p]
    lib.moe_oracle_wgrad.argtypes = [_f64p, _f64p, _i32p, _i32p, i32, i32, i32, _f64p]
    lib.moe_oracle_permute_bwd.argtypes = [_f64p, _i32p, i64, i32, i32, i64, _f64p]
    lib.moe_oracle_backward.argtypes = [_u16p, _f32p, _u16p, _u16p, _f64p, i64, i32, i32, i32, i32,
                                        _f64p, _f64p, _f64p, _f64p]
    lib.moe_oracle_router_logits.argtypes = [_u16p, _f32p, i64, i32, i32, _f64p]
    lib.moe_oracle_num_threads.argtypes = []
    lib.moe_oracle_num_threads.restype = ctypes.c_int
    lib.moe_oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.moe_oracle_set_num_threads.restype = None
    for name in ("moe_oracle_route_topk", "moe_oracle_layout", "moe_oracle_gather",
                 "moe_oracle_glu", "moe_oracle_down", "moe_oracle_combine",
                 "moe_oracle_forward", "moe_oracle_fp8_encode", "moe_oracle_fp8_decode",
                 "moe_oracle_quantize_fp8", "moe_oracle_dequantize_fp8", "moe_oracle_glu_w64",
                 "moe_oracle_down_w64", "moe_oracle_combine_bwd", "moe_oracle_route_bwd",
                 "moe_oracle_swiglu", "moe_oracle_swiglu_bwd", "moe_oracle_swiglu_clamped", "moe_oracle_gemm_nn",
                 "moe_oracle_wgrad", "moe_oracle_permute_bwd", "moe_oracle_backward",
                 "moe_oracle_router_logits"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def _lib():
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            build_oracle()
        _LIB = _load(path)
    return _LIB


def num_threads(lib=None) -> int:
    """OpenMP threads the oracle's loops run on."""
    return int((lib or _lib()).moe_oracle_num_threads())


def set_num_threads(n: int, lib=None) -> None:
    """OpenMP threads for later oracle calls made from this thread."""
    (lib or _lib()).moe_oracle_set_num_threads(int(n))


def _p(a: np.ndarray, ptype):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ptype)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what}: {_ERRORS.get(rc, rc)}")


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 tensors are passed as their raw uint16 bits")
    return a


def route_topk(logits: np.ndarray, k: int, lib=None):
    """Top-k expert ids (int32 [T,k]) and softmax-over-selected weights (float64 [T,k])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    _check((lib or _lib()).moe_oracle_route_topk(_p(logits, _f32p), T, E, k, _p(idx, _i32p),
                                        _p(w, _f64p)), "route_topk")
    return idx, w


def padded_rows_max(T: int, k: int, E: int, align: int) -> int:
    """Rows the padded layout can need: every route plus at most align-1 pad rows per expert."""
    return T * k + E * (align - 1)


def layout(topk_idx: np.ndarray, E: int, align: int, P_max: int | None = None, lib=None):
    """counts[E], offsets[E+1], route_row[T*k], row_token[P_max] (all int32)."""
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, k = topk_idx.shape
    if P_max is None:
        P_max = padded_rows_max(T, k, E, align)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    route_row = np.empty(T * k, np.int32)
    row_token = np.empty(P_max, np.int32)
    _check((lib or _lib()).moe_oracle_layout(_p(topk_idx, _i32p), T, k, E, align, P_max,
                                    _p(counts, _i32p), _p(offsets, _i32p),
                                    _p(route_row, _i32p), _p(row_token, _i32p)), "layout")
    return counts, offsets, route_row, row_token


def gather(x_bits: np.ndarray, row_token: np.ndarray, rows: int | None = None, lib=None) -> np.ndarray:
    """x_perm bits [rows, H]: token rows copied bit for bit, zero rows where row_token is -1."""
    x_bits = _u16(x_bits)
    row_token = np.ascontiguousarray(row_token, dtype=np.int32)
    T, H = x_bits.shape
    if rows is None:
        rows = row_token.shape[0]
    out = np.empty((rows, H), np.uint16)
    _check((lib or _lib()).moe_oracle_gather(_p(x_bits, _u16p), _p(row_token, _i32p), T, rows, H,
                                    _p(out, _u16p)), "gather")
    return out


def glu(x_perm_bits, w_gu_bits, counts, offsets, I: int, lib=None) -> np.ndarray:
    """h (float64 [rows, I]) = silu(x W_gate^T) * (x W_up^T) on every valid row; other rows NaN."""
    x_perm_bits = _u16(x_perm_bits)
    w_gu_bits = _u16(w_gu_bits)
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    rows, H = x_perm_bits.shape
    E = counts.shape[0]
    assert w_gu_bits.shape == (E, 2 * I, H)
    h = np.full((rows, I), np.nan)
    _check((lib or _lib()).moe_oracle_glu(_p(x_perm_bits, _u16p), _p(w_gu_bits, _u16p),
                                 _p(counts, _i32p), _p(offsets, _i32p), E, H, I,
                                 _p(h, _f64p)), "glu")
    return h


def down(h: np.ndarray, w_d_bits, counts, offsets, lib=None) -> np.ndarray:
    """y (float64 [rows, H]) = h W_down^T on every valid row; other rows NaN."""
    h = np.ascontiguousarray(h, dtype=np.float64)
    w_d_bits = _u16(w_d_bits)
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    rows, I = h.shape
    E, H, I2 = w_d_bits.shape
    assert I2 == I and counts.shape[0] == E
    y = np.full((rows, H), np.nan)
    _check((lib or _lib()).moe_oracle_down(_p(h, _f64p), _p(w_d_bits, _u16p), _p(counts, _i32p),
                                  _p(offsets, _i32p), E, H, I, _p(y, _f64p)), "down")
    return y


def combine(y: np.ndarray, route_row, topk_w, lib=None) -> np.ndarray:
    """out (float64 [T, H]) = sum_j w[t,j] * y[route_row[t*k+j]]."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    topk_w = np.ascontiguousarray(topk_w, dtype=np.float64)
    route_row = np.ascontiguousarray(route_row, dtype=np.int32).reshape(-1)
    T, k = topk_w.shape
    P_max, H = y.shape
    out = np.empty((T, H), np.float64)
    _check((lib or _lib()).moe_oracle_combine(_p(y, _f64p), _p(route_row, _i32p), _p(topk_w, _f64p),
                                     T, H, k, P_max, _p(out, _f64p)), "combine")
    return out


def forward(x_bits, logits, w_gu_bits, w_d_bits, k: int, tokens=None, lib=None) -> np.ndarray:
    """The whole layer as a per-token loop; out float64 [len(tokens) or T, H]."""
    x_bits = _u16(x_bits)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    w_gu_bits = _u16(w_gu_bits)
    w_d_bits = _u16(w_d_bits)
    T, H = x_bits.shape
    E, two_i, H2 = w_gu_bits.shape
    I = two_i // 2
    assert H2 == H and logits.shape == (T, E) and w_d_bits.shape == (E, H, I)
    if tokens is None:
        tok_p, n = None, T
    else:
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        tok_p, n = _p(tokens, _i64p), tokens.shape[0]
    out = np.empty((n, H), np.float64)
    _check((lib or _lib()).moe_oracle_forward(_p(x_bits, _u16p), _p(logits, _f32p), _p(w_gu_bits, _u16p),
                                     _p(w_d_bits, _u16p), T, H, E, k, I, tok_p, n,
                                     _p(out, _f64p)), "forward")
    return out


def fp8_encode(v, lib=None) -> np.ndarray:
    """OCP E4M3 codes (uint8) of float32 values, nearest with ties to even; |v| <= 448."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    _check((lib or _lib()).moe_oracle_fp8_encode(_p(v, _f32p), v.size, _p(out, _u8p)), "fp8_encode")
    return out


def fp8_decode(c, lib=None) -> np.ndarray:
    """float64 values of OCP E4M3 codes (NaN for S.1111.111)."""
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    _check((lib or _lib()).moe_oracle_fp8_decode(_p(c, _u8p), c.size, _p(out, _f64p)), "fp8_decode")
    return out


def quantize_fp8(w_bits, lib=None):
    """Block-scaled FP8 of expert weights [E, R, K] (bf16 bits): (w8 uint8 [E, R, K],
    scale float32 [E, R // 64]), one scale per 64 rows."""
    w_bits = _u16(w_bits)
    E, R, K = w_bits.shape
    w8 = np.empty((E, R, K), np.uint8)
    scale = np.empty((E, R // 64), np.float32)
    _check((lib or _lib()).moe_oracle_quantize_fp8(_p(w_bits, _u16p), E, R, K, _p(w8, _u8p),
                                                   _p(scale, _f32p)), "quantize_fp8")
    return w8, scale


def dequantize_fp8(w8, scale, lib=None) -> np.ndarray:
    """float64 [E, R, K] = scale[e, r // 64] * value(w8[e, r, c])."""
    w8 = np.ascontiguousarray(w8, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.float32)
    E, R, K = w8.shape
    w = np.empty((E, R, K), np.float64)
    _check((lib or _lib()).moe_oracle_dequantize_fp8(_p(w8, _u8p), _p(scale, _f32p), E, R, K,
                                                     _p(w, _f64p)), "dequantize_fp8")
    return w


def glu_w64(x_perm_bits, w_gu, counts, offsets, I: int, lib=None) -> np.ndarray:
    """glu() with float64 weights [E, 2I, H] (e.g. dequantized FP8)."""
    x_perm_bits = _u16(x_perm_bits)
    w_gu = np.ascontiguousarray(w_gu, dtype=np.float64)
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    rows, H = x_perm_bits.shape
    E = counts.shape[0]
    assert w_gu.shape == (E, 2 * I, H)
    h = np.full((rows, I), np.nan)
    _check((lib or _lib()).moe_oracle_glu_w64(_p(x_perm_bits, _u16p), _p(w_gu, _f64p),
                                              _p(counts, _i32p), _p(offsets, _i32p), E, H, I,
                                              _p(h, _f64p)), "glu_w64")
    return h


def down_w64(h: np.ndarray, w_d, counts, offsets, lib=None) -> np.ndarray:
    """down() with float64 weights [E, H, I] (e.g. dequantized FP8)."""
    h = np.ascontiguousarray(h, dtype=np.float64)
    w_d = np.ascontiguousarray(w_d, dtype=np.float64)
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    rows, I = h.shape
    E, H, I2 = w_d.shape
    assert I2 == I and counts.shape[0] == E
    y = np.full((rows, H), np.nan)
    _check((lib or _lib()).moe_oracle_down_w64(_p(h, _f64p), _p(w_d, _f64p), _p(counts, _i32p),
                                               _p(offsets, _i32p), E, H, I, _p(y, _f64p)), "down_w64")
    return y


def router_logits(x_bits, w_r, lib=None) -> np.ndarray:
    """logits [T, E] (float64) = x W_r with x bf16 bits [T, H], W_r fp32 [H, E]."""
    x_bits = _u16(x_bits)
    w_r = np.ascontiguousarray(w_r, dtype=np.float32)
    T, H = x_bits.shape
    H2, E = w_r.shape
    assert H2 == H
    out = np.empty((T, E))
    _check((lib or _lib()).moe_oracle_router_logits(_p(x_bits, _u16p), _p(w_r, _f32p), T, H, E, _p(out, _f64p)),
           "router_logits")
    return out


# ---- backward ----------------------------------------------------------------------

def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def combine_bwd(dout, y, route_row, topk_w, lib=None):
    """(dy [P_max, H], dw [T, k]): dy rows of routes = w * dout[t], other rows 0;
    dw = <dout[t], y[route_row]>."""
    dout, y, topk_w = _f64(dout), _f64(y), _f64(topk_w)
    route_row = np.ascontiguousarray(route_row, dtype=np.int32).reshape(-1)
    T, k = topk_w.shape
    P_max, H = y.shape
    dy = np.empty((P_max, H))
    dw = np.empty((T, k))
    _check((lib or _lib()).moe_oracle_combine_bwd(_p(dout, _f64p), _p(y, _f64p), _p(route_row, _i32p),
                                                  _p(topk_w, _f64p), T, H, k, P_max, _p(dy, _f64p),
                                                  _p(dw, _f64p)), "combine_bwd")
    return dy, dw


def route_bwd(topk_idx, topk_w, dw, E: int, lib=None):
    """dlogits [T, E] of the softmax over the selected logits."""
    topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    topk_w, dw = _f64(topk_w), _f64(dw)
    T, k = topk_idx.shape
    out = np.empty((T, E))
    _check((lib or _lib()).moe_oracle_route_bwd(_p(topk_idx, _i32p), _p(topk_w, _f64p), _p(dw, _f64p),
                                                T, E, k, _p(out, _f64p)), "route_bwd")
    return out


def swiglu(gu, lib=None):
    """h [rows, I] = silu(g) * u from gu = [g | u] [rows, 2I]."""
    gu = _f64(gu)
    rows, two_i = gu.shape
    h = np.empty((rows, two_i // 2))
    _check((lib or _lib()).moe_oracle_swiglu(_p(gu, _f64p), rows, two_i // 2, _p(h, _f64p)), "swiglu")
    return h


def swiglu_clamped(gu, limit: float, lib=None):
    """h [rows, I] = silu(min(g, limit)) * clip(u, -limit, limit) from gu = [g | u]."""
    gu = _f64(gu)
    rows, two_i = gu.shape
    h = np.empty((rows, two_i // 2))
    _check((lib or _lib()).moe_oracle_swiglu_clamped(_p(gu, _f64p), rows, two_i // 2, float(limit), _p(h, _f64p)),
           "swiglu_clamped")
    return h


def swiglu_bwd(dh, gu, lib=None):
    """dgu [rows, 2I] = [dh u silu'(g) | dh silu(g)]."""
    dh, gu = _f64(dh), _f64(gu)
    rows, I = dh.shape
    assert gu.shape == (rows, 2 * I)
    dgu = np.empty((rows, 2 * I))
    _check((lib or _lib()).moe_oracle_swiglu_bwd(_p(dh, _f64p), _p(gu, _f64p), rows, I, _p(dgu, _f64p)),
           "swiglu_bwd")
    return dgu


def gemm_nn(a, w_bits, counts, offsets, lib=None):
    """C[p] = a[p] W[e] on routed rows, W [E, K, N] bf16 bits; other rows NaN."""
    a = _f64(a)
    w_bits = _u16(w_bits)
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    rows, K = a.shape
    E, K2, N = w_bits.shape
    assert K2 == K and counts.shape[0] == E
    c = np.full((rows, N), np.nan)
    _check((lib or _lib()).moe_oracle_gemm_nn(_p(a, _f64p), _p(w_bits, _u16p), _p(counts, _i32p),
                                              _p(offsets, _i32p), E, K, N, _p(c, _f64p)), "gemm_nn")
    return c


def wgrad(a, b, counts, offsets, lib=None):
    """dW [E, M, N] = sum over each expert's routed rows of a[p]^T b[p]."""
    a, b = _f64(a), _f64(b)
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    E = counts.shape[0]
    M, N = a.shape[1], b.shape[1]
    assert a.shape[0] == b.shape[0]
    dW = np.empty((E, M, N))
    _check((lib or _lib()).moe_oracle_wgrad(_p(a, _f64p), _p(b, _f64p), _p(counts, _i32p),
                                            _p(offsets, _i32p), E, M, N, _p(dW, _f64p)), "wgrad")
    return dW


def permute_bwd(dx_perm, route_row, T: int, k: int, lib=None):
    """dx [T, H] = sum_j dx_perm[route_row[t*k+j]]."""
    dx_perm = _f64(dx_perm)
    route_row = np.ascontiguousarray(route_row, dtype=np.int32).reshape(-1)
    P_max, H = dx_perm.shape
    dx = np.empty((T, H))
    _check((lib or _lib()).moe_oracle_permute_bwd(_p(dx_perm, _f64p), _p(route_row, _i32p), T, H, k,
                                                  P_max, _p(dx, _f64p)), "permute_bwd")
    return dx


def backward(x_bits, logits, w_gu_bits, w_d_bits, dout, k: int, lib=None, weights: bool = True):
    """The whole backward as a per-token loop: (dx [T,H], dlogits [T,E],
    dw_gu [E,2I,H], dw_d [E,H,I]), all float64.  weights=False computes only dx
    and dlogits (tokens in parallel; the weight gradients come back as None)."""
    x_bits, w_gu_bits, w_d_bits = _u16(x_bits), _u16(w_gu_bits), _u16(w_d_bits)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    dout = _f64(dout)
    T, H = x_bits.shape
    E, two_i, _ = w_gu_bits.shape
    I = two_i // 2
    assert logits.shape == (T, E) and w_d_bits.shape == (E, H, I) and dout.shape == (T, H)
    dx, dl = np.empty((T, H)), np.empty((T, E))
    dwgu = np.empty((E, 2 * I, H)) if weights else None
    dwd = np.empty((E, H, I)) if weights else None
    _check((lib or _lib()).moe_oracle_backward(_p(x_bits, _u16p), _p(logits, _f32p), _p(w_gu_bits, _u16p),
                                               _p(w_d_bits, _u16p), _p(dout, _f64p), T, H, E, k, I,
                                               _p(dx, _f64p), _p(dl, _f64p),
                                               _p(dwgu, _f64p) if weights else None,
                                               _p(dwd, _f64p) if weights else None), "backward")
    return dx, dl, dwgu, dwd


class Oracle:
    """The oracle's functions bound to one built library (the default build, or
    a variant that a test compiled from an edited copy of the source)."""

    def __init__(self, path: str | None = None):
        self.lib = _lib() if path is None else _load(path)

    def route_topk(self, *a, **kw):
        return route_topk(*a, lib=self.lib, **kw)

    def layout(self, *a, **kw):
        return layout(*a, lib=self.lib, **kw)

    def gather(self, *a, **kw):
        return gather(*a, lib=self.lib, **kw)

    def glu(self, *a, **kw):
        return glu(*a, lib=self.lib, **kw)

    def down(self, *a, **kw):
        return down(*a, lib=self.lib, **kw)

    def combine(self, *a, **kw):
        return combine(*a, lib=self.lib, **kw)

    def forward(self, *a, **kw):
        return forward(*a, lib=self.lib, **kw)

    def fp8_encode(self, *a, **kw):
        return fp8_encode(*a, lib=self.lib, **kw)

    def fp8_decode(self, *a, **kw):
        return fp8_decode(*a, lib=self.lib, **kw)

    def quantize_fp8(self, *a, **kw):
        return quantize_fp8(*a, lib=self.lib, **kw)

    def dequantize_fp8(self, *a, **kw):
        return dequantize_fp8(*a, lib=self.lib, **kw)

    def glu_w64(self, *a, **kw):
        return glu_w64(*a, lib=self.lib, **kw)

    def down_w64(self, *a, **kw):
        return down_w64(*a, lib=self.lib, **kw)

    def combine_bwd(self, *a, **kw):
        return combine_bwd(*a, lib=self.lib, **kw)

    def route_bwd(self, *a, **kw):
        return route_bwd(*a, lib=self.lib, **kw)

    def swiglu(self, *a, **kw):
        return swiglu(*a, lib=self.lib, **kw)

    def swiglu_bwd(self, *a, **kw):
        return swiglu_bwd(*a, lib=self.lib, **kw)

    def swiglu_clamped(self, *a, **kw):
        return swiglu_clamped(*a, lib=self.lib, **kw)

    def gemm_nn(self, *a, **kw):
        return gemm_nn(*a, lib=self.lib, **kw)

    def wgrad(self, *a, **kw):
        return wgrad(*a, lib=self.lib, **kw)

    def permute_bwd(self, *a, **kw):
        return permute_bwd(*a, lib=self.lib, **kw)

    def backward(self, *a, **kw):
        return backward(*a, lib=self.lib, **kw)

    def router_logits(self, *a, **kw):
        return router_logits(*a, lib=self.lib, **kw)
