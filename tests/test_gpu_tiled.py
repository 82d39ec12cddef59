"""GPU: the row-pair tiled calls.

The tiled order is this library's own memory order, not a result the pages
define: element (r, c) of an [R, C] matrix sits at
((r / 2) * (C / 32) + c / 32) * 64 + (r % 2) * 32 + c % 32.  moe_tile_rows is
checked against that formula written out element by element; every tiled call
is then checked bit for bit against its row-major counterpart (the same fp32
arithmetic in the same order, only the operands' memory order differs), which
the parity tests hold to the oracle; and the tiled layer is also held to the
oracle directly.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_routed_router_amd import inputs as gen
from gpu_util import assert_close_bf16, dev, dev_bf16, host_bits, host_f64, sample_tokens
from test_gpu_parity import (FULL_SIZE, GEMM_CASES, PERMUTE_CASES, SMALL_LAYERS, _routing, _rows_of,
                             _synthetic_layout)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _tiled_index(R: int, C: int) -> np.ndarray:
    """Flat position of every element (r, c) in the tiled order, from the formula."""
    r = np.arange(R)[:, None]
    c = np.arange(C)[None, :]
    return ((r // 2) * (C // 32) + c // 32) * 64 + (r % 2) * 32 + c % 32


def _np_tile(a: np.ndarray) -> np.ndarray:
    R, C = a.shape
    out = np.empty(R * C, a.dtype)
    out[_tiled_index(R, C).ravel()] = a.ravel()
    return out.reshape(R, C)


def _same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


TILE_SHAPES = [(2, 32), (6, 64), (130, 96), (1000, 2048), (4098, 2880)]


@pytest.mark.parametrize("R,C", TILE_SHAPES, ids=[f"{r}x{c}" for r, c in TILE_SHAPES])
def test_tile_rows(gpu_lib, R, C):
    _say(f"tile_rows {R}x{C}")
    a = gen.random_bf16((R, C), seed=R + C)
    if R * C <= 6 * 64:
        # the formula, one element at a time
        flat = _np_tile(a).ravel()
        for r in range(R):
            for c in range(C):
                assert flat[((r // 2) * (C // 32) + c // 32) * 64 + (r % 2) * 32 + c % 32] == a[r, c]
    t = gpu_lib.tile_rows(dev_bf16(a))
    back = gpu_lib.untile_rows(t)
    torch.cuda.synchronize()
    assert (host_bits(t) == _np_tile(a)).all()
    assert (host_bits(back) == a).all()


def test_tile_weights_per_expert(gpu_lib):
    """Expert weights [E, R, C] tile as E separate [R, C] matrices (R even)."""
    w = gen.random_bf16((3, 6, 64), seed=5)
    tw = gpu_lib.tile_weights(dev_bf16(w))
    torch.cuda.synchronize()
    got = host_bits(tw.data)
    for e in range(3):
        assert (got[e] == _np_tile(w[e])).all()


# --------------------------------------------------------------------------------------
# GEMMs: tiled == row-major, bit for bit
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("case", GEMM_CASES, ids=[c[0] for c in GEMM_CASES])
def test_tiled_gemms_equal_row_major(gpu_lib, case):
    """Gate/up, gathering gate/up and down GEMMs on tiled operands against the
    row-major calls, over every row of every segment (odd segment starts
    included: the align-1 cases)."""
    name, counts, align, H, I = case
    _say(f"tiled gemms case {name}")
    counts, offsets = _synthetic_layout(counts, align)
    E, P = len(counts), int(offsets[-1])
    P_max = gpu_lib.even_rows(P + 64)
    rows = _rows_of(counts, offsets)
    x_perm = np.zeros((P_max, H), np.uint16)
    x_perm[rows] = gen.random_bf16((len(rows), H), seed=1)
    h_in = np.zeros((P_max, I), np.uint16)
    h_in[rows] = gen.random_bf16((len(rows), I), seed=3)
    w_gu = dev_bf16(gen.random_bf16((E, 2 * I, H), seed=2, std=0.02))
    w_d = dev_bf16(gen.random_bf16((E, H, I), seed=4, std=0.02))
    cd, od = dev(counts), dev(offsets)
    tw_gu, tw_d = gpu_lib.tile_weights(w_gu), gpu_lib.tile_weights(w_d)
    xd, hd = dev_bf16(x_perm), dev_bf16(h_in)

    h = gpu_lib.grouped_glu_gemm(xd, w_gu, cd, od)
    h_t = gpu_lib.grouped_glu_gemm_tiled(gpu_lib.tile_rows(xd), tw_gu, cd, od)
    y = gpu_lib.grouped_down_gemm(hd, w_d, cd, od)
    y_t = gpu_lib.grouped_down_gemm_tiled(gpu_lib.tile_rows(hd), tw_d, cd, od)
    T = max(1, len(rows) // 3 + 7)
    row_token = np.full(P_max, -1, np.int32)
    row_token[rows] = np.random.default_rng(len(name)).integers(0, T, size=len(rows))
    x_tok = dev_bf16(gen.random_bf16((T, H), seed=6))
    rt = dev(row_token)
    h_g = gpu_lib.grouped_glu_gemm_gather(x_tok, rt, w_gu, cd, od)
    h_gt = gpu_lib.grouped_glu_gemm_gather_tiled(x_tok, rt, tw_gu, cd, od)
    torch.cuda.synchronize()
    # rows past offsets[E] are written by neither; pad rows inside segments by both
    assert _same_bits(gpu_lib.untile_rows(h_t)[:P], h[:P]), "gate/up"
    assert _same_bits(y_t[:P], y[:P]), "down"
    ri = dev(rows)
    assert _same_bits(gpu_lib.untile_rows(h_gt)[ri], h_g[ri]), "gathering gate/up"
    # and one of them against the oracle, so this test stands on its own too
    h_ref = oracle.glu(x_perm, host_bits(w_gu), counts, offsets, I)
    assert_close_bf16(host_f64(gpu_lib.untile_rows(h_t)[:P])[rows], h_ref[rows], f"h_tiled[{name}]")


# --------------------------------------------------------------------------------------
# permute
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("case", PERMUTE_CASES, ids=[c[0] for c in PERMUTE_CASES])
def test_permute_tiled(gpu_lib, case):
    """The layout of moe_permute_tiled equals the oracle's; its x_perm, un-tiled,
    equals the oracle's gather on every used row (pad rows included)."""
    name, T, H, E, k, align, kind = case
    _say(f"tiled permute case {name}")
    x = gen.random_bf16((T, H), seed=T + H)
    idx = _routing(kind, T, E, k, seed=len(name))
    P_max = gpu_lib.even_rows(T * k + E * (align - 1))
    c_ref, o_ref, rr_ref, rt_ref = oracle.layout(idx, E, align, P_max)
    L = gpu_lib.permute(dev_bf16(x), dev(idx.astype(np.int32)), E, align, P_max, tiled=True)
    torch.cuda.synchronize()
    assert (L.counts.cpu().numpy() == c_ref).all()
    assert (L.offsets.cpu().numpy() == o_ref).all()
    assert (L.route_row.cpu().numpy() == rr_ref).all()
    assert (L.row_token.cpu().numpy() == rt_ref).all()
    used = int(o_ref[-1])
    xp = gpu_lib.untile_rows(L.x_perm)
    torch.cuda.synchronize()
    assert (host_bits(xp[:used]) == oracle.gather(x, rt_ref, rows=used)).all()
    if used & 1:  # the pair holding the last used row is written whole: a zero second row
        assert (host_bits(xp[used]) == 0).all()


# --------------------------------------------------------------------------------------
# the layer
# --------------------------------------------------------------------------------------

def _layers(gpu_lib, d, fused_gather):
    cfg = d["cfg"]
    x, logits = dev_bf16(d["x"]), dev(d["logits"])
    w_gu, w_d = dev_bf16(d["w_gu"]), dev_bf16(d["w_d"])
    ref = gpu_lib.MoELayer(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.align, fused_gather=fused_gather)
    ref(x, logits, w_gu, w_d)
    til = gpu_lib.MoELayer(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.align, fused_gather=fused_gather, tiled=True)
    til(x, logits, gpu_lib.tile_weights(w_gu), gpu_lib.tile_weights(w_d))
    torch.cuda.synchronize()
    return ref, til


def _check_tiled_layer(gpu_lib, d, fused_gather, oracle_tokens):
    cfg = d["cfg"]
    ref, til = _layers(gpu_lib, d, fused_gather)
    assert torch.equal(til.topk_idx, ref.topk_idx)
    assert torch.equal(til.layout.offsets, ref.layout.offsets)
    assert torch.equal(til.layout.route_row, ref.layout.route_row)
    assert torch.equal(til.layout.row_token[:ref.P_max], ref.layout.row_token)
    used = int(ref.layout.offsets[-1].item())
    if not fused_gather:
        assert _same_bits(gpu_lib.untile_rows(til.layout.x_perm)[:used], ref.layout.x_perm[:used]), "x_perm"
        assert _same_bits(gpu_lib.untile_rows(til.h)[:used], ref.h[:used]), "h"
        assert _same_bits(til.y[:used], ref.y[:used]), "y"
    assert _same_bits(til.out, ref.out), "out"
    if oracle_tokens:
        toks = sample_tokens(cfg.T, oracle_tokens, cfg.seed)
        want = oracle.forward(d["x"], d["logits"], d["w_gu"], d["w_d"], cfg.k, tokens=toks)
        got = host_f64(til.out[dev(toks.astype(np.int64))])
        rel = assert_close_bf16(got, want, f"tiled out[{cfg.name}]", tight=False)
        _say(f"  {cfg.name}: tiled layer max|d|/max|ref| = {rel:.3e} over {len(toks)} tokens")


@pytest.mark.parametrize("fused_gather", [False, True], ids=["x_perm", "fused_gather"])
@pytest.mark.parametrize("cfg", SMALL_LAYERS, ids=[c.name for c in SMALL_LAYERS])
def test_tiled_layer_small(gpu_lib, cfg, fused_gather):
    _say(f"tiled layer case {cfg.name} fused_gather={fused_gather}")
    _check_tiled_layer(gpu_lib, gen.make_inputs(cfg), fused_gather, oracle_tokens=cfg.T)


@pytest.mark.parametrize("fused_gather", [False, True], ids=["x_perm", "fused_gather"])
@pytest.mark.parametrize("name", [n for n, _ in FULL_SIZE], ids=[n for n, _ in FULL_SIZE])
def test_tiled_layer_full_size(gpu_lib, name, fused_gather):
    """Bit for bit against the row-major layer (which test_layer_full_size holds to
    the oracle), plus 256 sampled tokens against the oracle directly."""
    _say(f"full-size tiled layer {name} fused_gather={fused_gather}: generating inputs")
    d = gen.make_inputs(name)
    _say(f"full-size tiled layer {name}: running")
    _check_tiled_layer(gpu_lib, d, fused_gather, oracle_tokens=256)


def test_tiled_layer_rejects_mixed_weights(gpu_lib):
    cfg = SMALL_LAYERS[0]
    d = gen.make_inputs(cfg)
    til = gpu_lib.MoELayer(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.align, tiled=True)
    with pytest.raises(ValueError):
        til(dev_bf16(d["x"]), dev(d["logits"]), dev_bf16(d["w_gu"]), dev_bf16(d["w_d"]))


# --------------------------------------------------------------------------------------
# FP8 weights in 4-row tiled order
# --------------------------------------------------------------------------------------

def _np_tile_fp8(a: np.ndarray) -> np.ndarray:
    """Codes [R, K] -> 4-row tiled order, from the formula
    ((r/4)(K/32) + c/32) * 128 + (r%4) * 32 + c%32."""
    R, K = a.shape
    r = np.arange(R)[:, None]
    c = np.arange(K)[None, :]
    idx = ((r // 4) * (K // 32) + c // 32) * 128 + (r % 4) * 32 + c % 32
    out = np.empty(R * K, a.dtype)
    out[idx.ravel()] = a.ravel()
    return out.reshape(R, K)


@pytest.mark.parametrize("R,K", [(4, 32), (8, 64), (132, 96), (2048, 2880)], ids=["4x32", "8x64", "132x96", "2048x2880"])
def test_tile_fp8_rows(gpu_lib, R, K):
    _say(f"tile_fp8_rows {R}x{K}")
    a = np.random.default_rng(R + K).integers(0, 256, size=(R, K), dtype=np.uint8)
    if R * K <= 8 * 64:
        flat = _np_tile_fp8(a).ravel()
        for r in range(R):
            for c in range(K):
                assert flat[((r // 4) * (K // 32) + c // 32) * 128 + (r % 4) * 32 + c % 32] == a[r, c]
    q = gpu_lib.FP8Weights(dev(a.reshape(1, R, K)), torch.zeros((1, max(R // 64, 1)), device="cuda"))
    t = gpu_lib.tile_fp8_weights(q)
    back = gpu_lib.untile_fp8_rows(t.w8.view(R, K))
    torch.cuda.synchronize()
    assert (t.w8.view(R, K).cpu().numpy() == _np_tile_fp8(a)).all()
    assert (back.cpu().numpy() == a).all()


@pytest.mark.parametrize("case", GEMM_CASES, ids=[c[0] for c in GEMM_CASES])
def test_tiled_fp8_gemms(gpu_lib, case):
    """FP8-weight gate/up and down GEMMs on tiled operands against the row-major
    FP8 calls: bit for bit where those run the MFMA tiles (P_max > 64 E), within
    one bf16 rounding where they run the weight-streaming kernel."""
    name, counts, align, H, I = case
    _say(f"tiled fp8 gemms case {name}")
    counts, offsets = _synthetic_layout(counts, align)
    E, P = len(counts), int(offsets[-1])
    P_max = gpu_lib.even_rows(P + 64)
    rows = _rows_of(counts, offsets)
    x_perm = np.zeros((P_max, H), np.uint16)
    x_perm[rows] = gen.random_bf16((len(rows), H), seed=1)
    h_in = np.zeros((P_max, I), np.uint16)
    h_in[rows] = gen.random_bf16((len(rows), I), seed=3)
    q_gu = gpu_lib.quantize_fp8(dev_bf16(gen.random_bf16((E, 2 * I, H), seed=2, std=0.02)))
    q_d = gpu_lib.quantize_fp8(dev_bf16(gen.random_bf16((E, H, I), seed=4, std=0.02)))
    t_gu, t_d = gpu_lib.tile_fp8_weights(q_gu), gpu_lib.tile_fp8_weights(q_d)
    cd, od = dev(counts), dev(offsets)
    xd, hd = dev_bf16(x_perm), dev_bf16(h_in)
    h = gpu_lib.grouped_glu_gemm_fp8w(xd, q_gu, cd, od)
    h_t = gpu_lib.grouped_glu_gemm_fp8w(gpu_lib.tile_rows(xd), t_gu, cd, od)
    y = gpu_lib.grouped_down_gemm_fp8w(hd, q_d, cd, od)
    y_t = gpu_lib.grouped_down_gemm_fp8w(gpu_lib.tile_rows(hd), t_d, cd, od)
    torch.cuda.synchronize()
    h_u = gpu_lib.untile_rows(h_t)
    ri = dev(rows)
    if P_max > 64 * E:
        assert _same_bits(h_u[:P], h[:P]), "gate/up"
        assert _same_bits(y_t[:P], y[:P]), "down"
    else:
        assert_close_bf16(host_f64(h_u[ri]), host_f64(h[ri]), f"h_fp8_tiled[{name}]")
        assert_close_bf16(host_f64(y_t[ri]), host_f64(y[ri]), f"y_fp8_tiled[{name}]")


@pytest.mark.parametrize("cfg", SMALL_LAYERS + [gen.CONFIGS[n] for n, _ in FULL_SIZE],
                         ids=[c.name for c in SMALL_LAYERS] + [n for n, _ in FULL_SIZE])
def test_tiled_fp8_layer(gpu_lib, cfg):
    """The tiled layer with tiled FP8 weights against the row-major FP8 layer: bit for
    bit where the latter runs the MFMA tiles, else within the layer gate."""
    _say(f"tiled fp8 layer {cfg.name}")
    d = gen.make_inputs(cfg)
    x, logits = dev_bf16(d["x"]), dev(d["logits"])
    q_gu, q_d = gpu_lib.quantize_fp8(dev_bf16(d["w_gu"])), gpu_lib.quantize_fp8(dev_bf16(d["w_d"]))
    ref = gpu_lib.MoELayer(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.align)
    ref(x, logits, q_gu, q_d)
    til = gpu_lib.MoELayer(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.align, tiled=True)
    til(x, logits, gpu_lib.tile_fp8_weights(q_gu), gpu_lib.tile_fp8_weights(q_d))
    torch.cuda.synchronize()
    assert torch.equal(til.layout.offsets, ref.layout.offsets)
    if ref.P_max > 64 * cfg.E:
        assert _same_bits(til.out, ref.out), "out"
    else:
        assert_close_bf16(host_f64(til.out), host_f64(ref.out), f"tiled fp8 out[{cfg.name}]", tight=False)


# --------------------------------------------------------------------------------------
# training steps on tiled operands: == row-major, bit for bit
# --------------------------------------------------------------------------------------

TRAIN_STEP_CASES = [c for c in GEMM_CASES
                    if c[0] in ("many_tiles_k256", "many_tiles_align1", "ragged", "tails_align8", "align1",
                                "wide_H2880")]


def _same_f32(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("case", TRAIN_STEP_CASES, ids=[c[0] for c in TRAIN_STEP_CASES])
def test_tiled_training_steps_equal_row_major(gpu_lib, case):
    """The plain GEMM, the SwiGLU forward / backward and the weight gradient on
    tiled operands against the row-major calls (odd segment starts included: the
    align-1 cases), and the last pair's row past the used rows written as zeros."""
    name, counts, align, H, I = case
    _say(f"tiled training steps case {name}")
    counts, offsets = _synthetic_layout(counts, align)
    E, P = len(counts), int(offsets[-1])
    P_max = gpu_lib.even_rows(P + 64)
    rows = _rows_of(counts, offsets)
    cd, od = dev(counts), dev(offsets)
    x_perm = np.zeros((P_max, H), np.uint16)
    x_perm[rows] = gen.random_bf16((len(rows), H), seed=11)
    w_gu = dev_bf16(gen.random_bf16((E, 2 * I, H), seed=12, std=0.02))
    w_gu_t = gpu_lib.transpose_experts(w_gu)
    gu = dev_bf16(gen.random_bf16((P_max, 2 * I), seed=13))
    dh = dev_bf16(gen.random_bf16((P_max, I), seed=14))
    xd = dev_bf16(x_perm)

    # gate/up output (K = H, N = 2I) and the input gradient (K = 2I, N = H)
    c = gpu_lib.grouped_gemm(xd, w_gu, cd, od)
    c_t = gpu_lib.grouped_gemm_tiled(gpu_lib.tile_rows(xd), gpu_lib.tile_weights(w_gu), cd, od)
    dgu_in = gpu_lib.grouped_gemm(c, w_gu_t, cd, od)
    dgu_in_t = gpu_lib.grouped_gemm_tiled(gpu_lib.tile_rows(c), gpu_lib.tile_weights(w_gu_t), cd, od)
    # SwiGLU forward and backward with tiled outputs
    h = gpu_lib.swiglu(gu, od)
    h_t = gpu_lib.swiglu_tiled(gu, od)
    dgu = gpu_lib.swiglu_backward(dh, gu, od)
    dgu_t = gpu_lib.swiglu_backward_tiled(dh, gu, od)
    torch.cuda.synchronize()
    assert _same_bits(c_t[:P], c[:P]), "grouped_gemm_tiled, K = H"
    assert _same_bits(dgu_in_t[:P], dgu_in[:P]), "grouped_gemm_tiled, K = 2I"
    h_u, dgu_u = gpu_lib.untile_rows(h_t), gpu_lib.untile_rows(dgu_t)
    assert _same_bits(h_u[:P], h[:P]), "swiglu_tiled"
    assert _same_bits(dgu_u[:P], dgu[:P]), "swiglu_backward_tiled"
    if P % 2:
        assert not h_u[P].view(torch.int16).any() and not dgu_u[P].view(torch.int16).any()

    # weight gradients with every combination of tiled operands; a's pad rows zero
    for M, N, a_bits, b_bits in ((H, I, gen.random_bf16((len(rows), H), seed=15), gen.random_bf16((P_max, I), seed=16)),
                                 (2 * I, H, gen.random_bf16((len(rows), 2 * I), seed=17), x_perm)):
        a = np.zeros((P_max, M), np.uint16)
        a[rows] = a_bits
        ad, bd = dev_bf16(a), dev_bf16(b_bits)
        ref = gpu_lib.grouped_wgrad(ad, bd, cd, od)
        at_, bt_ = gpu_lib.tile_rows(ad), gpu_lib.tile_rows(bd)
        for a_tiled in (False, True):
            for b_tiled in (False, True):
                got = gpu_lib.grouped_wgrad_tiled(at_ if a_tiled else ad, bt_ if b_tiled else bd, cd, od,
                                                  a_tiled, b_tiled)
                torch.cuda.synchronize()
                assert _same_f32(got, ref), f"wgrad M={M} N={N} a_tiled={a_tiled} b_tiled={b_tiled}"


TRAIN_LAYERS = [
    gen.CONFIGS["tiny"],
    gen.MoEConfig("k1", 200, 256, 16, 1, 128, 21, "gaussian"),
    gen.MoEConfig("align1_odd_starts", 301, 256, 12, 3, 192, 27, "gaussian", align=1),
    gen.MoEConfig("sparse_experts", 12, 192, 64, 2, 128, 24, "gaussian"),
    gen.MoEConfig("skewed_small", 2048, 256, 32, 4, 128, 26, "zipf"),
    # degenerate: one token, one expert, top-1 (P_max 1 rounded up to a pair)
    gen.MoEConfig("one_token", 1, 128, 1, 1, 64, 31, "gaussian"),
    # more than 256 experts (weight gradients take experts by id), most of them empty
    gen.MoEConfig("e300_mostly_empty", 200, 128, 300, 2, 64, 32, "gaussian"),
    gen.CONFIGS["qwen3_30b_a3b"],
    # the skewed layer at full size: a 32k-row expert's weight gradients, the
    # non-temporal tiled gather
    gen.CONFIGS["skewed_zipf"],
]


def _train_layer(gpu_lib, d, tiled):
    cfg = d["cfg"]
    layer = gpu_lib.MoETrainingLayer(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.align, tiled=tiled)
    w_gu, w_d, w_gu_t, w_d_t = gpu_lib.training_weights(dev_bf16(d["w_gu"]), dev_bf16(d["w_d"]), tiled=tiled)
    out = layer.forward(dev_bf16(d["x"]), dev(d["logits"]), w_gu, w_d).clone()
    dout = dev_bf16(gen.random_bf16((cfg.T, cfg.H), seed=cfg.seed + 500))
    grads = [g.clone() for g in layer.backward(dout, w_gu_t, w_d_t)]
    torch.cuda.synchronize()
    return [out] + grads


@pytest.mark.parametrize("cfg", TRAIN_LAYERS, ids=[c.name for c in TRAIN_LAYERS])
def test_tiled_training_layer_equals_row_major(gpu_lib, cfg):
    """The whole training step on tiled operands gives the row-major step's output
    and gradients bit for bit (the row-major step is held to the oracle by the
    backward tests)."""
    _say(f"tiled training layer {cfg.name}")
    d = gen.make_inputs(cfg)
    a = _train_layer(gpu_lib, d, tiled=False)
    b = _train_layer(gpu_lib, d, tiled=True)
    for name, x, y in zip(("out", "dx", "dlogits", "dW_gu", "dW_d"), a, b):
        same = _same_bits(x, y) if x.dtype == torch.bfloat16 else _same_f32(x, y)
        assert same, f"{name}[{cfg.name}]"


def test_tiled_training_layer_rejects_row_major_weights(gpu_lib):
    cfg = gen.CONFIGS["tiny"]
    d = gen.make_inputs(cfg)
    layer = gpu_lib.MoETrainingLayer(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.align, tiled=True)
    w_gu, w_d = dev_bf16(d["w_gu"]), dev_bf16(d["w_d"])
    with pytest.raises(ValueError):
        layer.forward(dev_bf16(d["x"]), dev(d["logits"]), w_gu, w_d)
    with pytest.raises(ValueError):
        gpu_lib.MoETrainingLayer(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, cfg.align, tiled=True, fuse_swiglu_backward=True)
