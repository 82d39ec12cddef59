"""Pins of the CPU oracle to things other than itself (CPU only, no GPU).

Each check compares the oracle with brute force, a closed form, a library
routine or an invariant that the method's definition fixes, never with a retyped
copy of its own formula.  The checks are plain functions of an oracle instance
so that ``test_oracle_mutants.py`` can run them against builds of the oracle
with a mistake planted in them and show that they fail.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from mixture_experts_routed_router_amd import accounting, inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(bits):
    return gen.bf16_bits_to_f32(bits)


# --------------------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------------------

def _before(la, a, lb, b):
    """Routing order by definition: larger logit first; an exact tie (float ==,
    so -0 == +0) goes to the lower expert id."""
    return la > lb or (la == lb and a < b)


def brute_topk(row, k):
    """Enumerate every k-subset; exactly one has each member ranked before every
    non-member.  Its members are then ordered by how many members precede them."""
    row = [float(v) for v in row]
    E = len(row)
    winners = []
    for S in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in S]
        if all(_before(row[a], a, row[b], b) for a in S for b in rest):
            winners.append(S)
    assert len(winners) == 1, "the routing order must single out one subset"
    S = winners[0]
    return sorted(S, key=lambda a: sum(_before(row[b], b, row[a], a) for b in S))


def check_topk_brute_force(orc):
    for case, (E, k) in enumerate([(1, 1), (2, 1), (2, 2), (4, 2), (5, 3), (7, 4), (8, 2), (8, 8)]):
        for logits in (gen.tied_logits(24, E, seed=case), gen.tied_logits(24, E, seed=100 + case, levels=2),
                       np.random.default_rng(case).standard_normal((24, E)).astype(np.float32)):
            idx, _ = orc.route_topk(logits, k)
            for t in range(logits.shape[0]):
                assert list(idx[t]) == brute_topk(logits[t], k), (E, k, t, logits[t])


def check_topk_lexsort(orc):
    rng = np.random.default_rng(5)
    for E, k in [(128, 8), (512, 10), (32, 4)]:
        logits = rng.standard_normal((200, E)).astype(np.float32)
        logits[:, ::7] = logits[:, :1]  # plant exact ties with column 0
        idx, _ = orc.route_topk(logits, k)
        for t in range(logits.shape[0]):
            order = np.lexsort((np.arange(E), -logits[t]))  # primary: logit desc, then id asc
            assert list(idx[t]) == list(order[:k])


def check_topk_special_cases(orc):
    # all-equal logits: the first k ids, equal weights 1/k
    idx, w = orc.route_topk(np.full((3, 9), 0.25, np.float32), 4)
    assert (idx == np.arange(4)).all()
    assert np.all(np.abs(w - 0.25) <= 1e-15)
    # +0 and -0 compare equal: a tie resolved by id
    idx, _ = orc.route_topk(np.array([[-0.0, 0.0, -1.0]], np.float32), 2)
    assert list(idx[0]) == [0, 1]
    # k = 1: the argmax with the lowest id, weight exactly 1
    logits = np.random.default_rng(1).standard_normal((50, 16)).astype(np.float32)
    idx, w = orc.route_topk(logits, 1)
    assert (idx[:, 0] == np.argmax(logits, axis=1)).all()  # numpy's argmax takes the first max
    assert (w == 1.0).all()
    # k = E: the full order
    idx, _ = orc.route_topk(logits, 16)
    for t in range(50):
        assert list(idx[t]) == list(np.lexsort((np.arange(16), -logits[t])))


def check_softmax_weights(orc):
    rng = np.random.default_rng(2)
    logits = (rng.standard_normal((300, 64)) * 3).astype(np.float32)
    k = 6
    idx, w = orc.route_topk(logits, k)
    sel = np.take_along_axis(logits, idx, 1).astype(np.float64)
    assert np.all(np.abs(w.sum(1) - 1.0) <= 1e-14)            # a distribution over the k picks
    assert np.all(np.diff(w, axis=1) <= 0)                      # non-increasing in the slot
    # closed form of the softmax ratio: w_i / w_j = exp(L_i - L_j)
    ratio = w[:, 1:] / w[:, :1]
    assert np.allclose(ratio, np.exp(sel[:, 1:] - sel[:, :1]), rtol=1e-13, atol=0)
    # two selected logits that differ by ln 3 get weights 3/4 and 1/4
    L = np.array([[math.log(3.0), 0.0, -50.0]], np.float32)
    _, w2 = orc.route_topk(L, 2)
    d = float(np.float32(math.log(3.0)))  # the logit actually stored
    assert abs(w2[0, 0] - 1.0 / (1.0 + math.exp(-d))) < 1e-15
    assert abs(w2[0, 0] - 0.75) < 1e-7


# --------------------------------------------------------------------------------------
# layout
# --------------------------------------------------------------------------------------

def check_layout(orc, topk_idx, E, align):
    T, k = topk_idx.shape
    P_max = T * k + E * (align - 1)
    counts, offsets, route_row, row_token = orc.layout(topk_idx, E, align, P_max)
    flat = topk_idx.reshape(-1)
    assert (counts == np.bincount(flat, minlength=E)).all()
    assert counts.sum() == T * k
    padded = (counts + align - 1) // align * align
    assert offsets[0] == 0 and (np.diff(offsets) == padded).all() and (offsets % align == 0).all()
    assert offsets[-1] <= P_max
    # placement = a stable sort of the flat routes by expert, laid out from offsets[e]
    order = np.argsort(flat, kind="stable")
    expect = np.empty(T * k, np.int64)
    pos = 0
    for e in range(E):
        rs = order[pos:pos + counts[e]]
        expect[rs] = offsets[e] + np.arange(counts[e])
        pos += counts[e]
    assert (route_row == expect).all()
    # row_token: every token exactly k times, -1 everywhere else, ascending inside a segment
    assert (row_token[route_row] == np.arange(T * k) // k).all()
    assert np.bincount(row_token[row_token >= 0], minlength=T).tolist() == [k] * T
    assert (row_token >= 0).sum() == T * k
    for e in range(E):
        seg = row_token[offsets[e]:offsets[e] + counts[e]]
        assert (seg >= 0).all() and (np.diff(seg) > 0).all()
        assert (row_token[offsets[e] + counts[e]:offsets[e + 1]] == -1).all()
    assert (row_token[offsets[-1]:] == -1).all()
    return counts, offsets, route_row, row_token


def check_layout_cases(orc):
    rng = np.random.default_rng(3)
    check_layout(orc, gen.balanced_topk_idx(64, 8, 2), 8, 32)
    check_layout(orc, gen.balanced_topk_idx(100, 128, 8), 128, 16)
    idx, _ = orc.route_topk(rng.standard_normal((300, 40)).astype(np.float32), 5)
    check_layout(orc, idx, 40, 8)
    check_layout(orc, idx, 40, 1)
    # every token to the same experts (the rest get zero rows)
    check_layout(orc, np.tile(np.array([[3, 1]], np.int32), (50, 1)), 6, 32)


def check_gather(orc):
    rng = np.random.default_rng(4)
    T, H, E, k, a = 40, 64, 6, 2, 16
    x = gen.random_bf16((T, H), seed=4)
    idx, _ = orc.route_topk(rng.standard_normal((T, E)).astype(np.float32), k)
    counts, offsets, route_row, row_token = orc.layout(idx, E, a)
    xp = orc.gather(x, row_token, rows=int(offsets[-1]))
    assert (xp[route_row] == x[np.arange(T * k) // k]).all()
    pad = np.ones(int(offsets[-1]), bool)
    pad[route_row] = False
    assert (xp[pad] == 0).all()


# --------------------------------------------------------------------------------------
# expert MLPs and the whole layer
# --------------------------------------------------------------------------------------

def _silu(g):
    return g / (1.0 + np.exp(-g))


def check_dense_swiglu_reduction(orc):
    """E = 1, k = 1: the layer is a dense SwiGLU MLP (numpy float64 matmuls)."""
    T, H, I = 24, 64, 48
    x = gen.random_bf16((T, H), seed=11)
    w_gu = gen.random_bf16((1, 2 * I, H), seed=12, std=0.1)
    w_d = gen.random_bf16((1, H, I), seed=13, std=0.1)
    logits = np.random.default_rng(0).standard_normal((T, 1)).astype(np.float32)
    X = f32(x).astype(np.float64)
    Wg, Wu = f32(w_gu[0, :I]).astype(np.float64), f32(w_gu[0, I:]).astype(np.float64)
    Wd = f32(w_d[0]).astype(np.float64)
    ref = (_silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T
    out = orc.forward(x, logits, w_gu, w_d, 1)
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


def dense_masked_reference(x, logits, w_gu, w_d, k):
    """Every expert on every token (the dense work the routed layer avoids), then a
    gate matrix that is zero off each token's top-k (selected by lexsort)."""
    T, H = x.shape
    E, two_i, _ = w_gu.shape
    I = two_i // 2
    X = f32(x).astype(np.float64)
    gate = np.zeros((T, E))
    for t in range(T):
        sel = np.lexsort((np.arange(E), -logits[t]))[:k]
        z = np.exp(logits[t, sel].astype(np.float64) - float(logits[t, sel[0]]))
        gate[t, sel] = z / z.sum()
    out = np.zeros((T, H))
    for e in range(E):
        Wg = f32(w_gu[e, :I]).astype(np.float64)
        Wu = f32(w_gu[e, I:]).astype(np.float64)
        Wd = f32(w_d[e]).astype(np.float64)
        out += gate[:, e:e + 1] * ((_silu(X @ Wg.T) * (X @ Wu.T)) @ Wd.T)
    return out


def check_dense_masked(orc, cfg):
    d = gen.make_inputs(cfg)
    ref = dense_masked_reference(d["x"], d["logits"], d["w_gu"], d["w_d"], cfg.k)
    out = orc.forward(d["x"], d["logits"], d["w_gu"], d["w_d"], cfg.k)
    assert np.max(np.abs(out - ref)) <= 1e-11 * np.max(np.abs(ref))
    return d, out


def check_structured_closed_form(orc):
    """Weights with a closed-form answer: gate = a_e * Id, up = b_e * Id, down =
    c_e * (permutation pi_e), so y_e[c] = c_e * silu(a_e x[pi_e(c)]) * b_e x[pi_e(c)]."""
    T, n, E, k = 16, 32, 4, 2
    rng = np.random.default_rng(9)
    a = np.array([0.5, 1.25, -2.0, 0.75])
    b = np.array([1.5, -0.5, 0.25, 2.0])
    c = np.array([-1.0, 0.5, 1.75, -0.25])
    perms = [rng.permutation(n) for _ in range(E)]
    w_gu = np.zeros((E, 2 * n, n), np.float32)
    w_d = np.zeros((E, n, n), np.float32)
    for e in range(E):
        w_gu[e, :n] = a[e] * np.eye(n)
        w_gu[e, n:] = b[e] * np.eye(n)
        w_d[e][np.arange(n), perms[e]] = c[e]       # row c reads input pi_e(c)
    x = gen.random_bf16((T, n), seed=9)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    out = orc.forward(x, logits, gen.f32_to_bf16_bits(w_gu), gen.f32_to_bf16_bits(w_d), k)
    X = f32(x).astype(np.float64)
    for t in range(T):
        sel = np.lexsort((np.arange(E), -logits[t]))[:k]
        z = np.exp(logits[t, sel].astype(np.float64) - float(logits[t, sel[0]]))
        w = z / z.sum()
        expect = np.zeros(n)
        for j, e in enumerate(sel):
            xs = X[t, perms[e]]
            expect += w[j] * c[e] * _silu(a[e] * xs) * (b[e] * xs)
        assert np.max(np.abs(out[t] - expect)) <= 1e-13 * max(1.0, np.max(np.abs(expect))), t


def check_steps_compose(orc):
    """layout -> gather -> glu -> down -> combine equals the per-token loop."""
    cfg = gen.CONFIGS["tiny"]
    d = gen.make_inputs(cfg)
    idx, w = orc.route_topk(d["logits"], cfg.k)
    counts, offsets, route_row, row_token = orc.layout(idx, cfg.E, cfg.align)
    xp = orc.gather(d["x"], row_token)
    h = orc.glu(xp, d["w_gu"], counts, offsets, cfg.I)
    y = orc.down(np.nan_to_num(h), d["w_d"], counts, offsets)
    out = orc.combine(np.nan_to_num(y), route_row, w)
    ref = orc.forward(d["x"], d["logits"], d["w_gu"], d["w_d"], cfg.k)
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


def check_identity_experts(orc):
    """Identity experts reproduce the input: combine applied to the gathered rows
    themselves.  k = 1 gives weight 1.0 and an exact copy; for k > 1 the weights
    sum to 1 within a few ulps of double."""
    T, H, E = 50, 64, 8
    x = gen.random_bf16((T, H), seed=21)
    X = f32(x).astype(np.float64)
    logits = np.random.default_rng(21).standard_normal((T, E)).astype(np.float32)
    for k in (1, 3, 8):
        idx, w = orc.route_topk(logits, k)
        counts, offsets, route_row, row_token = orc.layout(idx, E, 16)
        xp = orc.gather(x, row_token)
        out = orc.combine(f32(xp).astype(np.float64), route_row, w)
        if k == 1:
            assert (out == X).all()
        else:
            assert np.max(np.abs(out - X)) <= 8 * k * 2.0 ** -52 * np.max(np.abs(X))


def check_linearity_and_symmetry(orc):
    cfg = gen.CONFIGS["tiny"]
    d = gen.make_inputs(cfg)
    x, logits, w_gu, w_d = d["x"], d["logits"], d["w_gu"], d["w_d"]
    out = orc.forward(x, logits, w_gu, w_d, cfg.k)
    # doubling W_down doubles the output exactly
    w_d2 = gen.f32_to_bf16_bits(f32(w_d) * 2)
    assert (orc.forward(x, logits, w_gu, w_d2, cfg.k) == 2 * out).all()
    # permuting tokens permutes output rows bit for bit
    perm = np.random.default_rng(1).permutation(cfg.T)
    assert (orc.forward(x[perm], logits[perm], w_gu, w_d, cfg.k) == out[perm]).all()
    # relabelling experts consistently leaves the output unchanged (no ties here)
    sigma = np.random.default_rng(2).permutation(cfg.E)   # new id of old expert e is sigma[e]
    inv = np.argsort(sigma)
    out2 = orc.forward(x, logits[:, inv], w_gu[inv], w_d[inv], cfg.k)
    assert (out2 == out).all()
    # a token subset gives the same rows
    toks = np.array([5, 0, 63, 17])
    assert (orc.forward(x, logits, w_gu, w_d, cfg.k, tokens=toks) == out[toks]).all()


# --------------------------------------------------------------------------------------
# FP8 expert weights (OCP E4M3, block-scaled)
# --------------------------------------------------------------------------------------

def _torch_e4m3_codes(v):
    """PyTorch's own float32 -> float8_e4m3fn cast (round to nearest even), as codes."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_e4m3_values(codes):
    import torch
    c = torch.from_numpy(np.ascontiguousarray(codes, np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def check_fp8_decode(orc):
    codes = np.arange(256, dtype=np.uint8)
    v = orc.fp8_decode(codes)
    # the library's decoding of every code, NaN for S.1111.111 only
    assert np.array_equal(v, _torch_e4m3_values(codes), equal_nan=True)
    assert [c for c in range(256) if np.isnan(v[c])] == [0x7F, 0xFF]
    # landmarks of the format: 1.0, the largest finite, the smallest subnormal and normal
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    # positive codes are strictly increasing; the sign bit mirrors them
    assert np.all(np.diff(v[:0x7F]) > 0)
    assert np.array_equal(v[0x80:0xFF], -v[:0x7F])


def check_fp8_encode(orc):
    codes = np.arange(256, dtype=np.uint8)
    vals = _torch_e4m3_values(codes)
    finite = codes[~np.isnan(vals)]
    # every finite value encodes to its own code (the two zeros keep their signs)
    assert np.array_equal(orc.fp8_encode(vals[finite].astype(np.float32)), finite)
    # midpoints between neighbours go to the code with an even mantissa
    pos = vals[:0x7F]
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[1:] + pos[:-1]) / 2)  # held exactly
    enc = orc.fp8_encode(mids)
    assert np.all(enc % 2 == 0) and np.all((enc == np.arange(126)) | (enc == np.arange(1, 127)))
    assert np.array_equal(orc.fp8_encode(-mids), enc | 0x80)
    # nearest code by brute force over all finite codes, on values of every magnitude
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(4000) * np.exp2(rng.uniform(-12, 9, 4000))).clip(-448, 448).astype(np.float32)
    enc = orc.fp8_encode(x)
    err = np.abs(x.astype(np.float64)[:, None] - vals[finite][None, :])
    assert np.allclose(np.abs(x - orc.fp8_decode(enc)), err.min(axis=1), rtol=0, atol=0)
    # and the library cast agrees code for code
    assert np.array_equal(enc, _torch_e4m3_codes(x))
    # out of range is refused, not saturated
    with pytest.raises(oracle.OracleError):
        orc.fp8_encode(np.array([448.5], np.float32))


def check_fp8_quantize(orc):
    rng = np.random.default_rng(12)
    E, R, K = 3, 192, 40
    w = (rng.standard_normal((E, R, K)) * np.exp2(rng.uniform(-6, 2, (E, R // 64, 1, 1)))
         .repeat(64, axis=1).reshape(E, R, 1)).astype(np.float32)
    w[1, 64:128] = 0.0                                   # an all-zero block
    w[2, 0, 0] = -np.abs(w[2, :64]).max() * 2            # a block whose absmax is negative
    bits = gen.f32_to_bf16_bits(w)
    wf = f32(bits).astype(np.float32)
    w8, scale = orc.quantize_fp8(bits)
    assert w8.shape == (E, R, K) and scale.shape == (E, R // 64)
    for e in range(E):
        for b in range(R // 64):
            blk = wf[e, 64 * b:64 * b + 64]
            amax = np.abs(blk).max()
            s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
            assert scale[e, b] == s
            q = np.clip(blk / s, -448, 448).astype(np.float32)
            assert np.array_equal(w8[e, 64 * b:64 * b + 64], _torch_e4m3_codes(q))
            if amax > 0:  # the block's largest magnitude lands on the largest code
                c = w8[e, 64 * b:64 * b + 64].reshape(-1)[np.argmax(np.abs(blk))]
                assert c & 0x7F == 0x7E
            else:
                assert (w8[e, 64 * b:64 * b + 64] == 0).all()
    # dequantized weights: within half a unit in the last place of E4M3 (2^-4 relative)
    # of each normal value, and within half a subnormal step of the small ones
    wd = orc.dequantize_fp8(w8, scale)
    sc = np.repeat(scale.astype(np.float64), 64, axis=1)[:, :, None]
    err = np.abs(wd - wf)
    assert np.all(err <= np.maximum(np.abs(wf) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-6))
    # weights that already are block scale x E4M3 values round-trip exactly
    codes = rng.integers(0, 0x7F, (2, 128, 16)).astype(np.uint8) | (rng.integers(0, 2, (2, 128, 16)) * 0x80).astype(np.uint8)
    codes[:, 0, 0] = 0x7E                                 # each block holds the largest code
    codes[:, 64, 0] = 0xFE
    vals = _torch_e4m3_values(codes) * np.array([2.0 ** -7, 2.0 ** 3])[:, None, None]
    w8b, scb = orc.quantize_fp8(gen.f32_to_bf16_bits(vals.astype(np.float32)))
    assert np.array_equal(orc.dequantize_fp8(w8b, scb), vals)


def check_glu_down_w64(orc):
    """glu_w64 / down_w64 on weights that are exactly the bf16 weights give the
    bf16 functions' results bit for bit."""
    cfg = gen.CONFIGS["tiny"]
    d = gen.make_inputs(cfg)
    idx, _ = orc.route_topk(d["logits"], cfg.k)
    counts, offsets, route_row, row_token = orc.layout(idx, cfg.E, 8)
    xp = orc.gather(d["x"], row_token)
    h = orc.glu(xp, d["w_gu"], counts, offsets, cfg.I)
    h64 = orc.glu_w64(xp, f32(d["w_gu"]).astype(np.float64), counts, offsets, cfg.I)
    assert np.array_equal(h, h64, equal_nan=True)
    y = orc.down(h, d["w_d"], counts, offsets)
    y64 = orc.down_w64(h, f32(d["w_d"]).astype(np.float64), counts, offsets)
    assert np.array_equal(y, y64, equal_nan=True)


# --------------------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------------------

def dense_forward64(X, L, Wgu, Wd, k):
    """The layer on float64 arrays (every expert on every token, then the top-k
    gate matrix), for finite differences: no bf16 anywhere."""
    T, H = X.shape
    E, two_i, _ = Wgu.shape
    I = two_i // 2
    gate = np.zeros((T, E))
    for t in range(T):
        sel = np.lexsort((np.arange(E), -L[t]))[:k]
        z = np.exp(L[t, sel] - L[t, sel[0]])
        gate[t, sel] = z / z.sum()
    out = np.zeros((T, H))
    for e in range(E):
        out += gate[:, e:e + 1] * ((_silu(X @ Wgu[e, :I].T) * (X @ Wgu[e, I:].T)) @ Wd[e].T)
    return out


def _bwd_case(seed=31, T=7, H=8, E=4, k=2, I=6, std=0.4):
    rng = np.random.default_rng(seed)
    x = gen.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w_gu = gen.f32_to_bf16_bits((rng.standard_normal((E, 2 * I, H)) * std).astype(np.float32))
    w_d = gen.f32_to_bf16_bits((rng.standard_normal((E, H, I)) * std).astype(np.float32))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    dout = rng.standard_normal((T, H))
    return x, logits, w_gu, w_d, dout, k


def check_backward_finite_differences(orc):
    """Every gradient of the per-token backward against central differences of an
    independent float64 forward, on random elements of x, logits, W_gu and W_d."""
    x, logits, w_gu, w_d, dout, k = _bwd_case()
    X, L = f32(x).astype(np.float64), logits.astype(np.float64)
    Wgu, Wd = f32(w_gu).astype(np.float64), f32(w_d).astype(np.float64)
    srt = np.sort(L, axis=1)[:, ::-1]
    assert np.all(srt[:, k - 1] - srt[:, k] > 1e-4)   # no selection change under the probe
    dx, dl, dwgu, dwd = orc.backward(x, logits, w_gu, w_d, dout, k)
    args = [X, L, Wgu, Wd]
    grads = [dx, dl, dwgu, dwd]
    rng = np.random.default_rng(5)
    eps = 1e-6
    for a_i, (A, G) in enumerate(zip(args, grads)):
        flat = rng.choice(A.size, size=min(A.size, 24), replace=False)
        scale = np.max(np.abs(G))
        assert scale > 0
        for f in flat:
            ix = np.unravel_index(f, A.shape)
            vals = []
            for sgn in (1, -1):
                B = [a.copy() for a in args]
                B[a_i][ix] += sgn * eps
                vals.append(np.sum(dout * dense_forward64(*B, k)))
            fd = (vals[0] - vals[1]) / (2 * eps)
            assert abs(fd - G[ix]) <= 1e-6 * scale, (a_i, ix, fd, G[ix])


def _oracle_forward_intermediates(orc, x, logits, w_gu, w_d, k, align=4):
    T, H = x.shape
    E, two_i, _ = w_gu.shape
    I = two_i // 2
    idx, w = orc.route_topk(logits, k)
    counts, offsets, route_row, row_token = orc.layout(idx, E, align)
    xp = orc.gather(x, row_token)
    gu = np.nan_to_num(orc.down(f32(xp).astype(np.float64), w_gu, counts, offsets))  # [g | u] = x_perm W_gu^T
    h = orc.swiglu(gu)
    y = np.nan_to_num(orc.down(h, w_d, counts, offsets))
    return idx, w, counts, offsets, route_row, row_token, xp, gu, h, y


def check_backward_steps_compose(orc):
    """combine_bwd -> route_bwd, gemm_nn (dh) -> swiglu_bwd -> gemm_nn (dx_perm) ->
    permute_bwd, and wgrad for both weights, equal the per-token loop (same
    terms in the same order)."""
    for case in (_bwd_case(), _bwd_case(seed=32, T=20, H=16, E=6, k=3, I=10, std=0.1)):
        x, logits, w_gu, w_d, dout, k = case
        T, H = x.shape
        E = w_gu.shape[0]
        idx, w, counts, offsets, route_row, row_token, xp, gu, h, y = \
            _oracle_forward_intermediates(orc, x, logits, w_gu, w_d, k)
        dy, dw = orc.combine_bwd(dout, y, route_row, w)
        dl = orc.route_bwd(idx, w, dw, E)
        dh = np.nan_to_num(orc.gemm_nn(dy, w_d, counts, offsets))
        dgu = orc.swiglu_bwd(dh, gu)
        dxp = np.nan_to_num(orc.gemm_nn(dgu, w_gu, counts, offsets))
        dx = orc.permute_bwd(dxp, route_row, T, k)
        dwd = orc.wgrad(dy, h, counts, offsets)
        dwgu = orc.wgrad(dgu, f32(xp).astype(np.float64), counts, offsets)
        ref = orc.backward(x, logits, w_gu, w_d, dout, k)
        for name, a, b in zip(("dx", "dlogits", "dw_gu", "dw_d"), (dx, dl, dwgu, dwd), ref):
            assert np.max(np.abs(a - b)) <= 1e-12 * max(1e-300, np.max(np.abs(b))), name


def check_backward_invariants(orc):
    """Softmax gradient rows sum to zero; k = 1 leaves no logit gradient; the
    backward is linear in dout (doubling is exact); unrouted experts get zero
    weight gradients; the input gradients alone equal the full backward's; the
    steps match numpy matmuls on their own."""
    x, logits, w_gu, w_d, dout, k = _bwd_case(seed=33, T=12, E=6, k=3)
    dx, dl, dwgu, dwd = orc.backward(x, logits, w_gu, w_d, dout, k)
    # the input gradients alone (tokens in parallel, no weight gradients) are the same numbers
    dx_only, dl_only, none_gu, none_d = orc.backward(x, logits, w_gu, w_d, dout, k, weights=False)
    assert none_gu is None and none_d is None
    assert np.array_equal(dx_only, dx) and np.array_equal(dl_only, dl)
    assert np.all(np.abs(dl.sum(axis=1)) <= 1e-15 * max(1.0, np.max(np.abs(dl))) * 8)
    sel = np.zeros_like(dl, dtype=bool)
    idx, _ = orc.route_topk(logits, k)
    np.put_along_axis(sel, idx.astype(np.int64), True, axis=1)
    assert np.all(dl[~sel] == 0)
    for a, b in zip(orc.backward(x, logits, w_gu, w_d, 2 * dout, k), (dx, dl, dwgu, dwd)):
        assert np.array_equal(a, 2 * b)
    _, dl1, _, _ = orc.backward(x, logits, w_gu, w_d, dout, 1)
    assert np.all(dl1 == 0)
    # experts no token selects get zero weight gradients
    L2 = logits.copy()
    L2[:, 0] = -50.0
    _, _, dwgu2, dwd2 = orc.backward(x, L2, w_gu, w_d, dout, k)
    assert np.all(dwgu2[0] == 0) and np.all(dwd2[0] == 0)
    # gemm_nn and wgrad against numpy matmuls, per expert
    idx, w, counts, offsets, route_row, row_token, xp, gu, h, y = \
        _oracle_forward_intermediates(orc, x, logits, w_gu, w_d, k)
    rng = np.random.default_rng(1)
    A = rng.standard_normal((len(row_token), w_d.shape[1]))
    C = orc.gemm_nn(A, w_d, counts, offsets)
    Wd = f32(w_d).astype(np.float64)
    B = rng.standard_normal((len(row_token), 5))
    dW = orc.wgrad(A, B, counts, offsets)
    for e in range(len(counts)):
        rows = np.arange(offsets[e], offsets[e] + counts[e])
        assert np.allclose(C[rows], A[rows] @ Wd[e], rtol=1e-13, atol=1e-13)
        assert np.allclose(dW[e], A[rows].T @ B[rows], rtol=1e-13, atol=1e-13)
    # permute_bwd against numpy's scatter-add of routed rows back to tokens
    dxp = rng.standard_normal((len(row_token), 4))
    ref = np.zeros((x.shape[0], 4))
    np.add.at(ref, np.repeat(np.arange(x.shape[0]), k), dxp[route_row])
    assert np.allclose(orc.permute_bwd(dxp, route_row, x.shape[0], k), ref, rtol=1e-14, atol=1e-14)


def check_swiglu_bwd_derivative(orc):
    """swiglu_bwd against central differences of swiglu itself."""
    rng = np.random.default_rng(4)
    gu = rng.standard_normal((5, 12)) * 3
    dh = rng.standard_normal((5, 6))
    dgu = orc.swiglu_bwd(dh, gu)
    eps = 1e-6
    for i in range(12):
        P, M = gu.copy(), gu.copy()
        P[:, i] += eps
        M[:, i] -= eps
        fd = (np.sum(dh * orc.swiglu(P), axis=1) - np.sum(dh * orc.swiglu(M), axis=1)) / (2 * eps)
        assert np.allclose(dgu[:, i], fd, rtol=1e-7, atol=1e-8), i


def check_swiglu_clamped(orc):
    """Clamped SwiGLU: textbook sigmoid values where the gate is capped and where it
    is not, the up clip on both sides, a zero limit, and limit = +inf and
    in-range inputs reducing to the plain SwiGLU."""
    sig1 = 0.7310585786300049      # 1 / (1 + e^-1)
    sigm3 = 0.04742587317756678    # 1 / (1 + e^3)
    # rows of [g | u] with I = 1
    gu = np.array([[50.0, 5.0],     # g capped to 1, u clipped to 1: silu(1) * 1 = sigma(1)
                   [50.0, -5.0],    # u clipped to -1 from below
                   [-3.0, -0.5],    # nothing clamped (g below the cap, |u| < 1): silu(-3) * -0.5
                   [1.0, 1.0]])     # exactly at the limit: unchanged
    h = orc.swiglu_clamped(gu, 1.0)[:, 0]
    assert h[0] == pytest.approx(sig1, rel=1e-15)
    assert h[1] == pytest.approx(-sig1, rel=1e-15)
    assert h[2] == pytest.approx(-3.0 * sigm3 * -0.5, rel=1e-14)
    assert h[3] == pytest.approx(sig1, rel=1e-15)
    rng = np.random.default_rng(9)
    big = rng.standard_normal((7, 10)) * 20
    assert np.all(orc.swiglu_clamped(big, 0.0) == 0.0)                         # u clipped to 0
    assert np.array_equal(orc.swiglu_clamped(big, np.inf), orc.swiglu(big))  # no clamp
    small = rng.uniform(-0.9, 0.9, (7, 10))
    assert np.array_equal(orc.swiglu_clamped(small, 1.0), orc.swiglu(small))  # inside the limits
    with pytest.raises(RuntimeError):
        orc.swiglu_clamped(small, -1.0)


# --------------------------------------------------------------------------------------
# tests
# --------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def test_topk_brute_force(orc):
    check_topk_brute_force(orc)


def test_topk_lexsort(orc):
    check_topk_lexsort(orc)


def test_topk_special_cases(orc):
    check_topk_special_cases(orc)


def test_softmax_weights(orc):
    check_softmax_weights(orc)


def test_layout(orc):
    check_layout_cases(orc)


def test_gather(orc):
    check_gather(orc)


def test_dense_swiglu_reduction(orc):
    check_dense_swiglu_reduction(orc)


@pytest.mark.parametrize("cfg", [gen.CONFIGS["tiny"],
                                 gen.CONFIGS["tiny"].with_(name="tiny_hot", weight_std=0.2, seed=10),
                                 gen.MoEConfig("odd", 37, 64, 5, 3, 64, 6, "gaussian")])
def test_dense_masked(orc, cfg):
    check_dense_masked(orc, cfg)


def test_structured_closed_form(orc):
    check_structured_closed_form(orc)


def test_steps_compose(orc):
    check_steps_compose(orc)


def test_identity_experts(orc):
    check_identity_experts(orc)


def test_linearity_and_symmetry(orc):
    check_linearity_and_symmetry(orc)


def test_fp8_decode(orc):
    check_fp8_decode(orc)


def test_fp8_encode(orc):
    check_fp8_encode(orc)


def test_fp8_quantize(orc):
    check_fp8_quantize(orc)


def test_glu_down_w64(orc):
    check_glu_down_w64(orc)


def test_backward_finite_differences(orc):
    check_backward_finite_differences(orc)


def test_backward_steps_compose(orc):
    check_backward_steps_compose(orc)


def test_backward_invariants(orc):
    check_backward_invariants(orc)


def test_swiglu_bwd_derivative(orc):
    check_swiglu_bwd_derivative(orc)


def test_router_logits(orc):
    """The router projection against numpy's float64 matmul, and against the
    generator's own logits for the projection-routed config (which sums in
    another order and rounds once to fp32: at most one fp32 ulp apart)."""
    rng = np.random.default_rng(8)
    x = gen.random_bf16((33, 96), seed=8)
    w = rng.standard_normal((96, 20)).astype(np.float32) * np.float32(0.05)
    ref = f32(x).astype(np.float64) @ w.astype(np.float64)
    assert np.allclose(orc.router_logits(x, w), ref, rtol=1e-13, atol=1e-15)
    cfg = gen.CONFIGS["tiny"]
    d = gen.make_inputs(cfg)
    lg = orc.router_logits(d["x"], gen.draw_router_weight(cfg)).astype(np.float32)
    ulp = np.spacing(np.abs(d["logits"]))
    assert np.all(np.abs(lg - d["logits"]) <= ulp)


def test_rejects_bad_inputs(orc):
    bad = np.zeros((2, 4), np.float32)
    bad[1, 2] = np.inf
    with pytest.raises(oracle.OracleError):
        orc.route_topk(bad, 2)
    with pytest.raises(oracle.OracleError):
        orc.layout(np.array([[0, 7]], np.int32), 4, 8)


# ---- figures the pages print --------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        return json.load(f)


def test_uniform_routing_distinct_experts(orc):
    """Gaussian logits + top-10 of 512: 8 tokens touch 74.7 distinct experts
    (closed form 512 * (1 - (1 - 10/512)^8) = 74.74)."""
    page = _golden()["distinct_experts_8_tokens_top10_of_512"]["value"]
    closed = 512 * (1 - (1 - 10 / 512) ** 8)
    assert abs(closed - page) < 0.05
    cfg = gen.MoEConfig("u", 8 * 1500, 64, 512, 10, 64, 77, "gaussian")
    idx, _ = orc.route_topk(gen.draw_logits(cfg), 10)
    distinct = [len(np.unique(idx[g * 8:(g + 1) * 8])) for g in range(1500)]
    assert abs(np.mean(distinct) - page) < 0.3


def test_expert_size_and_flop_accounting():
    g = _golden()
    cfg = gen.CONFIGS["fine_grained_512"]
    mib = 3 * cfg.H * cfg.I * 2 / 2 ** 20
    assert mib == g["bf16_expert_mib_512_expert_layer"]["value"]
    # the routed-MoE floor on the page: 1.326 s over 48 layers, one quarter of the
    # 8192-token layer's flops per rank at the measured 7.50 TFLOP/s bf16 GEMM roof
    f = g["routed_moe_floor_ms_per_layer_per_rank"]
    assert abs(f["total_s"] / f["layers"] * 1e3 - f["value"]) < 0.05
    per_rank_s = accounting.layer_flops(cfg.T, cfg.H, cfg.k, cfg.I) / f["ranks"] / (f["bf16_gemm_tflops"] * 1e12)
    assert abs(per_rank_s * 1e3 - f["value"]) / f["value"] < 0.05


def test_skew_generator(orc):
    """Zipf(1.2) bias: a heavy max load, close to its bound E/k (a token takes an
    expert at most once), with many near-idle experts.  Real routers reach ~20x
    the mean at other shapes (the page's figure)."""
    cfg = gen.CONFIGS["skewed_zipf"]
    idx, _ = orc.route_topk(gen.draw_logits(cfg), cfg.k)
    counts = np.bincount(idx.reshape(-1), minlength=cfg.E)
    mean = cfg.T * cfg.k / cfg.E
    assert 12 < counts.max() / mean <= cfg.E / cfg.k
    assert (counts <= 32).sum() >= 20
    assert np.sort(counts)[::-1][:8].sum() > 0.5 * cfg.T * cfg.k


def test_gaussian_generator_balanced(orc):
    cfg = gen.CONFIGS["qwen3_30b_a3b"]
    idx, _ = orc.route_topk(gen.draw_logits(cfg), cfg.k)
    counts = np.bincount(idx.reshape(-1), minlength=cfg.E)
    assert counts.min() > 400 and counts.max() < 640  # mean 512, binomial spread


def test_swiglu_clamped(orc):
    check_swiglu_clamped(orc)
