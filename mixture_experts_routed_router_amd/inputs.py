"""Seeded synthetic inputs for the routed-expert MoE layer.

This module draws inputs only; it holds none of the layer's arithmetic, and it
is the one piece that both the GPU path's tests/bench and the CPU oracle use.

Shapes, distributions and seeds (one config per workload the pages discuss):

* ``tiny``           T=64, H=128, E=8, k=2, I=256.  x ~ N(0,1) bf16; router
  weight W_r ~ N(0,0.02) fp32 and logits = x W_r (fp32, computed here once, in
  float64 then rounded, so the bits do not depend on the host's BLAS).
* ``qwen3_30b_a3b``  T=8192, H=2048, E=128, k=8, I=768 (a Qwen3-30B-A3B-shaped
  layer at M >= 8k rows [Halo "Performance", Rough numbers]).
* ``gpt_oss_20b_small_m`` T=128, H=2880, E=32, k=4, I=2880 (GPT-OSS-20B-shaped
  experts with few rows each: weight-bandwidth-bound [Halo "Performance", Levers
  that do not help here]).
* ``fine_grained_512`` T=8192, H=2560, E=512, k=10, I=640 (the 512-expert top-10
  layer of one 8192-token prefill chunk; one bf16 expert = 3*2560*640*2 B =
  9.375 MiB [PocketLLM "Qwen4-Exp Heterogeneous TP4 Performance", Runtime
  architecture]).
* ``skewed_zipf``    the Qwen3-30B-A3B shape at T=32768 with router logits
  N(0,1) + ln p(rank(e)), p(r) proportional to r^-1.2 over a seeded expert
  ranking, so a few experts take most rows (real routers reach a max expert load
  of ~20x the mean [prime-rl PR 3885, Earlier results]).

For every config but ``tiny`` the logits are drawn directly, iid N(0,1) fp32, so
each token's top-k set is a uniform k-subset.  Expert weights are N(0,0.02) bf16,
never zeros (zero weights made kernels look 1.5-3.5x too fast [prime-rl PR 3885,
Changes: debug.random_init]).  Draws are fp32 rounded to bf16 (round to nearest
even).  Every array comes from its own ``numpy.random.default_rng([seed, stream,
index])`` stream, so results do not depend on thread count or draw order.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, replace

import numpy as np

WEIGHT_STD = 0.02

_S_X, _S_ROUTER, _S_WGU, _S_WD, _S_RANK = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    seed: int
    router: str  # "projection" | "gaussian" | "zipf"
    zipf_s: float = 1.2
    weight_std: float = WEIGHT_STD
    align: int = 32

    @property
    def R(self) -> int:
        return self.T * self.k

    @property
    def P_max(self) -> int:
        return self.T * self.k + self.E * (self.align - 1)

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


CONFIGS = {
    "tiny": MoEConfig("tiny", 64, 128, 8, 2, 256, 0, "projection"),
    "qwen3_30b_a3b": MoEConfig("qwen3_30b_a3b", 8192, 2048, 128, 8, 768, 1, "gaussian"),
    "gpt_oss_20b_small_m": MoEConfig("gpt_oss_20b_small_m", 128, 2880, 32, 4, 2880, 2, "gaussian"),
    "fine_grained_512": MoEConfig("fine_grained_512", 8192, 2560, 512, 10, 640, 3, "gaussian"),
    "skewed_zipf": MoEConfig("skewed_zipf", 32768, 2048, 128, 8, 768, 4, "zipf"),
}


def _rng(seed: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, stream, index])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns the raw uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bits to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return f32_to_bf16_bits(a)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def draw_x(cfg: MoEConfig) -> np.ndarray:
    return _normal_bf16(_rng(cfg.seed, _S_X), (cfg.T, cfg.H), 1.0)


def draw_router_weight(cfg: MoEConfig) -> np.ndarray:
    """The router weight W_r [H, E] fp32 ~ N(0, weight_std) (the one the
    "projection" configs form their logits from)."""
    rng = _rng(cfg.seed, _S_ROUTER)
    return rng.standard_normal(size=(cfg.H, cfg.E), dtype=np.float32) * np.float32(cfg.weight_std)


def draw_logits(cfg: MoEConfig, x_bits: np.ndarray | None = None) -> np.ndarray:
    rng = _rng(cfg.seed, _S_ROUTER)
    if cfg.router == "projection":
        if x_bits is None:
            x_bits = draw_x(cfg)
        w_r = draw_router_weight(cfg)
        # Router projection (outside the layer's path): exact products in float64,
        # numpy's fixed pairwise summation, then one rounding to float32.
        prod = bf16_bits_to_f32(x_bits).astype(np.float64)[:, :, None] * w_r.astype(np.float64)[None]
        return prod.sum(axis=1).astype(np.float32)
    logits = rng.standard_normal(size=(cfg.T, cfg.E), dtype=np.float32)
    if cfg.router == "zipf":
        rank = _rng(cfg.seed, _S_RANK).permutation(cfg.E) + 1  # expert e has rank rank[e]
        p = rank.astype(np.float64) ** (-cfg.zipf_s)
        p /= p.sum()
        logits = (logits.astype(np.float64) + np.log(p)[None, :]).astype(np.float32)
    elif cfg.router != "gaussian":
        raise ValueError(f"unknown router kind {cfg.router!r}")
    return logits


def draw_expert_weights(cfg: MoEConfig):
    """w_gu bits [E, 2I, H] (rows [0,I) gate, [I,2I) up) and w_d bits [E, H, I]."""
    E, H, I = cfg.E, cfg.H, cfg.I
    w_gu = np.empty((E, 2 * I, H), np.uint16)
    w_d = np.empty((E, H, I), np.uint16)

    def fill(e):
        w_gu[e] = _normal_bf16(_rng(cfg.seed, _S_WGU, e), (2 * I, H), cfg.weight_std)
        w_d[e] = _normal_bf16(_rng(cfg.seed, _S_WD, e), (H, I), cfg.weight_std)

    with _cf.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(E)))
    return w_gu, w_d


def make_inputs(cfg: MoEConfig | str) -> dict:
    """All inputs of one layer call: x bits [T,H], logits f32 [T,E], w_gu, w_d bits."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    x = draw_x(cfg)
    logits = draw_logits(cfg, x)
    w_gu, w_d = draw_expert_weights(cfg)
    return {"cfg": cfg, "x": x, "logits": logits, "w_gu": w_gu, "w_d": w_d}


# ---- structured routing cases (test-only structures; fed straight to the permute) ----

def balanced_topk_idx(T: int, E: int, k: int, stride: int = 97) -> np.ndarray:
    """idx[t,j] = ((t*k + j) * stride) mod E: experts strided by 97 (spread balanced
    routing [prime-rl PR 3885, Changes]); distinct per token when gcd(stride, E) = 1."""
    r = np.arange(T * k, dtype=np.int64)
    return ((r * stride) % E).astype(np.int32).reshape(T, k)


def tied_logits(T: int, E: int, seed: int, levels: int = 3) -> np.ndarray:
    """Logits drawn from a few values (including +0 and -0) so exact ties are common."""
    rng = _rng(seed, 7)
    vals = np.array([0.0, -0.0, 1.5, -2.25, 0.75][: max(2, levels)], np.float32)
    return vals[rng.integers(0, len(vals), size=(T, E))]


def random_bf16(shape, seed: int, std: float = 1.0, stream: int = 8) -> np.ndarray:
    return _normal_bf16(_rng(seed, stream), shape, std)
