"""Helpers for the GPU parity tests: moving seeded numpy inputs to the device and
results back, and the comparison rules.

Comparison rules (per element, over the compared region):
  * index and layout arrays, and bit copies: equal bit for bit;
  * topk_w: |gpu - ref| <= 1e-6;
  * bf16 outputs: |gpu - ref| <= 1e-2 * max|ref| + 1e-3 (the gate), and, for a
    single step, also max|gpu - ref| <= 2^-8 * max|ref|: one step rounds its
    result to bf16 once (at most half an ulp, 2^-9 of the value) on top of fp32
    sums whose error is orders of magnitude smaller, so any larger error is a
    real mistake.  The whole layer rounds three times (h, y, out) and is held to
    the gate only.
"""
from __future__ import annotations

import numpy as np
import torch

from mixture_experts_routed_router_amd import inputs as gen


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return gen.bf16_bits_to_f32(host_bits(t)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def assert_close_bf16(gpu: np.ndarray, ref: np.ndarray, what: str, tight: bool = True) -> float:
    """Returns max|gpu-ref| / max|ref|."""
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite values"
    err = np.abs(gpu - ref)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    bound = 1e-2 * scale + 1e-3
    worst = float(err.max()) if err.size else 0.0
    assert worst <= bound, f"{what}: max|d| = {worst:.3e} > 1e-2*max|ref| + 1e-3 = {bound:.3e}"
    if tight and scale > 0:
        assert worst <= 2.0 ** -8 * scale, f"{what}: max|d|/max|ref| = {worst / scale:.3e} > 2^-8"
    return worst / scale if scale > 0 else 0.0


def sample_tokens(T: int, n: int, seed: int) -> np.ndarray:
    if n >= T:
        return np.arange(T)
    rng = np.random.default_rng([seed, 99])
    pick = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.sort(np.concatenate([[0, T - 1], pick]))
