"""Algorithmic work of each step of the routed-expert layer: the flops and HBM
bytes the method itself needs, used to place measured kernel times on the
MI355X roofline.

Flops count routed rows only: 2 flops per multiply-add, so the two expert GEMMs
are 4*R*H*I (gate and up) and 2*R*H*I (down), 6*R*H*I in all -- twice the active
expert parameters per routed token, the 6*N*D forward-and-backward rule's
forward third [prime-rl PR 3885, Pipeline-parallel push: MFU is 6ND].  Pad rows
of the layout are not counted as flops.

Bytes count each buffer once at its algorithmic size: every active expert's
weights read once (an expert with no rows reads none [PocketLLM "Qwen4-Exp
Heterogeneous TP4 Performance", Confirmed architecture decisions: active-only
traffic]), the activation buffers each written once and read once, the index
maps once.  P below is the number of rows actually used by the padded layout
(offsets[E]); it includes pad rows because they are written and read.

Variants: FP8 expert weights count one byte per weight plus a 4-byte scale per
64 rows; the fused gather (layout-only permute, gate/up GEMM reading token rows
in place) moves no x_perm, and its GEMM reads x once.
"""
from __future__ import annotations

from dataclasses import dataclass

# MI355X published peaks (dense, no sparsity).
PEAK_HBM_BYTES_PER_S = 8.0e12
PEAK_BF16_FLOPS = 2.5e15


@dataclass(frozen=True)
class StepWork:
    name: str
    flops: float
    bytes: float

    def roofline_seconds(self, peak_flops=PEAK_BF16_FLOPS, peak_bw=PEAK_HBM_BYTES_PER_S) -> float:
        return max(self.flops / peak_flops, self.bytes / peak_bw)

    def bound(self, peak_flops=PEAK_BF16_FLOPS, peak_bw=PEAK_HBM_BYTES_PER_S) -> str:
        return "mfma" if self.flops / peak_flops >= self.bytes / peak_bw else "hbm"


def layer_flops(T: int, H: int, k: int, I: int) -> float:
    """Forward flops of the routed experts: 6 * T * k * H * I."""
    return 6.0 * T * k * H * I


def step_work(T: int, H: int, E: int, k: int, I: int, P: int, active_experts: int,
              fp8_weights: bool = False, fused_gather: bool = False):
    """Per-step algorithmic work for one layer call (list of StepWork, path order)."""
    R = T * k
    bf, i32, f32 = 2, 4, 4
    # bytes of one expert's gate/up and down weights
    if fp8_weights:
        w_gu_bytes = 2 * I * H + (2 * I // 64) * f32
        w_d_bytes = H * I + (H // 64) * f32
    else:
        w_gu_bytes = 2 * I * H * bf
        w_d_bytes = H * I * bf
    route = StepWork("route_topk", 0.0, T * E * f32 + R * (i32 + f32))
    x_moved = 0 if fused_gather else T * H * bf + P * H * bf  # x read, x_perm written
    permute = StepWork(
        "permute",
        0.0,
        R * i32            # topk_idx read
        + x_moved
        + R * i32          # route_row written
        + P * i32          # row_token written
        + (2 * E + 1) * i32,
    )
    # gate/up A operand: x_perm (pad rows included), or x itself read once plus row_token
    a_bytes = T * H * bf + P * i32 if fused_gather else P * H * bf
    glu = StepWork(
        "grouped_glu_gemm",
        4.0 * R * H * I,
        active_experts * w_gu_bytes + a_bytes + P * I * bf + (2 * E + 1) * i32,
    )
    down = StepWork(
        "grouped_down_gemm",
        2.0 * R * H * I,
        active_experts * w_d_bytes + P * I * bf + P * H * bf + (2 * E + 1) * i32,
    )
    combine = StepWork("combine", 0.0, R * H * bf + R * (i32 + f32) + T * H * bf)
    return [route, permute, glu, down, combine]


def training_work(T: int, H: int, E: int, k: int, I: int, P: int, active_experts: int,
                  fused_swiglu_backward: bool = False):
    """Per-kernel algorithmic work of one training step (forward that keeps its
    gate/up output, then the backward), in launch order. Weight gradients are
    fp32 (4 bytes per element), everything else as in step_work. With the fused
    SwiGLU backward, dh = dy W_d and its SwiGLU backward are one kernel that reads
    dy, W_d and gu and writes dgu (dh never reaches memory)."""
    R = T * k
    bf, i32, f32 = 2, 4, 4
    wgu = active_experts * 2 * I * H
    wd = active_experts * H * I
    maps = (2 * E + 1) * i32
    fwd = step_work(T, H, E, k, I, P, active_experts)
    route, permute, _, down, combine = fwd
    return [
        route, permute,
        StepWork("gate_up_gemm", 4.0 * R * H * I, wgu * bf + P * H * bf + P * 2 * I * bf + maps),
        StepWork("swiglu", 0.0, P * 2 * I * bf + P * I * bf),
        down, combine,
        StepWork("combine_backward", 0.0, T * H * bf + R * H * bf + P * H * bf + R * (2 * i32 + 2 * f32)),
        StepWork("route_backward", 0.0, R * (i32 + 2 * f32) + T * E * f32),
    ] + ([
        StepWork("dgrad_down_swiglu_backward", 2.0 * R * H * I, wd * bf + P * H * bf + 2 * P * 2 * I * bf + maps),
    ] if fused_swiglu_backward else [
        StepWork("dgrad_down", 2.0 * R * H * I, wd * bf + P * H * bf + P * I * bf + maps),
        StepWork("swiglu_backward", 0.0, P * I * bf + 2 * P * 2 * I * bf),
    ]) + [
        StepWork("dgrad_gate_up", 4.0 * R * H * I, wgu * bf + P * 2 * I * bf + P * H * bf + maps),
        StepWork("permute_backward", 0.0, R * H * bf + R * i32 + T * H * bf),
        StepWork("wgrad_down", 2.0 * R * H * I, P * H * bf + P * I * bf + wd * f32 + maps),
        StepWork("wgrad_gate_up", 4.0 * R * H * I, P * 2 * I * bf + P * H * bf + wgu * f32 + maps),
    ]
