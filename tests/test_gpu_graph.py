"""The five-call layer captured as a HIP graph (MoELayer.graph): every replay,
with new inputs copied in and eager layer calls and synchronizations between
replays, equals the eager layer on the same inputs bit for bit (every kernel is
deterministic, so the two runs compute the same bits)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mixture_experts_routed_router_amd import inputs as gen
from gpu_util import dev, dev_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("tiled", [False, True], ids=["row_major", "tiled"])
@pytest.mark.parametrize("fused_gather", [False, True], ids=["five_call", "fused_gather"])
def test_layer_graph_replay(gpu_lib, fused_gather, tiled):
    T, H, E, k, I = 300, 256, 16, 4, 192
    print(f"graph replay fused_gather={fused_gather} tiled={tiled}", flush=True)
    rng = np.random.default_rng(5)
    w_gu = dev_bf16(gen.random_bf16((E, 2 * I, H), seed=1, std=0.05))
    w_d = dev_bf16(gen.random_bf16((E, H, I), seed=2, std=0.05))
    if tiled:
        w_gu, w_d = gpu_lib.tile_weights(w_gu), gpu_lib.tile_weights(w_d)
    xs = [gen.random_bf16((T, H), seed=10 + i) for i in range(3)]
    lgs = [rng.standard_normal((T, E)).astype(np.float32) for _ in range(3)]

    layer = gpu_lib.MoELayer(T, H, E, k, I, fused_gather=fused_gather, tiled=tiled)
    x_buf, lg_buf = dev_bf16(xs[0]), dev(lgs[0])
    g = layer.graph(x_buf, lg_buf, w_gu, w_d)
    eager = gpu_lib.MoELayer(T, H, E, k, I, fused_gather=fused_gather, tiled=tiled)
    for i in range(3):
        x_buf.copy_(dev_bf16(xs[i]))
        lg_buf.copy_(dev(lgs[i]))
        g.replay()
        got = layer.out.clone()
        ref = eager(dev_bf16(xs[i]), dev(lgs[i]), w_gu, w_d).clone()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
