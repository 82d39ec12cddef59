"""The allocation-free permute (moe_permute_noalloc) against moe_permute with a
workspace: the same layout and x_perm bit for bit, on two calls in a row (the
second smaller, so the fixed scratch holds the first call's histogram when the
second starts), and the size limit rejected on the host."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mixture_experts_routed_router_amd import inputs as gen
from gpu_util import dev, dev_bf16, host_bits

pytestmark = pytest.mark.gpu


def _case(lib, T, H, E, k, align, seed):
    x = dev_bf16(gen.random_bf16((T, H), seed=seed))
    logits = np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)
    idx, _ = lib.route_topk(dev(logits), k)
    P_max = lib.padded_rows_max(T, k, E, align)
    ref = lib.permute(x, idx, E, align, P_max)
    out = lib.alloc_layout(T, H, E, k, P_max, "cuda")
    lib.permute_noalloc(x, idx, E, align, out)
    torch.cuda.synchronize()
    return ref, out


def _same(ref, out):
    for name in ("counts", "offsets", "route_row", "row_token"):
        assert torch.equal(getattr(ref, name), getattr(out, name)), name
    used = int(ref.offsets[-1].item())
    assert (host_bits(ref.x_perm[:used]) == host_bits(out.x_perm[:used])).all()


def test_permute_noalloc_matches_permute(gpu_lib):
    print("no-alloc permute: 8192 x 2048, E 128, k 8, then 1000 x 256, E 40, k 5", flush=True)
    ref, out = _case(gpu_lib, 8192, 2048, 128, 8, 32, seed=1)
    _same(ref, out)
    ref, out = _case(gpu_lib, 1000, 256, 40, 5, 8, seed=2)   # smaller: stale scratch from the first call
    _same(ref, out)


def test_permute_noalloc_rejects_oversize(gpu_lib):
    cap = gpu_lib.permute_noalloc_max_workspace()
    T, H, E, k = 600000, 64, 1024, 8   # ceil(T*k/256) * E * 4 bytes > 4 MiB
    assert gpu_lib.permute_workspace_size(T, k, E) > cap
    x = torch.empty((1, H), dtype=torch.bfloat16, device="cuda")  # never read: rejected on the host
    idx = torch.empty((1, k), dtype=torch.int32, device="cuda")
    P_max = gpu_lib.padded_rows_max(T, k, E, 32)
    out = gpu_lib.Layout(torch.empty(E, dtype=torch.int32, device="cuda"),
                         torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                         torch.empty(T * k, dtype=torch.int32, device="cuda"),
                         torch.empty(P_max, dtype=torch.int32, device="cuda"), None, P_max)
    with pytest.raises(gpu_lib.MoEError, match="WORKSPACE_TOO_SMALL"):
        gpu_lib._call("moe_permute_noalloc", x.data_ptr(), idx.data_ptr(), T, H, E, k, 32, P_max,
                      out.counts.data_ptr(), out.offsets.data_ptr(), out.route_row.data_ptr(),
                      out.row_token.data_ptr(), None, None)
