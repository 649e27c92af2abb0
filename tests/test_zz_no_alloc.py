"""moe_expert_ffn_noalloc (the routed FFN on the library's own device scratch
array, for callers that cannot allocate) against moe_expert_ffn on a caller
workspace, through the C-ABI: bit for bit, on two calls in a row with the
second smaller, on the decode and the prefill kernels."""
import numpy as np
import pytest
import torch

from block_scaled_fp8xfp4_amd import mxmoe
from block_scaled_fp8xfp4_amd.layer import ExpertFFN
from gpu_common import dev, moe_workload, say

pytestmark = pytest.mark.gpu


def run_pair(layer, rows, path):
    """y from moe_expert_ffn (workspace) and from moe_expert_ffn_noalloc on the same rows."""
    c = layer.cfg
    d = layer.d
    idx = dev(np.asarray(rows, np.int64))
    x, xs = d["x"][idx].contiguous(), d["x_sc"][idx].contiguous()
    route = layer.gpu_route(rows)
    T = len(rows)
    old = mxmoe.set_ffn_path(path)
    try:
        ffn = ExpertFFN(T, c.H, c.E, c.I, c.k)
        y_ws = ffn(x, xs, route, d["w13"], d["w13_sc"], d["w2"], d["w2_sc"]).clone()
        v_ws = mxmoe.last_variant()
        y = torch.full((T, c.H), float("nan"), dtype=torch.float32, device="cuda")
        mxmoe.moe_expert_ffn_noalloc(x, xs, route.w, route.offsets, route.perm, route.slot_pos, c.k, d["w13"],
                                     d["w13_sc"], d["w2"], d["w2_sc"], c.E, c.I, y)
        v = mxmoe.last_variant()
    finally:
        mxmoe.set_ffn_path(old)
    assert v == v_ws, (v, v_ws)
    torch.cuda.synchronize()
    return y, y_ws, v


@pytest.mark.parametrize("path", [1, 2])
def test_noalloc_matches_workspace_entry_point(path):
    inp, r, layer = moe_workload("verify")
    T = inp.cfg.T
    for rows in (np.arange(T), np.array([3, 17, 40, 41, 5])):            # second call smaller
        y, y_ws, v = run_pair(layer, rows, path)
        assert torch.equal(y.view(torch.int32), y_ws.view(torch.int32)), (path, len(rows))
        say(f"noalloc path {path}, {len(rows)} rows ({v}): bitwise equal to the workspace entry point")


def test_noalloc_limit():
    assert mxmoe.moe_expert_ffn_noalloc_max_bytes() == 16 << 20
    assert mxmoe.moe_expert_ffn_workspace_bytes(48, 4096, 256, 576, 16) <= 16 << 20
