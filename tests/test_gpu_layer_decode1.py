"""moe_layer_decode1 (the gate inside the gate/up kernel, one row) against
moe_route followed by moe_expert_ffn: bit for bit on every route output and
on y, live and dead rows, ties, and several layer shapes; and against the
oracle end to end."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp8xfp4_amd import mxmoe, synth
from block_scaled_fp8xfp4_amd.layer import ExpertFFN, Route
from gpu_common import Layer, assert_close, dev, host, say, small_workload

pytestmark = pytest.mark.gpu


def run_both(layer, logits, survival=None, skip=0.2):
    c = layer.cfg
    E, k, H, I = c.E, c.k, c.H, c.I
    d = layer.d
    x, xs = d["x"][:1].contiguous(), d["x_sc"][:1].contiguous()
    lg = dev(np.ascontiguousarray(logits[:1], np.float32))
    sv = None if survival is None else dev(np.ascontiguousarray(survival[:1], np.float32))
    route = Route(1, E, k)
    route(lg, sv, skip)
    ffn = ExpertFFN(1, H, E, I, k)
    y_ref = ffn(x, xs, route, d["w13"], d["w13_sc"], d["w2"], d["w2_sc"])
    fused = Route(1, E, k)
    fused.ids.fill_(-7)
    fused.offsets.fill_(-7)
    y = torch.full((1, H), 7.0, device="cuda")
    ws = torch.empty(mxmoe.moe_expert_ffn_workspace_bytes(1, H, E, I, k), dtype=torch.uint8, device="cuda")
    mxmoe.moe_layer_decode1(lg, k, sv, skip, x, xs, d["w13"], d["w13_sc"], d["w2"], d["w2_sc"], E, I, fused.ids,
                            fused.w, fused.offsets, fused.perm, fused.slot_pos, y, ws)
    assert mxmoe.last_variant().startswith("layer1:")
    for key in ("ids", "w", "offsets", "perm", "slot_pos"):
        assert torch.equal(getattr(fused, key), getattr(route, key)), key
    assert torch.equal(y, y_ref)
    return host(y), route


def test_decode_workload_bitwise_and_oracle():
    from gpu_common import moe_workload
    inp, r, layer = moe_workload("decode")
    y, route = run_both(layer, inp.logits)
    ref = layer.oracle_y(r)
    err, cos = assert_close(y, ref, "layer_decode1 end to end")
    say(f"layer_decode1: end-to-end {err:.2e}, cosine {cos:.8f}")


@pytest.mark.parametrize("shape", [
    dict(seed=41, T=1, H=256, E=8, k=2, I=64),
    dict(seed=42, T=1, H=1152, E=384, k=8, I=96),                # 6 logits per lane, a non-exact step count
    dict(seed=43, T=1, H=512, E=64, k=16, I=160),
])
def test_small_shapes(shape):
    inp, r, layer = small_workload(**shape)
    run_both(layer, inp.logits)


def test_dead_row_and_ties():
    inp, r, layer = small_workload(seed=44, T=1, H=256, E=32, k=4, I=64)
    y, route = run_both(layer, inp.logits, np.array([0.1], np.float32), 0.2)   # dead: no bucket, y = +0
    assert not np.any(y) and not np.any(np.signbit(y))
    assert not host(route.offsets).any() and np.all(host(route.slot_pos) == -1)
    ties = np.zeros((1, 32), np.float32)                       # all equal: experts 0..k-1
    y, route = run_both(layer, ties, np.array([0.9], np.float32), 0.2)
    assert np.array_equal(host(route.ids)[0], np.arange(4))
