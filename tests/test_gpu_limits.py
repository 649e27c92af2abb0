"""The kernels at the largest shapes they accept: the decode path's largest
intermediate (I = 2048: the 16-step down kernels, on one row and on several),
the most experts and the largest top-k of the single-row layer (E = 1024,
k = 16), and the dense GEMM's largest K (16 384 = 16 canonical parts) on both
kernels; against the oracle, and the single-row layer bitwise against
moe_route + moe_expert_ffn (forum thread post #6, "How it works": the routed
experts and the MXFP8 projections; the limits are the ones include/mxmoe.h
documents)."""
import numpy as np
import pytest

from block_scaled_fp8xfp4_amd import mxmoe
from gpu_common import ffn_parity, say, small_workload
from test_gpu_layer_decode1 import run_both
from test_gpu_parity import check_gemm, gemm_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,variant", [(3, "ffn:gu_decode+down_decode+combine"), (1, "ffn:gu1_decode+down_combine1")])
def test_ffn_largest_intermediate(T, variant):
    inp, r, layer = small_workload(seed=70 + T, T=T, H=512, E=8, k=2, I=2048)
    say(f"ffn I=2048 T={T}")
    ffn_parity(inp, r, layer, what=f"I=2048 T={T}", path=1)
    assert mxmoe.last_variant() == variant


@pytest.mark.parametrize("shape", [dict(seed=75, T=1, H=256, E=1024, k=16, I=64),    # most experts, largest k
                                   dict(seed=76, T=1, H=512, E=16, k=4, I=2048)])    # largest intermediate
def test_layer_decode1_limits(shape):
    """The row's route + FFN against the oracle (staged), then the fused
    single-row layer bitwise against moe_route + moe_expert_ffn."""
    inp, r, layer = small_workload(**shape)
    say(f"layer_decode1 {shape}")
    y = ffn_parity(inp, r, layer, what=str(shape), path=1)
    y_fused, _ = run_both(layer, inp.logits)
    assert np.array_equal(y_fused.view(np.uint32), np.asarray(y, np.float32).view(np.uint32))


@pytest.mark.parametrize("M,prefix", [(2, "gemm:decode"), (320, "gemm:prefill")])
def test_gemm_largest_k(M, prefix):
    a, w = gemm_case(M, 64, 16384, 900 + M)
    rows = None if M < 16 else np.array([0, 1, 159, 318, 319], np.int32)
    check_gemm(a, w, rows=rows)
    assert mxmoe.last_variant().startswith(prefix)


@pytest.mark.parametrize("path", [1, 2])
def test_ffn_all_rows_dead(path):
    """A batch whose rows all skip the routed experts: no pair is bucketed, no
    expert item runs, and y is +0 everywhere (no sign bit), on both paths; the
    output buffer starts as garbage."""
    import torch
    from block_scaled_fp8xfp4_amd.layer import ExpertFFN, Route
    from gpu_common import dev, host
    inp, r, layer = small_workload(seed=77, T=40, H=256, E=16, k=4, I=64)
    c = layer.cfg
    route = Route(c.T, c.E, c.k)
    route(dev(inp.logits), dev(np.full(c.T, 0.1, np.float32)))
    assert not host(route.offsets).any() and np.all(host(route.slot_pos) == -1)
    ffn = ExpertFFN(c.T, c.H, c.E, c.I, c.k)
    ffn.y.fill_(float("nan"))
    old = mxmoe.set_ffn_path(path)
    try:
        y = ffn(layer.d["x"], layer.d["x_sc"], route, layer.d["w13"], layer.d["w13_sc"], layer.d["w2"], layer.d["w2_sc"])
    finally:
        mxmoe.set_ffn_path(old)
    yh = host(y)
    assert not np.any(yh) and not np.any(np.signbit(yh)), "dead rows must give +0"
