"""The hot path replayed from a HIP graph: route, expert FFN and the dense
projection captured once on the decode and verification workloads, replayed
several times with eager work and synchronizations between the replays; every
replay must give the eager results bit for bit (the library records kernels
only: no allocation, memset or host synchronization inside a call)."""
import numpy as np
import pytest
import torch

from block_scaled_fp8xfp4_amd import mxmoe, synth
from block_scaled_fp8xfp4_amd.layer import ExpertFFN, Route, quantize
from gpu_common import dev, host, moe_workload, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,fused", [("decode", False), ("decode", True), ("verify", False)])
def test_graph_replays_match_eager(name, fused):
    inp, r, layer = moe_workload(name)
    c = inp.cfg
    say(f"graph replay: {name}")
    logits = dev(inp.logits)
    surv = None if inp.survival is None else dev(inp.survival)
    d = synth.dense_inputs()
    g_q, g_sc = quantize(dev(d.w), mxmoe.MX_FMT_E4M3)
    a = np.resize(d.a, (c.T, d.cfg.K))
    a_q, a_sc = quantize(dev(a).to(torch.bfloat16).contiguous(), mxmoe.MX_FMT_E4M3)
    route = Route(c.T, c.E, c.k)
    ffn = ExpertFFN(c.T, c.H, c.E, c.I, c.k)
    yg = torch.empty((c.T, d.cfg.N), dtype=torch.bfloat16, device="cuda")
    L = layer.d

    def step():
        if fused:                                        # one row: the gate inside the gate/up kernel
            mxmoe.moe_layer_decode1(logits, c.k, surv, 0.2, L["x"], L["x_sc"], L["w13"], L["w13_sc"], L["w2"],
                                    L["w2_sc"], c.E, c.I, route.ids, route.w, route.offsets, route.perm,
                                    route.slot_pos, ffn.y, ffn.ws)
        else:
            route(logits, surv)
            ffn(L["x"], L["x_sc"], route, L["w13"], L["w13_sc"], L["w2"], L["w2_sc"])
        mxmoe.fp8_block_gemm(a_q, a_sc, g_q, g_sc, yg, mxmoe.MX_OUT_BF16)

    step()
    eager = [host(t).copy() for t in (route.ids, route.w, route.offsets, route.perm, route.slot_pos, ffn.y, yg.view(torch.int16))]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    outs = (route.ids, route.w, route.offsets, route.perm, route.slot_pos, ffn.y, yg.view(torch.int16))
    for rep in range(4):
        for t in outs:                                   # eager work between replays
            t.fill_(-1 if t.dtype in (torch.int32, torch.int16) else float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        got = [host(t) for t in outs]
        for g, e, n in zip(got, eager, ("ids", "w", "offsets", "perm", "slot_pos", "y", "dense y")):
            assert np.array_equal(g.view(np.uint8), e.view(np.uint8)), f"replay {rep}: {n} differs from eager"
