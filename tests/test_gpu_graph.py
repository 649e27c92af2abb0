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
from gpu_common import dev, host, moe_workload, say, shared_operands, status_offset

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


def test_graph_single_launch_forms_take_fresh_tags():
    """moe_layer_decode1, moe_layer_decode1_shared and moe_shared_expert on
    one row, captured in one HIP graph, keep their one-launch forms (each
    preceded by the kernel that advances its workspace's call counter, the
    tag source of a replay).  Every replay takes a new row copied into the
    captured inputs, with eager calls of other rows on the same workspaces
    between replays, and must equal the eager calls on its row bit for bit
    (a stale word from the call before could only pass with a repeated tag);
    the status words stay clear."""
    inp, r, layer = moe_workload("verify")
    c = inp.cfg
    E, k, H, I = c.E, c.k, c.H, c.I
    L = layer.d
    sw = shared_operands(c, H, I)
    rows = [0, 7, 13, 21, 30, 41, 47]
    lg_all = dev(np.ascontiguousarray(inp.logits, np.float32))
    a256 = lambda b: (b + 255) // 256 * 256
    hq = a256(2 * I * 4) + a256(I) + a256(I // 32)

    # static inputs and outputs of the captured calls
    lg_s = torch.empty((1, E), dtype=torch.float32, device="cuda")
    x_s = torch.empty((1, H), dtype=torch.uint8, device="cuda")
    xs_s = torch.empty((1, H // 32), dtype=torch.uint8, device="cuda")
    rt1, rt2 = Route(1, E, k), Route(1, E, k)
    y1 = torch.empty((1, H), dtype=torch.float32, device="cuda")
    y2 = torch.empty((1, H), dtype=torch.float32, device="cuda")
    ys2 = torch.empty((1, H), dtype=torch.float32, device="cuda")
    ys3 = torch.empty((1, H), dtype=torch.float32, device="cuda")
    ws1 = torch.randint(0, 256, (mxmoe.moe_expert_ffn_workspace_bytes(1, H, E, I, k),), dtype=torch.uint8, device="cuda")
    n2 = mxmoe.moe_layer_decode1_shared_workspace_bytes(H, E, I, k, I)
    ws2 = torch.randint(0, 256, (n2,), dtype=torch.uint8, device="cuda")
    n3 = mxmoe.moe_shared_expert_workspace_bytes(1, H, I)
    ws3 = torch.randint(0, 256, (n3,), dtype=torch.uint8, device="cuda")
    so = status_offset(H, I, k)
    for w, o in ((ws1, so), (ws2, so), (ws3, n3 - 256)):
        w[o:o + 4] = 0

    def calls(lg, x, xs):
        mxmoe.moe_layer_decode1(lg, k, None, 0.2, x, xs, L["w13"], L["w13_sc"], L["w2"], L["w2_sc"], E, I, rt1.ids,
                                rt1.w, rt1.offsets, rt1.perm, rt1.slot_pos, y1, ws1)
        v = [mxmoe.last_variant()]
        mxmoe.moe_layer_decode1_shared(lg, k, None, 0.2, x, xs, L["w13"], L["w13_sc"], L["w2"], L["w2_sc"], E, I,
                                       *sw, rt2.ids, rt2.w, rt2.offsets, rt2.perm, rt2.slot_pos, y2, ys2, ws2)
        v.append(mxmoe.last_variant())
        mxmoe.moe_shared_expert(x, xs, *sw, ys3, ws3)
        v.append(mxmoe.last_variant())
        return v

    def outs():
        return [host(t).copy() for t in (rt1.ids, rt1.w, y1, rt2.ids, y2, ys2, ys3)] + \
            [host(ws3[:hq]).copy(), host(ws2[a256(mxmoe.moe_expert_ffn_workspace_bytes(1, H, E, I, k)):][:hq]).copy()]

    def row_inputs(t):
        return lg_all[t:t + 1].contiguous(), L["x"][t:t + 1].contiguous(), L["x_sc"][t:t + 1].contiguous()

    ref = {}
    for t in rows:                                           # eager, each row
        v = calls(*row_inputs(t))
        assert all("one launch" in s for s in v), v
        ref[t] = outs()
    lg0, x0, xs0 = row_inputs(rows[0])
    lg_s.copy_(lg0), x_s.copy_(x0), xs_s.copy_(xs0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        v = calls(lg_s, x_s, xs_s)
    assert all("one launch" in s for s in v), v              # captured: still one launch each
    for rep, t in enumerate(rows[1:] + rows[:1] + rows[2:4]):
        if rep % 2 == 1:                                     # an eager call of another row on the same workspaces
            calls(*row_inputs(rows[(rep + 3) % len(rows)]))
        lg, x, xs = row_inputs(t)
        lg_s.copy_(lg), x_s.copy_(x), xs_s.copy_(xs)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outs()
        for i, (g, e) in enumerate(zip(got, ref[t])):
            assert np.array_equal(g.view(np.uint8), e.view(np.uint8)), f"replay {rep} (row {t}): output {i} differs"
    for w, o in ((ws1, so), (ws2, so), (ws3, n3 - 256)):
        assert int(w[o:o + 4].view(torch.int32).item()) == 0, "a handoff wait ran out of time"
    say("graph: single-launch layer, layer + shared and shared expert replayed on 9 rows between eager calls, "
        "each bitwise equal to its eager result")
