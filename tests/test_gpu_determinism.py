"""Determinism of the kernels that pace their global -> LDS transfers by hand
(explicit vmcnt counts the compiler cannot check) and hand out work through
atomic queues: the prefill gate/up and down kernels, the tiled dense GEMM and
the tiled router logits (forum thread post #4, "512K context", "Quality and
correctness" and "Testing": pipeline stages reused before their data landed
gave wrong results under co-resident load until fenced; post #6, "A race in
TileLang's warp-specialized pipeline").

Each call is repeated 200 times on its full-size workload and every result is
compared bit for bit with the first; then the same calls run while a
bandwidth-heavy copy streams on a second stream (default priority), so other
work shares the CUs, the caches and the memory system.  Each loop stops at its
first mismatch."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp8xfp4_amd import mxmoe, synth
from block_scaled_fp8xfp4_amd.layer import ExpertFFN, RouterLogits
from gpu_common import dev, moe_workload, say

pytestmark = pytest.mark.gpu

REPEATS = 200
STRESSED = 100


class Stressor:
    """Copies between two 512 MiB buffers on a second stream (default priority)."""

    def __init__(self):
        n = 128 << 20
        self.src = torch.randn(n, device="cuda")
        self.dst = torch.empty_like(self.src)
        self.stream = torch.cuda.Stream()
        self.stream.wait_stream(torch.cuda.current_stream())

    def enqueue(self, copies):
        with torch.cuda.stream(self.stream):
            for _ in range(copies):
                self.dst.copy_(self.src)

    def drain(self):
        self.stream.synchronize()


def repeat_bitwise(call, outs, what, copies):
    """Run call() REPEATS times alone, then STRESSED times beside the stressor;
    every run's outputs must equal the first run's bit for bit."""
    call()
    ref = [o.clone() for o in outs]
    for i in range(REPEATS):
        call()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"{what}: repeat {i} differs from the first run"
    st = Stressor()
    try:
        for i in range(STRESSED):
            st.enqueue(copies)
            call()
            for o, r in zip(outs, ref):
                assert torch.equal(o, r), f"{what}: run {i} beside the copy stream differs from the first run"
            if i % 10 == 9:
                st.drain()
    finally:
        st.drain()
    say(f"{what}: {REPEATS} repeats + {STRESSED} beside a copy stream, all bitwise equal")


def test_prefill_ffn_is_deterministic():
    """The 8192-token routed layer on the prefill kernels: y and the FP8
    intermediate (codes and scales)."""
    inp, r, layer = moe_workload("prefill")
    c = inp.cfg
    route = layer.gpu_route()
    ffn = ExpertFFN(c.T, c.H, c.E, c.I, c.k)
    d = layer.d

    def call():
        ffn(d["x"], d["x_sc"], route, d["w13"], d["w13_sc"], d["w2"], d["w2_sc"])

    call()
    assert mxmoe.last_variant().startswith("ffn:gu_prefill")
    q, qsc, _ = ffn.ws_views()
    P = c.T * c.k
    repeat_bitwise(call, [ffn.y, q[:P], qsc[:P]], "prefill FFN", copies=6)


def test_prefill_gemm_is_deterministic():
    """The tiled dense GEMM at M = 8192, K = N = 4096 (bf16 and fp32 out)."""
    inp = synth.dense_inputs()
    wq, wsc = oracle.quantize_e4m3(inp.w)
    a = synth.hidden_rows(11, 8192, 4096)
    aq, asc = oracle.quantize_e4m3(a)
    da, dasc, dw, dwsc = dev(aq), dev(asc), dev(wq), dev(wsc)
    y16 = torch.empty((8192, 4096), dtype=torch.bfloat16, device="cuda")
    y32 = torch.empty((8192, 4096), dtype=torch.float32, device="cuda")

    def call():
        mxmoe.fp8_block_gemm(da, dasc, dw, dwsc, y16, mxmoe.MX_OUT_BF16)
        mxmoe.fp8_block_gemm(da, dasc, dw, dwsc, y32, mxmoe.MX_OUT_F32)

    call()
    assert mxmoe.last_variant().startswith("gemm:prefill")
    repeat_bitwise(call, [y16, y32], "prefill GEMM", copies=2)


def test_prefill_router_logits_are_deterministic():
    """The tiled router logits at T = 8192, H = 4096, E = 256."""
    inp = synth.moe_inputs("prefill")
    c = inp.cfg
    hidden = dev(inp.x).to(torch.bfloat16)
    gate = dev(synth.router_gate("prefill")).to(torch.bfloat16)
    logits = torch.empty((c.T, c.E), dtype=torch.float32, device="cuda")
    rl = RouterLogits(c.T, c.H, c.E)

    def call():
        rl(hidden, gate, logits)

    call()
    assert mxmoe.last_variant().startswith("logits:prefill")
    repeat_bitwise(call, [logits], "prefill router logits", copies=1)


def test_single_launch_layer_is_deterministic_beside_other_work():
    """moe_layer_decode1 in one launch, whose down workgroups wait for the
    gate/up workgroups' requantized blocks: y, the route outputs and the
    intermediate bit for bit over every repeat, alone and while the copy
    stream shares the GPU (its workgroups can delay the gate/up side), and the
    handoff status word stays clear (no wait ran out of time)."""
    from block_scaled_fp8xfp4_amd.layer import Route
    inp, r, layer = moe_workload("decode")
    c = inp.cfg
    d = layer.d
    x, xs = d["x"][:1].contiguous(), d["x_sc"][:1].contiguous()
    lg = dev(np.ascontiguousarray(inp.logits[:1], np.float32))
    route = Route(1, c.E, c.k)
    y = torch.empty((1, c.H), dtype=torch.float32, device="cuda")
    ws = torch.zeros(mxmoe.moe_expert_ffn_workspace_bytes(1, c.H, c.E, c.I, c.k), dtype=torch.uint8, device="cuda")
    oq, oqs, oo = mxmoe.moe_ws_layout(1, c.H, c.I, c.k)
    so = oo + (c.k * max(c.H, c.I) * 4 + 255) // 256 * 256

    def call():
        mxmoe.moe_layer_decode1(lg, c.k, None, 0.2, x, xs, d["w13"], d["w13_sc"], d["w2"], d["w2_sc"], c.E, c.I,
                                route.ids, route.w, route.offsets, route.perm, route.slot_pos, y, ws)

    call()
    assert "one launch" in mxmoe.last_variant()
    outs = [y, route.ids, route.w, route.offsets, route.perm, route.slot_pos, ws[oq:oq + c.k * c.I],
            ws[oqs:oqs + c.k * c.I // 32]]
    repeat_bitwise(call, outs, "single-launch decode layer", copies=1)
    assert int(ws[so:so + 4].view(torch.int32).item()) == 0, "a handoff wait ran out of time"


def test_single_launch_shared_forms_are_deterministic_beside_other_work():
    """The shared expert of one row in one launch and the routed + shared
    layer in one launch (their down workgroups wait for the shared gate/up
    workgroups' SwiGLU words): y, y_shared and the shared h, q, q_sc bit for
    bit over every repeat, alone and beside the copy stream; the status
    words stay clear."""
    from block_scaled_fp8xfp4_amd.layer import Route
    inp, r, layer = moe_workload("decode")
    c = inp.cfg
    d = layer.d
    x, xs = d["x"][:1].contiguous(), d["x_sc"][:1].contiguous()
    lg = dev(np.ascontiguousarray(inp.logits[:1], np.float32))
    w13, w2 = synth.shared_expert_weights(c)
    q13, s13 = oracle.quantize_e4m3(w13)
    q2, s2 = oracle.quantize_e4m3(w2)
    sw = tuple(dev(t) for t in (q13, s13, q2, s2))
    Is = c.I
    a256 = lambda b: (b + 255) // 256 * 256
    hq = a256(2 * Is * 4) + a256(Is) + a256(Is // 32)
    # the shared expert alone
    sws = mxmoe.moe_shared_expert_workspace_bytes(1, c.H, Is)
    ws_s = torch.zeros(sws, dtype=torch.uint8, device="cuda")
    ys = torch.empty((1, c.H), dtype=torch.float32, device="cuda")

    def call_shared():
        mxmoe.moe_shared_expert(x, xs, *sw, ys, ws_s)

    call_shared()
    assert "one launch" in mxmoe.last_variant()
    repeat_bitwise(call_shared, [ys, ws_s[:hq]], "single-launch shared expert", copies=1)
    assert int(ws_s[sws - 256:sws - 252].view(torch.int32).item()) == 0, "a handoff wait ran out of time"
    # the routed + shared layer
    route = Route(1, c.E, c.k)
    y = torch.empty((1, c.H), dtype=torch.float32, device="cuda")
    y2 = torch.empty((1, c.H), dtype=torch.float32, device="cuda")
    need = mxmoe.moe_layer_decode1_shared_workspace_bytes(c.H, c.E, c.I, c.k, Is)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    rws = mxmoe.moe_expert_ffn_workspace_bytes(1, c.H, c.E, c.I, c.k)
    off = a256(rws)
    oq, oqs, oo = mxmoe.moe_ws_layout(1, c.H, c.I, c.k)
    so = oo + (c.k * max(c.H, c.I) * 4 + 255) // 256 * 256

    def call_layer():
        mxmoe.moe_layer_decode1_shared(lg, c.k, None, 0.2, x, xs, d["w13"], d["w13_sc"], d["w2"], d["w2_sc"], c.E,
                                       c.I, *sw, route.ids, route.w, route.offsets, route.perm, route.slot_pos, y, y2,
                                       ws)

    call_layer()
    assert "one launch" in mxmoe.last_variant()
    outs = [y, y2, route.ids, route.w, ws[oq:oq + c.k * c.I], ws[off:off + hq]]
    repeat_bitwise(call_layer, outs, "single-launch routed + shared layer", copies=1)
    assert int(ws[so:so + 4].view(torch.int32).item()) == 0, "a handoff wait ran out of time"
    assert torch.equal(y2, ys), "y_shared differs from the shared expert alone"
