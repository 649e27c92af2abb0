"""moe_layer_decode1 (the gate inside the gate/up kernel, one row) against
moe_route followed by moe_expert_ffn: bit for bit on every route output and
on y, live and dead rows, ties, and several layer shapes; and against the
oracle end to end."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp8xfp4_amd import mxmoe, synth
from block_scaled_fp8xfp4_amd.layer import ExpertFFN, Route, quantize
from gpu_common import Layer, assert_close, dev, host, say, shared_operands, small_workload, status_offset

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


# ------------------------------------------- routed + shared experts, one row
def run_with_shared(layer, logits, sw, survival=None, skip=0.2, single=True):
    """moe_layer_decode1_shared (one launch where it applies when `single`,
    else two) against moe_layer_decode1 followed by moe_shared_expert's
    two-launch form (T = 1): route outputs, y, y_shared and both workspace
    parts (the routed intermediate and SwiGLU rows; the shared h, q and q_sc,
    and with two launches the gate/up parts) bit for bit; the status word of
    the one-launch form clear."""
    c = layer.cfg
    E, k, H, I = c.E, c.k, c.H, c.I
    sw13, sw13s, sw2, sw2s = sw
    Is = sw2.shape[1]
    d = layer.d
    x, xs = d["x"][:1].contiguous(), d["x_sc"][:1].contiguous()
    lg = dev(np.ascontiguousarray(logits[:1], np.float32))
    sv = None if survival is None else dev(np.ascontiguousarray(survival[:1], np.float32))
    rws = mxmoe.moe_expert_ffn_workspace_bytes(1, H, E, I, k)
    sws = mxmoe.moe_shared_expert_workspace_bytes(1, H, Is)
    # the two calls
    ref = Route(1, E, k)
    y_ref = torch.empty((1, H), dtype=torch.float32, device="cuda")
    ws_r = torch.full((rws,), 0xFF, dtype=torch.uint8, device="cuda")
    so = status_offset(H, I, k)
    ws_r[so:so + 4] = 0                                        # the status word, as in the fused call's workspace
    mxmoe.moe_layer_decode1(lg, k, sv, skip, x, xs, d["w13"], d["w13_sc"], d["w2"], d["w2_sc"], E, I, ref.ids, ref.w,
                            ref.offsets, ref.perm, ref.slot_pos, y_ref, ws_r)
    ys_ref = torch.empty((1, H), dtype=torch.float32, device="cuda")
    ws_s = torch.full((sws,), 0xFF, dtype=torch.uint8, device="cuda")
    prev = mxmoe.set_layer1_single_launch(0)                   # the shared expert's two-launch form
    try:
        mxmoe.moe_shared_expert(x, xs, sw13, sw13s, sw2, sw2s, ys_ref, ws_s)
        assert mxmoe.last_variant() == "shared:decode1_gemm_parts+down_requant"
    finally:
        mxmoe.set_layer1_single_launch(prev)
    # the fused call
    fz = Route(1, E, k)
    for key in ("ids", "offsets", "perm", "slot_pos"):
        getattr(fz, key).fill_(-7)
    y = torch.full((1, H), 7.0, device="cuda")
    ys = torch.full((1, H), 7.0, device="cuda")
    need = mxmoe.moe_layer_decode1_shared_workspace_bytes(H, E, I, k, Is)
    assert need == (rws + 255) // 256 * 256 + sws
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    ws[so:so + 4] = 0
    prev = mxmoe.set_layer1_single_launch(1 if single else 0)
    try:
        mxmoe.moe_layer_decode1_shared(lg, k, sv, skip, x, xs, d["w13"], d["w13_sc"], d["w2"], d["w2_sc"], E, I,
                                       sw13, sw13s, sw2, sw2s, fz.ids, fz.w, fz.offsets, fz.perm, fz.slot_pos, y, ys,
                                       ws)
        v = mxmoe.last_variant()
    finally:
        mxmoe.set_layer1_single_launch(prev)
    one = single and k <= 8 and I <= 640 and Is <= 640
    assert v.startswith("layer1_shared:") and ("one launch" in v) == one, v
    if one:
        assert int(ws[so:so + 4].view(torch.int32).item()) == 0, "a handoff wait ran out of time"
    for key in ("ids", "w", "offsets", "perm", "slot_pos"):
        assert torch.equal(getattr(fz, key), getattr(ref, key)), key
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
    assert torch.equal(ys.view(torch.int32), ys_ref.view(torch.int32))
    off = (rws + 255) // 256 * 256
    flags = rws - (k * (I // 32) * 128 + 255) // 256 * 256     # the handoff words (a 128-byte line per block) end the region
    assert torch.equal(ws[:flags], ws_r[:flags]), "routed workspace"
    a256 = lambda b: (b + 255) // 256 * 256
    hq = a256(2 * Is * 4) + a256(Is) + a256(Is // 32)             # shared h, q, q_sc; then its parts or words
    assert torch.equal(ws[off:off + hq], ws_s[:hq]), "shared workspace (h, q, q_sc)"
    if not one:
        assert torch.equal(ws[off:off + sws - 256], ws_s[:sws - 256]), "shared workspace (gate/up parts)"
    return host(y), host(ys)


@pytest.mark.parametrize("single", [True, False], ids=["one_launch", "two_launches"])
def test_decode_workload_with_shared_expert_bitwise(single):
    from gpu_common import moe_workload
    inp, r, layer = moe_workload("decode")
    c = inp.cfg
    y, ys = run_with_shared(layer, inp.logits, shared_operands(c, c.H, c.I), single=single)
    assert np.any(ys) and np.any(y)
    say(f"layer_decode1_shared ({'one launch' if single else 'two launches'}): routed and shared outputs "
        "bitwise equal to the separate calls")


@pytest.mark.parametrize("single", [True, False], ids=["one_launch", "two_launches"])
@pytest.mark.parametrize("shape,Is", [
    (dict(seed=41, T=1, H=256, E=8, k=2, I=64), 64),
    (dict(seed=42, T=1, H=1152, E=384, k=8, I=96), 160),          # K tail in the shared down projection
    (dict(seed=43, T=1, H=512, E=64, k=16, I=160), 1024),         # the largest shared intermediate (two launches)
    (dict(seed=45, T=1, H=2048, E=32, k=4, I=128), 128),          # two K parts of the shared gate/up
    (dict(seed=46, T=1, H=5120, E=16, k=8, I=640), 640),         # five K parts; routed and shared I at the limit
    (dict(seed=47, T=1, H=4096, E=24, k=6, I=576), 32),          # one shared block: four producers
    (dict(seed=48, T=1, H=128, E=16, k=1, I=32), 576),            # shared I above the routed one
])
def test_small_shapes_with_shared_expert(shape, Is, single):
    inp, r, layer = small_workload(**shape)
    run_with_shared(layer, inp.logits, shared_operands(layer.cfg, shape["H"], Is), single=single)


@pytest.mark.parametrize("single", [True, False], ids=["one_launch", "two_launches"])
def test_dead_row_still_gets_its_shared_expert(single):
    inp, r, layer = small_workload(seed=44, T=1, H=256, E=32, k=4, I=64)
    y, ys = run_with_shared(layer, inp.logits, shared_operands(layer.cfg, 256, 96), np.array([0.1], np.float32), 0.2,
                            single=single)
    assert not np.any(y) and not np.any(np.signbit(y))
    assert np.any(ys)


def test_shared_layer_alternating_calls_share_one_workspace():
    """The routed + shared layer in one launch, called on one workspace for
    two rows in turn (live, then dead), six times: every call bitwise equal to
    its first result (the per-call tags keep each wait on that call's words)."""
    inp, r, layer = small_workload(seed=49, T=2, H=4096, E=32, k=8, I=576)
    c = layer.cfg
    sw13, sw13s, sw2, sw2s = shared_operands(c, c.H, 576)
    d = layer.d
    need = mxmoe.moe_layer_decode1_shared_workspace_bytes(c.H, c.E, c.I, c.k, 576)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda")
    so = status_offset(c.H, c.I, c.k)
    ws[so:so + 4] = 0
    firsts = {}
    for it in range(6):
        for row, surv in ((0, 1.0), (1, 0.1)):
            x, xs = d["x"][row:row + 1].contiguous(), d["x_sc"][row:row + 1].contiguous()
            lg = dev(np.ascontiguousarray(inp.logits[row:row + 1], np.float32))
            sv = dev(np.array([surv], np.float32))
            rt = Route(1, c.E, c.k)
            y = torch.full((1, c.H), 7.0, device="cuda")
            ys = torch.full((1, c.H), 7.0, device="cuda")
            mxmoe.moe_layer_decode1_shared(lg, c.k, sv, 0.2, x, xs, d["w13"], d["w13_sc"], d["w2"], d["w2_sc"], c.E,
                                           c.I, sw13, sw13s, sw2, sw2s, rt.ids, rt.w, rt.offsets, rt.perm,
                                           rt.slot_pos, y, ys, ws)
            assert "one launch" in mxmoe.last_variant()
            out = (host(y), host(ys), host(rt.ids))
            if row not in firsts:
                firsts[row] = out
            for a_, b_ in zip(out, firsts[row]):
                assert np.array_equal(a_.view(np.uint32), b_.view(np.uint32)), (it, row)
    assert int(ws[so:so + 4].view(torch.int32).item()) == 0, "a handoff wait ran out of time"
    assert not np.any(firsts[1][0]) and np.any(firsts[1][1])
    say("layer_decode1_shared: 12 alternating one-launch calls (live and dead rows) on one workspace, stable")


# ---------------------------------------- one launch against two launches
def layer1_call(layer, lg, sv, skip, x, xs, ws, single):
    c = layer.cfg
    d = layer.d
    prev = mxmoe.set_layer1_single_launch(1 if single else 0)
    try:
        r = Route(1, c.E, c.k)
        for key in ("ids", "offsets", "perm", "slot_pos"):
            getattr(r, key).fill_(-7)
        y = torch.full((1, c.H), 7.0, device="cuda")
        mxmoe.moe_layer_decode1(lg, c.k, sv, skip, x, xs, d["w13"], d["w13_sc"], d["w2"], d["w2_sc"], c.E, c.I,
                                r.ids, r.w, r.offsets, r.perm, r.slot_pos, y, ws)
        v = mxmoe.last_variant()
    finally:
        mxmoe.set_layer1_single_launch(prev)
    return r, y, v


def single_vs_two(layer, logits, survival=None, skip=0.2):
    """moe_layer_decode1 in one launch and in two launches: every route
    output, y and the workspace's intermediate (q, its scales and the SwiGLU
    rows) bit for bit; the handoff status word stays clear."""
    c = layer.cfg
    E, k, H, I = c.E, c.k, c.H, c.I
    d = layer.d
    x, xs = d["x"][:1].contiguous(), d["x_sc"][:1].contiguous()
    lg = dev(np.ascontiguousarray(logits[:1], np.float32))
    sv = None if survival is None else dev(np.ascontiguousarray(survival[:1], np.float32))
    n = mxmoe.moe_expert_ffn_workspace_bytes(1, H, E, I, k)
    ws2 = torch.zeros(n, dtype=torch.uint8, device="cuda")
    r2, y2, v2 = layer1_call(layer, lg, sv, skip, x, xs, ws2, False)
    assert v2 == "layer1:gu1_decode_topk+down_combine1", v2
    ws1 = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")   # garbage: nothing needs clearing
    so = status_offset(H, I, k)
    ws1[so:so + 4] = 0
    r1, y1, v1 = layer1_call(layer, lg, sv, skip, x, xs, ws1, True)
    assert "one launch" in v1, v1
    assert int(ws1[so:so + 4].view(torch.int32).item()) == 0, "a handoff wait ran out of time"
    for key in ("ids", "w", "offsets", "perm", "slot_pos"):
        assert torch.equal(getattr(r1, key), getattr(r2, key)), key
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    live = survival is None or not survival[0] < skip
    if live:
        oq, oqs, oo = mxmoe.moe_ws_layout(1, H, I, k)
        assert torch.equal(ws1[oq:oq + k * I], ws2[oq:oq + k * I]), "q"
        assert torch.equal(ws1[oqs:oqs + k * I // 32], ws2[oqs:oqs + k * I // 32]), "q scales"
        assert torch.equal(ws1[oo:oo + k * I * 4], ws2[oo:oo + k * I * 4]), "SwiGLU rows"
    return host(y1)


def test_single_launch_decode_workload():
    from gpu_common import moe_workload
    inp, r, layer = moe_workload("decode")
    y = single_vs_two(layer, inp.logits)
    err, cos = assert_close(y, layer.oracle_y(r), "layer_decode1 single launch end to end")
    say(f"layer_decode1 single launch: bitwise equal to two launches; end-to-end {err:.2e}, cosine {cos:.8f}")


@pytest.mark.parametrize("shape", [
    dict(seed=51, T=1, H=256, E=8, k=2, I=64),                  # one down step
    dict(seed=52, T=1, H=1152, E=384, k=8, I=96),               # 16 logits per lane, a non-exact gate/up step count
    dict(seed=53, T=1, H=512, E=64, k=1, I=640),                # the largest intermediate of the single launch
    dict(seed=54, T=1, H=5120, E=384, k=8, I=576),              # the pages' layer shape
    dict(seed=55, T=1, H=2048, E=256, k=6, I=288),              # k below 8, I not a multiple of 128
])
def test_single_launch_shapes(shape):
    inp, r, layer = small_workload(**shape)
    single_vs_two(layer, inp.logits)


def test_single_launch_dead_row_and_ties():
    inp, r, layer = small_workload(seed=56, T=1, H=256, E=32, k=4, I=64)
    y = single_vs_two(layer, inp.logits, np.array([0.1], np.float32), 0.2)
    assert not np.any(y) and not np.any(np.signbit(y))
    single_vs_two(layer, np.zeros((1, 32), np.float32), np.array([0.9], np.float32), 0.2)


def test_single_launch_alternating_inputs_share_one_workspace():
    """Calls with different rows on one workspace, one after another: each
    call waits for its own gate/up results (the tags of the call before never
    match), so every y equals its own two-launch result bit for bit."""
    from gpu_common import moe_workload
    inp, r, layer = moe_workload("decode")
    c = layer.cfg
    d = layer.d
    rng = np.random.default_rng(57)
    cases = []
    for i in range(3):
        lg = dev(rng.standard_normal((1, c.E)).astype(np.float32))
        xb = torch.from_numpy(rng.standard_normal((1, c.H)).astype(np.float32)).to("cuda").to(torch.bfloat16)
        xq, xsc = quantize(xb, mxmoe.MX_FMT_E4M3)
        ws = torch.zeros(mxmoe.moe_expert_ffn_workspace_bytes(1, c.H, c.E, c.I, c.k), dtype=torch.uint8,
                         device="cuda")
        _, y, _ = layer1_call(layer, lg, None, 0.2, xq, xsc, ws, False)
        cases.append((lg, xq, xsc, y))
    n = mxmoe.moe_expert_ffn_workspace_bytes(1, c.H, c.E, c.I, c.k)
    ws = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    so = status_offset(c.H, c.I, c.k)
    ws[so:so + 4] = 0
    for it in range(24):
        lg, xq, xsc, yref = cases[it % 3 if it < 12 else (it * 7) % 3]
        _, y, v = layer1_call(layer, lg, None, 0.2, xq, xsc, ws, True)
        assert "one launch" in v
        assert torch.equal(y.view(torch.int32), yref.view(torch.int32)), f"call {it}"
    assert int(ws[so:so + 4].view(torch.int32).item()) == 0


# ------------------------------------------- seeded sweep of the single launch
def sweep_shapes(n=12, seed=71):
    """Single-row layer shapes drawn once from a fixed seed, inside the single
    launch's domain (k <= 8, I <= 640): H a multiple of 128 up to 5120, E up
    to 1024, I a multiple of 32, some rows dead."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([8, 33, 128, 256, 300, 512, 1024]))
        out.append(dict(seed=seed + 1 + i, T=1, H=128 * int(rng.integers(1, 41)), E=E,
                        k=int(rng.integers(1, min(8, E) + 1)), I=32 * int(rng.integers(1, 21)),
                        dead=bool(rng.random() < 0.2)))
    return out


@pytest.mark.parametrize("shape", sweep_shapes(), ids=lambda s: f"H{s['H']}_E{s['E']}_k{s['k']}_I{s['I']}")
def test_single_launch_sweep(shape):
    """One launch against two, bit for bit, and end to end against the oracle."""
    s = dict(shape)
    dead = s.pop("dead")
    inp = synth.small_moe(s["seed"], s["T"], s["H"], s["E"], s["k"], s["I"])
    r = oracle.route(inp.logits, s["k"], inp.survival)
    layer = Layer(inp, np.unique(r["ids"]))                     # the row's experts alone get weights
    surv = np.array([0.1 if dead else 0.9], np.float32)
    y = single_vs_two(layer, inp.logits, surv, 0.2)
    if dead:
        assert not np.any(y) and not np.any(np.signbit(y))
    else:
        err, cos = assert_close(y, layer.oracle_y(r), f"single launch {shape}")
        say(f"single launch {shape}: end to end {err:.2e}, cosine {cos:.8f}")
