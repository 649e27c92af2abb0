"""GPU parity of the shared expert (moe_shared_expert: FP8 gate/up GEMM,
SwiGLU + E4M3 requant, FP8 down GEMM with K = I = 576 unpadded) against the
oracle through the C-ABI, staged on identical inputs like the routed FFN,
on the decode, verification and prefill row counts; rows bitwise
independent of the batch."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp8xfp4_amd import mxmoe, synth
from gpu_common import TOL_COS, TOL_REL_MAX, assert_close, dev, explain_code_differences, host, rel_err_cos, say

pytestmark = pytest.mark.gpu


class Shared:
    def __init__(self, cfg, H=None, I=None, T=None):
        inp = synth.moe_inputs(cfg)
        c = inp.cfg
        self.H = c.H if H is None else H
        self.I = c.I if I is None else I
        x = inp.x if H is None else synth.hidden_rows(c.seed, c.T, self.H)
        x = x if T is None else np.resize(x, (T, self.H))
        w13, w2 = synth.shared_expert_weights(c, self.H, self.I)
        self.x, self.x_sc = oracle.quantize_e4m3(x)
        self.w13, self.w13_sc = oracle.quantize_e4m3(w13)
        self.w2, self.w2_sc = oracle.quantize_e4m3(w2)
        self.d = {k: dev(getattr(self, k)) for k in ("x", "x_sc", "w13", "w13_sc", "w2", "w2_sc")}

    def gpu(self, rows=None):
        x, xs = self.d["x"], self.d["x_sc"]
        if rows is not None:
            idx = dev(np.asarray(rows, np.int64))
            x, xs = x[idx].contiguous(), xs[idx].contiguous()
        T = x.shape[0]
        y = torch.empty((T, self.H), dtype=torch.float32, device="cuda")
        ws = torch.full((mxmoe.moe_shared_expert_workspace_bytes(T, self.H, self.I),), 0xFF, dtype=torch.uint8,
                        device="cuda")
        mxmoe.moe_shared_expert(x, xs, self.d["w13"], self.d["w13_sc"], self.d["w2"], self.d["w2_sc"], y, ws)
        variant = mxmoe.last_variant()
        I = self.I
        hb = ((T * 2 * I * 4 + 255) // 256) * 256
        qb = ((T * I + 255) // 256) * 256
        wsh = host(ws)
        h = wsh[:T * 2 * I * 4].view(np.float32).reshape(T, 2 * I)
        q = wsh[hb:hb + T * I].reshape(T, I)
        q_sc = wsh[hb + qb:hb + qb + T * (I // 32)].reshape(T, I // 32)
        return host(y), h, q, q_sc, variant


def staged_parity(S, rows, what):
    """As the routed FFN's staged parity: (i) gate/up GEMM against the oracle,
    (ii) the requant of the GPU's own h bit for bit, (iii) the down GEMM from
    the GPU's own intermediate; end to end 2e-3 / 0.99999 where the GPU's
    intermediate codes equal the oracle's own, and every differing code
    explained by the h error carrying a across a rounding boundary."""
    y, h, q, q_sc, variant = S.gpu()
    rows = np.asarray(rows, np.int32)
    # (i) gate/up GEMM
    h_ref = oracle.block_gemm(S.x, S.x_sc, S.w13, S.w13_sc, rows=rows)
    ei, _ = assert_close(h[rows], h_ref, what + " gate/up")
    # (ii) SwiGLU + requant on the GPU's own h: bit for bit
    q2, sc2, a_g = oracle.swiglu_requant(h[rows])
    assert np.array_equal(sc2, q_sc[rows]) and np.array_equal(q2, q[rows]), what + ": requant differs on identical h"
    q_r, sc_r, a_r = oracle.swiglu_requant(h_ref)
    nel, nsc = explain_code_differences(q[rows], q_sc[rows], a_g, q_r, sc_r, a_r)
    # (iii) down GEMM from the GPU's intermediate
    y_mid = oracle.block_gemm(q, q_sc, S.w2, S.w2_sc, rows=rows)
    e3, _ = assert_close(y[rows], y_mid, what + " down")
    # end to end
    ref, *_ = oracle.shared_expert(S.x, S.x_sc, S.w13, S.w13_sc, S.w2, S.w2_sc, rows=rows)
    err, cos = rel_err_cos(y[rows], ref)
    say(f"{what}: gate/up {ei:.2e}, down {e3:.2e}, intermediate codes differing from the oracle's own {nel} "
        f"(+{nsc} scales); end-to-end max|diff|/max|ref| {err:.2e}, cosine {cos:.8f} ({variant})")
    if nel == 0 and nsc == 0:
        assert err <= TOL_REL_MAX and cos >= TOL_COS
    return y, variant


@pytest.mark.parametrize("name", ["decode", "verify"])
def test_shared_expert_workloads(name):
    S = Shared(name)
    T = S.x.shape[0]
    _, variant = staged_parity(S, np.arange(T), f"shared {name}")
    assert "decode" in variant


def test_shared_expert_prefill_sampled_rows():
    S = Shared("prefill")
    rows = np.concatenate([np.random.default_rng(9).choice(8192, 24, replace=False), [0, 8191]])
    _, variant = staged_parity(S, rows, "shared prefill")
    assert "prefill" in variant


@pytest.mark.parametrize("H,I", [(256, 64), (384, 96), (1152, 160)])
def test_shared_expert_small_shapes(H, I):
    S = Shared("tiny", H=H, I=I)
    staged_parity(S, np.arange(S.x.shape[0]), f"shared H={H} I={I}")


def test_shared_expert_rows_do_not_depend_on_the_batch():
    """Rows of a 400-row call (tiled GEMMs) equal the same rows run alone and
    in 16-row batches (decode GEMMs), bit for bit."""
    S = Shared("verify", T=400)
    full, *_ = S.gpu()
    for rows in ([0], [399], list(range(100, 116)), [5, 250, 17]):
        part, *_ , v = S.gpu(rows)
        assert "decode" in v
        assert np.array_equal(part, full[rows]), rows


# ------------------------------------------------------------ one row, one launch
def shared_ws_status_offset(H, I):
    """Byte offset of the one-launch form's status word: the workspace's last 256 bytes."""
    return mxmoe.moe_shared_expert_workspace_bytes(1, H, I) - 256


def shared_row_call(S, single, ws=None, row=0):
    """moe_shared_expert on one row with the one-launch form on or off:
    y, h, q, q_sc, the variant and the status word."""
    I, H = S.I, S.H
    x, xs = S.d["x"][row:row + 1].contiguous(), S.d["x_sc"][row:row + 1].contiguous()
    n = mxmoe.moe_shared_expert_workspace_bytes(1, H, I)
    if ws is None:                                              # garbage: nothing needs clearing but the status
        ws = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    so = shared_ws_status_offset(H, I)
    ws[so:so + 4] = 0
    y = torch.full((1, H), 7.0, device="cuda")
    prev = mxmoe.set_layer1_single_launch(1 if single else 0)
    try:
        mxmoe.moe_shared_expert(x, xs, S.d["w13"], S.d["w13_sc"], S.d["w2"], S.d["w2_sc"], y, ws)
        v = mxmoe.last_variant()
    finally:
        mxmoe.set_layer1_single_launch(prev)
    hb = (2 * I * 4 + 255) // 256 * 256
    qb = (I + 255) // 256 * 256
    wsh = host(ws[:n])
    h = wsh[:2 * I * 4].view(np.float32)
    q, q_sc = wsh[hb:hb + I], wsh[hb + qb:hb + qb + I // 32]
    status = int(wsh[so:so + 4].view(np.uint32)[0])
    return host(y)[0], h.copy(), q.copy(), q_sc.copy(), v, status


def single_vs_two_shared(S, row=0):
    y1, h1, q1, s1, v1, st = shared_row_call(S, True, row=row)
    y2, h2, q2, s2, v2, _ = shared_row_call(S, False, row=row)
    assert "one launch" in v1, v1
    assert v2 == "shared:decode1_gemm_parts+down_requant", v2
    assert st == 0, "a handoff wait ran out of time"
    assert np.array_equal(h1.view(np.uint32), h2.view(np.uint32)), "h"
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2), "intermediate"
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "y"
    return y1


@pytest.mark.parametrize("H,I", [
    (4096, 576),        # the decode shape: four K parts, I = 4.5 MFMA steps
    (5120, 576),        # five K parts: wavefront 0 takes parts 0 and 4
    (128, 32),          # one step, one block, four producers
    (256, 64),
    (1152, 160),        # K tail in the down projection
    (512, 1024),        # the largest intermediate: every handoff chunk in use
    (3072, 640),
])
def test_shared_single_launch_equals_two_launches(H, I):
    """The one-launch form (gate/up workgroups hand their SwiGLU values to the
    down workgroups through tagged words) against the two-launch form: h, the
    intermediate codes and scales, and y bit for bit; the status word clear.
    Staged parity against the oracle on the same row."""
    S = Shared("decode" if (H, I) == (4096, 576) else "tiny", H=H, I=I, T=1)
    single_vs_two_shared(S)
    y, h, q, q_sc, v, _ = shared_row_call(S, True)
    h_ref = oracle.block_gemm(S.x[:1], S.x_sc[:1], S.w13, S.w13_sc)
    assert_close(h[None, :], h_ref, f"shared one launch H={H} I={I} gate/up")
    q2, sc2, _ = oracle.swiglu_requant(h[None, :])
    assert np.array_equal(q2[0], q) and np.array_equal(sc2[0], q_sc), "requant differs on identical h"
    y_mid = oracle.block_gemm(q[None, :], q_sc[None, :], S.w2, S.w2_sc)
    e, _ = assert_close(y[None, :], y_mid, f"shared one launch H={H} I={I} down")
    say(f"shared one launch H={H} I={I}: bitwise equal to two launches; down {e:.2e} ({v})")


def test_shared_single_launch_falls_back_off_the_k_grid():
    """H % 128 != 0 keeps the two-launch form (the gate/up workgroups take no K tail)."""
    S = Shared("tiny", H=1056, I=96, T=1)
    *_, v, _ = shared_row_call(S, True)
    assert v == "shared:decode1_gemm_parts+down_requant", v


def test_shared_single_launch_alternating_shapes_share_one_workspace():
    """Calls of different rows and shapes reuse one workspace in turn, the
    second of each pair smaller: the per-call tags keep every wait on this
    call's words (a stale word from the call before never passes)."""
    big = Shared("verify", H=4096, I=576, T=4)
    small = Shared("tiny", H=1024, I=96, T=1)
    n = mxmoe.moe_shared_expert_workspace_bytes(1, 4096, 576)
    ws = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    ref_big = [shared_row_call(big, False, row=r)[0] for r in range(4)]
    ref_small = shared_row_call(small, False)[0]
    for it in range(3):
        for r in range(4):
            y, *_, v, st = shared_row_call(big, True, ws=ws, row=r)
            assert "one launch" in v and st == 0
            assert np.array_equal(y.view(np.uint32), ref_big[r].view(np.uint32)), (it, r)
            ys, *_, v, st = shared_row_call(small, True, ws=ws)
            assert "one launch" in v and st == 0
            assert np.array_equal(ys.view(np.uint32), ref_small.view(np.uint32)), (it, "small")
    say("shared one launch: 24 alternating calls on one workspace bitwise equal to two launches")
