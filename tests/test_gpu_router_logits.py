"""GPU parity of moe_router_logits (bf16 hidden . bf16 gate^T -> fp32) against
the oracle, through the C-ABI: both kernels (few rows / many rows), ragged
row, expert and K tails, the layer's own shapes, exact one-hot cases, and
bitwise row results that do not depend on the batch."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp8xfp4_amd import mxmoe, synth

from gpu_common import assert_close, dev, host, say

pytestmark = pytest.mark.gpu

PREFILL_MIN_T = 1024     # rows from which the tiled kernel runs
ONE_MAX_T = 16           # rows up to which one workgroup per expert runs


def few_rows_variant(T):
    return "logits:one" if T <= ONE_MAX_T else "logits:splitk"
# fp32 accumulation of bf16 products (exact in fp32): each 32-product MFMA
# step, 8-step chains and the ordered sum of H/256 parts each add at most a
# few units of 2^-24 of the running magnitude; 2^-16 of sum |h w| bounds all
# of it with room to spare for H <= 16384.
SUM_ABS_TOL = 2.0 ** -16


def bits(v):
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def run(hb, wb):
    T, H = hb.shape
    E = wb.shape[0]
    out = torch.empty((T, E), dtype=torch.float32, device="cuda")
    n = mxmoe.moe_router_logits_workspace_bytes(T, H, E)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda") if n else None   # contents must not matter
    mxmoe.moe_router_logits(dev(hb), dev(wb), out, ws)
    return host(out), mxmoe.last_variant()


def check(hf, wf, rows=None, what=""):
    hb, wb = bits(hf), bits(wf)
    got, variant = run(hb, wb)
    sel = np.arange(hb.shape[0]) if rows is None else np.asarray(rows)
    ref = oracle.router_logits(hb, wb, rows=sel.astype(np.int32))
    g = got[sel]
    assert_close(g, ref, what)
    sum_abs = np.abs(hf[sel].astype(np.float64)) @ np.abs(wf.astype(np.float64)).T
    err = np.abs(g.astype(np.float64) - ref)
    assert np.all(err <= SUM_ABS_TOL * sum_abs + 1e-30), f"{what}: worst {np.max(err / (sum_abs + 1e-30)):.2e} of sum|hw|"
    return got, variant


@pytest.mark.parametrize("T,H,E", [
    (4, 256, 8),          # the tiny layer
    (1, 4096, 256),       # decode row
    (16, 4096, 256),      # last row count of the one-workgroup-per-expert kernel
    (3, 5120, 40),        # 20 parts: waves take two parts
    (48, 4096, 256),      # verification rows
    (21, 96, 40),         # K of 3 steps (one short part), ragged experts
    (17, 5120, 24),       # 20 parts
    (127, 4352, 384),     # 17 parts
    (1023, 2048, 256),    # last row count of the few-rows path
    (1, 32, 1),           # one step, one expert
])
def test_few_rows_kernel(T, H, E):
    say(f"router logits T={T} H={H} E={E}")
    _, v = check(synth.hidden_rows(T + H, T, H), synth.router_gate("decode", E=E, H=H), what=f"{T}x{H}x{E}")
    assert v.startswith(few_rows_variant(T))


@pytest.mark.parametrize("T,H,E", [
    (1024, 4096, 256),    # first row count of the tiled kernel
    (1100, 1120, 72),     # K tail inside a stage (35 steps), experts < one tile
    (1089, 5120, 384),    # ragged row and expert tiles, 20 parts
    (1030, 32, 130),      # a single step
])
def test_many_rows_kernel(T, H, E):
    say(f"router logits T={T} H={H} E={E}")
    rows = np.unique(np.concatenate([np.arange(0, T, 37), [T - 1]]))
    _, v = check(synth.hidden_rows(T + H, T, H), synth.router_gate("prefill", E=E, H=H), rows=rows,
                 what=f"{T}x{H}x{E}")
    assert v.startswith("logits:prefill")


def test_prefill_layer_sampled_rows():
    """The prefill layer's own shape (T = 8192 hidden rows of the workload,
    H = 4096, E = 256), sampled rows against the oracle."""
    inp = synth.moe_inputs("prefill")
    rows = np.concatenate([np.random.default_rng(5).choice(8192, 40, replace=False), [0, 8191]])
    say("router logits prefill 8192x4096x256")
    full, _ = check(inp.x, synth.router_gate("prefill"), rows=rows, what="prefill")
    wb = bits(synth.router_gate("prefill"))
    for t in (0, 4097, 8191):                      # the same row alone: bit for bit
        one, _ = run(bits(inp.x[t:t + 1]), wb)
        assert np.array_equal(one[0], full[t]), t


@pytest.mark.parametrize("T", [5, 1030])
def test_one_hot_rows_are_exact(T):
    """Hidden row t = e_j: logits[t] is column j of the gate, bit for bit, on
    both paths (every K position pairs the right operands)."""
    H, E = 1056, 48
    wf = synth.router_gate("decode", E=E, H=H) * 8.0      # exact in bf16
    cols = np.random.default_rng(T).integers(0, H, T)
    hf = np.zeros((T, H), np.float32)
    hf[np.arange(T), cols] = 1.0
    got, v = run(bits(hf), bits(wf))
    assert v.startswith(few_rows_variant(T) if T < PREFILL_MIN_T else "logits:prefill")
    assert np.array_equal(got, wf[:, cols].T)


def test_rows_do_not_depend_on_the_batch():
    """Rows of a 1100-row call (tiled kernel) equal, bit for bit, the same rows
    computed 1..1023 at a time (few-rows path) and in another tiling."""
    T, H, E = 1100, 4096, 256
    hb, wb = bits(synth.hidden_rows(3, T, H)), bits(synth.router_gate("prefill"))
    full, v = run(hb, wb)
    assert v.startswith("logits:prefill")
    for t0, t1 in [(0, 1), (63, 64), (64, 80), (200, 327), (77, 1100), (1099, 1100)]:
        part, v = run(hb[t0:t1], wb)
        assert v.startswith(few_rows_variant(t1 - t0))
        assert np.array_equal(part, full[t0:t1]), (t0, t1)
    part, v = run(hb[5:1100], wb)                # another tiling of the same rows
    assert v.startswith("logits:prefill")
    assert np.array_equal(part, full[5:1100])


def test_workspace_reuse_and_changing_shapes():
    """One workspace serves calls of different T, H and E in a row: every
    result matches a fresh-workspace run."""
    n = max(mxmoe.moe_router_logits_workspace_bytes(T, H, E) for T, H, E in [(48, 4096, 256), (7, 1120, 72)])
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    for T, H, E in [(48, 4096, 256), (7, 1120, 72), (48, 4096, 256), (1, 4096, 256), (7, 1120, 72)]:
        hb, wb = bits(synth.hidden_rows(T, T, H)), bits(synth.router_gate("decode", E=E, H=H))
        out = torch.empty((T, E), dtype=torch.float32, device="cuda")
        mxmoe.moe_router_logits(dev(hb), dev(wb), out, ws)
        fresh, _ = run(hb, wb)
        assert np.array_equal(host(out), fresh), (T, H, E)


def test_empty_batch_is_a_no_op():
    out = torch.full((0, 8), 7.0, device="cuda")
    mxmoe.moe_router_logits(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"),
                            torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda"), out)
    assert mxmoe.last_variant() == "logits:empty"
