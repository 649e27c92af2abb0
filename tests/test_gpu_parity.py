"""GPU parity of every step of the hot path against the CPU oracle, through
the C-ABI: quantizer (bit-exact), top-k gate and bucketing (bit-exact ids,
offsets, perm, slot_pos; weights within 2^-22), routed-expert FFN and dense
GEMM (max|diff| <= 2e-3 max|ref|, cosine >= 0.99999 on fp32 outputs; bf16 =
RNE of the GPU's own fp32), on the five seeded workloads and edge cases."""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp8xfp4_amd import mxmoe, synth
from block_scaled_fp8xfp4_amd.layer import ExpertFFN, Route, quantize
from gpu_common import (Layer, assert_close, dev, ffn_parity, gpu_ffn_with_h, host, moe_workload, say,
                        small_workload)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ quantizer
def quant_inputs():
    rng = np.random.default_rng(21)
    v = rng.standard_normal((512, 256)).astype(np.float32)
    v[0] *= 1e-30
    v[1] *= 1e30
    v[2] *= 1e-40                      # fp32 subnormals
    v[3] = 0.0
    v[4, :32] = -0.0
    # exact E4M3 ties at scale 2^0 (block max 256 fixes the scale)
    v[5, ::32] = 256.0
    ties = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 464.0, 500.0, 15.5, 0.0146484375], np.float32)
    v[5, 1:9] = ties
    v[5, 33:41] = -ties
    # exact E2M1 ties at scale 2^0 (block max 4)
    v[6, ::32] = 4.0
    t4 = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0], np.float32)
    v[6, 1:9] = t4
    v[6, 33:41] = -t4
    v[7] = rng.standard_normal(256).astype(np.float32) * 0.02
    return v


@pytest.mark.parametrize("fmt", [mxmoe.MX_FMT_E4M3, mxmoe.MX_FMT_E2M1])
@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_quantizer_bit_exact(fmt, src):
    v = quant_inputs()
    t = dev(v)
    if src == "bf16":
        t = t.to(torch.bfloat16)
        v = t.float().cpu().numpy()
    q, sc = quantize(t, fmt)
    if fmt == mxmoe.MX_FMT_E4M3:
        rq, rsc = oracle.quantize_e4m3(v)
    else:
        rq, rsc = oracle.quantize_e2m1(v)
    assert np.array_equal(host(sc), rsc)
    assert np.array_equal(host(q), rq)


def test_quantizer_workload_bytes_match_oracle():
    inp = synth.moe_inputs("tiny")
    w13 = inp.w13()
    q, sc = quantize(dev(w13), mxmoe.MX_FMT_E2M1)
    rq, rsc = oracle.quantize_e2m1(w13.reshape(-1, w13.shape[-1]))
    assert np.array_equal(host(q).reshape(rq.shape), rq) and np.array_equal(host(sc).reshape(rsc.shape), rsc)
    qx, sx = quantize(dev(inp.x).to(torch.bfloat16), mxmoe.MX_FMT_E4M3)
    rqx, rsx = oracle.quantize_e4m3(inp.x)
    assert np.array_equal(host(qx), rqx) and np.array_equal(host(sx), rsx)


# ---------------------------------------------------------------------- route
def check_route(logits, k, survival=None, skip=0.2):
    T, E = logits.shape
    r = oracle.route(logits, k, survival, skip)
    g = Route(T, E, k)
    g(dev(logits), None if survival is None else dev(survival), skip)
    assert np.array_equal(host(g.ids), r["ids"])
    assert np.array_equal(host(g.offsets), r["offsets"])
    assert np.array_equal(host(g.perm), r["perm"])
    assert np.array_equal(host(g.slot_pos), r["slot_pos"])
    w = host(g.w)
    assert np.all(np.abs(w - r["w"]) <= 2.0 ** -22 * np.abs(r["w"]))
    return g


@pytest.mark.parametrize("name", ["tiny", "decode", "verify", "prefill"])
def test_route_workloads(name):
    inp = synth.moe_inputs(name)
    say(f"route {name} T={inp.cfg.T}")
    check_route(inp.logits, inp.cfg.k, inp.survival)


def test_route_edge_cases():
    rng = np.random.default_rng(3)
    ties = np.round(rng.standard_normal((300, 64)) * 2).astype(np.float32)      # many exact ties
    ties[7] = 0.0
    ties[8, ::2] = -0.0
    check_route(ties, 8)
    surv = rng.random(300).astype(np.float32)
    check_route(ties, 8, surv)                                                  # multi-chunk with dead rows
    check_route(rng.standard_normal((5, 1024)).astype(np.float32), 16)           # E = 1024, k = 16
    check_route(rng.standard_normal((100, 1024)).astype(np.float32), 16, surv[:100])   # the same, ranked over CUs
    check_route(rng.standard_normal((40, 512)).astype(np.float32), 8, surv[:40])        # E = 512
    check_route(rng.standard_normal((3, 1)).astype(np.float32), 1)              # E = 1
    check_route(rng.standard_normal((64, 32)).astype(np.float32), 4, np.zeros(64, np.float32))   # all dead
    check_route(rng.standard_normal((700, 256)).astype(np.float32), 8)          # ragged last chunk
    # around the row count where ranking moves out of the single bucketing workgroup
    for T, variant in ((32, "route:fused_single_workgroup"), (33, "route:topk_wave+bucket_single_workgroup"),
                       (256, "route:topk_wave+bucket_single_workgroup")):
        check_route(ties[:T], 8, surv[:T])
        assert mxmoe.last_variant() == variant, (T, mxmoe.last_variant())


# ----------------------------------------------------------------- expert FFN
# Both kernel paths are checked against the oracle on their own outputs
# (gpu_common.ffn_parity: gate/up of every live pair, the requant bit for bit
# on identical h, down + combine from the GPU's own intermediate, end to end).
def both_paths(layer):
    c = layer.cfg
    return (1, 2) if c.H % 256 == 0 and c.I <= 608 else (1,)


@pytest.mark.parametrize("shape", [
    dict(seed=31, T=37, H=384, E=12, k=3, I=96, skip=0.3),       # ragged rows, K tail of one step, I < 128
    dict(seed=32, T=5, H=1152, E=4, k=2, I=160, skip=0.0),       # several K parts (H > 1024), odd step count
    dict(seed=33, T=70, H=256, E=64, k=8, I=64, skip=0.0),       # many experts, ~9 rows each
    dict(seed=34, T=33, H=128, E=2, k=2, I=32, skip=0.0),        # every row hits both experts: 33 rows / expert
])
def test_ffn_small_shapes(shape):
    inp, r, layer = small_workload(**shape)
    say(f"ffn small {shape}")
    for path in both_paths(layer):
        ffn_parity(inp, r, layer, what=str(shape), path=path)


@pytest.mark.parametrize("path", [1, 2])
def test_ffn_tiny_workload(path):
    inp, r, layer = moe_workload("tiny")
    ffn_parity(inp, r, layer, what="tiny", path=path)


@pytest.mark.parametrize("path", [1, 2])
def test_ffn_decode_workload(path):
    inp, r, layer = moe_workload("decode")
    ffn_parity(inp, r, layer, what="decode", path=path, strict_e2e=True)


@pytest.mark.parametrize("path", [1, 2])
def test_ffn_verify_workload(path):
    inp, r, layer = moe_workload("verify")
    yg = ffn_parity(inp, r, layer, what="verify", path=path, strict_e2e=True)
    dead = ~r["live"].astype(bool)
    assert dead.any() and np.all(yg[dead] == 0)


def test_ffn_prefill_workload_prefill_kernels():
    """The 8192-token chunk on the prefill kernels (the path it takes):
    every pair of 64 sampled rows (plus the first and last) staged against
    the oracle; then the decode kernels on the same chunk give the same bits."""
    inp, r, layer = moe_workload("prefill")
    rows = np.random.default_rng(4).choice(inp.cfg.T, 62, replace=False).astype(np.int32)
    rows = np.concatenate([rows, [0, inp.cfg.T - 1]]).astype(np.int32)
    say("ffn prefill: prefill kernels, oracle on every pair of 64 sampled rows")
    y_pre = ffn_parity(inp, r, layer, rows=rows, what="prefill sample", path=2)
    y_dec, _, _, _ = gpu_ffn_with_h(layer, 1)
    assert np.array_equal(host(y_dec).view(np.uint32), y_pre.view(np.uint32))


# ----------------------------------------------------------------- dense GEMM
def gemm_case(M, N, K, seed):
    rng = np.random.default_rng(seed)
    a = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    return a, w


def check_gemm(a, w, rows=None):
    aq, asc = oracle.quantize_e4m3(a)
    wq, wsc = oracle.quantize_e4m3(w)
    M, N = a.shape[0], w.shape[0]
    da, dasc, dw, dwsc = dev(aq), dev(asc), dev(wq), dev(wsc)
    y32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    y16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mxmoe.fp8_block_gemm(da, dasc, dw, dwsc, y32, mxmoe.MX_OUT_F32)
    mxmoe.fp8_block_gemm(da, dasc, dw, dwsc, y16, mxmoe.MX_OUT_BF16)
    g32 = host(y32)
    ref = oracle.block_gemm(aq, asc, wq, wsc, rows=rows)
    assert_close(g32 if rows is None else g32[rows], ref, f"gemm {M}x{N}x{a.shape[1]}")
    # bf16 output is the round-to-nearest-even of the GPU's own fp32 result
    assert torch.equal(y16.cpu().view(torch.int16), y32.cpu().to(torch.bfloat16).view(torch.int16))
    return g32


@pytest.mark.parametrize("M", [1, 16])
def test_gemm_dense_workload(M):
    inp = synth.dense_inputs()
    check_gemm(inp.a[:M], inp.w, rows=None if M == 1 else np.arange(0, 16, 3, dtype=np.int32))


@pytest.mark.parametrize("M,N,K", [(21, 48, 384), (1, 16, 128), (40, 272, 2176), (3, 4096, 1024),
                                   (1, 64, 576), (5, 4096, 576), (16, 272, 96), (3, 48, 32), (7, 32, 1120)])
def test_gemm_shapes(M, N, K):
    a, w = gemm_case(M, N, K, M + N + K)
    check_gemm(a, w)


@pytest.mark.parametrize("M,N,K", [(320, 128, 1024), (333, 272, 2176), (520, 4096, 4096),
                                   (333, 272, 576), (330, 128, 1120), (321, 64, 32)])
def test_gemm_prefill_shapes(M, N, K):
    """The tiled kernel (M >= 320): ragged row and column tiles, a partial
    last K part; sampled rows against the oracle."""
    a, w = gemm_case(M, N, K, 7 * M + N + K)
    rows = np.unique(np.concatenate([np.arange(0, M, 37), [M - 1]])).astype(np.int32)
    check_gemm(a, w, rows=rows)
    assert mxmoe.last_variant().startswith("gemm:prefill")


def test_gemm_prefill_rows_equal_decode_rows():
    """Rows of a 333-row GEMM (tiled prefill kernel) equal, bit for bit, the
    same rows run 1..16 at a time (decode kernel)."""
    a, w = gemm_case(333, 272, 2176, 11)
    aq, asc = oracle.quantize_e4m3(a)
    wq, wsc = oracle.quantize_e4m3(w)
    full = torch.empty((333, 272), dtype=torch.float32, device="cuda")
    mxmoe.fp8_block_gemm(dev(aq), dev(asc), dev(wq), dev(wsc), full, mxmoe.MX_OUT_F32)
    assert mxmoe.last_variant().startswith("gemm:prefill")
    full = host(full)
    for m0, m1 in [(0, 1), (127, 128), (128, 144), (320, 333)]:
        y = torch.empty((m1 - m0, 272), dtype=torch.float32, device="cuda")
        mxmoe.fp8_block_gemm(dev(aq[m0:m1]), dev(asc[m0:m1]), dev(wq), dev(wsc), y, mxmoe.MX_OUT_F32)
        assert mxmoe.last_variant().startswith("gemm:decode")
        assert np.array_equal(host(y), full[m0:m1]), (m0, m1)


def test_gemm_k_tail_rows_equal_across_kernels():
    """K = 576 (4.5 MFMA steps, scale rows of 18 bytes): rows of the tiled
    kernel equal the decode kernel's, bit for bit."""
    a, w = gemm_case(333, 4096, 576, 13)
    aq, asc = oracle.quantize_e4m3(a)
    wq, wsc = oracle.quantize_e4m3(w)
    full = torch.empty((333, 4096), dtype=torch.float32, device="cuda")
    mxmoe.fp8_block_gemm(dev(aq), dev(asc), dev(wq), dev(wsc), full, mxmoe.MX_OUT_F32)
    assert "ktail" in mxmoe.last_variant() and mxmoe.last_variant().startswith("gemm:prefill")
    full = host(full)
    for m0, m1 in [(0, 1), (100, 116), (332, 333)]:
        y = torch.empty((m1 - m0, 4096), dtype=torch.float32, device="cuda")
        mxmoe.fp8_block_gemm(dev(aq[m0:m1]), dev(asc[m0:m1]), dev(wq), dev(wsc), y, mxmoe.MX_OUT_F32)
        assert mxmoe.last_variant().startswith("gemm:decode")
        assert np.array_equal(host(y), full[m0:m1]), (m0, m1)


def test_gemm_rows_do_not_depend_on_M():
    a, w = gemm_case(64, 256, 4096, 9)
    full = check_gemm(a, w, rows=np.arange(0, 64, 7, dtype=np.int32))
    aq, asc = oracle.quantize_e4m3(a)
    wq, wsc = oracle.quantize_e4m3(w)
    for m0, m1 in [(0, 1), (5, 6), (3, 20), (17, 64)]:
        y = torch.empty((m1 - m0, 256), dtype=torch.float32, device="cuda")
        mxmoe.fp8_block_gemm(dev(aq[m0:m1]), dev(asc[m0:m1]), dev(wq), dev(wsc), y, mxmoe.MX_OUT_F32)
        assert np.array_equal(host(y), full[m0:m1])


# ------------------------------------------------ the pages' own layer shape
def test_ffn_pages_shape_both_paths():
    """One TP4 rank's routed layer as the pages size it (384 experts, hidden
    5120, intermediate slice 576), top-8: the decode path (fused single row
    and T = 4) and the prefill kernels on the same rows, against the oracle,
    bitwise equal to each other."""
    inp = synth.small_moe(61, 4, 5120, 384, 8, 576)
    r = oracle.route(inp.logits, 8)
    layer = Layer(inp, np.unique(r["ids"]))
    say("pages shape H=5120 E=384 I=576: decode and prefill paths")
    y_dec = ffn_parity(inp, r, layer, what="pages shape", path=1)
    y_pre = ffn_parity(inp, r, layer, what="pages shape", path=2)
    assert np.array_equal(y_pre.view(np.uint32), y_dec.view(np.uint32))
    # the single-row fused layer on row 0
    d = layer.d
    route1 = Route(1, 384, 8)
    ffn1 = ExpertFFN(1, 5120, 384, 576, 8)
    mxmoe.moe_layer_decode1(dev(inp.logits[:1]), 8, None, 0.2, d["x"][:1].contiguous(), d["x_sc"][:1].contiguous(),
                            d["w13"], d["w13_sc"], d["w2"], d["w2_sc"], 384, 576, route1.ids, route1.w,
                            route1.offsets, route1.perm, route1.slot_pos, ffn1.y, ffn1.ws)
    assert np.array_equal(host(ffn1.y)[0], y_dec[0])
