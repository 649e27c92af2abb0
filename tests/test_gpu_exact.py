"""Integer-exact cases: operands whose every partial sum is exactly
representable in fp32, so the sum does not depend on its order or on the
matrix cores' accumulation, and the GPU must equal the oracle bit for bit
(forum thread post #6, "Why TileLang": DeepSeek's arithmetic term for term;
"How it works": block-scaled FP8 x FP4 experts and MXFP8 projections).

Each test checks the exactness condition itself before comparing: for every
output, with L the exponent of the lowest set bit over its nonzero products
and S the sum of their magnitudes, S < 2^(L + 24) makes every partial sum, in
any order, a multiple of 2^L below 2^(L + 24), hence exact in fp32."""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import dev, host, say
from block_scaled_fp8xfp4_amd import mxmoe
from block_scaled_fp8xfp4_amd.layer import ExpertFFN, Route

pytestmark = pytest.mark.gpu



def lowest_bit_exponent(v):
    """Exponent of the lowest set bit of each nonzero float64 (inf for zeros)."""
    v = np.abs(np.asarray(v, np.float64))
    m, e = np.frexp(v)                                   # v = m 2^e, m in [0.5, 1)
    mi = (m * 2.0 ** 53).astype(np.uint64)               # 53-bit integer mantissa
    tz = np.zeros(v.shape, np.int64)
    nz = mi != 0
    low = mi & (~mi + np.uint64(1))                      # lowest set bit
    tz[nz] = np.log2(low[nz].astype(np.float64)).astype(np.int64)
    out = (e - 53 + tz).astype(np.float64)
    out[~nz] = np.inf
    return out


def assert_exact_sums(products, what):
    """products [..., K]: every row's partial sums are exact in fp32."""
    L = lowest_bit_exponent(products).min(axis=-1)
    S = np.abs(products).sum(axis=-1)
    ok = (S == 0) | (S < 2.0 ** (L + 24))
    assert ok.all(), f"{what}: {int((~ok).sum())} outputs whose sum is not exact in fp32 (test construction)"


@pytest.mark.parametrize("M,N,K", [(1, 64, 256), (16, 4096, 1024), (5, 48, 576), (333, 272, 2176),
                                   (320, 128, 4096)])
def test_gemm_integer_operands_bitwise(M, N, K):
    """Small-integer activations and weights (quantized by the oracle: the
    decoded values are the integers themselves): y == oracle bit for bit on
    the decode kernel (M < 320) and the tiled kernel, K tails included."""
    rng = np.random.default_rng(M * 7 + N + K)
    vals = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 12, 16], np.float32)
    a = rng.choice(vals, (M, K)) * rng.choice([-1, 1], (M, K))
    w = rng.choice(vals, (N, K)) * rng.choice([-1, 1], (N, K))
    a[:, ::32] = 16                                        # block maximum 16 in every block
    w[:, ::32] = -16
    aq, asc = oracle.quantize_e4m3(a.astype(np.float32))
    wq, wsc = oracle.quantize_e4m3(w.astype(np.float32))
    ad, wd = oracle.dequantize(aq, asc, "e4m3"), oracle.dequantize(wq, wsc, "e4m3")
    assert np.array_equal(ad, a) and np.array_equal(wd, w)
    # integer products: every partial sum is an integer of magnitude <= sum |a||w| < 2^24
    assert (np.abs(ad) @ np.abs(wd).T).max() < 2 ** 24
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    mxmoe.fp8_block_gemm(dev(aq), dev(asc), dev(wq), dev(wsc), y, mxmoe.MX_OUT_F32)
    assert mxmoe.last_variant().startswith("gemm:prefill" if M >= 320 else "gemm:decode")
    got = host(y)
    ref = oracle.block_gemm(aq, asc, wq, wsc)
    assert np.array_equal(ref, (ad @ wd.T).astype(np.float32))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def exact_layer(seed, T=40, H=256, E=8, I=64):
    """A routed layer whose whole chain is exact on the matrix cores:
    activations 1 or 2; gate rows of positive E2M1 values 1..3 (gate 256..1536,
    whose SiLU equals the gate in double), up rows with one to three 1.0s (up
    1..6), so a = silu(gate) up lies within a factor 36 and requantizes to
    codes whose down products with half-integer E2M1 weights stay exact;
    top-2 of tied logits gives every slot weight 0.5 exactly."""
    rng = np.random.default_rng(seed)
    x = np.where(rng.random((T, H)) < 0.5, 0x38, 0x40).astype(np.uint8)     # 1.0 or 2.0
    x_sc = np.full((T, H // 32), 127, np.uint8)
    g = rng.choice([2, 3, 4, 5], (E, I, H))                                 # 1, 1.5, 2, 3
    u = np.zeros((E, I, H), np.int64)
    for e in range(E):
        for i in range(I):
            u[e, i, rng.choice(H, rng.integers(1, 4), replace=False)] = 2       # 1.0
    codes13 = np.concatenate([g, u], axis=1)
    w13 = (codes13[..., 0::2] | (codes13[..., 1::2] << 4)).astype(np.uint8)
    w13_sc = np.full((E, 2 * I, H // 32), 127, np.uint8)
    c2 = rng.choice([0, 1, 2, 3, 4, 5, 9, 10, 11, 12, 13], (E, H, I))       # 0, +-0.5 .. +-2, 3
    w2 = (c2[..., 0::2] | (c2[..., 1::2] << 4)).astype(np.uint8)
    w2_sc = np.full((E, H, I // 32), 127, np.uint8)
    logits = rng.uniform(-3, 0, (T, E)).astype(np.float32)
    for t in range(T):
        logits[t, rng.choice(E, 2, replace=False)] = 5.0
    return x, x_sc, w13, w13_sc, w2, w2_sc, logits


@pytest.mark.parametrize("path", [1, 2])
def test_ffn_integer_operands_bitwise(path):
    """The whole routed layer on exact operands: the gate/up values (diagnostic
    output), the FP8 intermediate and its scales, and y equal the oracle's bit
    for bit, on the decode and the prefill kernels."""
    x, x_sc, w13, w13_sc, w2, w2_sc, logits = exact_layer(7)
    T, H = x.shape
    E, I, k = w13.shape[0], w13.shape[1] // 2, 2
    r = oracle.route(logits, k)
    assert np.all(r["w"] == 0.5)
    ts = np.repeat(np.arange(T, dtype=np.int32), k)
    es = r["ids"].ravel().astype(np.int32)
    h_ref = oracle.gate_up_pairs(x, x_sc, ts, es, w13, w13_sc)
    xd = oracle.dequantize(x, x_sc, "e4m3")
    assert np.all(h_ref[:, :I] >= 256) and np.all(h_ref[:, I:] >= 1)
    q_ref, sc_ref, _ = oracle.swiglu_requant(h_ref)
    qd = oracle.dequantize(q_ref, sc_ref, "e4m3")
    w2d = oracle.dequantize(w2.reshape(E * H, I // 2), w2_sc.reshape(E * H, I // 32), "e2m1").reshape(E, H, I)
    for i in range(0, T * k, 7):
        assert_exact_sums(qd[i][None, :] * w2d[es[i]], "down products")
    w13d = oracle.dequantize(w13.reshape(E * 2 * I, H // 2), w13_sc.reshape(E * 2 * I, H // 32),
                             "e2m1").reshape(E, 2 * I, H)
    assert_exact_sums(xd[ts[0]][None, :] * w13d[es[0]], "gate/up products")
    y_ref = oracle.moe_rows(x, x_sc, r["ids"], r["w"], r["live"], w13, w13_sc, w2, w2_sc)

    route = Route(T, E, k)
    route(dev(logits))
    assert np.array_equal(host(route.slot_pos), r["slot_pos"]) and np.all(host(route.w) == 0.5)
    ffn = ExpertFFN(T, H, E, I, k)
    hbuf = torch.empty((T * k, 2 * I), dtype=torch.float32, device="cuda")
    old = mxmoe.set_ffn_path(path)
    mxmoe.set_ffn_diag(hbuf)
    try:
        y = ffn(dev(x), dev(x_sc), route, dev(w13), dev(w13_sc), dev(w2), dev(w2_sc))
        assert ("decode" if path == 1 else "prefill") in mxmoe.last_variant()
    finally:
        mxmoe.set_ffn_diag(None)
        mxmoe.set_ffn_path(old)
    q, qsc, _ = (host(t) for t in ffn.ws_views())
    sp = r["slot_pos"].ravel()
    assert np.array_equal(host(hbuf)[sp].view(np.uint32), h_ref.view(np.uint32))
    assert np.array_equal(q[sp], q_ref) and np.array_equal(qsc[sp], sc_ref)
    assert np.array_equal(host(y).view(np.uint32), y_ref.view(np.uint32))
    say(f"integer-exact layer, path {path}: h, intermediate and y bitwise equal to the oracle")
