"""Pins of the oracle's shared expert (FP8 block-32 gate/up GEMM, SwiGLU,
E4M3 requant, FP8 down GEMM with K = I, no padding) against a brute-force
float64 evaluation over torch-decoded operands with an independent requant,
and against exact integer arithmetic."""
import numpy as np
import pytest

import oracle
from test_oracle_moe import dec_e4m3, requant_e4m3_independent


def layer(seed, T, H, I, wstd=0.02):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    w13 = (rng.standard_normal((2 * I, H)) * wstd).astype(np.float32)
    w2 = (rng.standard_normal((H, I)) * wstd).astype(np.float32)
    return oracle.quantize_e4m3(x) + oracle.quantize_e4m3(w13) + oracle.quantize_e4m3(w2)


def brute(x, xs, w13, w13s, w2, w2s):
    X, W13, W2 = dec_e4m3(x, xs), dec_e4m3(w13, w13s), dec_e4m3(w2, w2s)
    I = W13.shape[0] // 2
    h = (X @ W13.T).astype(np.float32).astype(np.float64)
    g, u = h[:, :I], h[:, I:]
    a = (g / (1 + np.exp(-g)) * u).astype(np.float32)
    A = np.stack([requant_e4m3_independent(r) for r in a])
    return (A @ W2.T).astype(np.float32), h


@pytest.mark.parametrize("T,H,I", [(3, 256, 64), (5, 384, 576), (2, 1152, 96)])
def test_matches_brute_force_float64(T, H, I):
    x, xs, w13, w13s, w2, w2s = layer(T + H + I, T, H, I)
    y, h, q, q_sc = oracle.shared_expert(x, xs, w13, w13s, w2, w2s)
    yb, hb = brute(x, xs, w13, w13s, w2, w2s)
    assert np.all(np.abs(h - hb) <= np.spacing(np.abs(hb).astype(np.float32)))
    assert np.all(np.abs(y - yb) <= 2 * np.spacing(np.abs(yb)) + 1e-30)
    assert q.shape == (T, I) and q_sc.shape == (T, I // 32)


def test_rows_are_independent_and_selectable():
    x, xs, w13, w13s, w2, w2s = layer(1, 6, 256, 576)
    y, *_ = oracle.shared_expert(x, xs, w13, w13s, w2, w2s)
    ys, *_ = oracle.shared_expert(x, xs, w13, w13s, w2, w2s, rows=np.array([4, 1], np.int32))
    assert np.array_equal(ys, y[[4, 1]])


def test_exact_on_integer_operands():
    # unit scales, small integer codes: gate/up sums are exact; with up = 0 the
    # intermediate and the output are exactly zero, with gate = 0 as well
    H, I = 128, 64
    rng = np.random.default_rng(3)
    ints = np.array([0, 1, 2, 3, -1, -2, -3], np.float32)
    x = rng.choice(ints, (4, H)).astype(np.float32)
    w13 = rng.choice(ints, (2 * I, H)).astype(np.float32)
    w13[I:] = 0.0                                              # up rows zero
    w2 = rng.choice(ints, (H, I)).astype(np.float32)
    xq, xs = oracle.quantize_e4m3(x)
    q13, s13 = oracle.quantize_e4m3(w13)
    q2, s2 = oracle.quantize_e4m3(w2)
    y, h, q, q_sc = oracle.shared_expert(xq, xs, q13, s13, q2, s2)
    X, W = dec_e4m3(xq, xs), dec_e4m3(q13, s13)
    assert np.array_equal(h, (X @ W.T).astype(np.float32))       # integers: exact in double and fp32
    assert not np.any(q & 0x7F) and not np.any(y)
