"""Pins of the oracle's router logits (hidden . w_gate^T over bf16 operands,
fp32 result) against what the mathematics fixes, not against itself:
torch's own bf16 decoding on one-hot rows, exact integer arithmetic, a
library matmul in double, and exact scaling and sign symmetries."""
import numpy as np
import torch

import oracle


def bf16_bits(v):
    """fp32 values -> bf16 bit patterns through torch's rounding."""
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_decode(bits):
    """bf16 bit patterns -> float64 through torch's decoder."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def test_one_hot_rows_return_gate_columns_exactly():
    # hidden row t = e_{j_t} (bf16 1.0 = 0x3F80): logits[t][e] = w_gate[e][j_t], so a
    # transposed operand or a wrong decode shows up at once
    rng = np.random.default_rng(0)
    E, H = 24, 96
    wg = bf16_bits(rng.standard_normal((E, H)) * 3.0)
    cols = np.array([0, 1, 31, 32, 64, 95])
    h = np.zeros((len(cols), H), np.uint16)
    h[np.arange(len(cols)), cols] = 0x3F80
    out = oracle.router_logits(h, wg)
    want = bf16_decode(wg)[:, cols].T.astype(np.float32)
    assert np.array_equal(out.view(np.uint32), want.view(np.uint32))


def test_small_integers_are_exact():
    # integers |v| <= 8 are exact in bf16; every partial sum stays below 2^24
    rng = np.random.default_rng(1)
    T, E, H = 5, 7, 512
    hi = rng.integers(-8, 9, (T, H))
    wi = rng.integers(-8, 9, (E, H))
    out = oracle.router_logits(bf16_bits(hi), bf16_bits(wi))
    assert np.array_equal(out, (hi @ wi.T).astype(np.float32))


def test_matches_library_matmul_in_double():
    rng = np.random.default_rng(2)
    T, E, H = 9, 40, 4096
    h = bf16_bits(rng.standard_normal((T, H)))
    wg = bf16_bits(rng.standard_normal((E, H)) * 0.02)
    out = oracle.router_logits(h, wg)
    ref = bf16_decode(h) @ bf16_decode(wg).T              # float64, another summation order
    # both round a double sum (errors ~1e-16 relative) to fp32: at most one fp32 ulp apart
    ulp = np.spacing(np.abs(ref).astype(np.float32))
    assert np.all(np.abs(out.astype(np.float64) - ref) <= ulp)
    assert np.mean(out == ref.astype(np.float32)) > 0.999


def test_scaling_and_sign_symmetries_are_exact():
    rng = np.random.default_rng(3)
    T, E, H = 4, 16, 256
    hf = rng.standard_normal((T, H)).astype(np.float32)
    wf = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    base = oracle.router_logits(bf16_bits(hf), bf16_bits(wf))
    assert np.array_equal(oracle.router_logits(bf16_bits(hf * 4.0), bf16_bits(wf)), base * 4.0)
    assert np.array_equal(oracle.router_logits(bf16_bits(hf), bf16_bits(-wf)), -base)


def test_row_selection_and_threads_do_not_change_results():
    rng = np.random.default_rng(4)
    h = bf16_bits(rng.standard_normal((6, 128)))
    wg = bf16_bits(rng.standard_normal((10, 128)))
    full = oracle.router_logits(h, wg, threads=1)
    assert np.array_equal(oracle.router_logits(h, wg, threads=5), full)
    assert np.array_equal(oracle.router_logits(h, wg, rows=np.array([5, 0, 3])), full[[5, 0, 3]])
