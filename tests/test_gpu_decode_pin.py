"""Exhaustive pin of the operand decode inside the kernels' own scaled-MFMA
paths (OCP MX v1.0 element and scale encodings; forum thread post #6, "How it
works": block-scaled MMAs for MXFP8, FP8 x FP4 and MXFP4).

Every finite E4M3 code (254) and every E2M1 code (16) is combined with every
E8M0 scale code 0..254 and sent through the library's kernels with one-hot
operands: one element of a row is the code under test, every other element
is zero, and the other operand is all ones at scale 2^0.  Each output element
is then a sum of exactly one product, dec(code) * 2^(scale - 127), plus
zeros, so it must equal the oracle's decode of that code and scale (double,
rounded once to fp32, added to +0) bit for bit:
  - E4M3 activations and E4M3 weights through the dense GEMM (both kernels);
  - E4M3 activations and E2M1 gate/up weights through the routed experts'
    gate/up GEMM (both paths, read back through the diagnostic output);
  - E2M1 down-projection weights through the routed experts' down GEMM and
    combine (the fused single row, and both paths), with an intermediate
    built to requantize to exactly 1.0.
"""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp8xfp4_amd import mxmoe
from block_scaled_fp8xfp4_amd.layer import ExpertFFN, Route
from gpu_common import dev, host, say

pytestmark = pytest.mark.gpu

E4M3_CODES = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)   # 254 finite codes
E2M1_CODES = np.arange(16, dtype=np.uint8)
SCALES = np.arange(255, dtype=np.uint8)                                           # 255 = NaN is excluded
ONE_E4M3, ONE_E2M1 = 0x38, 0x2


def expected_single(values):
    """fp32 of (+0 + v) for each double v: the sum of one exact product and zeros."""
    with np.errstate(over="ignore"):
        return (np.float64(0.0) + np.asarray(values, np.float64)).astype(np.float32)


def combos(codes):
    c, s = np.meshgrid(codes, SCALES, indexing="ij")
    return c.ravel().astype(np.uint8), s.ravel().astype(np.uint8)


def one_hot_e4m3(codes, scales, K):
    """Rows [n][K] E4M3 with codes[i] at position i % K under scales[i]; other blocks at 2^0."""
    n = len(codes)
    pos = np.arange(n) % K
    q = np.zeros((n, K), np.uint8)
    q[np.arange(n), pos] = codes
    sc = np.full((n, K // 32), 127, np.uint8)
    sc[np.arange(n), pos // 32] = scales
    return q, sc


def one_hot_e2m1(codes, scales, K):
    """Rows [n][K/2] packed E2M1 with codes[i] at element i % K under scales[i]."""
    n = len(codes)
    pos = np.arange(n) % K
    q = np.zeros((n, K // 2), np.uint8)
    q[np.arange(n), pos // 2] = np.where(pos % 2 == 0, codes, codes.astype(np.uint16) << 4).astype(np.uint8)
    sc = np.full((n, K // 32), 127, np.uint8)
    sc[np.arange(n), pos // 32] = scales
    return q, sc


def compare_bits(got, want, what):
    """Bitwise equality, with the mismatches broken down by the class of the expected value."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    bad = got.view(np.uint32) != want.view(np.uint32)
    if bad.any():
        a = np.abs(want.astype(np.float64))
        classes = {"normal": (a >= 2.0 ** -126) & np.isfinite(a), "subnormal": (a > 0) & (a < 2.0 ** -126),
                   "zero": a == 0, "inf": np.isinf(a)}
        detail = {k: (int((bad & m).sum()), int(m.sum())) for k, m in classes.items()}
        i = np.flatnonzero(bad.ravel())[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} differ; by class (bad, total) {detail}; "
                             f"first got {got.ravel()[i]} want {want.ravel()[i]}")


def value_of(q, sc, fmt):
    """Single-product expectation through the oracle's own decode tables."""
    return expected_single(oracle.dequantize(q, sc, fmt).sum(axis=1))


# ------------------------------------------------------------- dense GEMM
def gemm_f32(a, a_sc, w, w_sc):
    y = torch.empty((a.shape[0], w.shape[0]), dtype=torch.float32, device="cuda")
    mxmoe.fp8_block_gemm(dev(a), dev(a_sc), dev(w), dev(w_sc), y, mxmoe.MX_OUT_F32)
    return y


def test_gemm_activation_codes_times_every_scale():
    """E4M3 activation codes x scales (64 770 one-hot rows) against all-ones
    weights: the tiled kernel on all rows at once, the decode kernel in
    256-row slices; every one of the 16 output columns equals the decode."""
    K, N = 256, 16
    codes, scales = combos(E4M3_CODES)
    a, a_sc = one_hot_e4m3(codes, scales, K)
    w = np.full((N, K), ONE_E4M3, np.uint8)
    w_sc = np.full((N, K // 32), 127, np.uint8)
    want = value_of(a, a_sc, "e4m3")
    y = host(gemm_f32(a, a_sc, w, w_sc))
    assert mxmoe.last_variant().startswith("gemm:prefill")
    compare_bits(y, np.repeat(want[:, None], N, axis=1), "gemm A codes, tiled kernel")
    da, dsc, dw, dwsc = dev(a), dev(a_sc), dev(w), dev(w_sc)
    out = torch.empty((len(a), N), dtype=torch.float32, device="cuda")
    for m0 in range(0, len(a), 256):
        m1 = min(len(a), m0 + 256)
        mxmoe.fp8_block_gemm(da[m0:m1], dsc[m0:m1], dw, dwsc, out[m0:m1], mxmoe.MX_OUT_F32)
    assert mxmoe.last_variant().startswith("gemm:decode")
    compare_bits(host(out), np.repeat(want[:, None], N, axis=1), "gemm A codes, decode kernel")
    say(f"gemm activation decode pin: {len(a)} code x scale pairs bitwise on both kernels")


def test_gemm_weight_codes_times_every_scale():
    """E4M3 weight codes x scales (64 770 one-hot weight rows, N padded to a
    multiple of 16 with zero rows) against an all-ones activation row: one row
    (decode kernel) and 320 identical rows (tiled kernel)."""
    K = 256
    codes, scales = combos(E4M3_CODES)
    n = len(codes)
    N = (n + 15) // 16 * 16
    w, w_sc = one_hot_e4m3(np.concatenate([codes, np.zeros(N - n, np.uint8)]),
                           np.concatenate([scales, np.full(N - n, 127, np.uint8)]), K)
    want = value_of(w, w_sc, "e4m3")
    for M, kern in ((1, "gemm:decode"), (320, "gemm:prefill")):
        a = np.full((M, K), ONE_E4M3, np.uint8)
        a_sc = np.full((M, K // 32), 127, np.uint8)
        y = host(gemm_f32(a, a_sc, w, w_sc))
        assert mxmoe.last_variant().startswith(kern)
        compare_bits(y, np.broadcast_to(want, y.shape), f"gemm W codes, M={M}")
    say(f"gemm weight decode pin: {n} code x scale pairs bitwise on both kernels")


# ------------------------------------------------------- routed experts
class PinLayer:
    """A routed layer built from given codes (device copies), and runs of it."""

    def __init__(self, x, x_sc, w13, w13_sc, w2, w2_sc, logits, k):
        self.x, self.x_sc, self.w13, self.w13_sc, self.w2, self.w2_sc = x, x_sc, w13, w13_sc, w2, w2_sc
        self.logits = np.ascontiguousarray(logits, np.float32)
        self.T, self.H = x.shape
        self.E, twoI = w13.shape[0], w13.shape[1]
        self.I, self.k = twoI // 2, k
        self.d = {n: dev(getattr(self, n)) for n in ("x", "x_sc", "w13", "w13_sc", "w2", "w2_sc")}

    def run(self, path):
        """(y, h, route) of moe_route + moe_expert_ffn on the given path, h from the diagnostic output."""
        route = Route(self.T, self.E, self.k)
        route(dev(self.logits))
        ffn = ExpertFFN(self.T, self.H, self.E, self.I, self.k)
        hbuf = torch.empty((self.T * self.k, 2 * self.I), dtype=torch.float32, device="cuda")
        old = mxmoe.set_ffn_path(path)
        mxmoe.set_ffn_diag(hbuf)
        try:
            y = ffn(self.d["x"], self.d["x_sc"], route, self.d["w13"], self.d["w13_sc"], self.d["w2"],
                    self.d["w2_sc"])
            v = mxmoe.last_variant()
        finally:
            mxmoe.set_ffn_diag(None)
            mxmoe.set_ffn_path(old)
        assert ("decode" if path == 1 else "prefill") in v, v
        return host(y), host(hbuf), route

    def run_fused_row(self):
        """y of moe_layer_decode1 on row 0 (the gate inside the gate/up kernel)."""
        ids = torch.empty((1, self.k), dtype=torch.int32, device="cuda")
        w = torch.empty((1, self.k), dtype=torch.float32, device="cuda")
        off = torch.empty(self.E + 1, dtype=torch.int32, device="cuda")
        perm = torch.empty(self.k, dtype=torch.int32, device="cuda")
        sp = torch.empty((1, self.k), dtype=torch.int32, device="cuda")
        y = torch.empty((1, self.H), dtype=torch.float32, device="cuda")
        ws = torch.empty(mxmoe.moe_expert_ffn_workspace_bytes(1, self.H, self.E, self.I, self.k), dtype=torch.uint8,
                         device="cuda")
        mxmoe.moe_layer_decode1(dev(self.logits[:1]), self.k, None, 0.2, self.d["x"][:1].contiguous(),
                                self.d["x_sc"][:1].contiguous(), self.d["w13"], self.d["w13_sc"], self.d["w2"],
                                self.d["w2_sc"], self.E, self.I, ids, w, off, perm, sp, y, ws)
        assert mxmoe.last_variant().startswith("layer1:")
        return host(y)


def test_ffn_gate_up_weight_codes_times_every_scale():
    """E2M1 gate/up weight codes x scales (4 080 one-hot W13 rows over 8
    experts of 2I = 512 rows) against all-ones activations: every row routes
    to all 8 experts (equal logits), so bucket position p = e T + t holds
    expert e's 512 decoded values."""
    H, I, E = 256, 256, 8
    codes, scales = combos(E2M1_CODES)
    n = len(codes)
    rows = E * 2 * I
    w13, w13_sc = one_hot_e2m1(np.concatenate([codes, np.zeros(rows - n, np.uint8)]),
                               np.concatenate([scales, np.full(rows - n, 127, np.uint8)]), H)
    want = value_of(w13, w13_sc, "e2m1").reshape(E, 2 * I)
    w13, w13_sc = w13.reshape(E, 2 * I, H // 2), w13_sc.reshape(E, 2 * I, H // 32)
    w2 = np.zeros((E, H, I // 2), np.uint8)
    w2_sc = np.full((E, H, I // 32), 127, np.uint8)
    for T, path in ((1, 1), (3, 1), (3, 2)):
        x = np.full((T, H), ONE_E4M3, np.uint8)
        x_sc = np.full((T, H // 32), 127, np.uint8)
        L = PinLayer(x, x_sc, w13, w13_sc, w2, w2_sc, np.zeros((T, E)), E)
        _, h, route = L.run(path)
        assert np.array_equal(host(route.offsets), np.arange(E + 1) * T)
        compare_bits(h, np.repeat(want, T, axis=0), f"gate/up W13 codes, T={T}, path {path}")
    say(f"gate/up weight decode pin: {n} code x scale pairs bitwise on both paths")


def test_ffn_gate_up_activation_codes_times_every_scale():
    """E4M3 activation codes x scales (64 770 one-hot activation rows, one
    expert, k = 1) against all-ones E2M1 gate/up weights: h[p] of row p holds
    the decoded code in every column, on both paths."""
    H, I = 256, 32
    codes, scales = combos(E4M3_CODES)
    x, x_sc = one_hot_e4m3(codes, scales, H)
    want = value_of(x, x_sc, "e4m3")
    T = len(x)
    w13 = np.full((1, 2 * I, H // 2), ONE_E2M1 | (ONE_E2M1 << 4), np.uint8)
    w13_sc = np.full((1, 2 * I, H // 32), 127, np.uint8)
    w2 = np.zeros((1, H, I // 2), np.uint8)
    w2_sc = np.full((1, H, I // 32), 127, np.uint8)
    L = PinLayer(x, x_sc, w13, w13_sc, w2, w2_sc, np.zeros((T, 1)), 1)
    for path in (1, 2):
        _, h, _ = L.run(path)
        compare_bits(h, np.repeat(want[:, None], 2 * I, axis=1), f"gate/up activation codes, path {path}")
    say(f"gate/up activation decode pin: {T} code x scale pairs bitwise on both paths")


def test_ffn_down_weight_codes_times_every_scale():
    """E2M1 down weight codes x scales (4 080 one-hot W2 rows of H = 4096).
    Activations are all ones, the gate rows all ones (gate = 4096, whose SiLU
    is 4096 in double), and the up rows one 1.0 under scale 2^-12 (up =
    2^-12), so every intermediate value is exactly 1.0 and requantizes to 1.0;
    with k = 1 (weight 1) each y column is the decoded W2 code.  The fused
    single row, T = 1 and T = 3 on the decode kernels, T = 3 on the prefill
    kernels; each also equal to the oracle's whole layer bit for bit."""
    H, I = 4096, 64
    codes, scales = combos(E2M1_CODES)
    n = len(codes)
    w2, w2_sc = one_hot_e2m1(np.concatenate([codes, np.zeros(H - n, np.uint8)]),
                             np.concatenate([scales, np.full(H - n, 127, np.uint8)]), I)
    want = value_of(w2, w2_sc, "e2m1")
    w2, w2_sc = w2[None], w2_sc[None]
    w13 = np.zeros((1, 2 * I, H // 2), np.uint8)
    w13_sc = np.full((1, 2 * I, H // 32), 127, np.uint8)
    w13[0, :I] = ONE_E2M1 | (ONE_E2M1 << 4)                   # gate rows: 4096 ones
    w13[0, I:, 0] = ONE_E2M1                                   # up rows: element 0 = 1.0 ...
    w13_sc[0, I:, 0] = 127 - 12                                # ... under 2^-12
    for T, path in ((1, 0), (1, 1), (3, 1), (3, 2)):
        x = np.full((T, H), ONE_E4M3, np.uint8)
        x_sc = np.full((T, H // 32), 127, np.uint8)
        L = PinLayer(x, x_sc, w13, w13_sc, w2, w2_sc, np.zeros((T, 1)), 1)
        if path == 0:
            y = L.run_fused_row()
        else:
            y, h, _ = L.run(path)
            assert np.all(h[:, :I] == 4096.0) and np.all(h[:, I:] == 2.0 ** -12)
        compare_bits(y, np.broadcast_to(want, y.shape), f"down W2 codes, T={T}, path {path or 'fused'}")
        r = oracle.route(L.logits, 1)
        ref = oracle.moe_rows(x, x_sc, r["ids"], r["w"], r["live"], w13, w13_sc, w2, w2_sc)
        compare_bits(y, ref, f"down W2 codes vs the oracle's layer, T={T}, path {path or 'fused'}")
    say(f"down weight decode pin: {n} code x scale pairs bitwise on the fused row and both paths")
