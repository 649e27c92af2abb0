"""Shared helpers of the GPU parity tests: seeded workloads quantized by the
oracle on the CPU, their device copies, and the comparison rules."""
import functools
import sys

import numpy as np
import torch

import oracle
from block_scaled_fp8xfp4_amd import mxmoe, synth
from block_scaled_fp8xfp4_amd.layer import ExpertFFN, Route

# fp32-accumulated outputs: max|diff| <= 2e-3 * max|ref| and cosine >= 0.99999
TOL_REL_MAX = 2e-3
TOL_COS = 0.99999

# magnitudes of the E4M3 codes 0x00..0x7E (0x7F is NaN)
E4M3_MAG = np.array([oracle.e4m3_value(c) for c in range(0x7F)])


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda") if dtype is None else t.to("cuda", dtype=dtype)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def rel_err_cos(got, ref):
    """(max|got - ref| / max|ref|, cosine) in float64; (0, 1) for two zero arrays."""
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    scale = np.abs(ref).max() if ref.size else 0.0
    err = np.abs(got - ref).max() if ref.size else 0.0
    if scale == 0:
        return (0.0 if err == 0 else np.inf), (1.0 if err == 0 else 0.0)
    cos = float(got @ ref / max(np.linalg.norm(got) * np.linalg.norm(ref), 1e-300))
    return err / scale, cos


def assert_close(got, ref, what):
    """The bar for fp32-accumulated outputs: max|diff| <= 2e-3 max|ref|, cosine >= 0.99999."""
    assert np.all(np.isfinite(np.asarray(got, np.float64))), f"{what}: non-finite output"
    err, cos = rel_err_cos(got, ref)
    assert err <= TOL_REL_MAX, f"{what}: max|diff|/max|ref| {err:.3e} > {TOL_REL_MAX}"
    assert cos >= TOL_COS, f"{what}: cosine {cos:.7f}"
    return err, cos


def explain_code_differences(q_g, sc_g, a_g, q_r, sc_r, a_r):
    """The GPU's intermediate (its requant of its own fp32 h, which stage (ii)
    shows equal, bit for bit, to the oracle's requant of that h) against the
    oracle's own intermediate (the requant of the oracle's h).  The two h
    differ by the matrix cores' accumulation error, so a = silu(gate) * up
    differs slightly, and a code may differ only where that difference
    carries a across a rounding boundary:
      - a block scale differs only if the two block maxima lie in different
        binades and within 1e-4 of each other;
      - in a block with equal scales, the two element codes must each be
        consistent with rounding the other side's value range: the rounding
        boundary next to each code, toward the other code, lies between
        a_gpu / X and a_ref / X (for +0 / -0, a sign change of a); and a_gpu
        stays within 1e-2 of the pair's max |a_ref| (an unrelated row would
        not).  Where the subnormal steps are small against the block maximum,
        such a difference can span several codes.
    Returns (element codes differing, block scales differing)."""
    n, I = q_r.shape
    a_g = np.asarray(a_g, np.float64)
    a_r = np.asarray(a_r, np.float64)
    nsc = 0
    for r, b in zip(*np.nonzero(sc_g != sc_r)):
        mg = np.abs(a_g[r, 32 * b:32 * b + 32]).max()
        mr = np.abs(a_r[r, 32 * b:32 * b + 32]).max()
        assert np.floor(np.log2(mg)) != np.floor(np.log2(mr)), ("scale flip without a binade change", r, b, mg, mr)
        assert abs(mg - mr) <= 1e-4 * max(mg, mr), ("scale flip far from a power of two", r, b, mg, mr)
        nsc += 1

    def val(pos):                                      # signed grid position -> value (scaled by 1/X)
        return np.copysign(E4M3_MAG[abs(pos)], pos)

    same = np.repeat(sc_g == sc_r, 32, axis=1)
    row_max = np.abs(a_r).max(axis=1)
    nel = 0
    for r, i in zip(*np.nonzero(same & (q_g != q_r))):
        cg, cr = int(q_g[r, i]), int(q_r[r, i])
        assert abs(a_g[r, i] - a_r[r, i]) <= 1e-2 * row_max[r], ("a far from the oracle's", r, i, a_g[r, i], a_r[r, i])
        X = 2.0 ** (int(sc_r[r, i // 32]) - 127)
        tg, tr = a_g[r, i] / X, a_r[r, i] / X
        lo, hi = min(tg, tr), max(tg, tr)
        if (cg & 0x7F) == 0 and (cr & 0x7F) == 0:
            assert np.signbit(tg) != np.signbit(tr), ("signed-zero flip without a sign change", r, i, tg, tr)
        else:
            # positions on the signed E4M3 grid (+0 and -0 share position 0)
            pg = -(cg & 0x7F) if cg & 0x80 else (cg & 0x7F)
            pr = -(cr & 0x7F) if cr & 0x80 else (cr & 0x7F)
            d = 1 if pr > pg else -1
            mid_g = (val(pg) + val(pg + d)) / 2         # boundary next to the GPU's code, toward the oracle's
            mid_r = (val(pr) + val(pr - d)) / 2         # and next to the oracle's, toward the GPU's
            assert lo <= mid_g <= hi and lo <= mid_r <= hi, ("code difference not across rounding boundaries", r, i,
                                                             cg, cr, tg, tr)
        nel += 1
    return nel, nsc


class Layer:
    """Oracle-quantized MoE layer (host arrays) plus device copies."""

    def __init__(self, inp, experts=None):
        c = inp.cfg
        self.cfg, self.inp = c, inp
        E, H, I = c.E, c.H, c.I
        self.x, self.x_sc = oracle.quantize_e4m3(inp.x)
        self.w13 = np.zeros((E, 2 * I, H // 2), np.uint8)
        self.w13_sc = np.full((E, 2 * I, H // 32), 127, np.uint8)
        self.w2 = np.zeros((E, H, I // 2), np.uint8)
        self.w2_sc = np.full((E, H, I // 32), 127, np.uint8)
        experts = list(range(E)) if experts is None else sorted(set(int(e) for e in experts))
        for i in range(0, len(experts), 32):
            chunk = experts[i:i + 32]
            w13 = inp.w13(chunk)
            q, s = oracle.quantize_e2m1(w13.reshape(-1, H))
            self.w13[chunk] = q.reshape(len(chunk), 2 * I, H // 2)
            self.w13_sc[chunk] = s.reshape(len(chunk), 2 * I, H // 32)
            del w13
            w2 = inp.w2(chunk)
            q, s = oracle.quantize_e2m1(w2.reshape(-1, I))
            self.w2[chunk] = q.reshape(len(chunk), H, I // 2)
            self.w2_sc[chunk] = s.reshape(len(chunk), H, I // 32)
            del w2
        self.d = {n: dev(getattr(self, n)) for n in ("x", "x_sc", "w13", "w13_sc", "w2", "w2_sc")}

    def oracle_y(self, r, rows=None):
        return oracle.moe_rows(self.x, self.x_sc, r["ids"], r["w"], r["live"], self.w13, self.w13_sc,
                               self.w2, self.w2_sc, rows=rows)

    def gpu_route(self, rows=None):
        c, inp = self.cfg, self.inp
        logits = inp.logits if rows is None else inp.logits[rows]
        surv = inp.survival if (rows is None or inp.survival is None) else inp.survival[rows]
        route = Route(len(logits), c.E, c.k)
        route(dev(logits), None if surv is None else dev(surv))
        return route

    def gpu_y(self, rows=None, route=None):
        c = self.cfg
        x = self.d["x"] if rows is None else self.d["x"][dev(np.asarray(rows, np.int64))]
        x_sc = self.d["x_sc"] if rows is None else self.d["x_sc"][dev(np.asarray(rows, np.int64))]
        route = self.gpu_route(rows) if route is None else route
        ffn = ExpertFFN(x.shape[0], c.H, c.E, c.I, c.k)
        y = ffn(x.contiguous(), x_sc.contiguous(), route, self.d["w13"], self.d["w13_sc"], self.d["w2"],
                self.d["w2_sc"])
        return y, route, ffn


def gpu_ffn_with_h(layer, path, route=None):
    """Run the routed FFN on the given path (1 decode, 2 prefill kernels) with
    the diagnostic gate/up output on; returns (y, route, ffn, h) on the host
    except route/ffn."""
    c = layer.cfg
    hbuf = torch.empty(max(1, c.T * c.k * 2 * c.I), dtype=torch.float32, device="cuda")
    old = mxmoe.set_ffn_path(path)
    mxmoe.set_ffn_diag(hbuf)
    try:
        y, route, ffn = layer.gpu_y(route=route)
        variant = mxmoe.last_variant()
    finally:
        mxmoe.set_ffn_diag(None)
        mxmoe.set_ffn_path(old)
    if path == 1:
        assert "decode" in variant, variant
    else:
        assert "prefill" in variant, variant
    return y, route, ffn, hbuf.view(c.T * c.k, 2 * c.I)


def ffn_parity(inp, r, layer, rows=None, what="", path=1, route=None, strict_e2e=False):
    """Staged parity of one FFN path against the oracle on identical inputs:
    (i) gate/up h of EVERY live pair of `rows` against the oracle's h
        (2e-3 / 0.99999), read from the diagnostic output of the path's own
        gate/up kernel;
    (ii) the requant of the GPU's own h against the oracle's requant of the
        same fp32 h: bit for bit (both evaluate the SwiGLU in double and round
        once to fp32);
    (iii) y against the oracle's down projection + combine of the GPU's own
        intermediate (2e-3 / 0.99999);
    end to end: y against the full oracle.  Where the GPU's codes equal the
    oracle's own, end to end is stage (iii) and holds 2e-3 / 0.99999.  Codes
    may differ only where the matrix cores' h error carries a across an E4M3
    rounding boundary (explain_code_differences asserts every one); their
    effect on y is reported.  strict_e2e also asserts 2e-3 / 0.99999 end to
    end with whatever flips there are."""
    c = inp.cfg
    y, route, ffn, h = gpu_ffn_with_h(layer, path, route)
    assert np.array_equal(host(route.perm), r["perm"]) and np.array_equal(host(route.offsets), r["offsets"])
    yg = host(y)
    q, qsc, _ = (host(t) for t in ffn.ws_views())
    rows = np.arange(c.T, dtype=np.int32) if rows is None else np.asarray(rows, np.int32)
    pairs = [(int(t), j, int(r["slot_pos"][t, j])) for t in rows for j in range(c.k) if r["slot_pos"][t, j] >= 0]
    tag = f"{what} [path {path}]"
    if pairs:
        ts = np.array([t for t, _, _ in pairs], np.int32)
        es = np.array([int(r["ids"][t, j]) for t, j, _ in pairs], np.int32)
        ps = np.array([p for _, _, p in pairs], np.int64)
        hg = host(h[dev(ps)])
        # (i) gate/up on the matrix cores vs the oracle's double accumulation
        h_ref = oracle.gate_up_pairs(layer.x, layer.x_sc, ts, es, layer.w13, layer.w13_sc)
        ei, ci = assert_close(hg, h_ref, tag + " gate/up")
        # (ii) SwiGLU + requant on identical fp32 h: bit for bit
        q2, sc2, a_g = oracle.swiglu_requant(hg)
        assert np.array_equal(sc2, qsc[ps]), f"{tag}: requant scales differ on identical h"
        assert np.array_equal(q2, q[ps]), f"{tag}: requant codes differ on identical h"
        # the oracle's own intermediate (from its own h) against the GPU's
        q_r, sc_r, a_r = oracle.swiglu_requant(h_ref)
        nel, nsc = explain_code_differences(q[ps], qsc[ps], a_g, q_r, sc_r, a_r)
    else:
        ei, ci, nel, nsc = 0.0, 1.0, 0, 0
    # (iii) down + combine from the GPU's intermediate
    y_mid = oracle.down_combine(q, qsc, r["slot_pos"], r["ids"], r["w"], layer.w2, layer.w2_sc, rows=rows)
    e3, c3 = assert_close(yg[rows], y_mid, tag + " down+combine")
    # end to end against the full oracle
    ref = layer.oracle_y(r, rows)
    err, cos = rel_err_cos(yg[rows], ref)
    flip_err, _ = rel_err_cos(y_mid, ref)
    say(f"{tag}: pairs {len(pairs)}; gate/up {ei:.2e}; down+combine {e3:.2e}; intermediate codes differing from "
        f"the oracle's own {nel} (+{nsc} block scales), their effect on y {flip_err:.2e}; end-to-end "
        f"max|diff|/max|ref| {err:.2e}, cosine {cos:.8f}")
    if nel == 0 and nsc == 0:
        assert np.array_equal(y_mid, ref), f"{tag}: identical intermediate, different oracle y"
    if strict_e2e or (nel == 0 and nsc == 0):
        assert err <= TOL_REL_MAX and cos >= TOL_COS, f"{tag}: end-to-end {err:.2e} / cosine {cos:.8f}"
    live = r["live"].astype(bool)
    assert np.all(yg[~live] == 0) and not np.any(np.signbit(yg[~live]))
    return yg


@functools.lru_cache(maxsize=None)
def moe_workload(name):
    """(inputs, oracle route, layer) of a named MoE workload; only routed experts get weights."""
    inp = synth.moe_inputs(name)
    r = oracle.route(inp.logits, inp.cfg.k, inp.survival)
    experts = np.unique(r["ids"][r["live"].astype(bool)])
    say(f"[workload {name}] T={inp.cfg.T} experts touched={len(experts)} generating + quantizing on the CPU")
    return inp, r, Layer(inp, experts)


@functools.lru_cache(maxsize=None)
def small_workload(seed, T, H, E, k, I, skip=0.0, logits="normal"):
    inp = synth.small_moe(seed, T, H, E, k, I, logits=logits, skip_frac=skip)
    r = oracle.route(inp.logits, k, inp.survival)
    return inp, r, Layer(inp)


def shared_operands(cfg, H, Is):
    """The shared expert's FP8 weights (quantized by the oracle) on the device."""
    w13, w2 = synth.shared_expert_weights(cfg, H, Is)
    q13, s13 = oracle.quantize_e4m3(w13)
    q2, s2 = oracle.quantize_e4m3(w2)
    return tuple(dev(t) for t in (q13, s13, q2, s2))


def status_offset(H, I, k):
    """Byte offset of the single-launch layer's handoff status word in its
    workspace (the 32-bit call counter of the graph form follows it)."""
    off_o = mxmoe.moe_ws_layout(1, H, I, k)[2]
    return off_o + (k * max(H, I) * 4 + 255) // 256 * 256
