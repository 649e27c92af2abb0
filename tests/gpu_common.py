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


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda") if dtype is None else t.to("cuda", dtype=dtype)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(got, ref, what):
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if scale == 0:
        assert err == 0, f"{what}: expected zeros, max |got| {err}"
        return
    cos = float(got @ ref / (np.linalg.norm(got) * np.linalg.norm(ref)))
    assert err <= TOL_REL_MAX * scale, f"{what}: max|diff| {err:.3e} > {TOL_REL_MAX} * {scale:.3e}"
    assert cos >= TOL_COS, f"{what}: cosine {cos:.7f}"


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
