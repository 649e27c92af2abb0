"""Seeded synthetic inputs for the routed-expert MoE layer and the dense
projection: the one module that both the oracle side (tests) and the HIP side
(tests, benchmark) draw their inputs from.

It holds random numbers only, none of the method's arithmetic: no encoding,
no scale rule, no routing.  Quantization of these values is done separately by
the oracle (on the CPU) and by the library's quantizer kernel (on the GPU).

Streams: ``numpy.random.SeedSequence(seed)`` spawns one child per tensor in the
fixed order logits, survival, activations, W13, W2; the weight children spawn
one grandchild per expert, so any expert can be drawn alone and the threads
that draw several never change a value.

Workloads (sizes, distributions and structure), one per seed 0..4:
  tiny   T=4,    H=256,  E=8,   k=2, I=64;  logits N(0,1)
  dense  M in {1, 16} of 16 drawn rows, K=N=4096; FP8 weights
  decode T=1,    H=4096, E=256, k=8, I=576; logits N(0,1)
  verify T=48 = 8 streams x (1 anchor + 5 drafts), same layer; survival U(0,1)
         for drafts and 1.0 for anchors; logits log p_pi(e) + Gumbel(0,1) with
         p_r ~ r^-1.1 over a seeded permutation pi (top-k = k draws without
         replacement, popularity Zipf(1.1))
  prefill T=8192, same layer; logits N(0,1)
Activations are N(0,1) rounded to bf16; weights are N(0, 0.02^2) in fp32.
Shared expert: W13 [2I][H] and W2 [H][I], N(0, 0.02^2) in fp32, from the
stream SeedSequence([seed, 9]) (quantized to E4M3 block-32 by each side).
Router gate (the linear map whose scores the top-k gate ranks): bf16-valued
N(0, 1/H) rows [E][H] from the stream SeedSequence([seed, 7]), so that the
workload's bf16 hidden rows give logits of unit variance, like the drawn
N(0,1) logits above.
"""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import os

import numpy as np

WEIGHT_STD = 0.02


@dataclass(frozen=True)
class MoEConfig:
    name: str
    seed: int
    T: int
    H: int
    E: int
    k: int
    I: int
    logits: str = "normal"        # "normal" or "zipf"
    streams: int = 0              # > 0: rows are streams x (1 anchor + drafts), with survival
    drafts: int = 0


@dataclass(frozen=True)
class DenseConfig:
    name: str
    seed: int
    M: tuple
    K: int
    N: int


TINY = MoEConfig("tiny", 0, T=4, H=256, E=8, k=2, I=64)
DENSE = DenseConfig("dense", 1, M=(1, 16), K=4096, N=4096)
DECODE = MoEConfig("decode", 2, T=1, H=4096, E=256, k=8, I=576)
VERIFY = MoEConfig("verify", 3, T=48, H=4096, E=256, k=8, I=576, logits="zipf", streams=8, drafts=5)
PREFILL = MoEConfig("prefill", 4, T=8192, H=4096, E=256, k=8, I=576)

CONFIGS = {c.name: c for c in (TINY, DENSE, DECODE, VERIFY, PREFILL)}


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def _gen(ss):
    return np.random.Generator(np.random.PCG64(ss))


def _children(seed):
    logits, survival, x, w13, w2 = np.random.SeedSequence(seed).spawn(5)
    return dict(logits=logits, survival=survival, x=x, w13=w13, w2=w2)


def _to_bf16_values(v):
    """Round fp32 values to bf16 (nearest even) and return them as fp32."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(v)).to(torch.bfloat16).to(torch.float32).numpy()


def _normal(ss, shape, std=1.0):
    g = _gen(ss)
    a = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


@dataclass
class MoEInputs:
    cfg: MoEConfig
    logits: np.ndarray            # fp32 [T, E]
    survival: object              # fp32 [T] or None
    x: np.ndarray                 # fp32 [T, H], bf16-valued
    _kids: dict = field(repr=False, default=None)

    def w13(self, experts=None):
        """fp32 [len(experts), 2I, H] gate (rows < I) and up (rows >= I) weights."""
        c = self.cfg
        return _per_expert(self._kids["w13"], c.E, (2 * c.I, c.H), experts)

    def w2(self, experts=None):
        """fp32 [len(experts), H, I] down-projection weights."""
        c = self.cfg
        return _per_expert(self._kids["w2"], c.E, (c.H, c.I), experts)


def _per_expert(ss, E, shape, experts):
    experts = range(E) if experts is None else list(experts)
    out = np.empty((len(experts),) + shape, np.float32)

    def fill(i_e):
        i, e = i_e
        out[i] = _normal(np.random.SeedSequence(ss.entropy, spawn_key=ss.spawn_key + (e,)), shape, WEIGHT_STD)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, enumerate(experts)))
    return out


def moe_inputs(cfg):
    """Logits, survival and activations of a MoE workload; weights on demand."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    kids = _children(cfg.seed)
    T, E = cfg.T, cfg.E
    if cfg.logits == "normal":
        logits = _normal(kids["logits"], (T, E))
    else:
        g = _gen(kids["logits"])
        pi = g.permutation(E)                      # expert at popularity rank r is pi[r]
        ranks = np.empty(E, np.int64)
        ranks[pi] = np.arange(E)
        p = (ranks + 1.0) ** -1.1
        p /= p.sum()
        gumbel = g.gumbel(size=(T, E))
        logits = (np.log(p)[None, :] + gumbel).astype(np.float32)
    survival = None
    if cfg.streams:
        u = _gen(kids["survival"]).random(T, dtype=np.float32)
        u[:: cfg.drafts + 1] = 1.0                 # anchor rows always survive
        survival = u
    x = _to_bf16_values(_normal(kids["x"], (T, cfg.H)))
    return MoEInputs(cfg, logits, survival, x, kids)


@dataclass
class DenseInputs:
    cfg: DenseConfig
    a: np.ndarray   # fp32 [max(M), K], bf16-valued
    w: np.ndarray   # fp32 [N, K]


def dense_inputs(cfg=DENSE, rows=None):
    """Activations (rows x K, bf16-valued) and fp32 weights of the dense projection."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    kids = _children(cfg.seed)
    rows = max(cfg.M) if rows is None else rows
    a = _to_bf16_values(_normal(kids["x"], (rows, cfg.K)))
    # weights drawn in 16 row bands, each from its own stream, for threading
    bands = 16
    w = np.empty((cfg.N, cfg.K), np.float32)
    step = cfg.N // bands
    wk = kids["w13"].spawn(bands)

    def fill(b):
        w[b * step:(b + 1) * step] = _normal(wk[b], (step, cfg.K), WEIGHT_STD)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(bands)))
    return DenseInputs(cfg, a, w)


def small_moe(seed, T, H, E, k, I, logits="normal", skip_frac=0.0):
    """A MoE workload of arbitrary (small) shape for parity and edge cases."""
    cfg = MoEConfig(f"custom{seed}", seed, T=T, H=H, E=E, k=k, I=I, logits=logits)
    inp = moe_inputs(cfg)
    if skip_frac > 0:
        inp.survival = _gen(np.random.SeedSequence([seed, 99])).random(T, dtype=np.float32)
        inp.survival = np.where(inp.survival < skip_frac, np.float32(0.1), np.float32(0.9))
    return inp


def router_gate(cfg, E=None, H=None):
    """bf16-valued fp32 router gate rows [E][H], N(0, 1/H) (shape defaults to the workload's)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    E = cfg.E if E is None else E
    H = cfg.H if H is None else H
    w = _normal(np.random.SeedSequence([cfg.seed, 7]), (E, H), float(H) ** -0.5)
    return _to_bf16_values(w)


def hidden_rows(seed, T, H):
    """bf16-valued N(0,1) hidden rows [T][H] of an arbitrary (small) shape."""
    return _to_bf16_values(_normal(np.random.SeedSequence([seed, 8]), (T, H)))


def shared_expert_weights(cfg, H=None, I=None):
    """fp32 shared-expert weights (W13 [2I][H], W2 [H][I]), N(0, 0.02^2)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    H = cfg.H if H is None else H
    I = cfg.I if I is None else I
    g = _gen(np.random.SeedSequence([cfg.seed, 9]))
    w13 = g.standard_normal((2 * I, H), dtype=np.float32) * np.float32(WEIGHT_STD)
    w2 = g.standard_normal((H, I), dtype=np.float32) * np.float32(WEIGHT_STD)
    return w13, w2
