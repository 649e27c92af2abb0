"""Device-side convenience wrapper around the C-ABI: uploads and quantizes a
MoE layer on the GPU (with the library's own quantizer kernel) and owns the
route / FFN workspaces.  Every computation is a libmxmoe.so call."""
import numpy as np
import torch

from . import mxmoe


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)) if isinstance(a, np.ndarray) else a
    return t.to("cuda", dtype=dtype) if dtype is not None else t.to("cuda")


def quantize(v, fmt):
    """fp32/bf16 device tensor [..., cols] -> (codes, scales) device uint8 tensors."""
    cols = v.shape[-1]
    rows = v.numel() // cols
    qcols = cols if fmt == mxmoe.MX_FMT_E4M3 else cols // 2
    q = torch.empty(v.shape[:-1] + (qcols,), dtype=torch.uint8, device=v.device)
    sc = torch.empty(v.shape[:-1] + (cols // 32,), dtype=torch.uint8, device=v.device)
    if rows:
        mxmoe.mx_quantize(v.contiguous(), q, sc, fmt)
    return q, sc


def quantize_experts(w_host, chunk=16):
    """fp32 host weights [E, R, C] -> packed E2M1 [E, R, C/2] + E8M0 [E, R, C/32] on the GPU."""
    E, R, C = w_host.shape
    q = torch.empty((E, R, C // 2), dtype=torch.uint8, device="cuda")
    sc = torch.empty((E, R, C // 32), dtype=torch.uint8, device="cuda")
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        src = _dev(w_host[e0:e1])
        mxmoe.mx_quantize(src, q[e0:e1], sc[e0:e1], mxmoe.MX_FMT_E2M1)
    torch.cuda.synchronize()
    return q, sc


class RouterLogits:
    """Owns the workspace of moe_router_logits for up to T rows."""

    def __init__(self, T, H, E):
        self.T, self.H, self.E = T, H, E
        n = max(mxmoe.moe_router_logits_workspace_bytes(t, H, E) for t in range(1, min(T, 1024) + 1))
        self.ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")

    def __call__(self, hidden, w_gate, logits, stream=None):
        if hidden.shape[0] > self.T:
            raise ValueError("RouterLogits: more rows than sized for")
        mxmoe.moe_router_logits(hidden, w_gate, logits, self.ws, stream)
        return logits


class Route:
    def __init__(self, T, E, k):
        dev = "cuda"
        self.T, self.E, self.k = T, E, k
        self.ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.perm = torch.empty(T * k, dtype=torch.int32, device=dev)
        self.slot_pos = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.ws = torch.empty(mxmoe.moe_route_workspace_bytes(T, E, k), dtype=torch.uint8, device=dev)

    def __call__(self, logits, survival=None, skip_below=0.2, stream=None, anchor=None):
        """Skip mode, or router-live mode when anchor (int32 [T]) is given
        (then skip_below is the reuse threshold)."""
        if anchor is None:
            mxmoe.moe_route(logits, self.k, survival, skip_below, self.ids, self.w, self.offsets, self.perm,
                            self.slot_pos, self.ws, stream)
        else:
            mxmoe.moe_route_live(logits, self.k, survival, skip_below, anchor, self.ids, self.w, self.offsets,
                                 self.perm, self.slot_pos, self.ws, stream)
        return self


class ExpertFFN:
    def __init__(self, T, H, E, I, k):
        self.T, self.H, self.E, self.I, self.k = T, H, E, I, k
        self.ws = torch.empty(mxmoe.moe_expert_ffn_workspace_bytes(T, H, E, I, k), dtype=torch.uint8, device="cuda")
        self.y = torch.empty((T, H), dtype=torch.float32, device="cuda")

    def __call__(self, x, x_sc, route, w13, w13_sc, w2, w2_sc, stream=None):
        mxmoe.moe_expert_ffn(x, x_sc, route.w, route.offsets, route.perm, route.slot_pos, self.k, w13, w13_sc,
                             w2, w2_sc, self.E, self.I, self.y, self.ws, stream)
        return self.y

    def ws_views(self):
        """Workspace regions as tensors: q [T*k, I], q_sc [T*k, I/32] (uint8)
        and o [T*k, H] (fp32, T > 1)."""
        Tk, H, I = self.T * self.k, self.H, self.I
        oq, oqs, oo = mxmoe.moe_ws_layout(self.T, H, I, self.k)
        q = self.ws[oq:oq + Tk * I].view(Tk, I)
        sc = self.ws[oqs:oqs + Tk * (I // 32)].view(Tk, I // 32)
        o = self.ws[oo:oo + Tk * H * 4].view(torch.float32).view(Tk, H)
        return q, sc, o
