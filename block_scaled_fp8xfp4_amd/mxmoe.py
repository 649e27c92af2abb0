"""Thin ctypes binding of libmxmoe.so (include/mxmoe.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's kernels.  The
binding raises if the library is missing, never falls back to another path.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmxmoe.so")

MX_OK, MX_EINVAL, MX_EUNSUPPORTED, MX_EWORKSPACE, MX_EHIP = 0, -1, -2, -3, -4
MX_FMT_E4M3, MX_FMT_E2M1 = 0, 1
MX_IN_F32, MX_IN_BF16 = 0, 1
MX_OUT_BF16, MX_OUT_F32 = 0, 1

# every entry point declared in include/mxmoe.h
EXPORTS = ("mx_quantize", "moe_router_logits_workspace_bytes", "moe_router_logits", "moe_route_workspace_bytes", "moe_route", "moe_route_live", "moe_expert_ffn_workspace_bytes",
           "moe_ws_layout", "moe_expert_ffn", "fp8_block_gemm", "mx_status_string",
           "mx_last_variant", "mx_set_ffn_path", "mx_set_layer1_single_launch", "mx_check_requant", "mx_set_phase_events",
           "moe_shared_expert_workspace_bytes", "moe_shared_expert", "mx_prefetch",
           "moe_layer_decode1", "mx_set_ffn_diag", "moe_expert_ffn_noalloc", "moe_expert_ffn_noalloc_max_bytes",
           "moe_layer_decode1_shared_workspace_bytes", "moe_layer_decode1_shared")

_lib = None


class MXError(RuntimeError):
    def __init__(self, status, name):
        self.status = status
        super().__init__(f"{name}: {status_string(status)} ({status})")


def load():
    """Load libmxmoe.so (built by block_scaled_fp8xfp4_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m block_scaled_fp8xfp4_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, F32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    lib.mx_quantize.restype = I32
    lib.mx_quantize.argtypes = [P, I32, I64, I64, I32, P, P, P]
    lib.moe_router_logits.restype = I32
    lib.moe_router_logits.argtypes = [P, I32, I32, P, I32, P, P, SZ, P]
    lib.moe_router_logits_workspace_bytes.restype = SZ
    lib.moe_router_logits_workspace_bytes.argtypes = [I32, I32, I32]
    lib.moe_route_workspace_bytes.restype = SZ
    lib.moe_route_workspace_bytes.argtypes = [I32, I32, I32]
    lib.moe_route.restype = I32
    lib.moe_route.argtypes = [P, I32, I32, I32, P, F32, P, P, P, P, P, P, SZ, P]
    lib.moe_route_live.restype = I32
    lib.moe_route_live.argtypes = [P, I32, I32, I32, P, F32, P, P, P, P, P, P, P, SZ, P]
    lib.moe_expert_ffn_workspace_bytes.restype = SZ
    lib.moe_expert_ffn_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    lib.moe_ws_layout.restype = I32
    lib.moe_ws_layout.argtypes = [I32, I32, I32, I32, P, P, P]
    lib.mx_set_ffn_diag.restype = I32
    lib.mx_set_ffn_diag.argtypes = [P, SZ]
    lib.moe_expert_ffn.restype = I32
    lib.moe_expert_ffn.argtypes = [P, P, I32, I32, P, P, P, P, I32, P, P, P, P, I32, I32, P, P, SZ, P]
    lib.moe_expert_ffn_noalloc.restype = I32
    lib.moe_expert_ffn_noalloc.argtypes = [P, P, I32, I32, P, P, P, P, I32, P, P, P, P, I32, I32, P, P]
    lib.moe_expert_ffn_noalloc_max_bytes.restype = SZ
    lib.moe_expert_ffn_noalloc_max_bytes.argtypes = []
    lib.fp8_block_gemm.restype = I32
    lib.fp8_block_gemm.argtypes = [P, P, P, P, I32, I32, I32, P, I32, P]
    lib.moe_shared_expert_workspace_bytes.restype = SZ
    lib.moe_shared_expert_workspace_bytes.argtypes = [I32, I32, I32]
    lib.moe_shared_expert.restype = I32
    lib.moe_shared_expert.argtypes = [P, P, I32, I32, P, P, P, P, I32, P, P, SZ, P]
    lib.moe_layer_decode1.restype = I32
    lib.moe_layer_decode1.argtypes = [P, I32, I32, P, F32, P, P, I32, P, P, P, P, I32, P, P, P, P, P, P, P, SZ, P]
    lib.moe_layer_decode1_shared_workspace_bytes.restype = SZ
    lib.moe_layer_decode1_shared_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    lib.moe_layer_decode1_shared.restype = I32
    lib.moe_layer_decode1_shared.argtypes = [P, I32, I32, P, F32, P, P, I32, P, P, P, P, I32, P, P, P, P, I32,
                                             P, P, P, P, P, P, P, P, SZ, P]
    lib.mx_prefetch.restype = I32
    lib.mx_prefetch.argtypes = [P, ctypes.c_uint64, ctypes.c_uint64, P]
    lib.mx_status_string.restype = ctypes.c_char_p
    lib.mx_status_string.argtypes = [I32]
    lib.mx_last_variant.restype = ctypes.c_char_p
    lib.mx_last_variant.argtypes = []
    lib.mx_set_ffn_path.restype = I32
    lib.mx_set_ffn_path.argtypes = [I32]
    lib.mx_set_layer1_single_launch.restype = I32
    lib.mx_set_layer1_single_launch.argtypes = [I32]
    lib.mx_check_requant.restype = I32
    lib.mx_check_requant.argtypes = [ctypes.c_uint32, ctypes.c_uint32, P, P]
    lib.mx_set_phase_events.restype = I32
    lib.mx_set_phase_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), I32]
    _lib = lib
    return lib


def status_string(status):
    return load().mx_status_string(status).decode()


def last_variant():
    return load().mx_last_variant().decode()


def set_layer1_single_launch(on):
    """1 = moe_layer_decode1(_shared) and moe_shared_expert (T = 1) in one launch where it applies, 0 = two;
    returns the previous setting."""
    r = load().mx_set_layer1_single_launch(int(on))
    if r < 0:
        raise MXError(r, "mx_set_layer1_single_launch")
    return r


def set_ffn_path(path):
    """0 = automatic, 1 = decode kernels, 2 = prefill kernels; returns the previous setting."""
    r = load().mx_set_ffn_path(int(path))
    if r < 0:
        raise MXError(r, "mx_set_ffn_path")
    return r


# Plain ints for the c_void_p arguments: ctypes converts them by the
# argtypes, which costs less per call than building a c_void_p per argument
# (at decode sizes the Python side of a call is as long as the kernel).
def _ptr(t):
    return None if t is None else t.data_ptr()


_raw_stream = None


def _stream(stream):
    """The given stream handle, else the current torch stream of the current device (its raw handle)."""
    global _raw_stream
    if stream is not None:
        return stream
    import torch
    if _raw_stream is None:
        f = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _raw_stream = (lambda: f(torch.cuda.current_device())) if f is not None else \
            (lambda: torch.cuda.current_stream().cuda_stream)
    return _raw_stream()


def _check(status, name):
    if status != MX_OK:
        raise MXError(status, name)


# ------------------------------------------------------------------ calls
def mx_quantize(src, q, sc, fmt, stream=None):
    """Quantize src [rows, cols] (fp32 or bf16 tensor) into q / sc (uint8 tensors)."""
    import torch
    dt = {torch.float32: MX_IN_F32, torch.bfloat16: MX_IN_BF16}[src.dtype]
    cols = src.shape[-1]
    rows = src.numel() // cols if cols else 0
    _check(load().mx_quantize(_ptr(src), dt, rows, cols, fmt, _ptr(q), _ptr(sc), _stream(stream)), "mx_quantize")


def moe_router_logits_workspace_bytes(T, H, E):
    return load().moe_router_logits_workspace_bytes(T, H, E)


def moe_router_logits(hidden, w_gate, logits, ws=None, stream=None):
    """logits [T, E] fp32 = hidden [T, H] bf16 . w_gate [E, H] bf16 (ws: uint8 device tensor of
    moe_router_logits_workspace_bytes(T, H, E) bytes, or None when that size is 0)."""
    T, H = hidden.shape
    E = w_gate.shape[0]
    if w_gate.shape[1] != H or tuple(logits.shape) != (T, E):
        raise ValueError("moe_router_logits: shape mismatch")
    for t in (hidden, w_gate):
        if t.element_size() != 2 or not t.is_contiguous():
            raise ValueError("moe_router_logits: hidden and w_gate must be contiguous 16-bit (bf16) tensors")
    ws_bytes = 0 if ws is None else ws.nbytes
    _check(load().moe_router_logits(_ptr(hidden), T, H, _ptr(w_gate), E, _ptr(logits), _ptr(ws), ws_bytes,
                                    _stream(stream)), "moe_router_logits")


def moe_route_workspace_bytes(T, E, k):
    return load().moe_route_workspace_bytes(T, E, k)


def moe_route(logits, k, survival, skip_below, topk_ids, topk_w, expert_offsets, perm, slot_pos, ws, stream=None):
    T, E = logits.shape
    _check(load().moe_route(_ptr(logits), T, E, k, _ptr(survival), float(skip_below), _ptr(topk_ids), _ptr(topk_w),
                            _ptr(expert_offsets), _ptr(perm), _ptr(slot_pos), _ptr(ws), ws.nbytes,
                            _stream(stream)), "moe_route")


def moe_route_live(logits, k, survival, reuse_below, anchor, topk_ids, topk_w, expert_offsets, perm, slot_pos, ws,
                   stream=None):
    T, E = logits.shape
    _check(load().moe_route_live(_ptr(logits), T, E, k, _ptr(survival), float(reuse_below), _ptr(anchor),
                                 _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets), _ptr(perm), _ptr(slot_pos),
                                 _ptr(ws), ws.nbytes, _stream(stream)), "moe_route_live")


def moe_expert_ffn_workspace_bytes(T, H, E, I, k):
    return load().moe_expert_ffn_workspace_bytes(T, H, E, I, k)


def moe_ws_layout(T, H, I, k):
    """Byte offsets (q, q_sc, o) of the FFN workspace regions."""
    offs = [ctypes.c_size_t() for _ in range(3)]
    _check(load().moe_ws_layout(T, H, I, k, *[ctypes.byref(o) for o in offs]), "moe_ws_layout")
    return tuple(o.value for o in offs)


def moe_expert_ffn(x, x_sc, topk_w, expert_offsets, perm, slot_pos, k, w13, w13_sc, w2, w2_sc, E, I, y, ws,
                   stream=None):
    T, H = x.shape
    _check(load().moe_expert_ffn(_ptr(x), _ptr(x_sc), T, H, _ptr(topk_w), _ptr(expert_offsets), _ptr(perm),
                                 _ptr(slot_pos), k, _ptr(w13), _ptr(w13_sc), _ptr(w2), _ptr(w2_sc), E, I, _ptr(y),
                                 _ptr(ws), ws.nbytes, _stream(stream)), "moe_expert_ffn")


def moe_expert_ffn_noalloc(x, x_sc, topk_w, expert_offsets, perm, slot_pos, k, w13, w13_sc, w2, w2_sc, E, I, y,
                           stream=None):
    """moe_expert_ffn without a caller workspace (the library's own device scratch array)."""
    T, H = x.shape
    _check(load().moe_expert_ffn_noalloc(_ptr(x), _ptr(x_sc), T, H, _ptr(topk_w), _ptr(expert_offsets), _ptr(perm),
                                         _ptr(slot_pos), k, _ptr(w13), _ptr(w13_sc), _ptr(w2), _ptr(w2_sc), E, I,
                                         _ptr(y), _stream(stream)), "moe_expert_ffn_noalloc")


def moe_expert_ffn_noalloc_max_bytes():
    return load().moe_expert_ffn_noalloc_max_bytes()


def moe_layer_decode1(logits, k, survival, skip_below, x, x_sc, w13, w13_sc, w2, w2_sc, E, I, topk_ids, topk_w,
                      expert_offsets, perm, slot_pos, y, ws, stream=None):
    """Route + routed-expert FFN of one row (logits [1, E] or [E]) in one launch (or two)."""
    H = x.shape[-1]
    _check(load().moe_layer_decode1(_ptr(logits), E, k, _ptr(survival), float(skip_below), _ptr(x), _ptr(x_sc), H,
                                    _ptr(w13), _ptr(w13_sc), _ptr(w2), _ptr(w2_sc), I, _ptr(topk_ids), _ptr(topk_w),
                                    _ptr(expert_offsets), _ptr(perm), _ptr(slot_pos), _ptr(y), _ptr(ws),
                                    ws.nbytes, _stream(stream)), "moe_layer_decode1")


def moe_layer_decode1_shared_workspace_bytes(H, E, I, k, Is):
    return load().moe_layer_decode1_shared_workspace_bytes(H, E, I, k, Is)


def moe_layer_decode1_shared(logits, k, survival, skip_below, x, x_sc, w13, w13_sc, w2, w2_sc, E, I,
                             sw13, sw13_sc, sw2, sw2_sc, topk_ids, topk_w, expert_offsets, perm, slot_pos, y,
                             y_shared, ws, stream=None):
    """moe_layer_decode1 plus the row's shared expert (sw13 FP8 [2Is, H], sw2 FP8 [H, Is] + scales) in the
    same launches (one where moe_layer_decode1 takes one and Is <= 640); y_shared [H] fp32 as moe_shared_expert."""
    H = x.shape[-1]
    Is = sw2.shape[-1]
    _check(load().moe_layer_decode1_shared(_ptr(logits), E, k, _ptr(survival), float(skip_below), _ptr(x), _ptr(x_sc),
                                           H, _ptr(w13), _ptr(w13_sc), _ptr(w2), _ptr(w2_sc), I, _ptr(sw13),
                                           _ptr(sw13_sc), _ptr(sw2), _ptr(sw2_sc), Is, _ptr(topk_ids), _ptr(topk_w),
                                           _ptr(expert_offsets), _ptr(perm), _ptr(slot_pos), _ptr(y), _ptr(y_shared),
                                           _ptr(ws), ws.nbytes, _stream(stream)),
           "moe_layer_decode1_shared")


def fp8_block_gemm(a, a_sc, w, w_sc, y, y_dtype, stream=None):
    M, K = a.shape
    N = w.shape[0]
    _check(load().fp8_block_gemm(_ptr(a), _ptr(a_sc), _ptr(w), _ptr(w_sc), M, N, K, _ptr(y), y_dtype,
                                 _stream(stream)), "fp8_block_gemm")


def moe_shared_expert_workspace_bytes(T, H, I):
    return load().moe_shared_expert_workspace_bytes(T, H, I)


def moe_shared_expert(x, x_sc, w13, w13_sc, w2, w2_sc, y, ws, stream=None):
    """y [T, H] fp32 = shared expert of x (FP8 [T, H] + scales); w13 [2I, H], w2 [H, I] FP8 + scales.
    One row (T = 1, H % 128 == 0, I <= 1024, not under graph capture) runs in one launch."""
    T, H = x.shape
    I = w2.shape[1]
    if tuple(w13.shape) != (2 * I, H) or tuple(y.shape) != (T, H):
        raise ValueError("moe_shared_expert: shape mismatch")
    _check(load().moe_shared_expert(_ptr(x), _ptr(x_sc), T, H, _ptr(w13), _ptr(w13_sc), _ptr(w2), _ptr(w2_sc), I,
                                    _ptr(y), _ptr(ws), ws.nbytes, _stream(stream)),
           "moe_shared_expert")


def prefetch(t, chunk_bytes=0, stream=None, nbytes=None):
    """Read tensor t's bytes (or its first nbytes) into cache; see mx_prefetch."""
    n = t.numel() * t.element_size() if nbytes is None else nbytes
    _check(load().mx_prefetch(_ptr(t), n, chunk_bytes, _stream(stream)), "mx_prefetch")


def check_requant(lo, hi, mismatches, stream=None):
    """Add to mismatches (int64 device tensor of one element) the number of
    finite floats with magnitude bits in [lo, hi), both signs, whose E4M3 code
    from the FFN's hardware conversion differs from the quantize encoder's."""
    _check(load().mx_check_requant(lo, hi, _ptr(mismatches), _stream(stream)), "mx_check_requant")


def set_ffn_diag(h):
    """Have this thread's later FFN calls also write their fp32 gate/up values
    into h (float32 device tensor of at least T*k*2I elements); None stops it."""
    if h is None:
        _check(load().mx_set_ffn_diag(None, 0), "mx_set_ffn_diag")
        return
    _check(load().mx_set_ffn_diag(_ptr(h), h.numel() * h.element_size()), "mx_set_ffn_diag")


def set_phase_events(events):
    """Record torch.cuda.Event objects (4, created with enable_timing=True) at
    the phase boundaries of this thread's later moe_expert_ffn calls: before
    the first kernel, after gate/up, after the down projection, after the last
    kernel.  None stops the recording."""
    if events is None:
        _check(load().mx_set_phase_events(None, 0), "mx_set_phase_events")
        return
    for e in events:
        e.record()                                   # materialise the HIP event handle
    arr = (ctypes.c_void_p * 4)(*[e.cuda_event for e in events])
    _check(load().mx_set_phase_events(arr, 4), "mx_set_phase_events")
