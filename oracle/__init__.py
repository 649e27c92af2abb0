"""CPU oracle for the block-scaled routed-expert MoE layer and the dense
block-32 FP8 projection.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the CPU-baseline leg
of the benchmark use it; the product package never imports it.  It is a plain
C++ implementation (``oracle.cpp``) of the definitions, in double precision,
sharing no code with the HIP library; this module only marshals numpy arrays.

Every function is pinned by a ``-m "not gpu"`` test (tests/test_oracle_*.py)
against something other than itself: torch's float8 codecs, exact rational
arithmetic, brute force on tiny inputs, closed forms and invariants.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build():
    """Compile liboracle.so with g++ (strict IEEE double, no contraction)."""
    cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-pthread", _SRC, "-o", _LIB + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
    for name in ("or_e4m3_value", "or_e2m1_value", "or_e8m0_value"):
        getattr(lib, name).restype = ctypes.c_double
        getattr(lib, name).argtypes = [ctypes.c_uint8]
    for name in ("or_quantize_e4m3", "or_quantize_e2m1"):
        getattr(lib, name).restype = i32
        getattr(lib, name).argtypes = [P, i64, i64, P, P, i32]
    lib.or_dequantize.restype = i32
    lib.or_dequantize.argtypes = [P, P, i64, i64, i32, P]
    lib.or_route.restype = i32
    lib.or_route.argtypes = [P, i32, i32, i32, P, f32, P, P, P, P, P]
    lib.or_route_live.restype = i32
    lib.or_route_live.argtypes = [P, i32, i32, i32, P, f32, P, P, P, P, P, P]
    lib.or_moe_rows.restype = i32
    lib.or_moe_rows.argtypes = [P, P, i32, P, P, P, i32, P, P, P, P, i32, i32, P, i32, P, i32]
    lib.or_pair_ffn.restype = i32
    lib.or_pair_ffn.argtypes = [P, P, i32, i32, i32, P, P, P, P, i32, P, P, P, P, P]
    lib.or_gate_up_pairs.restype = i32
    lib.or_gate_up_pairs.argtypes = [P, P, i32, P, P, i32, P, P, i32, P, i32]
    lib.or_down_combine.restype = i32
    lib.or_down_combine.argtypes = [P, P, P, P, P, i32, P, P, i32, i32, i32, P, i32, P, i32]
    lib.or_swiglu_requant.restype = i32
    lib.or_swiglu_requant.argtypes = [P, i64, i32, P, P, P]
    lib.or_block_gemm.restype = i32
    lib.or_block_gemm.argtypes = [P, P, P, P, i32, i32, P, i32, P, i32]
    lib.or_router_logits.restype = i32
    lib.or_router_logits.argtypes = [P, P, i32, i32, P, i32, P, i32]
    lib.or_f32_to_bf16.restype = None
    lib.or_f32_to_bf16.argtypes = [P, i64, P]
    lib.or_hardware_threads.restype = i32
    lib.or_hardware_threads.argtypes = []
    _lib = lib
    return lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def hardware_threads():
    return _load().or_hardware_threads()


# ------------------------------------------------------------------ formats
def e4m3_value(code):
    return _load().or_e4m3_value(int(code))


def e2m1_value(code):
    return _load().or_e2m1_value(int(code))


def e8m0_value(code):
    return _load().or_e8m0_value(int(code))


def quantize_e4m3(v, threads=0):
    """fp32 [rows, cols] -> (E4M3 codes uint8 [rows, cols], E8M0 uint8 [rows, cols/32])."""
    v = _c(v, np.float32)
    rows, cols = v.shape
    q = np.empty((rows, cols), np.uint8)
    sc = np.empty((rows, cols // 32), np.uint8)
    if _load().or_quantize_e4m3(_p(v), rows, cols, _p(q), _p(sc), threads):
        raise ValueError("cols must be a multiple of 32")
    return q, sc


def quantize_e2m1(v, threads=0):
    """fp32 [rows, cols] -> (packed E2M1 uint8 [rows, cols/2], E8M0 uint8 [rows, cols/32])."""
    v = _c(v, np.float32)
    rows, cols = v.shape
    q = np.empty((rows, cols // 2), np.uint8)
    sc = np.empty((rows, cols // 32), np.uint8)
    if _load().or_quantize_e2m1(_p(v), rows, cols, _p(q), _p(sc), threads):
        raise ValueError("cols must be a multiple of 32")
    return q, sc


def dequantize(q, sc, fmt):
    """Codes + scales -> float64 values; fmt 'e4m3' (bytes) or 'e2m1' (packed)."""
    q = _c(q, np.uint8)
    sc = _c(sc, np.uint8)
    rows = q.shape[0]
    cols = q.shape[1] if fmt == "e4m3" else 2 * q.shape[1]
    out = np.empty((rows, cols), np.float64)
    _load().or_dequantize(_p(q), _p(sc), rows, cols, 0 if fmt == "e4m3" else 1, _p(out))
    return out


# ------------------------------------------------------------------- route
def route(logits, k, survival=None, skip_below=0.2):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    surv = _c(survival, np.float32) if survival is not None else None
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    slot_pos = np.empty((T, k), np.int32)
    rc = _load().or_route(_p(logits), T, E, k, _p(surv), skip_below,
                          _p(ids), _p(w), _p(offsets), _p(perm), _p(slot_pos))
    if rc:
        raise ValueError("bad route arguments")
    live = np.ones(T, np.uint8) if surv is None else (~(surv < np.float32(skip_below))).astype(np.uint8)
    return dict(ids=ids, w=w, offsets=offsets, perm=perm, slot_pos=slot_pos, live=live)


def route_live(logits, k, survival, anchor, reuse_below=0.1):
    """Top-k gate where rows with survival < reuse_below take their anchor row's
    experts (weighted by their own logits); every pair is bucketed."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    surv = _c(survival, np.float32) if survival is not None else None
    anc = _c(anchor, np.int32)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    slot_pos = np.empty((T, k), np.int32)
    rc = _load().or_route_live(_p(logits), T, E, k, _p(surv), reuse_below, _p(anc),
                               _p(ids), _p(w), _p(offsets), _p(perm), _p(slot_pos))
    if rc:
        raise ValueError("bad route_live arguments")
    return dict(ids=ids, w=w, offsets=offsets, perm=perm, slot_pos=slot_pos, live=np.ones(T, np.uint8))


# ------------------------------------------------------------- expert FFN
def moe_rows(x, x_sc, ids, w, live, w13, w13_sc, w2, w2_sc, rows=None, threads=0):
    """y [len(rows), H] fp32 for the listed token rows (all rows by default).

    x [T, H] E4M3 + x_sc [T, H/32]; w13 [E, 2I, H/2] packed E2M1 + w13_sc
    [E, 2I, H/32]; w2 [E, H, I/2] + w2_sc [E, H, I/32]; ids/w [T, k]; live [T].
    """
    x, x_sc = _c(x, np.uint8), _c(x_sc, np.uint8)
    T, H = x.shape
    E, twoI = w13.shape[0], w13.shape[1]
    I = twoI // 2
    k = ids.shape[1]
    ids, w, live = _c(ids, np.int32), _c(w, np.float32), _c(live, np.uint8)
    w13, w13_sc, w2, w2_sc = (_c(a, np.uint8) for a in (w13, w13_sc, w2, w2_sc))
    rows = np.arange(T, dtype=np.int32) if rows is None else _c(rows, np.int32)
    y = np.empty((len(rows), H), np.float32)
    rc = _load().or_moe_rows(_p(x), _p(x_sc), H, _p(ids), _p(w), _p(live), k,
                             _p(w13), _p(w13_sc), _p(w2), _p(w2_sc), E, I,
                             _p(rows), len(rows), _p(y), threads)
    if rc:
        raise ValueError("bad moe arguments")
    return y


def pair_ffn(x, x_sc, t, e, w13, w13_sc, w2, w2_sc):
    """One (token, expert) pair with intermediates: dict(h, a, q, q_sc, o)."""
    x, x_sc = _c(x, np.uint8), _c(x_sc, np.uint8)
    H = x.shape[1]
    I = w13.shape[1] // 2
    w13, w13_sc, w2, w2_sc = (_c(a, np.uint8) for a in (w13, w13_sc, w2, w2_sc))
    h = np.empty(2 * I, np.float32)
    a = np.empty(I, np.float32)
    q = np.empty(I, np.uint8)
    q_sc = np.empty(I // 32, np.uint8)
    o = np.empty(H, np.float32)
    _load().or_pair_ffn(_p(x), _p(x_sc), H, int(t), int(e), _p(w13), _p(w13_sc), _p(w2), _p(w2_sc),
                        I, _p(h), _p(a), _p(q), _p(q_sc), _p(o))
    return dict(h=h, a=a, q=q, q_sc=q_sc, o=o)


def gate_up_pairs(x, x_sc, ts, es, w13, w13_sc, threads=0):
    """fp32 gate/up values h [n, 2I] of the pairs (ts[i], es[i]) (gate columns, then up)."""
    x, x_sc = _c(x, np.uint8), _c(x_sc, np.uint8)
    H = x.shape[1]
    I = w13.shape[1] // 2
    ts, es = _c(ts, np.int32), _c(es, np.int32)
    w13, w13_sc = _c(w13, np.uint8), _c(w13_sc, np.uint8)
    h = np.empty((len(ts), 2 * I), np.float32)
    if _load().or_gate_up_pairs(_p(x), _p(x_sc), H, _p(ts), _p(es), len(ts), _p(w13), _p(w13_sc), I, _p(h),
                                threads):
        raise ValueError("bad gate_up_pairs arguments")
    return h


def swiglu_requant(h):
    """fp32 gate/up rows h [n, 2I] -> (q [n, I], q_sc [n, I/32], a [n, I])."""
    h = _c(h, np.float32)
    n, twoI = h.shape
    I = twoI // 2
    q = np.empty((n, I), np.uint8)
    q_sc = np.empty((n, I // 32), np.uint8)
    a = np.empty((n, I), np.float32)
    if _load().or_swiglu_requant(_p(h), n, I, _p(q), _p(q_sc), _p(a)):
        raise ValueError("I must be a multiple of 32")
    return q, q_sc, a


def down_combine(q, q_sc, slot_pos, ids, w, w2, w2_sc, rows=None, threads=0):
    """y [len(rows), H] from a given FP8 intermediate q [P, I] (bucket-position rows)."""
    q, q_sc = _c(q, np.uint8), _c(q_sc, np.uint8)
    slot_pos, ids, w = _c(slot_pos, np.int32), _c(ids, np.int32), _c(w, np.float32)
    w2, w2_sc = _c(w2, np.uint8), _c(w2_sc, np.uint8)
    E, H, I = w2.shape[0], w2.shape[1], 2 * w2.shape[2]
    T, k = ids.shape
    rows = np.arange(T, dtype=np.int32) if rows is None else _c(rows, np.int32)
    y = np.empty((len(rows), H), np.float32)
    if _load().or_down_combine(_p(q), _p(q_sc), _p(slot_pos), _p(ids), _p(w), k, _p(w2), _p(w2_sc), H, E, I,
                               _p(rows), len(rows), _p(y), threads):
        raise ValueError("bad down_combine arguments")
    return y


# ------------------------------------------------------------- dense GEMM
def block_gemm(a, a_sc, w, w_sc, rows=None, threads=0):
    """fp32 y [len(rows), N] = decoded a[rows] @ decoded w^T (a [M, K], w [N, K] E4M3)."""
    a, a_sc, w, w_sc = (_c(t, np.uint8) for t in (a, a_sc, w, w_sc))
    M, K = a.shape
    N = w.shape[0]
    rows = np.arange(M, dtype=np.int32) if rows is None else _c(rows, np.int32)
    y = np.empty((len(rows), N), np.float32)
    if _load().or_block_gemm(_p(a), _p(a_sc), _p(w), _p(w_sc), N, K, _p(rows), len(rows), _p(y), threads):
        raise ValueError("K must be a multiple of 32")
    return y


# ---------------------------------------------------------- shared expert
def shared_expert(x, x_sc, w13, w13_sc, w2, w2_sc, rows=None, threads=0):
    """The shared expert, a dense SwiGLU MLP on every row with block-32 FP8
    operands (forum thread post #6, "Kernel by kernel against B12X": the shared
    expert's two kernels per call; TP4 README, settings table, row "Kernels",
    and its boot-log lines: the shared expert's down weight (5120, 576), K = 576
    padded to 640 there): h = x . W13^T (fp32, W13 [2I][H], rows [0, I) gate,
    [I, 2I) up), a = silu(gate) * up requantized to E4M3 block-32 (the same
    routine as the routed experts), y = a . W2^T (fp32, W2 [H][I]).  Returns
    y [len(rows), H] and the intermediate (h, q, q_sc)."""
    h = block_gemm(x, x_sc, w13, w13_sc, rows=rows, threads=threads)
    q, q_sc, _ = swiglu_requant(h)
    y = block_gemm(q, q_sc, w2, w2_sc, threads=threads)
    return y, h, q, q_sc


# ---------------------------------------------------------- router logits
def router_logits(h, wg, rows=None, threads=0):
    """fp32 logits [len(rows), E] = decoded h[rows] @ decoded wg^T (bf16 bit patterns h [T, H], wg [E, H])."""
    h, wg = _c(h, np.uint16), _c(wg, np.uint16)
    T, H = h.shape
    E = wg.shape[0]
    if wg.shape[1] != H:
        raise ValueError("hidden width mismatch")
    rows = np.arange(T, dtype=np.int32) if rows is None else _c(rows, np.int32)
    out = np.empty((len(rows), E), np.float32)
    if _load().or_router_logits(_p(h), _p(wg), E, H, _p(rows), len(rows), _p(out), threads):
        raise ValueError("bad router_logits arguments")
    return out


def f32_to_bf16(v):
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    _load().or_f32_to_bf16(_p(v), v.size, _p(out))
    return out
