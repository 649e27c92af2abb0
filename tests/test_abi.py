"""The C-ABI library loads without a GPU, exports every entry point that
include/mxmoe.h declares, and rejects bad arguments on the host, before any
HIP call, with the documented status codes."""
import ctypes
import os
import re

import pytest

from block_scaled_fp8xfp4_amd import mxmoe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxmoe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mxmoe.LIB_PATH):
        import block_scaled_fp8xfp4_amd.build as b
        b.build()
    return mxmoe.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("moe_route", "moe_expert_ffn", "fp8_block_gemm", "mx_quantize"):
        assert required in names
    assert sorted(mxmoe.EXPORTS) == names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4):
        assert mxmoe.status_string(s).startswith("MX_")
    assert "unknown" in mxmoe.status_string(7)


def test_workspace_sizes_are_pure_host_functions(lib):
    assert mxmoe.moe_route_workspace_bytes(8192, 256, 8) >= 32 * 256 * 4
    b = mxmoe.moe_expert_ffn_workspace_bytes(8192, 4096, 256, 576, 8)
    assert b >= 65536 * 4096 * 4 + 65536 * 576
    oq, oqs, oo = mxmoe.moe_ws_layout(8192, 4096, 576, 8)
    assert oq == 0 and oqs >= 65536 * 576 and oo >= oqs + 65536 * 18
    assert oo + 65536 * 4096 * 4 <= b
    # no fp32 gate/up region: those values go to the caller's diagnostic buffer only
    assert b < oo + 65536 * 4096 * 4 + 65536 * 1152 * 4
    assert mxmoe.moe_expert_ffn_workspace_bytes(1, 64, 1, 32, 1) == 0       # H < 128: invalid


FAKE = ctypes.c_void_p(1 << 20)        # aligned, never dereferenced: validation fails first
FAKE_WS = ctypes.c_void_p(1 << 24)


def test_quantize_rejects_bad_arguments(lib):
    q = lib.mx_quantize
    assert q(None, 0, 4, 64, 0, FAKE, FAKE, None) == mxmoe.MX_EINVAL
    assert q(FAKE, 0, 4, 48, 0, FAKE, FAKE, None) == mxmoe.MX_EINVAL              # cols % 32
    assert q(FAKE, 2, 4, 64, 0, FAKE, FAKE, None) == mxmoe.MX_EINVAL              # dtype
    assert q(FAKE, 0, 4, 64, 3, FAKE, FAKE, None) == mxmoe.MX_EINVAL              # format
    assert q(ctypes.c_void_p((1 << 20) + 4), 0, 4, 64, 0, FAKE, FAKE, None) == mxmoe.MX_EINVAL  # alignment
    assert q(FAKE, 0, -1, 64, 0, FAKE, FAKE, None) == mxmoe.MX_EINVAL


def route(lib, T=4, E=8, k=2, ws=FAKE_WS, ws_bytes=1 << 20, logits=FAKE, ids=FAKE):
    return lib.moe_route(logits, T, E, k, None, 0.2, ids, FAKE, FAKE, FAKE, FAKE, ws, ws_bytes, None)


def test_route_rejects_bad_arguments(lib):
    assert route(lib, k=0) == mxmoe.MX_EINVAL
    assert route(lib, k=9, E=8) == mxmoe.MX_EINVAL
    assert route(lib, k=17, E=64) == mxmoe.MX_EINVAL
    assert route(lib, E=0) == mxmoe.MX_EINVAL
    assert route(lib, E=1025) == mxmoe.MX_EINVAL
    assert route(lib, T=-1) == mxmoe.MX_EINVAL
    assert route(lib, T=1 << 28, k=16, E=64) == mxmoe.MX_EINVAL                 # T*k overflows int32
    assert route(lib, logits=None) == mxmoe.MX_EINVAL
    assert route(lib, ids=None) == mxmoe.MX_EINVAL
    assert route(lib, ws=None) == mxmoe.MX_EWORKSPACE
    assert route(lib, T=8192, E=256, k=8, ws_bytes=100) == mxmoe.MX_EWORKSPACE


def route_live(lib, T=4, E=8, k=2, anchor=FAKE, ws=FAKE_WS, ws_bytes=1 << 20, logits=FAKE):
    return lib.moe_route_live(logits, T, E, k, FAKE, 0.1, anchor, FAKE, FAKE, FAKE, FAKE, FAKE, ws, ws_bytes, None)


def test_route_live_rejects_bad_arguments(lib):
    assert route_live(lib, anchor=None) == mxmoe.MX_EINVAL
    assert route_live(lib, anchor=ctypes.c_void_p((1 << 20) + 2)) == mxmoe.MX_EINVAL   # alignment
    assert route_live(lib, k=9, E=8) == mxmoe.MX_EINVAL
    assert route_live(lib, logits=None) == mxmoe.MX_EINVAL
    assert route_live(lib, ws=None) == mxmoe.MX_EWORKSPACE
    assert route_live(lib, T=8192, E=256, k=8, ws_bytes=100) == mxmoe.MX_EWORKSPACE


def ffn(lib, T=4, H=256, E=8, I=64, k=2, ws=FAKE_WS, ws_bytes=1 << 34, x=FAKE, w13=FAKE, w2_sc=FAKE):
    return lib.moe_expert_ffn(x, FAKE, T, H, FAKE, FAKE, FAKE, FAKE, k, w13, FAKE, FAKE, w2_sc, E, I, FAKE,
                              ws, ws_bytes, None)


def test_ffn_rejects_bad_arguments(lib):
    assert ffn(lib, k=0) == mxmoe.MX_EINVAL
    assert ffn(lib, k=17) == mxmoe.MX_EINVAL
    assert ffn(lib, H=100) == mxmoe.MX_EINVAL                                   # H < 128
    assert ffn(lib, H=300) == mxmoe.MX_EINVAL                                   # H % 32
    assert ffn(lib, H=320) == mxmoe.MX_EUNSUPPORTED                             # H % 128
    assert ffn(lib, I=48) == mxmoe.MX_EINVAL                                    # I % 32
    assert ffn(lib, I=4096) == mxmoe.MX_EUNSUPPORTED                            # I > 2048
    assert ffn(lib, x=None) == mxmoe.MX_EINVAL
    assert ffn(lib, w13=ctypes.c_void_p((1 << 20) + 8)) == mxmoe.MX_EINVAL      # alignment
    assert ffn(lib, w2_sc=ctypes.c_void_p((1 << 20) + 2)) == mxmoe.MX_EINVAL    # scale rows are read as dwords
    assert ffn(lib, ws=None) == mxmoe.MX_EWORKSPACE
    assert ffn(lib, ws_bytes=1000) == mxmoe.MX_EWORKSPACE
    assert ffn(lib, E=0) == mxmoe.MX_EINVAL
    assert ffn(lib, T=1 << 20, H=4096, k=1) == mxmoe.MX_EUNSUPPORTED             # T*H >= 2^32


@pytest.mark.parametrize("H,I", [(6144, 1024), (5248, 576), (5376, 640), (16384, 2048)])
def test_ffn_rejects_shapes_no_path_implements(lib, H, I):
    """(H, I) beyond the decode kernels (H <= 5120, I <= 2048) and the prefill
    kernels (H % 256 == 0, I <= 608) is refused on the host, whatever T, for
    the automatic setting and for each forced path; nothing runs silently."""
    for T in (1, 48, 8192):
        assert ffn(lib, T=T, H=H, I=I, k=8, E=256) == mxmoe.MX_EUNSUPPORTED, (T, H, I)
    for path in (1, 2):
        old = mxmoe.set_ffn_path(path)
        try:
            assert ffn(lib, T=48, H=H, I=I, k=8, E=256) == mxmoe.MX_EUNSUPPORTED, (path, H, I)
        finally:
            mxmoe.set_ffn_path(old)
    assert layer1(lib, H=H, I=I) == mxmoe.MX_EUNSUPPORTED


def test_ffn_forced_path_rejects_what_that_path_lacks(lib):
    old = mxmoe.set_ffn_path(1)
    try:
        assert ffn(lib, T=4, H=5248, I=64) == mxmoe.MX_EUNSUPPORTED             # decode: H > 5120
        assert ffn(lib, T=4, H=6144, I=64, ws=None) == mxmoe.MX_EUNSUPPORTED    # reported before the workspace
    finally:
        mxmoe.set_ffn_path(old)
    old = mxmoe.set_ffn_path(2)
    try:
        assert ffn(lib, T=4, H=4096, I=640) == mxmoe.MX_EUNSUPPORTED            # prefill: I > 608
        assert ffn(lib, T=4, H=384, I=64) == mxmoe.MX_EUNSUPPORTED              # prefill: H % 256
    finally:
        mxmoe.set_ffn_path(old)


def layer1(lib, H=256, I=64, E=8, k=2, ws=FAKE_WS, ws_bytes=1 << 30, w2_sc=FAKE):
    return lib.moe_layer_decode1(FAKE, E, k, None, 0.2, FAKE, FAKE, H, FAKE, FAKE, FAKE, w2_sc, I, FAKE, FAKE, FAKE,
                                 FAKE, FAKE, FAKE, ws, ws_bytes, None)


def test_layer_decode1_rejects_bad_arguments(lib):
    assert layer1(lib, k=0) == mxmoe.MX_EINVAL
    assert layer1(lib, k=9, E=8) == mxmoe.MX_EINVAL
    assert layer1(lib, H=320) == mxmoe.MX_EUNSUPPORTED
    assert layer1(lib, w2_sc=ctypes.c_void_p((1 << 20) + 1)) == mxmoe.MX_EINVAL
    assert layer1(lib, ws=None) == mxmoe.MX_EWORKSPACE


def layer1s(lib, H=256, I=64, E=8, k=2, Is=64, ws=FAKE_WS, ws_bytes=1 << 30, sw2=FAKE, ys=FAKE):
    return lib.moe_layer_decode1_shared(FAKE, E, k, None, 0.2, FAKE, FAKE, H, FAKE, FAKE, FAKE, FAKE, I,
                                        FAKE, FAKE, sw2, FAKE, Is, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ys,
                                        ws, ws_bytes, None)


def test_layer_decode1_shared_rejects_bad_arguments(lib):
    """The routed part's checks as moe_layer_decode1, and the shared expert's:
    Is a multiple of 32 up to 1024 (its down projection is one K part), every
    pointer, the combined workspace; all before any launch."""
    assert layer1s(lib, k=0) == mxmoe.MX_EINVAL
    assert layer1s(lib, H=320) == mxmoe.MX_EUNSUPPORTED
    assert layer1s(lib, Is=48) == mxmoe.MX_EINVAL
    assert layer1s(lib, Is=16) == mxmoe.MX_EINVAL
    assert layer1s(lib, Is=1056) == mxmoe.MX_EUNSUPPORTED
    assert layer1s(lib, sw2=None) == mxmoe.MX_EINVAL
    assert layer1s(lib, ys=None) == mxmoe.MX_EINVAL
    assert layer1s(lib, ys=ctypes.c_void_p((1 << 20) + 2)) == mxmoe.MX_EINVAL
    assert layer1s(lib, ws=None) == mxmoe.MX_EWORKSPACE
    need = lib.moe_layer_decode1_shared_workspace_bytes(256, 8, 64, 2, 64)
    routed = lib.moe_expert_ffn_workspace_bytes(1, 256, 8, 64, 2)
    shared = lib.moe_shared_expert_workspace_bytes(1, 256, 64)
    assert need == (routed + 255) // 256 * 256 + shared
    assert layer1s(lib, ws_bytes=need - 1) == mxmoe.MX_EWORKSPACE
    assert lib.moe_layer_decode1_shared_workspace_bytes(256, 8, 64, 2, 48) == 0
    assert lib.moe_layer_decode1_shared_workspace_bytes(256, 8, 64, 9, 64) == 0


def test_ffn_diagnostic_buffer(lib):
    """mx_set_ffn_diag: misaligned buffers are refused; a call whose gate/up
    values do not fit the buffer fails with MX_EWORKSPACE before any launch."""
    assert lib.mx_set_ffn_diag(ctypes.c_void_p((1 << 20) + 4), 1 << 20) == mxmoe.MX_EINVAL
    assert lib.mx_set_ffn_diag(FAKE, 4 * 2 * 2 * 64 * 4 - 4) == mxmoe.MX_OK   # T*k*2I*4 - 4 bytes
    try:
        assert ffn(lib, T=4, k=2, I=64) == mxmoe.MX_EWORKSPACE
        assert layer1(lib, k=8, I=64) == mxmoe.MX_EWORKSPACE                  # 1 row x k = 8 pairs do not fit
    finally:
        assert lib.mx_set_ffn_diag(None, 0) == mxmoe.MX_OK


def gemm(lib, M=1, N=64, K=256, ydt=0, a=FAKE):
    return lib.fp8_block_gemm(a, FAKE, FAKE, FAKE, M, N, K, FAKE, ydt, None)


def test_gemm_rejects_bad_arguments(lib):
    assert gemm(lib, M=(1 << 20), N=1024, K=4096) == mxmoe.MX_EUNSUPPORTED   # M*K >= 2^32 (32-bit operand offsets)
    assert gemm(lib, M=16, N=(1 << 19), K=8192) == mxmoe.MX_EUNSUPPORTED     # N*K >= 2^32
    assert gemm(lib, M=(1 << 16), N=(1 << 15), K=64) == mxmoe.MX_EUNSUPPORTED   # M*N >= 2^31
    assert gemm(lib, M=0) == mxmoe.MX_EINVAL
    assert gemm(lib, K=100) == mxmoe.MX_EINVAL
    assert gemm(lib, K=16384 + 128) == mxmoe.MX_EUNSUPPORTED
    assert gemm(lib, N=40) == mxmoe.MX_EUNSUPPORTED
    assert gemm(lib, ydt=5) == mxmoe.MX_EINVAL
    assert gemm(lib, a=None) == mxmoe.MX_EINVAL


def logits(lib, T=4, H=256, E=8, h=FAKE, w=FAKE, out=FAKE, ws=FAKE_WS, ws_bytes=1 << 30):
    return lib.moe_router_logits(h, T, H, w, E, out, ws, ws_bytes, None)


def test_router_logits_rejects_bad_arguments(lib):
    assert logits(lib, T=-1) == mxmoe.MX_EINVAL
    assert logits(lib, E=0) == mxmoe.MX_EINVAL
    assert logits(lib, H=100) == mxmoe.MX_EINVAL                       # H % 32
    assert logits(lib, H=0) == mxmoe.MX_EINVAL
    assert logits(lib, H=16384 + 32) == mxmoe.MX_EUNSUPPORTED
    assert logits(lib, T=1 << 20, H=4096) == mxmoe.MX_EUNSUPPORTED      # T*H >= 2^31
    assert logits(lib, w=None) == mxmoe.MX_EINVAL
    assert logits(lib, h=None) == mxmoe.MX_EINVAL
    assert logits(lib, out=None) == mxmoe.MX_EINVAL
    assert logits(lib, h=ctypes.c_void_p((1 << 20) + 8)) == mxmoe.MX_EINVAL   # 16-byte alignment
    assert logits(lib, out=ctypes.c_void_p((1 << 20) + 2)) == mxmoe.MX_EINVAL
    assert logits(lib, ws=ctypes.c_void_p((1 << 24) + 64)) == mxmoe.MX_EINVAL
    need = mxmoe.moe_router_logits_workspace_bytes(100, 256, 8)
    assert need >= 100 * 8 * 4                                          # at least one part sum per element
    assert logits(lib, T=100, ws=None) == mxmoe.MX_EWORKSPACE
    assert logits(lib, T=100, ws_bytes=need - 1) == mxmoe.MX_EWORKSPACE
    assert mxmoe.moe_router_logits_workspace_bytes(16, 256, 8) == 0       # one launch, no workspace
    assert logits(lib, T=0, h=None, out=None, ws=None) == mxmoe.MX_OK   # nothing to do, nothing launched
    assert mxmoe.moe_router_logits_workspace_bytes(1, 100, 8) == 0      # invalid shape


def shared(lib, T=4, H=256, I=64, x=FAKE, y=FAKE, ws=FAKE_WS, ws_bytes=1 << 30):
    return lib.moe_shared_expert(x, FAKE, T, H, FAKE, FAKE, FAKE, FAKE, I, y, ws, ws_bytes, None)


def test_shared_expert_rejects_bad_arguments(lib):
    assert shared(lib, T=-1) == mxmoe.MX_EINVAL
    assert shared(lib, H=100) == mxmoe.MX_EINVAL
    assert shared(lib, I=48) == mxmoe.MX_EINVAL
    assert shared(lib, H=16384 + 32) == mxmoe.MX_EUNSUPPORTED
    assert shared(lib, x=None) == mxmoe.MX_EINVAL
    assert shared(lib, y=ctypes.c_void_p((1 << 20) + 2)) == mxmoe.MX_EINVAL
    assert shared(lib, ws=None) == mxmoe.MX_EWORKSPACE
    need = mxmoe.moe_shared_expert_workspace_bytes(4, 256, 64)
    assert need >= 4 * 128 * 4 + 4 * 64 + 4 * 2
    assert shared(lib, ws_bytes=need - 1) == mxmoe.MX_EWORKSPACE
    assert shared(lib, T=0, x=None, y=None, ws=None) == mxmoe.MX_OK       # nothing to do, nothing launched


def test_shared_expert_one_row_workspace_layout(lib):
    """One row: h, q, q_sc, then room for the gate/up parts (two-launch form)
    or the handoff words (one-launch form: I / 8 lines of 128 bytes), then
    the one-launch form's status word in the last 256 bytes."""
    a = lambda b: (b + 255) // 256 * 256
    for H, I in ((4096, 576), (256, 64), (5120, 1024), (128, 32), (1024, 640)):
        parts = (H + 1023) // 1024
        assert lib.moe_shared_expert_workspace_bytes(1, H, I) == \
            a(2 * I * 4) + a(I) + a(I // 32) + a(max(parts * 2 * I * 4, I // 8 * 128)) + 256
    assert lib.moe_shared_expert_workspace_bytes(1, 256, 1056) == a(2 * 1056 * 4) + a(1056) + a(33)


def test_prefetch_rejects_bad_arguments(lib):
    assert lib.mx_prefetch(None, 64, 0, None) == mxmoe.MX_EINVAL
    assert lib.mx_prefetch(ctypes.c_void_p((1 << 20) + 4), 64, 0, None) == mxmoe.MX_EINVAL   # alignment
    assert lib.mx_prefetch(FAKE, 64, 24, None) == mxmoe.MX_EINVAL                             # chunk % 16
    assert lib.mx_prefetch(None, 0, 0, None) == mxmoe.MX_OK                                   # nothing to read


def test_path_switch(lib):
    old = mxmoe.set_ffn_path(1)
    assert mxmoe.set_ffn_path(old) == 1
    with pytest.raises(mxmoe.MXError):
        mxmoe.set_ffn_path(3)


def test_check_requant_rejects_bad_arguments(lib):
    assert lib.mx_check_requant(0, 16, None, None) == mxmoe.MX_EINVAL
    assert lib.mx_check_requant(0, 16, ctypes.c_void_p((1 << 20) + 4), None) == mxmoe.MX_EINVAL   # alignment
    assert lib.mx_check_requant(32, 16, FAKE, None) == mxmoe.MX_EINVAL                          # lo > hi
    assert lib.mx_check_requant(0, 0x7F800001, FAKE, None) == mxmoe.MX_EINVAL                   # past the finite floats


def test_phase_events_reject_bad_arguments(lib):
    assert lib.mx_set_phase_events(None, 3) == mxmoe.MX_EINVAL
    assert lib.mx_set_phase_events(None, 4) == mxmoe.MX_EINVAL
    assert lib.mx_set_phase_events(None, 0) == mxmoe.MX_OK


def test_noalloc_rejects_what_does_not_fit(lib):
    """moe_expert_ffn_noalloc: argument errors as moe_expert_ffn, and a shape
    whose workspace exceeds the built-in 16 MiB array is refused on the host."""
    def call(T=4, H=256, E=8, I=64, k=2, x=FAKE):
        return lib.moe_expert_ffn_noalloc(x, FAKE, T, H, FAKE, FAKE, FAKE, FAKE, k, FAKE, FAKE, FAKE, FAKE, E, I,
                                          FAKE, None)
    assert lib.moe_expert_ffn_noalloc_max_bytes() == 16 << 20
    assert call(k=0) == mxmoe.MX_EINVAL
    assert call(x=None) == mxmoe.MX_EINVAL
    assert call(H=6144, I=1024) == mxmoe.MX_EUNSUPPORTED
    assert mxmoe.moe_expert_ffn_workspace_bytes(8192, 4096, 256, 576, 8) > 16 << 20
    assert call(T=8192, H=4096, E=256, I=576, k=8) == mxmoe.MX_EWORKSPACE
    assert call(T=1024, H=4096, E=256, I=576, k=8) == mxmoe.MX_EWORKSPACE
