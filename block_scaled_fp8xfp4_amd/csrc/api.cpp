// C-ABI of the library (include/mxmoe.h): argument validation on the host,
// then kernel launches on the caller's stream.  Nothing here allocates,
// synchronizes or reads device memory; every error is reported before the
// first launch of a call.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "mxmoe.h"
#include "mx_launch.hpp"

namespace {

thread_local const char* g_variant = "";
std::atomic<int> g_ffn_path{0};
thread_local float* g_diag_h = nullptr;          // mx_set_ffn_diag: gate/up values of this thread's FFN calls
thread_local size_t g_diag_h_bytes = 0;

// The diagnostic gate/up buffer must hold T*k rows of 2I floats.
bool diag_h_fits(int64_t Tk, int I) { return g_diag_h == nullptr || g_diag_h_bytes >= (size_t)Tk * 2 * I * 4; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

mx_status from_hip(hipError_t e) { return e == hipSuccess ? MX_OK : MX_EHIP; }

}  // namespace

namespace mx {
int num_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}
}  // namespace mx

extern "C" {

const char* mx_status_string(mx_status s) {
  switch (s) {
    case MX_OK: return "MX_OK";
    case MX_EINVAL: return "MX_EINVAL: null pointer, bad shape or value out of range";
    case MX_EUNSUPPORTED: return "MX_EUNSUPPORTED: valid request that the kernels do not implement";
    case MX_EWORKSPACE: return "MX_EWORKSPACE: workspace missing or smaller than required";
    case MX_EHIP: return "MX_EHIP: a HIP launch or runtime call failed";
    default: return "unknown mx_status";
  }
}

const char* mx_last_variant(void) { return g_variant; }

int mx_set_ffn_path(int path) {
  if (path < 0 || path > 2) return MX_EINVAL;
  return g_ffn_path.exchange(path);
}

int mx_set_layer1_single_launch(int on) {
  if (on != 0 && on != 1) return MX_EINVAL;
  static std::atomic<int> cur{1};
  mx::set_layer1_onepass(on == 1);
  return cur.exchange(on);
}

mx_status mx_quantize(const void* src, int src_dtype, int64_t rows, int64_t cols, int fmt, uint8_t* q, uint8_t* sc,
                      void* stream) {
  if (!src || !q || !sc) return MX_EINVAL;
  if (rows < 0 || cols < 0 || cols % 32 != 0) return MX_EINVAL;
  if (src_dtype != MX_IN_F32 && src_dtype != MX_IN_BF16) return MX_EINVAL;
  if (fmt != MX_FMT_E4M3 && fmt != MX_FMT_E2M1) return MX_EINVAL;
  if (!aligned(src, 16) || !aligned(q, 16)) return MX_EINVAL;
  if (rows > 0 && cols / 32 > (int64_t(1) << 40) / rows) return MX_EUNSUPPORTED;
  const hipError_t e = mx::launch_quantize(src, src_dtype == MX_IN_BF16, rows, cols, fmt == MX_FMT_E2M1, q, sc,
                                           static_cast<hipStream_t>(stream));
  if (e == hipSuccess) g_variant = fmt == MX_FMT_E2M1 ? "quantize:e2m1_block32" : "quantize:e4m3_block32";
  return from_hip(e);
}

size_t moe_router_logits_workspace_bytes(int T, int H, int E) {
  if (T < 0 || E < 1 || H < 32 || H % 32 != 0 || H > mx::LG_MAX_H) return 0;
  return mx::router_logits_ws_bytes(T, H, E);
}

mx_status moe_router_logits(const uint16_t* hidden, int T, int H, const uint16_t* w_gate, int E, float* logits,
                            void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || E < 1 || H < 32 || H % 32 != 0) return MX_EINVAL;
  if (H > mx::LG_MAX_H) return MX_EUNSUPPORTED;
  if ((int64_t)T * H >= (int64_t(1) << 31) || (int64_t)E * H >= (int64_t(1) << 31) ||
      (int64_t)T * E >= (int64_t(1) << 31))
    return MX_EUNSUPPORTED;
  if (!w_gate || (T > 0 && (!hidden || !logits))) return MX_EINVAL;
  if (!aligned(hidden, 16) || !aligned(w_gate, 16) || !aligned(logits, 4) || !aligned(ws, 256)) return MX_EINVAL;
  const size_t need = mx::router_logits_ws_bytes(T, H, E);
  if (need > 0 && (!ws || ws_bytes < need)) return MX_EWORKSPACE;
  if (T == 0) { g_variant = "logits:empty"; return MX_OK; }
  const char* v = "";
  const hipError_t e = mx::launch_router_logits(hidden, T, H, w_gate, E, logits, ws,
                                                static_cast<hipStream_t>(stream), &v);
  if (e == hipSuccess) g_variant = v;
  return from_hip(e);
}

size_t moe_route_workspace_bytes(int T, int E, int k) {
  (void)k;
  if (T < 0 || E < 1) return 0;
  return mx::route_ws_bytes(T, E);
}

namespace {
mx_status route_common(const float* logits, int T, int E, int k, const float* survival, float threshold,
                       const int32_t* anchor, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                       int32_t* perm, int32_t* slot_pos, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || E < 1 || E > mx::MAX_E || k < 1 || k > E || k > mx::MAX_K) return MX_EINVAL;
  if ((int64_t)T * k >= (int64_t(1) << 31)) return MX_EINVAL;
  if (!expert_offsets) return MX_EINVAL;
  if (T > 0 && (!logits || !topk_ids || !topk_w || !perm || !slot_pos)) return MX_EINVAL;
  if (!ws || ws_bytes < mx::route_ws_bytes(T, E)) return MX_EWORKSPACE;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(expert_offsets, 4) ||
      !aligned(perm, 4) || !aligned(slot_pos, 4) || !aligned(survival, 4) || !aligned(anchor, 4) ||
      !aligned(ws, 256))
    return MX_EINVAL;
  const char* v = "";
  const hipError_t e = mx::launch_route(logits, T, E, k, survival, threshold, anchor, topk_ids, topk_w,
                                        expert_offsets, perm, slot_pos, ws, static_cast<hipStream_t>(stream), &v);
  if (e == hipSuccess) g_variant = v;
  return from_hip(e);
}
}  // namespace

mx_status moe_route(const float* logits, int T, int E, int k, const float* survival, float skip_below,
                    int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* perm, int32_t* slot_pos,
                    void* ws, size_t ws_bytes, void* stream) {
  return route_common(logits, T, E, k, survival, skip_below, nullptr, topk_ids, topk_w, expert_offsets, perm,
                      slot_pos, ws, ws_bytes, stream);
}

mx_status moe_route_live(const float* logits, int T, int E, int k, const float* survival, float reuse_below,
                         const int32_t* anchor, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                         int32_t* perm, int32_t* slot_pos, void* ws, size_t ws_bytes, void* stream) {
  if (T > 0 && !anchor) return MX_EINVAL;
  if (T == 0) anchor = reinterpret_cast<const int32_t*>(ws);   // any non-null pointer: nothing is read
  return route_common(logits, T, E, k, survival, reuse_below, anchor, topk_ids, topk_w, expert_offsets, perm,
                      slot_pos, ws, ws_bytes, stream);
}

mx_status moe_ws_layout(int T, int H, int I, int k, size_t* off_q, size_t* off_q_sc, size_t* off_o) {
  if (T < 0 || H < 128 || I < 32 || k < 1 || !off_q || !off_q_sc || !off_o) return MX_EINVAL;
  mx::ffn_ws_layout(T, H, I, k, off_q, off_q_sc, off_o);
  return MX_OK;
}

mx_status mx_set_ffn_diag(float* h, size_t h_bytes) {
  if (h != nullptr && !aligned(h, 16)) return MX_EINVAL;
  g_diag_h = h;
  g_diag_h_bytes = h ? h_bytes : 0;
  return MX_OK;
}

size_t moe_expert_ffn_workspace_bytes(int T, int H, int E, int I, int k) {
  if (T < 0 || H < 128 || E < 1 || I < 32 || k < 1) return 0;
  return mx::ffn_ws_bytes(T, H, E, I, k);
}

mx_status moe_expert_ffn(const uint8_t* x, const uint8_t* x_sc, int T, int H, const float* topk_w,
                         const int32_t* expert_offsets, const int32_t* perm, const int32_t* slot_pos, int k,
                         const uint8_t* w13, const uint8_t* w13_sc, const uint8_t* w2, const uint8_t* w2_sc, int E,
                         int I, float* y, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k < 1 || k > mx::MAX_K || E < 1 || E > mx::MAX_E || H < 128 || I < 32) return MX_EINVAL;
  if (H % 32 != 0 || I % 32 != 0) return MX_EINVAL;
  if (H % 128 != 0 || H > 128 * 8 * mx::MAX_PARTS || I > mx::MAX_I) return MX_EUNSUPPORTED;
  if ((int64_t)T * k >= (int64_t(1) << 31)) return MX_EINVAL;
  if ((int64_t)T * H >= (int64_t(1) << 32)) return MX_EUNSUPPORTED;
  if (!x || !x_sc || !topk_w || !expert_offsets || !perm || !slot_pos || !w13 || !w13_sc || !w2 || !w2_sc || !y)
    return MX_EINVAL;
  if (!aligned(x, 16) || !aligned(w13, 16) || !aligned(w2, 16) || !aligned(y, 16) || !aligned(x_sc, 4) ||
      !aligned(w13_sc, 4) || !aligned(w2_sc, 4) || !aligned(topk_w, 4) || !aligned(expert_offsets, 4) ||
      !aligned(perm, 4) || !aligned(slot_pos, 4))
    return MX_EINVAL;
  // the kernels of the requested path (automatic: either path) must support (H, I): never a silent fallback
  const int path = mx::ffn_resolve_path(g_ffn_path.load(), (int64_t)T * k, H, I);
  if (path == 0) return MX_EUNSUPPORTED;
  if (!ws || ws_bytes < mx::ffn_ws_bytes(T, H, E, I, k) || !diag_h_fits((int64_t)T * k, I)) return MX_EWORKSPACE;
  if (!aligned(ws, 256)) return MX_EINVAL;
  if (T == 0) { g_variant = "ffn:empty"; return MX_OK; }
  const mx::FfnArgs a{x, x_sc, T, H, topk_w, expert_offsets, perm, slot_pos, k, w13, w13_sc, w2, w2_sc, E, I, y};
  const char* v = "";
  const hipError_t e = mx::launch_ffn(a, ws, path, static_cast<hipStream_t>(stream), &v, nullptr, g_diag_h);
  if (e == hipSuccess) g_variant = v;
  return from_hip(e);
}

size_t moe_expert_ffn_noalloc_max_bytes(void) { return mx::NOALLOC_SCRATCH_BYTES; }

mx_status moe_expert_ffn_noalloc(const uint8_t* x, const uint8_t* x_sc, int T, int H, const float* topk_w,
                                 const int32_t* expert_offsets, const int32_t* perm, const int32_t* slot_pos, int k,
                                 const uint8_t* w13, const uint8_t* w13_sc, const uint8_t* w2, const uint8_t* w2_sc,
                                 int E, int I, float* y, void* stream) {
  if (T < 0 || k < 1 || k > mx::MAX_K || E < 1 || E > mx::MAX_E || H < 128 || I < 32) return MX_EINVAL;
  if (H % 32 != 0 || I % 32 != 0) return MX_EINVAL;
  if (H % 128 != 0 || H > 128 * 8 * mx::MAX_PARTS || I > mx::MAX_I) return MX_EUNSUPPORTED;
  if ((int64_t)T * k >= (int64_t(1) << 31)) return MX_EINVAL;
  if ((int64_t)T * H >= (int64_t(1) << 32)) return MX_EUNSUPPORTED;
  if (!x || !x_sc || !topk_w || !expert_offsets || !perm || !slot_pos || !w13 || !w13_sc || !w2 || !w2_sc || !y)
    return MX_EINVAL;
  if (!aligned(x, 16) || !aligned(w13, 16) || !aligned(w2, 16) || !aligned(y, 16) || !aligned(x_sc, 4) ||
      !aligned(w13_sc, 4) || !aligned(w2_sc, 4) || !aligned(topk_w, 4) || !aligned(expert_offsets, 4) ||
      !aligned(perm, 4) || !aligned(slot_pos, 4))
    return MX_EINVAL;
  const int path = mx::ffn_resolve_path(g_ffn_path.load(), (int64_t)T * k, H, I);
  if (path == 0) return MX_EUNSUPPORTED;
  // the built-in scratch holds what moe_expert_ffn_workspace_bytes asks of a caller
  if (mx::ffn_ws_bytes(T, H, E, I, k) > mx::NOALLOC_SCRATCH_BYTES || !diag_h_fits((int64_t)T * k, I))
    return MX_EWORKSPACE;
  if (T == 0) { g_variant = "ffn:empty"; return MX_OK; }
  void* ws = nullptr;
  hipError_t e = mx::noalloc_scratch(&ws);
  if (e != hipSuccess) return MX_EHIP;
  const mx::FfnArgs a{x, x_sc, T, H, topk_w, expert_offsets, perm, slot_pos, k, w13, w13_sc, w2, w2_sc, E, I, y};
  const char* v = "";
  e = mx::launch_ffn(a, ws, path, static_cast<hipStream_t>(stream), &v, nullptr, g_diag_h);
  if (e == hipSuccess) g_variant = v;
  return from_hip(e);
}

mx_status moe_layer_decode1(const float* logits, int E, int k, const float* survival, float skip_below,
                            const uint8_t* x, const uint8_t* x_sc, int H, const uint8_t* w13, const uint8_t* w13_sc,
                            const uint8_t* w2, const uint8_t* w2_sc, int I, int32_t* topk_ids, float* topk_w,
                            int32_t* expert_offsets, int32_t* perm, int32_t* slot_pos, float* y, void* ws,
                            size_t ws_bytes, void* stream) {
  if (E < 1 || E > mx::MAX_E || k < 1 || k > E || k > mx::MAX_K || H < 128 || I < 32) return MX_EINVAL;
  if (H % 32 != 0 || I % 32 != 0) return MX_EINVAL;
  if (H % 128 != 0 || H > 128 * 8 * mx::MAX_PARTS || I > mx::MAX_I || mx::ffn_resolve_path(1, k, H, I) != 1)
    return MX_EUNSUPPORTED;
  if (!logits || !x || !x_sc || !w13 || !w13_sc || !w2 || !w2_sc || !topk_ids || !topk_w || !expert_offsets ||
      !perm || !slot_pos || !y)
    return MX_EINVAL;
  if (!aligned(logits, 4) || !aligned(survival, 4) || !aligned(x, 16) || !aligned(w13, 16) || !aligned(w2, 16) ||
      !aligned(y, 16) || !aligned(x_sc, 4) || !aligned(w13_sc, 4) || !aligned(w2_sc, 4) || !aligned(topk_ids, 4) ||
      !aligned(topk_w, 4) || !aligned(expert_offsets, 4) || !aligned(perm, 4) || !aligned(slot_pos, 4))
    return MX_EINVAL;
  if (!ws || ws_bytes < mx::ffn_ws_bytes(1, H, E, I, k) || !diag_h_fits(k, I)) return MX_EWORKSPACE;
  if (!aligned(ws, 256)) return MX_EINVAL;
  const mx::FfnArgs a{x, x_sc, 1, H, topk_w, expert_offsets, perm, slot_pos, k, w13, w13_sc, w2, w2_sc, E, I, y};
  const mx::FusedRoute fr{logits, survival, skip_below, topk_ids, topk_w, expert_offsets, perm, slot_pos};
  const char* v = "";
  const hipError_t e = mx::launch_ffn(a, ws, 1, static_cast<hipStream_t>(stream), &v, &fr, g_diag_h);
  if (e == hipSuccess) g_variant = v;
  return from_hip(e);
}

static size_t layer1_routed_ws(int H, int E, int I, int k) { return (mx::ffn_ws_bytes(1, H, E, I, k) + 255) / 256 * 256; }

size_t moe_layer_decode1_shared_workspace_bytes(int H, int E, int I, int k, int Is) {
  if (H < 128 || E < 1 || k < 1 || k > E || I < 32 || Is < 32 || H % 32 || I % 32 || Is % 32) return 0;
  return layer1_routed_ws(H, E, I, k) + mx::shared_ws_bytes(1, H, Is);
}

mx_status moe_layer_decode1_shared(const float* logits, int E, int k, const float* survival, float skip_below,
                                   const uint8_t* x, const uint8_t* x_sc, int H, const uint8_t* w13,
                                   const uint8_t* w13_sc, const uint8_t* w2, const uint8_t* w2_sc, int I,
                                   const uint8_t* sw13, const uint8_t* sw13_sc, const uint8_t* sw2,
                                   const uint8_t* sw2_sc, int Is, int32_t* topk_ids, float* topk_w,
                                   int32_t* expert_offsets, int32_t* perm, int32_t* slot_pos, float* y,
                                   float* y_shared, void* ws, size_t ws_bytes, void* stream) {
  if (E < 1 || E > mx::MAX_E || k < 1 || k > E || k > mx::MAX_K || H < 128 || I < 32 || Is < 32) return MX_EINVAL;
  if (H % 32 != 0 || I % 32 != 0 || Is % 32 != 0) return MX_EINVAL;
  if (H % 128 != 0 || H > 128 * 8 * mx::MAX_PARTS || I > mx::MAX_I || mx::ffn_resolve_path(1, k, H, I) != 1 ||
      Is > mx::KPART_MAX_SHARED1)
    return MX_EUNSUPPORTED;
  if (!logits || !x || !x_sc || !w13 || !w13_sc || !w2 || !w2_sc || !sw13 || !sw13_sc || !sw2 || !sw2_sc ||
      !topk_ids || !topk_w || !expert_offsets || !perm || !slot_pos || !y || !y_shared)
    return MX_EINVAL;
  if (!aligned(logits, 4) || !aligned(survival, 4) || !aligned(x, 16) || !aligned(w13, 16) || !aligned(w2, 16) ||
      !aligned(y, 16) || !aligned(x_sc, 4) || !aligned(w13_sc, 4) || !aligned(w2_sc, 4) || !aligned(topk_ids, 4) ||
      !aligned(topk_w, 4) || !aligned(expert_offsets, 4) || !aligned(perm, 4) || !aligned(slot_pos, 4) ||
      !aligned(sw13, 16) || !aligned(sw2, 16) || !aligned(sw13_sc, 4) || !aligned(sw2_sc, 4) || !aligned(y_shared, 4))
    return MX_EINVAL;
  const size_t rws = layer1_routed_ws(H, E, I, k);
  if (!ws || ws_bytes < rws + mx::shared_ws_bytes(1, H, Is) || !diag_h_fits(k, I)) return MX_EWORKSPACE;
  if (!aligned(ws, 256)) return MX_EINVAL;
  const mx::FfnArgs a{x, x_sc, 1, H, topk_w, expert_offsets, perm, slot_pos, k, w13, w13_sc, w2, w2_sc, E, I, y};
  const mx::FusedRoute fr{logits, survival, skip_below, topk_ids, topk_w, expert_offsets, perm, slot_pos};
  const mx::Shared1Args sh =
      mx::shared1_args(x, x_sc, H, sw13, sw13_sc, sw2, sw2_sc, Is, y_shared, static_cast<uint8_t*>(ws) + rws);
  const char* v = "";
  const hipError_t e = mx::launch_ffn(a, ws, 1, static_cast<hipStream_t>(stream), &v, &fr, g_diag_h, &sh);
  if (e == hipSuccess) g_variant = v;
  return from_hip(e);
}

mx_status fp8_block_gemm(const uint8_t* a, const uint8_t* a_sc, const uint8_t* w, const uint8_t* w_sc, int M, int N,
                         int K, void* y, int y_dtype, void* stream) {
  if (!a || !a_sc || !w || !w_sc || !y) return MX_EINVAL;
  if (M < 1 || N < 1 || K < 32 || K % 32 != 0) return MX_EINVAL;
  if (y_dtype != MX_OUT_BF16 && y_dtype != MX_OUT_F32) return MX_EINVAL;
  if (N % 16 != 0 || K > 128 * 8 * mx::MAX_PARTS) return MX_EUNSUPPORTED;
  // the tiled kernel addresses both operands with 32-bit byte offsets
  if ((int64_t)M * N >= (int64_t(1) << 31) || (int64_t)M * K >= (int64_t(1) << 32) ||
      (int64_t)N * K >= (int64_t(1) << 32))
    return MX_EUNSUPPORTED;
  if (!aligned(a, 16) || !aligned(w, 16) || !aligned(a_sc, 4) || !aligned(w_sc, 4) || !aligned(y, 4)) return MX_EINVAL;
  const char* v = "";
  const hipError_t e =
      mx::launch_block_gemm(a, a_sc, w, w_sc, M, N, K, y, y_dtype == MX_OUT_BF16, static_cast<hipStream_t>(stream), &v);
  if (e == hipSuccess) g_variant = v;
  return from_hip(e);
}

size_t moe_shared_expert_workspace_bytes(int T, int H, int I) {
  if (T < 0 || H < 32 || I < 32 || H % 32 != 0 || I % 32 != 0) return 0;
  return mx::shared_ws_bytes(T, H, I);
}

mx_status moe_shared_expert(const uint8_t* x, const uint8_t* x_sc, int T, int H, const uint8_t* w13,
                            const uint8_t* w13_sc, const uint8_t* w2, const uint8_t* w2_sc, int I, float* y, void* ws,
                            size_t ws_bytes, void* stream) {
  if (T < 0 || H < 32 || I < 32 || H % 32 != 0 || I % 32 != 0) return MX_EINVAL;
  const int kmax = 128 * 8 * mx::MAX_PARTS;
  if (H > kmax || I > kmax) return MX_EUNSUPPORTED;
  if ((int64_t)T * H >= (int64_t(1) << 31) || (int64_t)T * 2 * I >= (int64_t(1) << 31)) return MX_EUNSUPPORTED;
  if (!w13 || !w13_sc || !w2 || !w2_sc || (T > 0 && (!x || !x_sc || !y))) return MX_EINVAL;
  if (!aligned(x, 16) || !aligned(w13, 16) || !aligned(w2, 16) || !aligned(y, 4) || !aligned(x_sc, 4) ||
      !aligned(w13_sc, 4) || !aligned(w2_sc, 4) || !aligned(ws, 256))
    return MX_EINVAL;
  if (T == 0) { g_variant = "shared:empty"; return MX_OK; }
  if (!ws || ws_bytes < mx::shared_ws_bytes(T, H, I)) return MX_EWORKSPACE;
  const char* v = "";
  const hipError_t e = mx::launch_shared_expert(x, x_sc, T, H, w13, w13_sc, w2, w2_sc, I, y, ws,
                                                static_cast<hipStream_t>(stream), &v);
  if (e == hipSuccess) g_variant = v;
  return from_hip(e);
}

mx_status mx_prefetch(const void* p, uint64_t bytes, uint64_t chunk_bytes, void* stream) {
  if (bytes == 0) return MX_OK;
  if (!p || !aligned(p, 16)) return MX_EINVAL;
  if (chunk_bytes == 0) chunk_bytes = 65536;
  if (chunk_bytes % 16 != 0) return MX_EINVAL;
  if ((bytes + chunk_bytes - 1) / chunk_bytes > (uint64_t(1) << 31) - 1) return MX_EUNSUPPORTED;
  const hipError_t e = mx::launch_prefetch(p, bytes, chunk_bytes, static_cast<hipStream_t>(stream));
  if (e == hipSuccess) g_variant = "prefetch:lds_dma";
  return from_hip(e);
}

mx_status mx_check_requant(uint32_t lo, uint32_t hi, unsigned long long* mismatches, void* stream) {
  if (!mismatches || !aligned(mismatches, 8) || lo > hi || hi > 0x7F800000u) return MX_EINVAL;
  return from_hip(mx::launch_check_requant(lo, hi, mismatches, static_cast<hipStream_t>(stream)));
}

mx_status mx_set_phase_events(void* const* events, int n) {
  if (n != 0 && n != 4) return MX_EINVAL;
  if (n == 4)
    for (int i = 0; i < 4; ++i)
      if (!events || !events[i]) return MX_EINVAL;
  hipEvent_t ev[4] = {};
  for (int i = 0; i < n; ++i) ev[i] = static_cast<hipEvent_t>(events[i]);
  mx::set_ffn_phase_events(ev, n);
  return MX_OK;
}

}  // extern "C"
