// Internal launchers behind the C-ABI (api.cpp validates, these launch).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mx {

// limits the kernels are built for (checked on the host before any launch)
constexpr int MAX_E = 1024;      // experts (route LDS lists)
constexpr int MAX_K = 16;        // top-k
constexpr int MAX_I = 2048;      // expert intermediate (decode LDS staging)
constexpr int MAX_PARTS = 16;    // K parts of 1024 -> H, K <= 16384
constexpr int ROUTE_CHUNK = 256; // rows per bucketing chunk
constexpr int ROUTE_FUSED_MAX_T = 32;  // rows ranked inside the single-workgroup route (more: a top-k launch first)
constexpr int LG_MAX_H = 16384;     // router logits: hidden width
constexpr int LG_PREFILL_MIN_T = 1024; // router logits: rows from which the tiled kernel runs (measured crossover)
constexpr int KPART_MAX_SHARED1 = 1024; // one-row shared expert: its down projection is one K part

hipError_t launch_quantize(const void* src, bool bf16, int64_t rows, int64_t cols, bool fp4,
                           uint8_t* q, uint8_t* sc, hipStream_t stream);

size_t route_ws_bytes(int T, int E);
// anchor == NULL: skip mode; otherwise router-live mode
hipError_t launch_route(const float* logits, int T, int E, int k, const float* survival, float skip_below,
                        const int32_t* anchor, int32_t* ids, float* w, int32_t* offsets, int32_t* perm,
                        int32_t* slot_pos, void* ws, hipStream_t stream, const char** variant);

struct FfnArgs {
  const uint8_t* x; const uint8_t* x_sc; int T; int H;
  const float* topk_w; const int32_t* offsets; const int32_t* perm; const int32_t* slot_pos; int k;
  const uint8_t* w13; const uint8_t* w13_sc; const uint8_t* w2; const uint8_t* w2_sc; int E; int I;
  float* y;
};
// single-row layer: the gate runs inside the gate/up kernel (route outputs written there)
struct FusedRoute {
  const float* logits; const float* survival; float skip_below;
  int32_t* ids; float* w; int32_t* offsets; int32_t* perm; int32_t* slot_pos;
};
// one row's shared expert (T = 1, I <= 1024): x FP8 [H] + SC; W13 FP8 [2I][H]
// + SC; W2 FP8 [H][I] + SC; pbuf the gate/up parts [ceil(H / 1024)][2I]; y
// [H]; h [2I], q [I], q_sc [I/32] receive the intermediate (diagnostics)
struct Shared1Args {
  const uint8_t* x; const uint8_t* x_sc; const uint8_t* w13; const uint8_t* w13_sc;
  const uint8_t* w2; const uint8_t* w2_sc; int H, I;
  float* pbuf; float* y; float* h; uint8_t* q; uint8_t* q_sc;
};
size_t ffn_ws_bytes(int T, int H, int E, int I, int k);
void ffn_ws_layout(int T, int H, int I, int k, size_t* off_q, size_t* off_q_sc, size_t* off_o);
// path: 0 automatic, 1 decode kernels, 2 prefill kernels.  Returns the path
// that runs T*k pairs of an (H, I) layer under the requested setting, or 0
// when no kernel supports the shape (then nothing may be launched).
int ffn_resolve_path(int path, int64_t Tk, int H, int I);
// h: NULL, or fp32 [T*k][2I] that receives the gate/up values (diagnostics)
// sh (single-row fused layer only): the shared expert's tiles run in the same
// two launches as the routed experts'
hipError_t launch_ffn(const FfnArgs& a, void* ws, int path, hipStream_t stream, const char** variant,
                      const FusedRoute* fr = nullptr, float* h = nullptr, const Shared1Args* sh = nullptr);
void set_ffn_phase_events(const hipEvent_t* ev, int n);
void set_layer1_onepass(bool on);

// Cross-workgroup handoff of the single-launch forms: producers store 8-byte
// words (payload, then this call's 32-bit tag) with system-scope stores;
// consumers read them with system-scope loads until every word carries the
// tag, each wait bounded by `limit` wall-clock ticks (then bit 0 of *status).
// A launch replayed from a graph cannot carry a fresh host tag; there
// (graph = 1) a one-thread kernel recorded before it advances the
// workspace's call counter *epoch, and the call's tag is that count with
// bit 31 set.  Host tags keep bit 31 clear, so consecutive calls on one
// workspace never share a tag, whichever form each takes.
struct Handoff {
  uint64_t* words;                 // the (payload, tag) words
  uint32_t* status;                // bit 0: a wait ran past its limit
  uint32_t tag;                    // this call's tag (eager form; bit 31 clear)
  long long limit;                 // wall-clock ticks one consumer may wait in all
  int nprod;                       // producer workgroups (they come first in the grid)
  const uint32_t* epoch;           // the workspace's call counter (graph form: advanced before the launch)
  int graph;                       // 1: the graph form (tag = *epoch | 2^31), run by the GRAPH kernels
};
bool single_launch_on();           // mx_set_layer1_single_launch
uint32_t next_call_tag();          // unique per call in the process (a random start, then +1), bit 31 clear
long long handoff_limit_ticks();   // 20 ms of the current device's wall clock
// Records the epoch advance before a graph-form launch (a kernel: no memset node).
hipError_t launch_handoff_epoch(uint32_t* epoch, hipStream_t stream);

// The call counter (GRAPH: the kernels built for the graph form; issue early,
// resolve at first use, so the wait for it lands where the tag is first
// needed).  An ordinary cached load: an earlier kernel on the stream wrote
// the counter, which the stream order makes visible.
template <bool GRAPH>
__device__ __forceinline__ uint32_t handoff_epoch_issue(const Handoff& ho) {
  if constexpr (!GRAPH) return 0u;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)ho.epoch, (short)0, 4u, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, 0);
}
template <bool GRAPH>
__device__ __forceinline__ uint32_t handoff_tag(const Handoff& ho, uint32_t epoch_value) {
  return GRAPH ? (epoch_value | 0x80000000u) : ho.tag;
}
// moe_expert_ffn_noalloc: the library's own device scratch array (per GPU,
// NOALLOC_SCRATCH_BYTES) in place of a caller workspace; *ptr receives its
// address on the current device.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(16) << 20;
hipError_t noalloc_scratch(void** ptr);

constexpr int GEMM_PREFILL_MIN_M = 320;  // dense GEMM: rows from which the tiled kernel beats the decode kernel (measured)
hipError_t launch_block_gemm(const uint8_t* a, const uint8_t* a_sc, const uint8_t* w, const uint8_t* w_sc,
                             int M, int N, int K, void* y, bool bf16_out, hipStream_t stream, const char** variant);

size_t router_logits_ws_bytes(int T, int H, int E);
hipError_t launch_router_logits(const uint16_t* h, int T, int H, const uint16_t* wg, int E, float* logits, void* ws,
                                hipStream_t stream, const char** variant);

// shared expert of one row (I <= 1024): gate/up as canonical parts into pbuf
// [H / 1024 rounded up][2I], then the down kernel with the part sum, SwiGLU and
// requant in its prologue; h, q, q_sc receive the intermediate (diagnostics)
hipError_t launch_shared_down1(const uint8_t* x, const uint8_t* x_sc, int H, const uint8_t* w13,
                               const uint8_t* w13_sc, const uint8_t* w2, const uint8_t* w2_sc, int I, float* y,
                               float* h, uint8_t* q, uint8_t* q_sc, float* pbuf, hipStream_t stream);
size_t shared_ws_bytes(int T, int H, int I);
// the pointers of the one-row shared expert inside a moe_shared_expert workspace
Shared1Args shared1_args(const uint8_t* x, const uint8_t* x_sc, int H, const uint8_t* w13, const uint8_t* w13_sc,
                         const uint8_t* w2, const uint8_t* w2_sc, int I, float* y, void* ws);
hipError_t launch_shared_expert(const uint8_t* x, const uint8_t* x_sc, int T, int H, const uint8_t* w13,
                                const uint8_t* w13_sc, const uint8_t* w2, const uint8_t* w2_sc, int I, float* y,
                                void* ws, hipStream_t stream, const char** variant);

hipError_t launch_prefetch(const void* p, uint64_t bytes, uint64_t chunk, hipStream_t stream);

int num_cus();
hipError_t launch_check_requant(uint32_t lo, uint32_t hi, unsigned long long* nbad, hipStream_t stream);

}  // namespace mx
