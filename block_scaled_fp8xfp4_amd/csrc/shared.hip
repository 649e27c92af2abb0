// Shared expert: a dense SwiGLU MLP applied to every row, with block-32 FP8
// operands ("New Deepseek 4.1 flash recipe" thread, post #6, "Kernel by
// kernel against B12X": the shared expert's two kernels per call, on a side
// stream; DeepSeek-V4.1-Flash-4x-DGX-Spark-TP4 README, settings table, row
// "Kernels", and its boot-log lines: the shared expert's down weight is
// (5120, 576) and was padded to K = 640 for the kernels there).
//
// h = x . W13^T (fp32, dense FP8 GEMM), a = silu(gate) * up requantized to
// E4M3 block-32 by the routed experts' own routine, y = a . W2^T with K = I
// (576 is 4.5 MFMA steps: the GEMM kernels zero the half step in registers
// or LDS, no padded copy of the weight exists).  The GEMMs keep the dense
// projection's canonical order, so rows do not depend on the batch.
#include "mx_device.hpp"
#include "mx_launch.hpp"
#include "shared1_device.hpp"

namespace mx {

// One thread per pair of adjacent intermediate columns: 16 lanes (a DPP row)
// cover one block of 32, so the block's amax is a row maximum in registers.
// h row t: gate at [0, I), up at [I, 2I).
__global__ __launch_bounds__(256) void swiglu_requant_kernel(const float* __restrict__ h, int T, int I,
                                                             uint8_t* __restrict__ q, uint8_t* __restrict__ q_sc) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // pair index over [T][I / 2]
  const int64_t n = (int64_t)T * (I / 2);
  const bool ok = i < n;                                        // whole DPP rows are in or out (I / 2 % 16 == 0)
  const int64_t t = ok ? i / (I / 2) : 0;
  const int c = ok ? (int)(i % (I / 2)) * 2 : 0;
  const float* hr = h + t * 2 * I;
  float2 g = {0.f, 0.f}, u = {0.f, 0.f};
  if (ok) {
    g = *reinterpret_cast<const float2*>(hr + c);
    u = *reinterpret_cast<const float2*>(hr + I + c);
  }
  uint32_t sc;
  const uint32_t d = swiglu_requant2(g.x, u.x, g.y, u.y, &sc);
  if (!ok) return;
  *reinterpret_cast<uint16_t*>(q + t * I + c) = (uint16_t)d;
  if ((c & 31) == 0) q_sc[t * (I / 32) + c / 32] = (uint8_t)sc;
}

// The shared expert of one row in ONE launch: workgroups [0, I / 8) compute
// gate/up (shared1_gate_up8), the H / 16 after them the down projection
// (shared1_down_wait), which waits on the former's tagged words.  Producers
// come first in the grid and never wait, so every wait can end; each is
// bounded by ho.limit.  Same bits as the two-launch form.  H % 128 == 0.
template <bool TAIL, bool GRAPH>
__global__ __launch_bounds__(256) void shared1_onepass_kernel(Shared1Args sh, Handoff ho) {
  if ((int)blockIdx.x < ho.nprod) shared1_gate_up8<GRAPH>(sh, ho.words, ho, (int)blockIdx.x);
  else shared1_down_wait<TAIL, GRAPH>(sh, ho, (int)blockIdx.x - ho.nprod);
}

static size_t a256(size_t b) { return (b + 255) / 256 * 256; }

// one row with I <= 1024 takes the one-row path (one launch, or gate/up parts + down with the requant prologue)
static bool one_row_path(int T, int I) { return T == 1 && I <= KPART; }

// [h: T x 2I fp32][q: T x I][q_sc: T x I/32], then on the one-row path
// [parts: the gate/up parts (two launches) or the handoff words, I / 8
// lines of 128 bytes (one)][status word, 256 bytes]
size_t shared_ws_bytes(int T, int H, int I) {
  const size_t base = a256((size_t)T * 2 * I * 4) + a256((size_t)T * I) + a256((size_t)T * (I / 32));
  const size_t parts = (size_t)((H + KPART - 1) / KPART) * 2 * I * 4;
  return base + (one_row_path(T, I) ? a256(parts > shared1_words_bytes(I) ? parts : shared1_words_bytes(I)) + 256 : 0);
}

Shared1Args shared1_args(const uint8_t* x, const uint8_t* x_sc, int H, const uint8_t* w13, const uint8_t* w13_sc,
                         const uint8_t* w2, const uint8_t* w2_sc, int I, float* y, void* ws) {
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* h = reinterpret_cast<float*>(base);
  uint8_t* q = base + a256((size_t)2 * I * 4);
  uint8_t* q_sc = q + a256((size_t)I);
  float* pbuf = reinterpret_cast<float*>(q_sc + a256((size_t)(I / 32)));
  return Shared1Args{x, x_sc, w13, w13_sc, w2, w2_sc, H, I, pbuf, y, h, q, q_sc};
}
hipError_t launch_shared_expert(const uint8_t* x, const uint8_t* x_sc, int T, int H, const uint8_t* w13,
                                const uint8_t* w13_sc, const uint8_t* w2, const uint8_t* w2_sc, int I, float* y,
                                void* ws, hipStream_t stream, const char** variant) {
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* h = reinterpret_cast<float*>(base);
  uint8_t* q = base + a256((size_t)T * 2 * I * 4);
  uint8_t* q_sc = q + a256((size_t)T * I);
  const char* v = "";
  if (one_row_path(T, I)) {
    const Shared1Args sh = shared1_args(x, x_sc, H, w13, w13_sc, w2, w2_sc, I, y, ws);
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (H % KSTEP == 0 && single_launch_on() && hipStreamIsCapturing(stream, &cap) == hipSuccess &&
        (cap == hipStreamCaptureStatusNone || cap == hipStreamCaptureStatusActive)) {
      uint32_t* status = reinterpret_cast<uint32_t*>(base + shared_ws_bytes(1, H, I) - 256);   // then the call counter
      const bool graph = cap == hipStreamCaptureStatusActive;   // captured: the counter advance is recorded first
      if (graph) {
        const hipError_t e = launch_handoff_epoch(status + 1, stream);
        if (e != hipSuccess) return e;
      }
      const Handoff ho{reinterpret_cast<uint64_t*>(sh.pbuf), status, graph ? 0u : next_call_tag(), handoff_limit_ticks(),
                       I / 8, status + 1, graph ? 1 : 0};
      const dim3 grid(I / 8 + H / 16);
      if (graph && I % KSTEP) hipLaunchKernelGGL((shared1_onepass_kernel<true, true>), grid, dim3(256), 0, stream, sh, ho);
      else if (graph) hipLaunchKernelGGL((shared1_onepass_kernel<false, true>), grid, dim3(256), 0, stream, sh, ho);
      else if (I % KSTEP) hipLaunchKernelGGL((shared1_onepass_kernel<true, false>), grid, dim3(256), 0, stream, sh, ho);
      else hipLaunchKernelGGL((shared1_onepass_kernel<false, false>), grid, dim3(256), 0, stream, sh, ho);
      *variant = "shared:decode1_onepass(gate_up+down_requant, one launch)";
      return hipGetLastError();
    }
    *variant = "shared:decode1_gemm_parts+down_requant";
    return launch_shared_down1(x, x_sc, H, w13, w13_sc, w2, w2_sc, I, y, sh.h, sh.q, sh.q_sc, sh.pbuf, stream);
  }
  hipError_t e = launch_block_gemm(x, x_sc, w13, w13_sc, T, 2 * I, H, h, false, stream, &v);
  if (e != hipSuccess) return e;
  const int64_t pairs = (int64_t)T * (I / 2);
  hipLaunchKernelGGL(swiglu_requant_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0, stream, h, T, I, q,
                     q_sc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_block_gemm(q, q_sc, w2, w2_sc, T, H, I, y, false, stream, &v);
  *variant = T >= GEMM_PREFILL_MIN_M ? "shared:gemm_prefill+swiglu_requant+gemm_prefill"
                                     : "shared:gemm_decode+swiglu_requant+gemm_decode";
  return e;
}

}  // namespace mx
