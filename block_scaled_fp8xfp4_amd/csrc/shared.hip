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

// ------------------------------------------------- one row in one launch --
// Gate/up of intermediate columns [8 item, 8 item + 8) over the whole K: the
// W13 rows of those 8 gate and 8 up columns, wavefront w taking K parts w,
// w + 4, ... (each part's chain from zero, exactly shared1_part's); wavefront
// 0 adds the parts in part order (shared1_down's sum), writes the 16 h
// values, and publishes the 8 SwiGLU values as tagged words words[c].
__device__ void shared1_gate_up8(const Shared1Args& sh, const Handoff& ho, int item) {
  constexpr int MAXP = 16;                                      // K parts: H <= 16384
  __shared__ float ps[MAXP][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, col = lane & 15, g = lane >> 4;
  const int H = sh.H, I = sh.I, nparts = shared1_nparts(H), nsteps = H / KSTEP;
  const int c0 = 8 * item;
  const int64_t n = col < 8 ? c0 + col : I + c0 + col - 8;    // lanes 0..7 gate rows, 8..15 up rows
  const uint8_t* ap = sh.x + g * 16;
  const uint8_t* wp = sh.w13 + n * H + g * 16;
  const uint32_t* xsp = reinterpret_cast<const uint32_t*>(sh.x_sc);
  const uint32_t* wsp = reinterpret_cast<const uint32_t*>(sh.w13_sc + n * (H / 32));
  for (int q = wave; q < nparts; q += 4) {                      // wavefront-uniform
    const int s0 = q * KPART_STEPS;
    u32x4 alo[KPART_STEPS], ahi[KPART_STEPS], blo[KPART_STEPS], bhi[KPART_STEPS];
    uint32_t as[KPART_STEPS], bs[KPART_STEPS];
#pragma unroll
    for (int m = 0; m < KPART_STEPS; ++m) {
      const int s = min(s0 + m, nsteps - 1);
      alo[m] = ldg16(ap + s * KSTEP);
      ahi[m] = ldg16(ap + s * KSTEP + 64);
      as[m] = xsp[s];
    }
#pragma unroll
    for (int m = 0; m < KPART_STEPS; ++m) {
      const int s = min(s0 + m, nsteps - 1);
      blo[m] = ldg16(wp + s * KSTEP);
      bhi[m] = ldg16(wp + s * KSTEP + 64);
      bs[m] = wsp[s];
    }
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < KPART_STEPS; ++m)
      if (s0 + m < nsteps)
        acc = mfma_fp8_fp8(fp8_pair(alo[m], ahi[m]), fp8_pair(blo[m], bhi[m]), acc, as[m] >> (8 * g), bs[m] >> (8 * g));
    if (lane < 16) ps[q][col] = acc[0];                         // output row 0 (every A row is the row)
  }
  lds_barrier();
  if (wave != 0) return;
  float v = lane < 16 ? ps[0][col] : 0.f;
  for (int q = 1; q < nparts; ++q) v = v + (lane < 16 ? ps[q][col] : 0.f);
  if (lane < 16) sh.h[n] = v;
  const float up = __shfl_down(v, 8, 16);                       // lanes 0..7: the gate and up values of column c0 + lane
  if (lane < 8)
    __hip_atomic_store(ho.words + c0 + lane, (uint64_t)__float_as_uint(swiglu(v, up)) | ((uint64_t)ho.tag << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Down projection of output columns [16 tile, 16 tile + 16): wavefront 0
// requests its 16 W2 rows first; the four wavefronts then wait for the I
// SwiGLU words (16-byte system-scope reads, wavefront w, lane l: chunks
// 64 w + l and 256 + 64 w + l, two words each), copy them to LDS, and the
// requant, the tails and the chain follow shared1_down exactly.  Tile 0
// writes q and q_sc.  I <= 1024.
template <bool TAIL>
__device__ void shared1_down_wait(const Shared1Args& sh, const Handoff& ho, int tile) {
  constexpr int NSD = KPART_STEPS;                              // steps of K = I <= 1024
  __shared__ __attribute__((aligned(16))) float av[NSD * KSTEP];
  __shared__ __attribute__((aligned(16))) uint8_t q1[NSD * KSTEP];
  __shared__ uint8_t s1[NSD * 4];
  const uint64_t t0 = wall_clock64();
  const int I = sh.I;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int nsteps = (I + KSTEP - 1) / KSTEP, nblk = I / 32;
  const int64_t n = (int64_t)tile * 16 + col;
  u32x4 blo[NSD], bhi[NSD];
  uint32_t bs[NSD];
  if (wave == 0) {
    const uint8_t* wp = sh.w2 + n * I + g * 16;
    const uint8_t* wsp = sh.w2_sc + n * (I / 32);
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
      const int ss = min(s, nsteps - 1);
      blo[s] = ld_chunk<TAIL>(wp + ss * KSTEP, ss * KSTEP + 16 * g, I);
      bhi[s] = ld_chunk<TAIL>(wp + ss * KSTEP + 64, ss * KSTEP + 64 + 16 * g, I);
      bs[s] = ld_scale<TAIL>(wsp, ss, g, nblk);
    }
  }
  for (int idx = tid; idx < NSD * KSTEP - I; idx += 256) q1[I + idx] = 0;   // K past I: zero elements
  for (int idx = tid; idx < NSD * 4 - nblk; idx += 256) s1[nblk + idx] = 127;   // and unit scales
  const __amdgpu_buffer_rsrc_t r =                              // reads past the I words return zeros
      __builtin_amdgcn_make_buffer_rsrc((void*)ho.words, (short)0, (uint32_t)I * 8u, 0x00020000);
  for (;;) {
    u32x4 v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) v[h] = __builtin_amdgcn_raw_buffer_load_b128(r, (256 * h + 64 * wave + lane) * 16, 0, 17);
    bool ok = true;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int wi = 2 * (256 * h + 64 * wave + lane) + e;
        ok = ok && (wi >= I || v[h][2 * e + 1] == ho.tag);
      }
    if (__ballot(ok) == ~0ull) {                                // wavefront-uniform
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int wi = 2 * (256 * h + 64 * wave + lane) + e;
          if (wi < I) av[wi] = __uint_as_float(v[h][2 * e]);
        }
      break;
    }
    if ((long long)(wall_clock64() - t0) > ho.limit) {
      if (lane == 0) __hip_atomic_fetch_or(ho.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  lds_barrier();
  // requant: 16 lanes per block of 32, columns c and c + 16 (swiglu_requant2 past its SwiGLU)
  for (int b0 = 0; b0 < nblk; b0 += 16) {
    const int b = b0 + (tid >> 4), c = tid & 15;
    const bool ok = b < nblk;
    const int cb = ok ? b * 32 : 0;
    const float a0 = av[cb + c], a1 = av[cb + 16 + c];
    const uint32_t sc = e8m0_code_for_amax(row16_max(fmaxf(__builtin_fabsf(a0), __builtin_fabsf(a1))), 8);
    const uint32_t d = requant2_e4m3(a0, a1, sc);
    if (ok) {
      q1[cb + c] = (uint8_t)d;
      q1[cb + 16 + c] = (uint8_t)(d >> 8);
      if (c == 0) s1[b] = (uint8_t)sc;
      if (tile == 0) {
        sh.q[cb + c] = (uint8_t)d;
        sh.q[cb + 16 + c] = (uint8_t)(d >> 8);
        if (c == 0) sh.q_sc[b] = (uint8_t)sc;
      }
    }
  }
  lds_barrier();
  if (wave != 0) return;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NSD; ++s)
    if (s < nsteps) {
      const u32x4 alo = *reinterpret_cast<const u32x4*>(&q1[s * KSTEP + g * 16]);
      const u32x4 ahi = *reinterpret_cast<const u32x4*>(&q1[s * KSTEP + 64 + g * 16]);
      const uint32_t sa = (uint32_t)s1[4 * s + g] << (8 * g);
      acc = mfma_fp8_fp8(fp8_pair(alo, ahi), fp8_pair(blo[s], bhi[s]), acc, sa >> (8 * g), bs[s] >> (8 * g));
    }
  if (g == 0) sh.y[n] = acc[0];
}

// The shared expert of one row in ONE launch: workgroups [0, I / 8) compute
// gate/up (shared1_gate_up8), the H / 16 after them the down projection
// (shared1_down_wait), which waits on the former's tagged words.  Producers
// come first in the grid and never wait, so every wait can end; each is
// bounded by ho.limit.  Same bits as the two-launch form.  H % 128 == 0.
template <bool TAIL>
__global__ __launch_bounds__(256) void shared1_onepass_kernel(Shared1Args sh, Handoff ho) {
  if ((int)blockIdx.x < ho.nprod) shared1_gate_up8(sh, ho, (int)blockIdx.x);
  else shared1_down_wait<TAIL>(sh, ho, (int)blockIdx.x - ho.nprod);
}

static size_t a256(size_t b) { return (b + 255) / 256 * 256; }

// one row with I <= 1024 takes the one-row path (one launch, or gate/up parts + down with the requant prologue)
static bool one_row_path(int T, int I) { return T == 1 && I <= KPART; }

// [h: T x 2I fp32][q: T x I][q_sc: T x I/32], then on the one-row path
// [parts: the gate/up parts (two launches) or the I handoff words (one)]
// [status word, 256 bytes]
size_t shared_ws_bytes(int T, int H, int I) {
  const size_t base = a256((size_t)T * 2 * I * 4) + a256((size_t)T * I) + a256((size_t)T * (I / 32));
  return base + (one_row_path(T, I) ? a256((size_t)((H + KPART - 1) / KPART) * 2 * I * 4) + 256 : 0);
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
        cap == hipStreamCaptureStatusNone) {
      uint32_t* status = reinterpret_cast<uint32_t*>(base + shared_ws_bytes(1, H, I) - 256);
      const Handoff ho{reinterpret_cast<uint64_t*>(sh.pbuf), status, next_call_tag(), handoff_limit_ticks(), I / 8};
      const dim3 grid(I / 8 + H / 16);
      if (I % KSTEP) hipLaunchKernelGGL(shared1_onepass_kernel<true>, grid, dim3(256), 0, stream, sh, ho);
      else hipLaunchKernelGGL(shared1_onepass_kernel<false>, grid, dim3(256), 0, stream, sh, ho);
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
