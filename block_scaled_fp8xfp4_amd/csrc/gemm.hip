// Dense block-32 FP8 GEMM, decode shapes: y[M][N] = a[M][K] . w[N][K]^T with
// E8M0 block scales on both operands ("New Deepseek 4.1 flash recipe" thread,
// post #2, "Known issues and next steps": dense FP8 GEMMs, the largest
// remaining decode lever; post #6, "How it works": MXFP8 projections, decode
// rows on small row tiles).
//
// One workgroup per 16 output columns.  Its four wavefronts take the
// canonical K parts (1024 each, part q by wavefront q mod 4) and stream their
// slice of the 16 weight rows straight from HBM into registers (two 16-byte
// loads per lane per MFMA step, so every load instruction covers 64
// contiguous bytes of 16 rows).  Every load is unconditional: lanes of rows
// past M read row M - 1 again and their results are discarded (rows of the
// product are independent), and a part past K reloads its last step without
// using it, so a wavefront's loads issue back to back.  The row tile's
// activations (re-read from L2 by every column tile) are requested before
// the weights.  The parts are added in part order through LDS, so an
// element's result does not depend on M.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mx {

__device__ __forceinline__ v8i fp8_pair(const u32x4& lo, const u32x4& hi) {
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <bool BF16_OUT, bool WHOLE>                            // WHOLE: K = 4 parts of 1024 exactly
__global__ __launch_bounds__(256) void gemm_decode_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ a_sc,
                                                          const uint8_t* __restrict__ w, const uint8_t* __restrict__ w_sc,
                                                          int M, int N, int K, void* __restrict__ y) {
  __shared__ float red[MAX_PARTS][16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int nsteps = WHOLE ? 4 * KPART_STEPS : K / KSTEP;
  const int nparts = (nsteps + KPART_STEPS - 1) / KPART_STEPS;
  const int Kb = WHOLE ? 4 * KPART : K;
  const int n0 = blockIdx.x * 16;
  const int64_t n = n0 + col;
  const uint8_t* wp = w + n * Kb + g * 16;
  const uint32_t* wsp = reinterpret_cast<const uint32_t*>(w_sc + n * (Kb / 32));
  u32x4 blo[KPART_STEPS], bhi[KPART_STEPS];
  uint32_t bs[KPART_STEPS];
  auto load_w = [&](int s0) {
#pragma unroll
    for (int m = 0; m < KPART_STEPS; ++m) {
      const int s = WHOLE ? s0 + m : min(s0 + m, nsteps - 1);
      blo[m] = ldg16(wp + s * KSTEP);
      bhi[m] = ldg16(wp + s * KSTEP + 64);
      bs[m] = wsp[s];
    }
  };
  // the activations of row tile rt for part q
  struct ATile { u32x4 lo[KPART_STEPS], hi[KPART_STEPS]; uint32_t s[KPART_STEPS]; };
  auto load_a = [&](int rt, int q, ATile& A) {
    const int s0 = q * KPART_STEPS;
    const int m_row = min(rt * 16 + col, M - 1);               // rows past M repeat row M - 1
    const uint8_t* ap = a + (int64_t)m_row * Kb + g * 16;
    const uint32_t* asp = reinterpret_cast<const uint32_t*>(a_sc + (int64_t)m_row * (Kb / 32));
#pragma unroll
    for (int m = 0; m < KPART_STEPS; ++m) {
      const int s = WHOLE ? s0 + m : min(s0 + m, nsteps - 1);
      A.lo[m] = ldg16(ap + s * KSTEP);
      A.hi[m] = ldg16(ap + s * KSTEP + 64);
      A.s[m] = asp[s];
    }
  };
  // row tile against part q, whose weights are in registers
  auto part = [&](const ATile& A, int q) {
    const int s0 = q * KPART_STEPS;
    __builtin_amdgcn_sched_barrier(0);                          // every load of the part issued before the first MFMA
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < KPART_STEPS; ++m)
      if (WHOLE || s0 + m < nsteps)
        acc = mfma_fp8_fp8(fp8_pair(A.lo[m], A.hi[m]), fp8_pair(blo[m], bhi[m]), acc, A.s[m] >> (8 * g), bs[m] >> (8 * g));
#pragma unroll
    for (int i = 0; i < 4; ++i) red[q][4 * g + i][col] = acc[i];
  };
  auto finish = [&](int rt) {
    lds_barrier();                                              // only LDS is shared; loads stay in flight
    const int row = threadIdx.x >> 4, c = threadIdx.x & 15;
    float v = red[0][row][c];
    for (int q = 1; q < nparts; ++q) v = v + red[q][row][c];
    const int mr = rt * 16 + row;
    if (mr < M) {
      if (BF16_OUT) static_cast<uint16_t*>(y)[(int64_t)mr * N + n0 + c] = f32_to_bf16_rne(v);
      else static_cast<float*>(y)[(int64_t)mr * N + n0 + c] = v;
    }
    lds_barrier();
  };
  if (WHOLE) {
    // one part per wavefront: its weights stay in registers for every row
    // tile; the first tile's activations are requested before them
    ATile A;
    load_a(0, wave, A);
    __builtin_amdgcn_sched_barrier(0);
    load_w(wave * KPART_STEPS);
    for (int rt = 0; rt * 16 < M; ++rt) {
      if (rt > 0) load_a(rt, wave, A);
      part(A, wave);
      finish(rt);
    }
  } else {
    for (int rt = 0; rt * 16 < M; ++rt) {
      for (int q = wave; q < nparts; q += 4) {
        ATile A;
        load_a(rt, q, A);
        load_w(q * KPART_STEPS);
        part(A, q);
      }
      finish(rt);
    }
  }
}

hipError_t launch_block_gemm(const uint8_t* a, const uint8_t* a_sc, const uint8_t* w, const uint8_t* w_sc,
                             int M, int N, int K, void* y, bool bf16_out, hipStream_t stream, const char** variant) {
  const dim3 grid(N / 16), block(256);
  const bool whole = K == 4 * KPART;
  if (bf16_out && whole) hipLaunchKernelGGL((gemm_decode_kernel<true, true>), grid, block, 0, stream, a, a_sc, w, w_sc, M, N, K, y);
  else if (bf16_out) hipLaunchKernelGGL((gemm_decode_kernel<true, false>), grid, block, 0, stream, a, a_sc, w, w_sc, M, N, K, y);
  else if (whole) hipLaunchKernelGGL((gemm_decode_kernel<false, true>), grid, block, 0, stream, a, a_sc, w, w_sc, M, N, K, y);
  else hipLaunchKernelGGL((gemm_decode_kernel<false, false>), grid, block, 0, stream, a, a_sc, w, w_sc, M, N, K, y);
  *variant = bf16_out ? "gemm:decode16_kpart4_bf16" : "gemm:decode16_kpart4_f32";
  return hipGetLastError();
}

}  // namespace mx
