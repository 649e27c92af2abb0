// Dense block-32 FP8 GEMM, decode shapes: y[M][N] = a[M][K] . w[N][K]^T with
// E8M0 block scales on both operands ("New Deepseek 4.1 flash recipe" thread,
// post #2, "Known issues and next steps": dense FP8 GEMMs, the largest
// remaining decode lever; post #6, "How it works": MXFP8 projections, decode
// rows on small row tiles).
//
// One workgroup per 16 output columns.  Its four wavefronts take the
// canonical K parts (1024 each) and stream their slice of the 16 weight rows
// straight from HBM into registers (two 16-byte loads per lane per MFMA
// step, so every load instruction covers 64 contiguous bytes of 16 rows);
// the row tile of activations is re-read from L2 by every column tile.  The
// parts are added in part order through LDS, so an element's result does not
// depend on M.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mx {

__device__ __forceinline__ v8i fp8_pair(const u32x4& lo, const u32x4& hi) {
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <bool BF16_OUT>
__global__ __launch_bounds__(256) void gemm_decode_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ a_sc,
                                                          const uint8_t* __restrict__ w, const uint8_t* __restrict__ w_sc,
                                                          int M, int N, int K, void* __restrict__ y) {
  __shared__ float red[MAX_PARTS][16][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int nsteps = K / KSTEP, nparts = (nsteps + KPART_STEPS - 1) / KPART_STEPS;
  const int n0 = blockIdx.x * 16;
  const int64_t n = n0 + col;
  const uint8_t* wp = w + n * K;
  const uint32_t* wsp = reinterpret_cast<const uint32_t*>(w_sc + n * (K / 32));
  for (int rt = 0; rt * 16 < M; ++rt) {
    const int m_row = rt * 16 + col;
    const bool rv = m_row < M;
    const uint8_t* ap = a + (int64_t)(rv ? m_row : 0) * K;
    const uint32_t* asp = reinterpret_cast<const uint32_t*>(a_sc + (int64_t)(rv ? m_row : 0) * (K / 32));
    for (int q = wave; q < nparts; q += 4) {
      const int s0 = q * KPART_STEPS;
      u32x4 blo[KPART_STEPS], bhi[KPART_STEPS], alo[KPART_STEPS], ahi[KPART_STEPS];
      uint32_t bs[KPART_STEPS], as[KPART_STEPS];
      // weights then activations: every load of the part is in flight before
      // any is used; scale dwords stay raw until the MFMA
      if (s0 + KPART_STEPS <= nsteps) {
#pragma unroll
        for (int m = 0; m < KPART_STEPS; ++m) {
          const int s = s0 + m;
          blo[m] = ldg16(wp + s * KSTEP + g * 16);
          bhi[m] = ldg16(wp + s * KSTEP + 64 + g * 16);
          bs[m] = wsp[s];
        }
#pragma unroll
        for (int m = 0; m < KPART_STEPS; ++m) {
          const int s = s0 + m;
          const u32x4 z = {0u, 0u, 0u, 0u};
          alo[m] = rv ? ldg16(ap + s * KSTEP + g * 16) : z;
          ahi[m] = rv ? ldg16(ap + s * KSTEP + 64 + g * 16) : z;
          as[m] = rv ? asp[s] : bs[m];
        }
      } else {
#pragma unroll
        for (int m = 0; m < KPART_STEPS; ++m) {
          const int s = s0 + m;
          if (s < nsteps) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            blo[m] = ldg16(wp + s * KSTEP + g * 16);
            bhi[m] = ldg16(wp + s * KSTEP + 64 + g * 16);
            bs[m] = wsp[s];
            alo[m] = rv ? ldg16(ap + s * KSTEP + g * 16) : z;
            ahi[m] = rv ? ldg16(ap + s * KSTEP + 64 + g * 16) : z;
            as[m] = rv ? asp[s] : bs[m];
          }
        }
      }
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < KPART_STEPS; ++m)
        if (s0 + m < nsteps)
          acc = mfma_fp8_fp8(fp8_pair(alo[m], ahi[m]), fp8_pair(blo[m], bhi[m]), acc, as[m] >> (8 * g), bs[m] >> (8 * g));
#pragma unroll
      for (int i = 0; i < 4; ++i) red[q][4 * g + i][col] = acc[i];
    }
    __syncthreads();
    {
      const int row = threadIdx.x >> 4, c = threadIdx.x & 15;
      float v = red[0][row][c];
      for (int q = 1; q < nparts; ++q) v = v + red[q][row][c];
      const int mr = rt * 16 + row;
      if (mr < M) {
        if (BF16_OUT) static_cast<uint16_t*>(y)[(int64_t)mr * N + n0 + c] = f32_to_bf16_rne(v);
        else static_cast<float*>(y)[(int64_t)mr * N + n0 + c] = v;
      }
    }
    __syncthreads();
  }
}

hipError_t launch_block_gemm(const uint8_t* a, const uint8_t* a_sc, const uint8_t* w, const uint8_t* w_sc,
                             int M, int N, int K, void* y, bool bf16_out, hipStream_t stream, const char** variant) {
  const dim3 grid(N / 16), block(256);
  if (bf16_out) hipLaunchKernelGGL(gemm_decode_kernel<true>, grid, block, 0, stream, a, a_sc, w, w_sc, M, N, K, y);
  else hipLaunchKernelGGL(gemm_decode_kernel<false>, grid, block, 0, stream, a, a_sc, w, w_sc, M, N, K, y);
  *variant = bf16_out ? "gemm:decode16_kpart4_bf16" : "gemm:decode16_kpart4_f32";
  return hipGetLastError();
}

}  // namespace mx
