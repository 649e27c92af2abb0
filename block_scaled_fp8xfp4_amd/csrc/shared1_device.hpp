// The shared expert on one row (T = 1) as two tile functions, used by its
// own two kernels and by the fused single-row layer, whose two launches carry
// these tiles beside the routed experts' ("New Deepseek 4.1 flash recipe"
// thread, post #6, "Kernel by kernel against B12X": the shared expert runs
// beside the routed experts on a side stream; TP4 README, settings table,
// row "Kernels").  Both keep the dense projection's canonical order: gate/up
// as K parts of 1024 chained from zero and added in part order, the down
// projection (K = I <= 1024) as one chain.
#pragma once
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mx {

__device__ __forceinline__ v8i fp8_pair(const u32x4& lo, const u32x4& hi) {
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// K tail (TAIL: K % 128 != 0, e.g. the shared expert's K = 576): the last
// step's 16-byte chunks past K are zero in registers and its scale blocks
// past K are 127 (1.0), on both operands, in every kernel; scale rows are
// then not dword-aligned and are read a byte at a time.
template <bool TAIL>
__device__ __forceinline__ u32x4 ld_chunk(const uint8_t* p, int kpos, int K) {   // p: 16 bytes at K position kpos
  if (TAIL && kpos >= K) return u32x4{0u, 0u, 0u, 0u};
  return ldg16(p);
}
// lane group g's scale of step s, in byte g (the MFMA is passed dword >> 8 g)
template <bool TAIL>
__device__ __forceinline__ uint32_t ld_scale(const uint8_t* row_sc, int s, int g, int nblk) {
  if (!TAIL) return reinterpret_cast<const uint32_t*>(row_sc)[s];
  const int b = 4 * s + g;
  return (uint32_t)(b < nblk ? row_sc[b] : 127) << (8 * g);
}

__host__ __device__ inline int shared1_nparts(int H) { return (H + KPART - 1) / KPART; }

// Gate/up part q of W13 rows [16 cb, 16 cb + 16): one wavefront (threads
// 0..63 of the caller), the part's chain from zero written to pbuf[q][2I].
// (The decode GEMM would run 4 wavefronts per 16 columns on 2I / 16 CUs;
// parts spread the row's gate/up weights over every CU.)
template <bool TAIL>
__device__ __forceinline__ void shared1_part(const Shared1Args& sh, int cb, int q) {
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  const int K = sh.H, N = 2 * sh.I;
  const int s0 = q * KPART_STEPS;
  const int nsteps = (K + KSTEP - 1) / KSTEP, nblk = K / 32;
  const int64_t n = (int64_t)cb * 16 + col;
  const uint8_t* ap = sh.x + g * 16;
  const uint8_t* wp = sh.w13 + n * K + g * 16;
  const uint8_t* wsp = sh.w13_sc + n * (K / 32);
  u32x4 alo[KPART_STEPS], ahi[KPART_STEPS], blo[KPART_STEPS], bhi[KPART_STEPS];
  uint32_t as[KPART_STEPS], bs[KPART_STEPS];
#pragma unroll
  for (int m = 0; m < KPART_STEPS; ++m) {                       // the row first, then the weights
    const int s = min(s0 + m, nsteps - 1);
    alo[m] = ld_chunk<TAIL>(ap + s * KSTEP, s * KSTEP + 16 * g, K);
    ahi[m] = ld_chunk<TAIL>(ap + s * KSTEP + 64, s * KSTEP + 64 + 16 * g, K);
    as[m] = ld_scale<TAIL>(sh.x_sc, s, g, nblk);
  }
#pragma unroll
  for (int m = 0; m < KPART_STEPS; ++m) {
    const int s = min(s0 + m, nsteps - 1);
    blo[m] = ld_chunk<TAIL>(wp + s * KSTEP, s * KSTEP + 16 * g, K);
    bhi[m] = ld_chunk<TAIL>(wp + s * KSTEP + 64, s * KSTEP + 64 + 16 * g, K);
    bs[m] = ld_scale<TAIL>(wsp, s, g, nblk);
  }
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < KPART_STEPS; ++m)
    if (s0 + m < nsteps)
      acc = mfma_fp8_fp8(fp8_pair(alo[m], ahi[m]), fp8_pair(blo[m], bhi[m]), acc, as[m] >> (8 * g), bs[m] >> (8 * g));
  if (g == 0) sh.pbuf[(int64_t)q * N + n] = acc[0];             // output row 0 (every A row is the row)
}

// Down projection of output columns [16 tile, 16 tile + 16) with the SwiGLU
// and the requant in its prologue, by 256 threads: h = the gate/up parts
// added in part order (left to right, fp32), a = swiglu(gate, up), block-32
// E4M3 requant (the routed experts' routine) into LDS; then the 16 columns as
// the decode GEMM computes them (K = I in one part: a chain from zero over
// the steps; past K zero elements and unit scales on both operands).  Tile 0
// also writes h, q and q_sc to the workspace.  I <= 1024.
template <bool TAIL>
__device__ __forceinline__ void shared1_down(const Shared1Args& sh, int tile) {
  constexpr int NSD = KPART_STEPS;                              // steps of K = I <= 1024
  __shared__ __attribute__((aligned(16))) float hs[2 * NSD * KSTEP];
  __shared__ __attribute__((aligned(16))) uint8_t q1[NSD * KSTEP];
  __shared__ uint8_t s1[NSD * 4];
  const int I = sh.I, nparts = shared1_nparts(sh.H);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int nsteps = (I + KSTEP - 1) / KSTEP, nblk = I / 32;
  const int64_t n = (int64_t)tile * 16 + col;
  // wavefront 0: the 16 W2 rows, requested first
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
  // h = ((p0 + p1) + p2) + ... per column, 4 columns per thread
  const int c4n = 2 * I / 4;
  for (int c4 = tid; c4 < c4n; c4 += 256) {
    v4f v = *reinterpret_cast<const v4f*>(sh.pbuf + 4 * c4);
    for (int q = 1; q < nparts; ++q) {
      const v4f p = *reinterpret_cast<const v4f*>(sh.pbuf + (int64_t)q * 2 * I + 4 * c4);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = v[i] + p[i];
    }
    *reinterpret_cast<v4f*>(&hs[4 * c4]) = v;
    if (tile == 0) *reinterpret_cast<v4f*>(sh.h + 4 * c4) = v;
  }
  for (int idx = tid; idx < NSD * KSTEP - I; idx += 256) q1[I + idx] = 0;   // K past I: zero elements
  for (int idx = tid; idx < NSD * 4 - nblk; idx += 256) s1[nblk + idx] = 127;   // and unit scales
  lds_barrier();
  // SwiGLU + requant: 16 lanes per block of 32, columns c and c + 16
  for (int b0 = 0; b0 < nblk; b0 += 16) {
    const int b = b0 + (tid >> 4), c = tid & 15;
    const bool ok = b < nblk;
    const int cb = ok ? b * 32 : 0;
    uint32_t sc;
    const uint32_t d = swiglu_requant2(hs[cb + c], hs[I + cb + c], hs[cb + 16 + c], hs[I + cb + 16 + c], &sc);
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

}  // namespace mx
