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
#include "shared1_device.hpp"

namespace mx {

constexpr int XCDS_GEMM = 8;                      // XCDs of an MI355X (block scheduling)

template <bool BF16_OUT, bool WHOLE, bool TAIL>                 // WHOLE: K = 4 parts of 1024 exactly
__global__ __launch_bounds__(256) void gemm_decode_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ a_sc,
                                                          const uint8_t* __restrict__ w, const uint8_t* __restrict__ w_sc,
                                                          int M, int N, int K, void* __restrict__ y) {
  __shared__ float red[MAX_PARTS][16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int nsteps = WHOLE ? 4 * KPART_STEPS : (K + KSTEP - 1) / KSTEP;
  const int nblk = K / 32;
  const int nparts = (nsteps + KPART_STEPS - 1) / KPART_STEPS;
  const int Kb = WHOLE ? 4 * KPART : K;
  const int n0 = blockIdx.x * 16;
  const int64_t n = n0 + col;
  const uint8_t* wp = w + n * Kb + g * 16;
  const uint8_t* wsp = w_sc + n * (Kb / 32);
  u32x4 blo[KPART_STEPS], bhi[KPART_STEPS];
  uint32_t bs[KPART_STEPS];
  auto load_w = [&](int s0) {
#pragma unroll
    for (int m = 0; m < KPART_STEPS; ++m) {
      const int s = WHOLE ? s0 + m : min(s0 + m, nsteps - 1);
      blo[m] = ld_chunk<TAIL>(wp + s * KSTEP, s * KSTEP + 16 * g, K);
      bhi[m] = ld_chunk<TAIL>(wp + s * KSTEP + 64, s * KSTEP + 64 + 16 * g, K);
      bs[m] = ld_scale<TAIL>(wsp, s, g, nblk);
    }
  };
  // the activations of row tile rt for part q
  struct ATile { u32x4 lo[KPART_STEPS], hi[KPART_STEPS]; uint32_t s[KPART_STEPS]; };
  auto load_a = [&](int rt, int q, ATile& A) {
    const int s0 = q * KPART_STEPS;
    const int m_row = min(rt * 16 + col, M - 1);               // rows past M repeat row M - 1
    const uint8_t* ap = a + (int64_t)m_row * Kb + g * 16;
    const uint8_t* asp = a_sc + (int64_t)m_row * (Kb / 32);
#pragma unroll
    for (int m = 0; m < KPART_STEPS; ++m) {
      const int s = WHOLE ? s0 + m : min(s0 + m, nsteps - 1);
      A.lo[m] = ld_chunk<TAIL>(ap + s * KSTEP, s * KSTEP + 16 * g, K);
      A.hi[m] = ld_chunk<TAIL>(ap + s * KSTEP + 64, s * KSTEP + 64 + 16 * g, K);
      A.s[m] = ld_scale<TAIL>(asp, s, g, nblk);
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

// Dense block-32 FP8 GEMM, prefill shapes (many rows): 128 x 128 output
// tiles, two 4-wavefront workgroups per CU, each wavefront 64 x 64.  Per
// MFMA step (K = 128) the tile's activation rows (16 KB), weight rows (16 KB)
// and their scale dwords go global -> LDS by LDS DMA into one of two
// XOR-swizzled buffers, one step ahead of the matrix cores, ordered by
// explicit vmcnt waits and LDS-only barriers.  The canonical order is kept:
// each part of 8 steps is a chain from zero, added to the running total in
// part order, so every element equals the decode kernel's bit for bit.
// Tiles are handed out in 8 x 8 blocks, one block per XCD per round, so that a
// block's 8 activation panels and 8 weight panels are shared in that XCD's
// L2 while its 64 workgroups move through K together.
constexpr int GP_BM = 128, GP_BN = 128;
__device__ __forceinline__ int gp_phys(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }   // 16-byte chunk
struct GpStage {
  u32x4 a[GP_BM * 8];                             // [row][8 chunks] swizzled
  u32x4 b[GP_BN * 8];
  uint32_t as[GP_BM];                             // the step's 4 scale bytes per row
  uint32_t bs[GP_BN];
};

template <bool BF16_OUT, bool TAIL>
__global__ __launch_bounds__(256, 2) void gemm_prefill_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ a_sc,
                                                              const uint8_t* __restrict__ w, const uint8_t* __restrict__ w_sc,
                                                              int M, int N, int K, void* __restrict__ y) {
  __shared__ GpStage st[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int nsteps = (K + KSTEP - 1) / KSTEP;
  const int nblk = K / 32;
  const int nrt = (M + GP_BM - 1) / GP_BM, nct = (N + GP_BN - 1) / GP_BN;
  const int nsbr = (nrt + 7) / 8, nsbc = (nct + 7) / 8;
  const uint32_t st_lds = __builtin_amdgcn_readfirstlane(lds_addr(&st[0]));
  const int per_xcd = gridDim.x / XCDS_GEMM;                    // workgroups per XCD (<= 64)
  const int x = blockIdx.x % XCDS_GEMM, j = blockIdx.x / XCDS_GEMM;
  const int al0 = gp_phys(col, g), al1 = gp_phys(col, 4 + g);

  for (int sb = x; sb < nsbr * nsbc; sb += XCDS_GEMM) {
    for (int tj = j; tj < 64; tj += per_xcd) {
      const int rt = (sb / nsbc) * 8 + tj / 8, ct = (sb % nsbc) * 8 + tj % 8;
      if (rt >= nrt || ct >= nct) continue;                     // workgroup-uniform
      const int m0 = rt * GP_BM, n0 = ct * GP_BN;
      lds_barrier();                                            // the previous tile's LDS reads are done
      // this thread's slots: rows past M / N repeat the last row (results discarded)
      uint32_t aoff[4], boff[4];
      int cpos[4];                                              // K position of each slot's chunk within a step
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int p = q * 256 + tid;
        const int r = p >> 3, c = (p & 7) ^ ((r >> 1) & 7);
        aoff[q] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)K + c * 16;
        boff[q] = (uint32_t)min(n0 + r, N - 1) * (uint32_t)K + c * 16;
        cpos[q] = c * 16;
      }
      const int sr = (wave & 1) * 64 + lane;                    // scale row of this lane: waves 0-1 A, 2-3 B
      const uint32_t soff = (uint32_t)min((wave < 2 ? m0 : n0) + sr, (wave < 2 ? M : N) - 1) * (uint32_t)(K / 32);
      const uint8_t* srow = (wave < 2 ? a_sc : w_sc) + soff;    // TAIL: scale rows are read a byte at a time
      uint32_t sreg = 0;                                        // TAIL: the issued step's scale dword
      auto issue = [&](int s, int bf) {
        const uint32_t d = st_lds + bf * (uint32_t)sizeof(GpStage);
        if (!TAIL) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dma16_to_lds(a + s * KSTEP, aoff[q], d + (uint32_t)offsetof(GpStage, a) + (q * 256 + wave * 64) * 16);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dma16_to_lds(w + s * KSTEP, boff[q], d + (uint32_t)offsetof(GpStage, b) + (q * 256 + wave * 64) * 16);
          if (wave < 2) dma4_to_lds(a_sc + s * 4, soff, d + (uint32_t)offsetof(GpStage, as) + (wave & 1) * 256);
          else dma4_to_lds(w_sc + s * 4, soff, d + (uint32_t)offsetof(GpStage, bs) + (wave & 1) * 256);
        } else {
          // chunks past K read their row's first chunk (in bounds) and are
          // zeroed in LDS once they have landed
          const uint32_t k0 = (uint32_t)s * KSTEP;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bool in = (int)k0 + cpos[q] < K;
            dma16_to_lds(a, in ? aoff[q] + k0 : aoff[q] - cpos[q], d + (uint32_t)offsetof(GpStage, a) + (q * 256 + wave * 64) * 16);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bool in = (int)k0 + cpos[q] < K;
            dma16_to_lds(w, in ? boff[q] + k0 : boff[q] - cpos[q], d + (uint32_t)offsetof(GpStage, b) + (q * 256 + wave * 64) * 16);
          }
          uint32_t v = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int blk = 4 * s + b;
            v |= (uint32_t)(blk < nblk ? srow[blk] : 127) << (8 * b);
          }
          sreg = v;
        }
      };

      v4f tot[4][4], cur[4][4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) tot[m][n] = cur[m][n] = v4f{0.f, 0.f, 0.f, 0.f};
      auto compute = [&](const GpStage& S) {
        v8i bf[4];
        uint32_t bsv[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const int rb = wn * 64 + n * 16;
          bf[n] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
          const u32x4 lo = S.b[rb * 8 + al0], hi = S.b[rb * 8 + al1];
          bf[n] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          bsv[n] = S.bs[rb + col];
        }
        const int ra0 = wm * 64;
        u32x4 alo = S.a[ra0 * 8 + al0], ahi = S.a[ra0 * 8 + al1];
        uint32_t sa = S.as[ra0 + col];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = 0; n < 4; ++n) bsv[n] >>= 8 * g;
        sa >>= 8 * g;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          u32x4 nlo, nhi;
          uint32_t san = 0;
          if (m < 3) {
            const int ra = wm * 64 + (m + 1) * 16;
            nlo = S.a[ra * 8 + al0];
            nhi = S.a[ra * 8 + al1];
            san = S.as[ra + col];
          }
          __builtin_amdgcn_sched_barrier(0);
          const v8i af = v8i{(int)alo[0], (int)alo[1], (int)alo[2], (int)alo[3], (int)ahi[0], (int)ahi[1], (int)ahi[2], (int)ahi[3]};
#pragma unroll
          for (int n = 0; n < 4; ++n) cur[m][n] = mfma_fp8_fp8(af, bf[n], cur[m][n], sa, bsv[n]);
          __builtin_amdgcn_sched_barrier(0);
          if (m < 3) {
            alo = nlo;
            ahi = nhi;
            sa = san >> (8 * g);
          }
        }
      };
      // step s: wait for its DMA (the next step's stays in flight), make every
      // wavefront's part visible, refill the other buffer, multiply; at the
      // end of each part of 8 steps its chain joins the total
      issue(0, 0);
      for (int s = 0; s < nsteps; ++s) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (TAIL) {
          // this stage's scale dwords, and zeros in the chunks past K
          GpStage& S = st[s & 1];
          if (wave < 2) S.as[sr] = sreg;
          else S.bs[sr] = sreg;
          if (s == nsteps - 1) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (s * KSTEP + cpos[q] >= K) {
                S.a[q * 256 + tid] = u32x4{0u, 0u, 0u, 0u};
                S.b[q * 256 + tid] = u32x4{0u, 0u, 0u, 0u};
              }
          }
        }
        lds_barrier();
        if (s + 1 < nsteps) issue(s + 1, (s + 1) & 1);
        compute(st[s & 1]);
        if ((s + 1) % KPART_STEPS == 0 || s + 1 == nsteps) {
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int n = 0; n < 4; ++n) {
              tot[m][n] = s < KPART_STEPS ? cur[m][n] : tot[m][n] + cur[m][n];
              cur[m][n] = v4f{0.f, 0.f, 0.f, 0.f};
            }
        }
      }
      // results: lane holds column n0 + 64 wn + 16 n + col, rows m0 + 64 wm + 16 m + 4 g + i
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = m0 + wm * 64 + m * 16 + 4 * g + i;
          if (row < M) {
#pragma unroll
            for (int n = 0; n < 4; ++n) {
              const int c = n0 + wn * 64 + n * 16 + col;
              if (c < N) {
                if (BF16_OUT) static_cast<uint16_t*>(y)[(int64_t)row * N + c] = f32_to_bf16_rne(tot[m][n][i]);
                else static_cast<float*>(y)[(int64_t)row * N + c] = tot[m][n][i];
              }
            }
          }
        }
    }
  }
}

// ---------------------------------------------- shared expert, one row (T = 1)
// (the tile bodies are in shared1_device.hpp, shared with the fused
// single-row layer's kernels)
template <bool TAIL>
__global__ __launch_bounds__(64) void gemm1_parts_kernel(Shared1Args sh) {
  shared1_part<TAIL>(sh, blockIdx.x, blockIdx.y);
}

template <bool TAIL>
__global__ __launch_bounds__(256) void shared_down1_kernel(Shared1Args sh) {
  shared1_down<TAIL>(sh, blockIdx.x);
}

hipError_t launch_shared_down1(const uint8_t* x, const uint8_t* x_sc, int H, const uint8_t* w13,
                               const uint8_t* w13_sc, const uint8_t* w2, const uint8_t* w2_sc, int I, float* y,
                               float* h, uint8_t* q, uint8_t* q_sc, float* pbuf, hipStream_t stream) {
  const Shared1Args sh{x, x_sc, w13, w13_sc, w2, w2_sc, H, I, pbuf, y, h, q, q_sc};
  const dim3 g1(2 * I / 16, shared1_nparts(H));
  if (H % KSTEP) hipLaunchKernelGGL(gemm1_parts_kernel<true>, g1, dim3(64), 0, stream, sh);
  else hipLaunchKernelGGL(gemm1_parts_kernel<false>, g1, dim3(64), 0, stream, sh);
  const dim3 g2(H / 16);
  if (I % KSTEP) hipLaunchKernelGGL(shared_down1_kernel<true>, g2, dim3(256), 0, stream, sh);
  else hipLaunchKernelGGL(shared_down1_kernel<false>, g2, dim3(256), 0, stream, sh);
  return hipGetLastError();
}

hipError_t launch_block_gemm(const uint8_t* a, const uint8_t* a_sc, const uint8_t* w, const uint8_t* w_sc,
                             int M, int N, int K, void* y, bool bf16_out, hipStream_t stream, const char** variant) {
  const bool tail = K % KSTEP != 0;
  if (M >= GEMM_PREFILL_MIN_M) {
    const int tiles = ((M + GP_BM - 1) / GP_BM) * ((N + GP_BN - 1) / GP_BN);
    const int per_xcd = tiles / XCDS_GEMM < 64 ? (tiles + XCDS_GEMM - 1) / XCDS_GEMM : 64;   // 2 per CU at most
    const dim3 gp(per_xcd * XCDS_GEMM);
#define MX_GP(B, T) hipLaunchKernelGGL((gemm_prefill_kernel<B, T>), gp, dim3(256), 0, stream, a, a_sc, w, w_sc, M, N, K, y)
    if (bf16_out) { if (tail) MX_GP(true, true); else MX_GP(true, false); }
    else { if (tail) MX_GP(false, true); else MX_GP(false, false); }
#undef MX_GP
    *variant = bf16_out ? (tail ? "gemm:prefill128x128_ktail_bf16" : "gemm:prefill128x128_bf16")
                        : (tail ? "gemm:prefill128x128_ktail_f32" : "gemm:prefill128x128_f32");
    return hipGetLastError();
  }
  const dim3 grid(N / 16), block(256);
  const bool whole = K == 4 * KPART;
#define MX_GD(B, W, T) hipLaunchKernelGGL((gemm_decode_kernel<B, W, T>), grid, block, 0, stream, a, a_sc, w, w_sc, M, N, K, y)
  if (bf16_out) {
    if (whole) MX_GD(true, true, false);
    else if (tail) MX_GD(true, false, true);
    else MX_GD(true, false, false);
  } else {
    if (whole) MX_GD(false, true, false);
    else if (tail) MX_GD(false, false, true);
    else MX_GD(false, false, false);
  }
#undef MX_GD
  *variant = bf16_out ? (tail ? "gemm:decode16_kpart4_ktail_bf16" : "gemm:decode16_kpart4_bf16")
                      : (tail ? "gemm:decode16_kpart4_ktail_f32" : "gemm:decode16_kpart4_f32");
  return hipGetLastError();
}

}  // namespace mx
