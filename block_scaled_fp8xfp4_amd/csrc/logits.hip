// Router logits: logits[t][e] = hidden[t] . w_gate[e] with bf16 operands and
// fp32 results, the score the MoE top-k gate ranks ("New Deepseek 4.1 flash
// recipe" thread, post #6, "How it works": the MoE top-k gate; "Kernel by
// kernel against B12X": the router's time per decode step).
//
// Matrix-core step: gfx950 V_MFMA_F32_16X16X32_BF16, A 16 rows x 32 K,
// B 32 K x 16 columns, fp32 C/D.  Lane l serves row (A) / column (B) l % 16
// and holds the 8 bf16 values K = 8 (l / 16) + [0, 8) of the step; D as for
// every 16x16 MFMA (lane l: column l % 16, rows 4 (l / 16) + r).  A and B use
// the same placement, so which K a lane position carries never changes the
// product.
//
// Canonical order of an element (every path, every batch size): K is cut
// into steps of 32 and parts of LG_PART_STEPS steps (256; the last part may
// be shorter); each part is one MFMA chain started from zero, and the parts
// are added left to right in fp32: total = ((p0 + p1) + p2) + ...
//
// Three paths compute it:
//   * up to 16 rows: one workgroup per expert, its parts added in LDS;
//   * few rows: one workgroup per (16 experts, part), the part sums written
//     to a workspace and added in part order by a second kernel;
//   * many rows: 64 x 128 output tiles staged through LDS by LDS DMA, three
//     buffers of 128 K, two steps ahead of the matrix cores.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mx {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int LG_STEP = 32;                       // K per MFMA step
constexpr int LG_PART_STEPS = 8;                  // steps per part (K = 256)
constexpr int LG_PART = LG_STEP * LG_PART_STEPS;
constexpr int LG_MAX_PARTS = LG_MAX_H / LG_PART;
constexpr int LG_XCDS = 8;                        // XCDs of an MI355X (block scheduling)

__device__ __forceinline__ v4f mfma_bf16(const u32x4& a, const u32x4& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// ----------------------------------------------------------- one to 16 rows
// One workgroup per expert (matrix-core column c serves the expert for
// every c; the other 15 columns repeat it and are discarded), one wavefront
// per part (LG_ONE_WAVES of them, parts w, w + LG_ONE_WAVES, ...), the part
// sums added in part order through LDS: one launch, and each CU streams one
// 8 KB gate row plus the rows' activations.  Measured at T = 1: 4.6 us per
// launch against 2.7 + 4.1 us for the split-K kernel and its sum kernel.
constexpr int LG_ONE_WAVES = 16;
constexpr int LG_ONE_MAX_T = 16;

template <bool FULL>
__global__ __launch_bounds__(64 * LG_ONE_WAVES) void logits_one_kernel(const uint16_t* __restrict__ h,
                                                                        const uint16_t* __restrict__ wg, int T, int H,
                                                                        int E, float* __restrict__ logits) {
  __shared__ float red[LG_MAX_PARTS][16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int nsteps = H / LG_STEP;
  const int nparts = (nsteps + LG_PART_STEPS - 1) / LG_PART_STEPS;
  const int e = blockIdx.x;
  const uint16_t* wp = wg + (int64_t)e * H + g * 8;
  const uint16_t* ap = h + (int64_t)min(col, T - 1) * H + g * 8;   // rows past T repeat the last one
  for (int q = wave; q < nparts; q += LG_ONE_WAVES) {
    u32x4 a[LG_PART_STEPS], b[LG_PART_STEPS];
#pragma unroll
    for (int m = 0; m < LG_PART_STEPS; ++m) {                  // a short part repeats its last step (never multiplied)
      const int s = FULL ? q * LG_PART_STEPS + m : min(q * LG_PART_STEPS + m, nsteps - 1);
      a[m] = *reinterpret_cast<const u32x4*>(ap + s * LG_STEP);
    }
#pragma unroll
    for (int m = 0; m < LG_PART_STEPS; ++m) {
      const int s = FULL ? q * LG_PART_STEPS + m : min(q * LG_PART_STEPS + m, nsteps - 1);
      b[m] = *reinterpret_cast<const u32x4*>(wp + s * LG_STEP);
    }
    const int ns = FULL ? LG_PART_STEPS : min(LG_PART_STEPS, nsteps - q * LG_PART_STEPS);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < LG_PART_STEPS; ++m)
      if (FULL || m < ns) acc = mfma_bf16(a[m], b[m], acc);
    if (col == 0) {                                             // column 0: rows 4 g + i
#pragma unroll
      for (int i = 0; i < 4; ++i) red[q][4 * g + i] = acc[i];
    }
  }
  lds_barrier();
  if (threadIdx.x < T) {
    float v = red[0][threadIdx.x];
    for (int q = 1; q < nparts; ++q) v = v + red[q][threadIdx.x];
    logits[(int64_t)threadIdx.x * E + e] = v;
  }
}

// ---------------------------------------------------------------- few rows
// Split over K, so that few rows still spread the gate over every CU (one CU
// keeps only so many loads in flight: a 2 MB gate streamed by 16 CUs is
// latency-bound).  Workgroup (g, q): 16 experts g, part q; its four
// wavefronts take 16-row tiles in turn and write the part's chain results to
// the workspace as part_sums[q][t][e]; a second kernel adds the parts of
// every element left to right.  (Adding them in the last workgroup of each
// group to finish, after a device-scope release of the part sums, was
// measured 3-13x slower: every release writes back the XCD's L2.)  Rows past
// T and experts past E repeat the last one (their results are never stored).
// FULL: every part has 8 steps.
template <bool FULL>
__global__ __launch_bounds__(256) void logits_part_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ wg,
                                                          int T, int H, int E, float* __restrict__ part_sums) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int nsteps = H / LG_STEP;
  const int nparts = (nsteps + LG_PART_STEPS - 1) / LG_PART_STEPS;
  const int q = blockIdx.x % nparts, e0 = (blockIdx.x / nparts) * 16;
  const int ns = FULL ? LG_PART_STEPS : min(LG_PART_STEPS, nsteps - q * LG_PART_STEPS);
  const int e = e0 + col;
  // 8 steps of part q of one operand row; in a short part the slots past K
  // repeat its last step (never multiplied)
  auto load = [&](const uint16_t* p, u32x4* v) {
    p += g * 8;
    if (FULL) {
      p += q * LG_PART;
#pragma unroll
      for (int m = 0; m < LG_PART_STEPS; ++m) v[m] = *reinterpret_cast<const u32x4*>(p + m * LG_STEP);
    } else {
#pragma unroll
      for (int m = 0; m < LG_PART_STEPS; ++m)
        v[m] = *reinterpret_cast<const u32x4*>(p + min(q * LG_PART_STEPS + m, nsteps - 1) * LG_STEP);
    }
  };
  auto arow = [&](int rt) { return h + (int64_t)min(rt * 16 + col, T - 1) * H; };
  u32x4 b[LG_PART_STEPS], a[LG_PART_STEPS], an[LG_PART_STEPS];
  const int nrt = (T + 15) / 16;
  if (wave >= nrt) return;                                      // no barrier follows
  load(arow(wave), a);                                          // the first row tile before the weights
  __builtin_amdgcn_sched_barrier(0);
  load(wg + (int64_t)min(e, E - 1) * H, b);
  for (int rt = wave; rt < nrt; rt += 4) {
    if (rt + 4 < nrt) load(arow(rt + 4), an);                   // the next tile stays in flight
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < LG_PART_STEPS; ++m)
      if (FULL || m < ns) acc = mfma_bf16(a[m], b[m], acc);
    if (e < E) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = rt * 16 + 4 * g + i;
        if (t < T) part_sums[((int64_t)q * T + t) * E + e] = acc[i];
      }
    }
#pragma unroll
    for (int m = 0; m < LG_PART_STEPS; ++m) a[m] = an[m];
  }
}

// logits[t][e] = ((p0 + p1) + p2) + ... over the parts in the workspace
__global__ __launch_bounds__(256) void logits_sum_kernel(const float* __restrict__ part_sums, int nparts, int64_t n,
                                                         float* __restrict__ logits) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = part_sums[i];
  for (int q = 1; q < nparts; ++q) v = v + part_sums[q * n + i];
  logits[i] = v;
}

// --------------------------------------------------------------- many rows
// Workgroup tile: 64 rows x 128 experts, four wavefronts of 32 x 64 (2 x 4
// MFMA tiles).  One LDS stage holds 128 K (4 steps) of the tile's 64 hidden
// rows and 128 gate rows, 256 bytes per row in 16-byte chunks; chunk c of row
// r sits at position c ^ (r & 15), so the 16 rows a fragment read touches
// hit distinct banks.  Each thread moves 4 + 8 chunks per stage by LDS DMA;
// a stage is waited for with an explicit vmcnt (the next one stays in
// flight) and published by an LDS-only barrier.  Tiles go to XCDs in
// contiguous ranges, so a row tile's two expert halves share that XCD's L2.
// (measured: 2 workgroups per CU with 64-K stages, or 4-6 shallower stages,
// were all slower; the time per stage is set by the DMA rate per CU)
constexpr int LP_BM = 64, LP_BN = 128, LP_STAGE_K = 128, LP_STAGES = 3;
constexpr int LP_WGS = 1;                         // workgroups per CU
constexpr int LP_KSTEPS = LP_STAGE_K / LG_STEP;   // MFMA steps per stage
constexpr int LP_CHUNKS = LP_STAGE_K * 2 / 16;    // 16-byte chunks per row per stage
constexpr int LP_SWZ = LP_CHUNKS - 1;
constexpr int LP_A_DMA = LP_BM * LP_CHUNKS / 256, LP_B_DMA = LP_BN * LP_CHUNKS / 256;
struct LpStage {
  u32x4 a[LP_BM * LP_CHUNKS];
  u32x4 b[LP_BN * LP_CHUNKS];
};

// wait until at most n stages of LDS DMA (LP_A_DMA + LP_B_DMA operations
// each) are still in flight; loads complete in issue order
__device__ __forceinline__ void wait_stages(int n) {
  constexpr int D = LP_A_DMA + LP_B_DMA;
  static_assert(LP_STAGES - 2 <= 4 && 4 * D <= 63, "vmcnt range");
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(%0)" :: "n"(D) : "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * D) : "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(%0)" :: "n"(3 * D) : "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(%0)" :: "n"(4 * D) : "memory"); break;
  }
}

__global__ __launch_bounds__(256, LP_WGS) void logits_prefill_kernel(const uint16_t* __restrict__ h,
                                                                 const uint16_t* __restrict__ wg, int T, int H, int E,
                                                                 float* __restrict__ logits) {
  __shared__ LpStage st[LP_STAGES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int nsteps = H / LG_STEP;                               // MFMA steps
  const int nstages = (H + LP_STAGE_K - 1) / LP_STAGE_K;
  const int nrt = (T + LP_BM - 1) / LP_BM, nct = (E + LP_BN - 1) / LP_BN;
  const int tiles = nrt * nct;
  const int chunk = (tiles + LG_XCDS - 1) / LG_XCDS;            // tiles per XCD
  const int per_xcd = gridDim.x / LG_XCDS;
  const int x = blockIdx.x % LG_XCDS, j = blockIdx.x / LG_XCDS;
  const uint32_t st_lds = __builtin_amdgcn_readfirstlane(lds_addr(&st[0]));
  // fragment chunk positions of this lane for the steps of a stage (rows r with r % 16 == col)
  int fl[LP_KSTEPS];
#pragma unroll
  for (int m = 0; m < LP_KSTEPS; ++m) fl[m] = (4 * m + g) ^ (col & LP_SWZ);

  const int t_end = min((x + 1) * chunk, tiles);
  for (int tile = x * chunk + j; tile < t_end; tile += per_xcd) {
    const int rt = tile / nct, ct = tile % nct;
    const int m0 = rt * LP_BM, n0 = ct * LP_BN;
    lds_barrier();                                              // the previous tile's LDS reads are done
    // this thread's DMA slots.  In a stage that runs past H the chunks beyond
    // the row are never multiplied; they only have to stay inside the
    // matrix, so they are clamped to its last chunk.
    uint32_t aoff[LP_A_DMA], boff[LP_B_DMA];
#pragma unroll
    for (int q = 0; q < LP_A_DMA; ++q) {
      const int p = q * 256 + tid, r = p / LP_CHUNKS, c = (p % LP_CHUNKS) ^ (r & LP_SWZ);
      aoff[q] = ((uint32_t)min(m0 + r, T - 1) * (uint32_t)H + c * 8) * 2;
    }
#pragma unroll
    for (int q = 0; q < LP_B_DMA; ++q) {
      const int p = q * 256 + tid, r = p / LP_CHUNKS, c = (p % LP_CHUNKS) ^ (r & LP_SWZ);
      boff[q] = ((uint32_t)min(n0 + r, E - 1) * (uint32_t)H + c * 8) * 2;
    }
    const uint32_t a_last = (uint32_t)T * (uint32_t)H * 2 - 16, b_last = (uint32_t)E * (uint32_t)H * 2 - 16;
    auto issue = [&](int s, int bf) {
      const uint32_t d = st_lds + bf * (uint32_t)sizeof(LpStage);
      const uint32_t k0 = (uint32_t)s * LP_STAGE_K * 2;
      const bool tail = (s + 1) * LP_STAGE_K > H;               // uniform
#pragma unroll
      for (int q = 0; q < LP_A_DMA; ++q) {
        const uint32_t o = tail ? min(aoff[q] + k0, a_last) : aoff[q] + k0;
        dma16_to_lds(h, o, d + (uint32_t)offsetof(LpStage, a) + (q * 256 + wave * 64) * 16);
      }
#pragma unroll
      for (int q = 0; q < LP_B_DMA; ++q) {
        const uint32_t o = tail ? min(boff[q] + k0, b_last) : boff[q] + k0;
        dma16_to_lds(wg, o, d + (uint32_t)offsetof(LpStage, b) + (q * 256 + wave * 64) * 16);
      }
    };

    v4f tot[2][4], cur[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) tot[m][n] = cur[m][n] = v4f{0.f, 0.f, 0.f, 0.f};
    // MFMA steps [0, ns) of a stage: every fragment read is issued first, so
    // the reads of later steps overlap the matrix work of earlier ones
    auto stage = [&](const LpStage& S, int ns) {
      u32x4 af[LP_KSTEPS][2], bfr[LP_KSTEPS][4];
#pragma unroll
      for (int k = 0; k < LP_KSTEPS; ++k)
        if (k < ns) {
#pragma unroll
          for (int m = 0; m < 2; ++m) af[k][m] = S.a[(wm * 32 + m * 16 + col) * LP_CHUNKS + fl[k]];
#pragma unroll
          for (int n = 0; n < 4; ++n) bfr[k][n] = S.b[(wn * 64 + n * 16 + col) * LP_CHUNKS + fl[k]];
        }
#pragma unroll
      for (int k = 0; k < LP_KSTEPS; ++k)
        if (k < ns) {
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int n = 0; n < 4; ++n) cur[m][n] = mfma_bf16(af[k][m], bfr[k][n], cur[m][n]);
        }
    };
    // stages s + 1 .. s + LP_STAGES - 2 stay in flight while stage s is used
    for (int s = 0; s < LP_STAGES - 1 && s < nstages; ++s) issue(s, s);
    for (int s = 0; s < nstages; ++s) {
      const int ahead = min(nstages - 1 - s, LP_STAGES - 2);    // stages issued after s (uniform)
      wait_stages(ahead);
      lds_barrier();
      if (s + LP_STAGES - 1 < nstages) issue(s + LP_STAGES - 1, (s + LP_STAGES - 1) % LP_STAGES);
      const LpStage& S = st[s % LP_STAGES];
      const int k_steps = min(LP_KSTEPS, nsteps - s * LP_KSTEPS);   // uniform
      if (k_steps == LP_KSTEPS) stage(S, LP_KSTEPS);
      else stage(S, k_steps);
      const int done = s * LP_KSTEPS + k_steps;                 // steps finished so far
      if (done % LG_PART_STEPS == 0 || done == nsteps) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            tot[m][n] = done <= LG_PART_STEPS ? cur[m][n] : tot[m][n] + cur[m][n];
            cur[m][n] = v4f{0.f, 0.f, 0.f, 0.f};
          }
      }
    }
    // lane holds experts n0 + 64 wn + 16 n + col, rows m0 + 32 wm + 16 m + 4 g + i
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = m0 + wm * 32 + m * 16 + 4 * g + i;
        if (t < T) {
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            const int e = n0 + wn * 64 + n * 16 + col;
            if (e < E) logits[(int64_t)t * E + e] = tot[m][n][i];
          }
        }
      }
  }
}

size_t router_logits_ws_bytes(int T, int H, int E) {
  if (T <= LG_ONE_MAX_T || T >= LG_PREFILL_MIN_T) return 0;
  const int64_t nparts = (H / LG_STEP + LG_PART_STEPS - 1) / LG_PART_STEPS;
  return (size_t)(nparts * T * E * 4);
}

hipError_t launch_router_logits(const uint16_t* h, int T, int H, const uint16_t* wg, int E, float* logits, void* ws,
                                hipStream_t stream, const char** variant) {
  if (T >= LG_PREFILL_MIN_T) {
    const int tiles = ((T + LP_BM - 1) / LP_BM) * ((E + LP_BN - 1) / LP_BN);
    const int cap = num_cus() * LP_WGS;
    const int per_xcd = min((tiles + LG_XCDS - 1) / LG_XCDS, cap / LG_XCDS);
    hipLaunchKernelGGL(logits_prefill_kernel, dim3(per_xcd * LG_XCDS), dim3(256), 0, stream, h, wg, T, H, E, logits);
    *variant = "logits:prefill64x128";
    return hipGetLastError();
  }
  if (T <= LG_ONE_MAX_T) {
    if (H % LG_PART == 0)
      hipLaunchKernelGGL((logits_one_kernel<true>), dim3(E), dim3(64 * LG_ONE_WAVES), 0, stream, h, wg, T, H, E, logits);
    else
      hipLaunchKernelGGL((logits_one_kernel<false>), dim3(E), dim3(64 * LG_ONE_WAVES), 0, stream, h, wg, T, H, E, logits);
    *variant = "logits:one16_part256";
    return hipGetLastError();
  }
  const int nparts = (H / LG_STEP + LG_PART_STEPS - 1) / LG_PART_STEPS;
  float* part_sums = static_cast<float*>(ws);
  const dim3 grid(((E + 15) / 16) * nparts);
  if (H % LG_PART == 0)
    hipLaunchKernelGGL((logits_part_kernel<true>), grid, dim3(256), 0, stream, h, wg, T, H, E, part_sums);
  else
    hipLaunchKernelGGL((logits_part_kernel<false>), grid, dim3(256), 0, stream, h, wg, T, H, E, part_sums);
  const int64_t n = (int64_t)T * E;
  hipLaunchKernelGGL(logits_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, part_sums, nparts, n,
                     logits);
  *variant = "logits:splitk16_part256+sum";
  return hipGetLastError();
}

}  // namespace mx
