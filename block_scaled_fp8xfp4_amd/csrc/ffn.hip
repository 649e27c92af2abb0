// Routed-expert FFN kernels: gate/up GEMM, SwiGLU + FP8 requant, down GEMM
// and the fixed-order weighted combine ("New Deepseek 4.1 flash recipe"
// thread, post #6, "How it works": routed experts with FP8 activations x FP4
// weights, decode rows on small tiles, prefill on 64-row tiles; "Why
// TileLang": SwiGLU with per-block FP8 quantization, reductions in a fixed
// order; DeepSeek-V4.1-Flash-4x-DGX-Spark-TP4 README, settings table, row
// "Experts": per-slot buffer and a fixed-order sum instead of atomics, 64-row
// tiles for 576-wide experts at prefill sizes).
//
// Both paths evaluate every output element with the same MFMA chain (all K
// steps in order, see mx_device.hpp) and the same SwiGLU/requant routine, so
// they give the same bits; they differ only in how rows and weights reach the
// matrix cores.
//
// Decode path (few rows per expert, weight streaming):
//   gu_decode_kernel    one wavefront per (expert, 16 W13 rows): the whole K
//                       of its weight rows is loaded into registers at once;
//                       the expert's activation rows are staged in LDS, at
//                       most min(16, T) at a time; writes fp32 h = [gate |
//                       up] per bucket position.
//   down_decode_kernel  one workgroup per (expert, 64 W2 rows): W2 first,
//                       then SwiGLU + requant of the rows' h into LDS (8
//                       lanes per block of 32), then the down chain.
// Prefill path (hundreds of rows per expert, matrix-core bound):
//   gu_prefill_kernel   expert tile of up to 128 rows x 128 intermediate
//                       columns (256 W13 rows) per workgroup, 2 x 2
//                       wavefronts; gathered activation rows and weight rows
//                       staged through swizzled, double-buffered LDS one MFMA
//                       step at a time; SwiGLU + requant in the epilogue.
//   down_prefill_kernel 64-row tile x 256 W2 rows per workgroup; the tile's
//                       whole intermediate (K = I) sits in LDS.
//   Both run persistent grids whose blocks are remapped so that each XCD
//   walks a contiguous range of (expert, row tile, column tile) items and
//   shares weights and activations in its own L2.
// combine_kernel adds w_tj * o_tj over the slots in order j = 0..k-1.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mx {

constexpr int DEC_MAX_STEPS = 32;                 // decode gate/up: H <= 4096 held in registers
constexpr int DOWN_MAX_STEPS = MAX_I / KSTEP;     // 16
constexpr int PF_ROWS = 64;                       // prefill expert tile rows
constexpr int PF_ICOLS = 128;                     // prefill gate/up: intermediate columns per workgroup
constexpr int PF_KCH = 2;                         // prefill gate/up: MFMA steps per LDS stage
constexpr int PF_AROW = PF_KCH * KSTEP + 16;      // LDS row pitch of the staged activations (padded)
constexpr int PF_NCOLS = 256;                     // prefill down: W2 rows per workgroup
constexpr int PF_MAX_I = 640;                     // prefill down: intermediate held in LDS (5 steps)
constexpr int XCDS = 8;

// ---------------------------------------------------------------- work lists
__device__ __forceinline__ int wave_excl_scan(int v, int lane) {
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x - v;
}

// Wavefront 0 writes tile_start[e] (e = 0..E): the first tile index of each
// expert, where an expert with n live pairs owns ceil(n / rows) tiles
// (rows == 0: one tile per expert with any pair).  All offsets are read in
// one round of independent loads.
__device__ void build_tiles(const int32_t* __restrict__ offsets, int E, int rows, int* tile_start) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (E + 63) / 64;                  // <= MAX_E / 64 = 16
    int o[17];
#pragma unroll
    for (int i = 0; i < 17; ++i) {
      const int e = lane * per + i;
      o[i] = (i <= per && e <= E) ? offsets[e] : 0;
    }
    int cnt[16], local = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane * per + i;
      int n = (i < per && e < E) ? o[i + 1] - o[i] : 0;
      n = n < 0 ? 0 : n;
      cnt[i] = rows > 0 ? (n + rows - 1) / rows : (n > 0 ? 1 : 0);
      local += cnt[i];
    }
    int run = wave_excl_scan(local, lane);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane * per + i;
      if (i < per && e < E) tile_start[e] = run;
      run += cnt[i];
    }
    if (lane == 63) tile_start[E] = run;
  }
  __syncthreads();
}

// The expert that owns tile `tile` (tile_start non-decreasing, tile < tile_start[E]).
__device__ __forceinline__ int tile_expert(const int* tile_start, int E, int tile) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_start[mid] <= tile) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Logical item of a persistent block in a round: each XCD (blocks b with the
// same b % 8) takes a contiguous range of items.  G is a multiple of 8.
__device__ __forceinline__ int xcd_item(int round, int b, int G) {
  const int per = G / XCDS;
  return round * G + (b % XCDS) * per + b / XCDS;
}

__device__ __forceinline__ v8i fp8_operand(const u32x4& lo, const u32x4& hi) {
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
__device__ __forceinline__ v8i fp4_operand(const u32x4& b) {
  return v8i{(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
}

// =========================================================== decode path ==
// Gate/up: one wavefront per (expert, 16 W13 rows).  It first issues the
// loads of the whole K of its 16 weight rows (registers), then stages the
// expert's activation rows, at most R = min(16, T) at a time, in its own LDS
// (dynamic, R * (H + 16) + R * H / 32 bytes) and runs the chain.
__global__ __launch_bounds__(64) void gu_decode_kernel(FfnArgs a, float* __restrict__ h, int Tk, int R) {
  __shared__ int tile_start[MAX_E + 1];
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
  build_tiles(a.offsets, a.E, 0, tile_start);
  const int lane = threadIdx.x, col = lane & 15, g = lane >> 4;
  const int H = a.H, twoI = 2 * a.I;
  const int nsteps = H / KSTEP;
  const int pitch = H + 16;
  uint8_t* xlds = dyn_lds;                                      // [R][H + 16]
  uint32_t* xslds = reinterpret_cast<uint32_t*>(dyn_lds + (size_t)R * pitch);   // [R][nsteps]
  const int ntiles = twoI / 16;
  const int nitems = tile_start[a.E] * ntiles;
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int e = tile_expert(tile_start, a.E, item / ntiles), nt = item % ntiles;
    const int p0 = a.offsets[e];
    int cnt = a.offsets[e + 1] - p0;
    if (p0 < 0 || p0 + cnt > Tk) cnt = 0;                       // malformed route: skip
    const int64_t wrow = (int64_t)e * twoI + nt * 16 + col;     // B column of this lane
    const uint8_t* wp = a.w13 + wrow * (H / 2);
    const uint32_t* wsp = reinterpret_cast<const uint32_t*>(a.w13_sc + wrow * (H / 32));
    // every weight load of the 16 rows is issued before anything waits on one;
    // scale dwords stay raw (the lane's byte is picked at the MFMA)
    u32x4 bw[DEC_MAX_STEPS];
    uint32_t bsr[DEC_MAX_STEPS];
#pragma unroll
    for (int c = 0; c < DEC_MAX_STEPS / 8; ++c) {
      if (c * 8 + 8 <= nsteps) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          bw[c * 8 + m] = ldg16(wp + (c * 8 + m) * 64 + g * 16);
          bsr[c * 8 + m] = wsp[c * 8 + m];
        }
      } else if (c * 8 < nsteps) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
          if (c * 8 + m < nsteps) {
            bw[c * 8 + m] = ldg16(wp + (c * 8 + m) * 64 + g * 16);
            bsr[c * 8 + m] = wsp[c * 8 + m];
          }
      }
    }
    for (int r0 = 0; r0 < cnt; r0 += R) {
      const int nrows = min(R, cnt - r0);
      // token of staged row `lane` (lanes < nrows), read once
      int my_tok = -1;
      if (lane < nrows) {
        const int pr = a.perm[p0 + r0 + lane];
        my_tok = (pr >= 0 && pr < Tk) ? pr / a.k : -1;
      }
      lds_barrier();                                            // previous rows' LDS reads are done
      for (int r = 0; r < nrows; ++r) {
        const int tok = __shfl(my_tok, r);
        const uint8_t* src = a.x + (int64_t)(tok < 0 ? 0 : tok) * H;
        uint8_t* dst = xlds + (size_t)r * pitch;
        const u32x4 z = {0u, 0u, 0u, 0u};
        u32x4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int off = (j * 64 + lane) * 16;
          v[j] = (tok >= 0 && off < H) ? ldg16(src + off) : z;
        }
        const int sidx = lane;
        const uint32_t sv = (tok >= 0 && sidx < nsteps)
                                ? reinterpret_cast<const uint32_t*>(a.x_sc + (int64_t)tok * (H / 32))[sidx]
                                : 0x7F7F7F7Fu;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int off = (j * 64 + lane) * 16;
          if (off < H) *reinterpret_cast<u32x4*>(dst + off) = v[j];
        }
        if (sidx < nsteps) xslds[r * nsteps + sidx] = sv;
      }
      lds_barrier();
      for (int rt = 0; rt < nrows; rt += 16) {
        const int rr = rt + col;                                // staged row of this lane
        const bool rv = rr < nrows;
        const uint8_t* arow = xlds + (size_t)(rv ? rr : 0) * pitch;
        const uint32_t* asrow = xslds + (rv ? rr : 0) * nsteps;
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DEC_MAX_STEPS; ++s) {
          if (s < nsteps) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            const u32x4 alo = rv ? *reinterpret_cast<const u32x4*>(arow + s * KSTEP + g * 16) : z;
            const u32x4 ahi = rv ? *reinterpret_cast<const u32x4*>(arow + s * KSTEP + 64 + g * 16) : z;
            const uint32_t sb = bsr[s] >> (8 * g);
            const uint32_t sa = rv ? (asrow[s] >> (8 * g)) : sb;
            acc = mfma_fp8_fp4(fp8_operand(alo, ahi), fp4_operand(bw[s]), acc, sa, sb);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rt + 4 * g + i;
          if (row < nrows) h[(int64_t)(p0 + r0 + row) * twoI + nt * 16 + col] = acc[i];
        }
      }
    }
  }
}

// SwiGLU + requant of pair rows [p0, p0 + n) (n <= 16) from h into LDS, and
// into the workspace when `publish`.  Block-wide; 8 consecutive lanes share
// a block of 32 intermediate values (4 each), the block maximum is a
// butterfly over those 8 lanes.
__device__ void stage_intermediate(const float* __restrict__ h, int p0, int n, int I, uint8_t (*qlds)[MAX_I + 16],
                                   uint8_t (*slds)[MAX_I / 32], uint8_t* __restrict__ qws, uint8_t* __restrict__ qsc_ws,
                                   bool publish) {
  const int q4 = I / 4, nb = I / 32;
  const int total = 16 * q4;                                     // multiple of 128
  for (int base = 0; base < total; base += blockDim.x) {
    const int idx = base + (int)threadIdx.x;
    const int r = idx / q4, c4 = idx % q4;
    const bool in = idx < total && r < n;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (in) {
      const float* hp = h + (int64_t)(p0 + r) * 2 * I + 4 * c4;
      const float4 gg = *reinterpret_cast<const float4*>(hp);
      const float4 uu = *reinterpret_cast<const float4*>(hp + I);
      v[0] = swiglu(gg.x, uu.x);
      v[1] = swiglu(gg.y, uu.y);
      v[2] = swiglu(gg.z, uu.z);
      v[3] = swiglu(gg.w, uu.w);
    }
    float m = fmaxf(fmaxf(__builtin_fabsf(v[0]), __builtin_fabsf(v[1])), fmaxf(__builtin_fabsf(v[2]), __builtin_fabsf(v[3])));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    if (in) {
      const uint32_t sc = e8m0_code_for_amax(m, 8);
      const uint32_t d = requant_e4m3(v[0], sc) | (requant_e4m3(v[1], sc) << 8) | (requant_e4m3(v[2], sc) << 16) |
                         (requant_e4m3(v[3], sc) << 24);
      *reinterpret_cast<uint32_t*>(&qlds[r][4 * c4]) = d;
      if ((c4 & 7) == 0) slds[r][c4 >> 3] = (uint8_t)sc;
      if (publish) {
        *reinterpret_cast<uint32_t*>(qws + (int64_t)(p0 + r) * I + 4 * c4) = d;
        if ((c4 & 7) == 0) qsc_ws[(int64_t)(p0 + r) * nb + (c4 >> 3)] = (uint8_t)sc;
      }
    }
  }
}

__global__ __launch_bounds__(256) void down_decode_kernel(FfnArgs a, const float* __restrict__ h,
                                                          uint8_t* __restrict__ qws, uint8_t* __restrict__ qsc_ws,
                                                          float* __restrict__ o, int Tk) {
  __shared__ int tile_start[MAX_E + 1];
  __shared__ __attribute__((aligned(16))) uint8_t qlds[16][MAX_I + 16];   // padded rows: fewer bank conflicts
  __shared__ uint8_t slds[16][MAX_I / 32];
  build_tiles(a.offsets, a.E, 0, tile_start);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int H = a.H, I = a.I, nb = I / 32;
  const int nsteps = (I + KSTEP - 1) / KSTEP;
  const int ntiles = H / 64;
  const int nitems = tile_start[a.E] * ntiles;

  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int e = tile_expert(tile_start, a.E, item / ntiles), tile = item % ntiles;
    const int p0 = a.offsets[e];
    int cnt = a.offsets[e + 1] - p0;
    if (p0 < 0 || p0 + cnt > Tk) cnt = 0;
    const int n = tile * 64 + wave * 16 + col;                  // W2 row = output column of this lane
    const uint8_t* wp = a.w2 + ((int64_t)e * H + n) * (I / 2);
    const uint8_t* wsp = a.w2_sc + ((int64_t)e * H + n) * nb;
    u32x4 bw[DOWN_MAX_STEPS];
    uint32_t bs[DOWN_MAX_STEPS];
#pragma unroll
    for (int s = 0; s < DOWN_MAX_STEPS; ++s) {
      if (s < nsteps) {
        const bool bv = 4 * s + g < nb;
        const u32x4 z = {0u, 0u, 0u, 0u};
        bw[s] = bv ? ldg16(wp + s * 64 + g * 16) : z;
        bs[s] = wsp[bv ? 4 * s + g : 0];
      }
    }
    for (int rt = 0; rt * 16 < cnt; ++rt) {
      const int nrows = min(16, cnt - rt * 16);
      stage_intermediate(h, p0 + rt * 16, nrows, I, qlds, slds, qws, qsc_ws, tile == 0);
      lds_barrier();
      const bool rv = col < nrows;
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DOWN_MAX_STEPS; ++s) {
        if (s < nsteps) {
          const int klo = s * KSTEP + g * 16, khi = klo + 64;
          const u32x4 z = {0u, 0u, 0u, 0u};
          const u32x4 alo = (rv && klo < I) ? *reinterpret_cast<const u32x4*>(&qlds[col][klo]) : z;
          const u32x4 ahi = (rv && khi < I) ? *reinterpret_cast<const u32x4*>(&qlds[col][khi]) : z;
          const uint32_t sa = (rv && 4 * s + g < nb) ? (uint32_t)slds[col][4 * s + g] : bs[s];
          acc = mfma_fp8_fp4(fp8_operand(alo, ahi), fp4_operand(bw[s]), acc, sa, bs[s]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * g + i;
        if (row < nrows) o[(int64_t)(p0 + rt * 16 + row) * H + n] = acc[i];
      }
      lds_barrier();
    }
  }
}

// ========================================================== prefill path ==
// Gate/up over an expert tile of up to 128 rows and 128 intermediate columns
// (256 W13 rows: the 128 gate rows, then the 128 up rows).  Wavefront (wm,
// wn) computes rows [64 wm, 64 wm + 64) x intermediate columns [64 wn, 64 wn
// + 64): four 16-row A tiles against eight 16-row B tiles (4 gate + 4 up).
// One MFMA step (K = 128) per stage: the gathered activation rows (16 KB),
// the weight rows (16 KB) and their scale dwords go global -> registers ->
// LDS, double-buffered, the next stage's loads in flight during the MFMAs.
// LDS rows are XOR-swizzled by 16-byte chunk so that the 16 rows one MFMA
// operand read touches fall in distinct banks.
constexpr int GU_BM = 128;
constexpr int GU_BN = 256;                        // W13 rows per tile (128 intermediate columns)
constexpr int GU_ICOLS = GU_BN / 2;

__device__ __forceinline__ int a_phys(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }   // 16-byte chunk
__device__ __forceinline__ int b_phys(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

struct GuStage {
  u32x4 a[GU_BM * 8];                             // [row][8 chunks] swizzled
  u32x4 b[GU_BN * 4];                             // [row][4 chunks] swizzled
  uint32_t as[GU_BM];
  uint32_t bs[GU_BN];
};

__global__ __launch_bounds__(256, 1) void gu_prefill_kernel(FfnArgs a, uint8_t* __restrict__ qws,
                                                            uint8_t* __restrict__ qsc_ws, int Tk) {
  __shared__ int tile_start[MAX_E + 1];
  __shared__ int tok[GU_BM];
  __shared__ GuStage st[2];
  build_tiles(a.offsets, a.E, GU_BM, tile_start);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int H = a.H, I = a.I, nb = I / 32;
  const int nsteps = H / KSTEP;
  const int nct = (I + GU_ICOLS - 1) / GU_ICOLS;
  const int nitems = tile_start[a.E] * nct;

  for (int round = 0;; ++round) {
    const int item = xcd_item(round, blockIdx.x, gridDim.x);
    if (item >= nitems) break;
    const int tile = item / nct, ct = item % nct;
    const int e = tile_expert(tile_start, a.E, tile);
    const int p0 = a.offsets[e] + (tile - tile_start[e]) * GU_BM;
    int nrows = a.offsets[e + 1] - p0;
    nrows = nrows > GU_BM ? GU_BM : nrows;
    if (p0 < 0 || p0 + nrows > Tk) nrows = 0;
    const int c0 = ct * GU_ICOLS;                               // first intermediate column of the tile
    const int ncols = min(GU_ICOLS, I - c0);
    lds_barrier();                                              // previous item's LDS reads are done
    if (tid < GU_BM) {
      int t = -1;
      if (tid < nrows) {
        const int pr = a.perm[p0 + tid];
        t = (pr >= 0 && pr < Tk) ? pr / a.k : -1;
      }
      tok[tid] = t;
    }
    lds_barrier();

    // this thread's staging slots: 4 activation chunks, 4 weight chunks, one scale dword each
    const uint8_t* asrc[4];
    const uint8_t* bsrc[4];
    bool aok[4], bok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int qa = tid + 256 * j, r = qa >> 3, c = qa & 7;
      const int t = tok[r];
      aok[j] = t >= 0;
      asrc[j] = a.x + (int64_t)(t < 0 ? 0 : t) * H + c * 16;
      const int qb = tid + 256 * j, rb = qb >> 2, cb = qb & 3;
      const int icol = (rb & 127);                              // intermediate column within the tile
      bok[j] = icol < ncols;
      const int r13 = (rb < 128 ? 0 : I) + c0 + (bok[j] ? icol : 0);
      bsrc[j] = a.w13 + ((int64_t)e * 2 * I + r13) * (H / 2) + cb * 16;
    }
    const int tas = tok[tid & (GU_BM - 1)];
    const uint32_t* asc_src = reinterpret_cast<const uint32_t*>(a.x_sc + (int64_t)(tas < 0 ? 0 : tas) * (H / 32));
    const bool asc_ok = tid < GU_BM && tas >= 0;
    const int icol_s = tid & 127;
    const bool bsc_ok = icol_s < ncols;
    const uint32_t* bsc_src = reinterpret_cast<const uint32_t*>(
        a.w13_sc + ((int64_t)e * 2 * I + (tid < 128 ? 0 : I) + c0 + (bsc_ok ? icol_s : 0)) * (H / 32));

    // two register sets of staged loads: stage s + 2 is requested while stage
    // s is multiplied and stage s + 1 waits in registers for its LDS buffer
    struct Regs { u32x4 a[4], b[4]; uint32_t as, bs; };
    Regs R0, R1;                                                // named, never indexed: they stay in registers
    auto load_stage = [&](int s, Regs& r) {
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        r.a[j] = aok[j] ? ldg16(asrc[j] + s * KSTEP) : z;
        r.b[j] = bok[j] ? ldg16(bsrc[j] + s * 64) : z;
      }
      r.as = asc_ok ? asc_src[s] : 0x7F7F7F7Fu;
      r.bs = bsc_ok ? bsc_src[s] : 0x7F7F7F7Fu;
    };
    auto store_stage = [&](GuStage& S, const Regs& r) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int qa = tid + 256 * j;
        S.a[a_phys(qa >> 3, qa & 7)] = r.a[j];
        S.b[b_phys(qa >> 2, qa & 3)] = r.b[j];
      }
      if (tid < GU_BM) S.as[tid] = r.as;
      S.bs[tid] = r.bs;
    };

    v4f acc[4][8];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 8; ++n) acc[m][n] = v4f{0.f, 0.f, 0.f, 0.f};
    // waves whose rows or columns fall outside the tile skip the matrix work
    const bool wact = wm * 64 < nrows && wn * 64 < ncols;

    // one MFMA step from LDS buffer s & 1; `nxt` holds stage s + 1, `fut` receives stage s + 2
    auto step = [&](int s, Regs& nxt, Regs& fut) {
      GuStage& S = st[s & 1];
      lds_barrier();                                            // stage s is in LDS; stage s-1 reads are done
      if (s + 2 < nsteps) load_stage(s + 2, fut);               // in flight during two steps of MFMAs
      if (wact) {
        v8i bf[8];
        uint32_t bsv[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          const int r = (n < 4 ? 0 : 128) + wn * 64 + (n & 3) * 16 + col;
          const u32x4 v = S.b[b_phys(r, g)];
          bf[n] = fp4_operand(v);
          bsv[n] = S.bs[r] >> (8 * g);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int r = wm * 64 + m * 16 + col;
          const v8i af = fp8_operand(S.a[a_phys(r, g)], S.a[a_phys(r, 4 + g)]);
          const uint32_t sa = S.as[r] >> (8 * g);
#pragma unroll
          for (int n = 0; n < 8; ++n) acc[m][n] = mfma_fp8_fp4(af, bf[n], acc[m][n], sa, bsv[n]);
        }
      }
      if (s + 1 < nsteps) store_stage(st[(s + 1) & 1], nxt);
    };
    load_stage(0, R0);
    if (nsteps > 1) load_stage(1, R1);
    store_stage(st[0], R0);
    for (int s = 0; s < nsteps; s += 2) {
      step(s, R1, R0);
      if (s + 1 < nsteps) step(s + 1, R0, R1);
    }

    // epilogue: SwiGLU + requant; one block of 32 = two 16-column subtiles of one row
    if (wact) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v0 = swiglu(acc[m][2 * blk][i], acc[m][4 + 2 * blk][i]);
            const float v1 = swiglu(acc[m][2 * blk + 1][i], acc[m][5 + 2 * blk][i]);
            float mx = fmaxf(__builtin_fabsf(v0), __builtin_fabsf(v1));
            mx = fmaxf(mx, __shfl_xor(mx, 1));
            mx = fmaxf(mx, __shfl_xor(mx, 2));
            mx = fmaxf(mx, __shfl_xor(mx, 4));
            mx = fmaxf(mx, __shfl_xor(mx, 8));
            const uint32_t sc = e8m0_code_for_amax(mx, 8);
            const int row = wm * 64 + m * 16 + 4 * g + i;
            const int cb = c0 + wn * 64 + blk * 32;           // first column of the block
            if (row < nrows && cb < I) {
              uint8_t* qrow = qws + (int64_t)(p0 + row) * I;
              qrow[cb + col] = (uint8_t)requant_e4m3(v0, sc);
              qrow[cb + 16 + col] = (uint8_t)requant_e4m3(v1, sc);
              if (col == 0) qsc_ws[(int64_t)(p0 + row) * nb + cb / 32] = (uint8_t)sc;
            }
          }
        }
      }
    }
  }
}

// Down over a 64-row expert tile and 256 W2 rows (64 per wavefront, four
// 16-row B tiles); the tile's intermediate rows are contiguous bucket rows.
__global__ __launch_bounds__(256, 2) void down_prefill_kernel(FfnArgs a, const uint8_t* __restrict__ qws,
                                                              const uint8_t* __restrict__ qsc_ws,
                                                              float* __restrict__ o, int Tk) {
  __shared__ int tile_start[MAX_E + 1];
  __shared__ __attribute__((aligned(16))) uint8_t qlds[PF_ROWS][PF_MAX_I + 16];
  __shared__ uint8_t slds[PF_ROWS][PF_MAX_I / 32 + 4];
  build_tiles(a.offsets, a.E, PF_ROWS, tile_start);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int H = a.H, I = a.I, nb = I / 32;
  const int nsteps = (I + KSTEP - 1) / KSTEP;                   // <= 5
  const int nnt = H / PF_NCOLS;
  const int nitems = tile_start[a.E] * nnt;

  for (int round = 0;; ++round) {
    const int item = xcd_item(round, blockIdx.x, gridDim.x);
    if (item >= nitems) break;
    const int tile = item / nnt, nt = item % nnt;
    const int e = tile_expert(tile_start, a.E, tile);
    const int p0 = a.offsets[e] + (tile - tile_start[e]) * PF_ROWS;
    int nrows = a.offsets[e + 1] - p0;
    nrows = nrows > PF_ROWS ? PF_ROWS : nrows;
    if (p0 < 0 || p0 + nrows > Tk) nrows = 0;

    // W2 of this lane's four columns first (whole K = I in registers)
    const int n0 = nt * PF_NCOLS + wave * 64;
    u32x4 bw[4][5];
    uint32_t bs[4][5];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int64_t row = (int64_t)e * H + n0 + n * 16 + col;
      const uint8_t* wp = a.w2 + row * (I / 2);
      const uint8_t* wsp = a.w2_sc + row * nb;
#pragma unroll
      for (int s = 0; s < 5; ++s) {
        const bool bv = s < nsteps && 4 * s + g < nb;
        const u32x4 z = {0u, 0u, 0u, 0u};
        bw[n][s] = bv ? ldg16(wp + s * 64 + g * 16) : z;
        bs[n][s] = wsp[bv ? 4 * s + g : 0];
      }
    }
    lds_barrier();                                              // previous item's LDS reads are done
    const int q16 = I / 16;
    for (int idx = tid; idx < PF_ROWS * q16; idx += 256) {
      const int r = idx / q16, c16 = idx % q16;
      const u32x4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&qlds[r][c16 * 16]) = r < nrows ? ldg16(qws + (int64_t)(p0 + r) * I + c16 * 16) : z;
    }
    for (int idx = tid; idx < PF_ROWS * nb; idx += 256) {
      const int r = idx / nb, b = idx % nb;
      slds[r][b] = r < nrows ? qsc_ws[(int64_t)(p0 + r) * nb + b] : (uint8_t)127;
    }
    lds_barrier();

    v4f acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[m][n] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 5; ++s) {
      if (s < nsteps) {
        const int klo = s * KSTEP + g * 16, khi = klo + 64;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int r = m * 16 + col;
          const u32x4 z = {0u, 0u, 0u, 0u};
          const u32x4 alo = klo < I ? *reinterpret_cast<const u32x4*>(&qlds[r][klo]) : z;
          const u32x4 ahi = khi < I ? *reinterpret_cast<const u32x4*>(&qlds[r][khi]) : z;
          const uint32_t sa = (4 * s + g < nb) ? (uint32_t)slds[r][4 * s + g] : bs[0][s];
          const v8i av = fp8_operand(alo, ahi);
#pragma unroll
          for (int n = 0; n < 4; ++n) acc[m][n] = mfma_fp8_fp4(av, fp4_operand(bw[n][s]), acc[m][n], sa, bs[n][s]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m * 16 + 4 * g + i;
        if (row < nrows) {
          float* orow = o + (int64_t)(p0 + row) * H + n0 + col;
#pragma unroll
          for (int n = 0; n < 4; ++n) orow[n * 16] = acc[m][n][i];
        }
      }
  }
}

// ============================================================== combine ===
// y_t = sum_j w_tj * o[slot_pos[t][j]], j = 0..k-1 in order; 4 columns per thread.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o, const float* __restrict__ w,
                                                      const int32_t* __restrict__ slot_pos, int T, int H, int k, int Tk,
                                                      float* __restrict__ y) {
  const int n = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (n >= H) return;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int p = slot_pos[(int64_t)t * k + j];
      if (p < 0 || p >= Tk) continue;
      const float wj = w[(int64_t)t * k + j];
      const float4 v = *reinterpret_cast<const float4*>(o + (int64_t)p * H + n);
      acc.x = fmaf(wj, v.x, acc.x);
      acc.y = fmaf(wj, v.y, acc.y);
      acc.z = fmaf(wj, v.z, acc.z);
      acc.w = fmaf(wj, v.w, acc.w);
    }
    *reinterpret_cast<float4*>(y + (int64_t)t * H + n) = acc;
  }
}

// ================================================================= host ===
static size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// workspace: [q: Tk*I][q_sc: Tk*I/32][h: Tk*2I fp32][o: Tk*H fp32], each 256-byte aligned
void ffn_ws_layout(int T, int H, int I, int k, size_t* off_q, size_t* off_q_sc, size_t* off_h, size_t* off_o) {
  const size_t Tk = (size_t)T * k;
  *off_q = 0;
  *off_q_sc = align256(Tk * I);
  *off_h = *off_q_sc + align256(Tk * (I / 32));
  *off_o = *off_h + align256(Tk * 2 * I * 4);
  (void)H;
}

size_t ffn_ws_bytes(int T, int H, int E, int I, int k) {
  (void)E;
  size_t q, qs, h, o;
  ffn_ws_layout(T, H, I, k, &q, &qs, &h, &o);
  return o + align256((size_t)T * k * H * 4) + 256;
}

// Row pairs at or below which the decode kernels are chosen.
constexpr int DECODE_MAX_PAIRS = 1024;

bool ffn_path_supported(int path, int H, int I) {
  if (path == 1) return H <= KSTEP * DEC_MAX_STEPS;
  if (path == 2) return I <= PF_MAX_I && H % PF_NCOLS == 0;
  return true;
}

hipError_t launch_ffn(const FfnArgs& a, void* ws, int path, hipStream_t stream, const char** variant) {
  const int Tk = a.T * a.k;
  uint8_t* base = static_cast<uint8_t*>(ws);
  size_t oq, oqs, oh, oo;
  ffn_ws_layout(a.T, a.H, a.I, a.k, &oq, &oqs, &oh, &oo);
  uint8_t* qws = base + oq;
  uint8_t* qsc = base + oqs;
  float* h = reinterpret_cast<float*>(base + oh);
  float* o = reinterpret_cast<float*>(base + oo);
  const int cus = num_cus();
  const int max_active = a.E < Tk ? a.E : Tk;
  if (path == 0) {
    const bool dec_ok = ffn_path_supported(1, a.H, a.I), pre_ok = ffn_path_supported(2, a.H, a.I);
    path = ((Tk <= DECODE_MAX_PAIRS && dec_ok) || !pre_ok) ? 1 : 2;
  }
  if (path == 1) {
    const int R = a.T < 16 ? a.T : 16;                          // rows of one expert never exceed T
    const size_t lds = (size_t)R * (a.H + 16) + (size_t)R * (a.H / KSTEP) * 4;
    const int gu_items = max_active * (2 * a.I / 16);
    const int dn_items = max_active * (a.H / 64);
    const int gu_grid = gu_items < cus * 8 ? gu_items : cus * 8;
    const int dn_grid = dn_items < cus * 4 ? dn_items : cus * 4;
    hipLaunchKernelGGL(gu_decode_kernel, dim3(gu_grid), dim3(64), lds, stream, a, h, Tk, R);
    hipLaunchKernelGGL(down_decode_kernel, dim3(dn_grid), dim3(256), 0, stream, a, h, qws, qsc, o, Tk);
    *variant = "ffn:gu_decode+down_decode+combine";
  } else {
    const int tiles_bound = Tk / PF_ROWS + max_active;
    const int gu_items = (Tk / GU_BM + max_active) * ((a.I + GU_ICOLS - 1) / GU_ICOLS);
    const int dn_items = tiles_bound * (a.H / PF_NCOLS);
    int gu_grid = gu_items < cus ? gu_items : cus;             // one 4-wavefront workgroup per CU
    int dn_grid = dn_items < cus * 2 ? dn_items : cus * 2;
    gu_grid = (gu_grid + XCDS - 1) / XCDS * XCDS;
    dn_grid = (dn_grid + XCDS - 1) / XCDS * XCDS;
    hipLaunchKernelGGL(gu_prefill_kernel, dim3(gu_grid), dim3(256), 0, stream, a, qws, qsc, Tk);
    hipLaunchKernelGGL(down_prefill_kernel, dim3(dn_grid), dim3(256), 0, stream, a, qws, qsc, o, Tk);
    *variant = "ffn:gu_prefill64+down_prefill64+combine";
  }
  const dim3 cgrid((a.H / 4 + 255) / 256, a.T < 65535 ? a.T : 65535);
  hipLaunchKernelGGL(combine_kernel, cgrid, dim3(256), 0, stream, o, a.topk_w, a.slot_pos, a.T, a.H, a.k, Tk, a.y);
  return hipGetLastError();
}

}  // namespace mx
