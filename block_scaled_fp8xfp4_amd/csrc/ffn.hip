// Routed-expert FFN kernels: gate/up GEMM, SwiGLU + FP8 requant, down GEMM
// and the fixed-order weighted combine ("New Deepseek 4.1 flash recipe"
// thread, post #6, "How it works": routed experts with FP8 activations x FP4
// weights, decode rows on small tiles, prefill on 64-row tiles; "Why
// TileLang": SwiGLU with per-block FP8 quantization, reductions in a fixed
// order; DeepSeek-V4.1-Flash-4x-DGX-Spark-TP4 README, settings table, row
// "Experts": per-slot buffer and a fixed-order sum instead of atomics, 64-row
// tiles for 576-wide experts at prefill sizes).  The prefill kernels here use
// 128-row expert tiles for gate/up and 32-row tiles for the down projection
// (measured faster on MI355X than 64-row tiles; a tile never changes a
// result, since every element runs the same chain).
//
// Both paths evaluate every output element with the same MFMA chain (all K
// steps in order, see mx_device.hpp) and the same SwiGLU/requant routine, so
// they give the same bits; they differ only in how rows and weights reach the
// matrix cores.
//
// Decode path (few rows per expert, weight streaming), T > 1:
//   gu_decode_kernel    one workgroup per (expert, block of 32 intermediate
//                       columns) = 64 W13 rows, 16 per wavefront: the whole K
//                       of the weight rows is loaded into registers at once,
//                       the expert's activation rows are staged in LDS, and
//                       the gate/up tile is turned into the requantized
//                       intermediate block in the same workgroup.
//   down_decode_kernel  one workgroup per (expert, 128 W2 rows); intermediate
//                       rows from the workspace through LDS; writes o.
// One row (T = 1):
//   gu1_kernel          one wavefront per (slot, 8 intermediate columns): the
//                       MFMA's 16 output columns are 8 gate rows and the
//                       matching 8 up rows, so each tile yields 8 SwiGLU
//                       values (fp32, in slot order in the workspace); may
//                       rank the row's logits itself (the fused gate).
//   down_combine1_kernel  one workgroup per 16 output columns: requantizes the
//                       k SwiGLU rows to FP8 blocks in LDS while its W2 rows
//                       stream in, runs the down chains of all k slots and
//                       the combine, so o never leaves the chip.
//   layer1_kernel       the same layer in ONE launch (moe_layer_decode1, k <=
//                       8): gate/up workgroups of one requant block each
//                       (four wavefronts = the gu1 tile four times) hand the
//                       block's FP8 codes to down + combine workgroups (16
//                       output columns, two slots per wavefront) through
//                       tagged words in the workspace; every wait is bounded.
//                       SH = true (moe_layer_decode1_shared): the shared
//                       expert's gate/up workgroups join the grid and the
//                       down workgroups also run its down projection.
// Prefill path (hundreds of rows per expert, matrix-core bound):
//   gu_prefill_kernel   expert tile of up to 128 rows x 128 intermediate
//                       columns (256 W13 rows) per workgroup, 2 x 2
//                       wavefronts; gathered activation rows and weight rows
//                       staged through swizzled, double-buffered LDS one MFMA
//                       step at a time; SwiGLU + requant in the epilogue.
//   down_prefill_kernel (expert, 256 W2 rows) items: the W2 rows stay in
//                       registers while the expert's 32-row tiles of the
//                       intermediate stream through LDS.
//   Both run persistent grids whose blocks are remapped so that each XCD
//   walks a contiguous range of (expert, row tile, column tile) items and
//   shares weights and activations in its own L2.
// combine_kernel adds w_tj * o_tj over the slots in order j = 0..k-1.
#include <atomic>
#include <chrono>

#include "mx_device.hpp"
#include "mx_launch.hpp"
#include "route_device.hpp"
#include "shared1_device.hpp"

namespace mx {

constexpr int DEC_MAX_STEPS = 40;                 // decode gate/up: H <= 5120 held in registers
constexpr int DOWN_MAX_STEPS = MAX_I / KSTEP;     // 16
constexpr int PF_NCOLS = 256;                     // prefill down: W2 rows per workgroup
constexpr int PF_MAX_I = 608;                     // prefill down: W2 slice of 256 rows x (I/32 + 1) chunks in LDS
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

// The expert list seen by one wavefront, from its own registers (no LDS, no
// barrier): lane l holds offsets[l * per + i], i = 0..per (per = ceil(E / 64)
// <= EPL).  A "tile" here is an expert with at least one live pair, in expert
// order.  EPL = 4 serves E <= 256 and EPL = 16 every E up to MAX_E: the loops
// over a lane's entries are unrolled to EPL, and at E = 256 the four-entry
// form takes 3.8 us off the verification batch's FFN call (two kernels, and
// one list lookup per item).
template <int EPL>
struct WaveExperts {
  int o[EPL + 1];
  int per, cnt, incl;                             // this lane's tiles and their inclusive prefix
};

// Entries per lane of the expert list for E experts.
constexpr int epl_for(int E) { return E <= 256 ? 4 : 16; }

template <int EPL>
__device__ __forceinline__ void wave_experts_load(const int32_t* __restrict__ offsets, int E, WaveExperts<EPL>& w) {
  static_assert(EPL == 4 || EPL == 16, "expert-list capacity");
  const int lane = threadIdx.x & 63;
  w.per = (E + 63) / 64;                          // <= EPL (the launcher picks EPL from E)
#pragma unroll
  for (int i = 0; i < EPL + 1; ++i) {             // branch-free: entries past per are never used
    const int e = lane * w.per + i;
    w.o[i] = offsets[e < E ? e : E];
  }
}

// Count this lane's tiles and scan them over the wavefront; returns the total.
template <int EPL>
__device__ __forceinline__ int wave_experts_scan(int E, WaveExperts<EPL>& w) {
  const int lane = threadIdx.x & 63;
  int c = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (i < w.per && lane * w.per + i < E && w.o[i + 1] > w.o[i]) ++c;
  w.cnt = c;
  w.incl = c + wave_excl_scan(c, lane);
  return __builtin_amdgcn_readlane(w.incl, 63);
}

// Tile t (< total): its expert, first bucket position and pair count.
template <int EPL>
__device__ __forceinline__ void wave_tile(const WaveExperts<EPL>& w, int E, int t, int& e, int& p0, int& cnt) {
  const int lane = threadIdx.x & 63;
  const unsigned long long past = __ballot(w.incl > t);
  const int L = __builtin_ctzll(past);            // lowest lane whose tiles reach past t
  int k = t - (w.incl - w.cnt), ei = 0, pe = 0, ce = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const bool live = i < w.per && lane * w.per + i < E && w.o[i + 1] > w.o[i];
    if (live && k == 0) { ei = lane * w.per + i; pe = w.o[i]; ce = w.o[i + 1] - w.o[i]; }
    if (live) --k;
  }
  e = __builtin_amdgcn_readlane(ei, L);
  p0 = __builtin_amdgcn_readlane(pe, L);
  cnt = __builtin_amdgcn_readlane(ce, L);
}

// The expert whose bucket holds position p (offsets[e] <= p < offsets[e + 1]), or -1.
template <int EPL>
__device__ __forceinline__ int wave_owner(const WaveExperts<EPL>& w, int E, int p) {
  const int lane = threadIdx.x & 63;
  int ei = -1;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (i < w.per && lane * w.per + i < E && w.o[i] <= p && p < w.o[i + 1]) ei = lane * w.per + i;
  const unsigned long long has = __ballot(ei >= 0);
  return has ? __builtin_amdgcn_readlane(ei, __builtin_ctzll(has)) : -1;
}

// Logical item of a persistent block in a round: each XCD (blocks b with the
// same b % 8) takes a contiguous range of items.  G is a multiple of 8.
__device__ __forceinline__ int xcd_item(int round, int b, int G) {
  const int per = G / XCDS;
  return round * G + (b % XCDS) * per + b / XCDS;
}

// Work queue of a persistent kernel: items [0, n) are split into XCDS
// contiguous ranges, one per XCD (the items that share activation rows and
// weights then meet in one L2).  A workgroup takes the next item of its own
// XCD's range from that range's counter and, once the range is drained, of
// the following ones.  Called by one thread; returns -1 when every range is
// drained.  Counters start at zero (cleared before the launch) and only grow.
__device__ __forceinline__ int queue_next(int* ctr, int n, int& q) {
  const int x0 = blockIdx.x % XCDS;
  while (q < XCDS) {
    const int x = (x0 + q) % XCDS;
    const int lo = (int)((int64_t)n * x / XCDS), hi = (int)((int64_t)n * (x + 1) / XCDS);
    const int c = atomicAdd(&ctr[x], 1);
    if (c < hi - lo) return lo + c;
    ++q;
  }
  return -1;
}

// The same in two halves, so that the counter's round trip overlaps other
// work: queue_take() starts the increment of the current range's counter,
// queue_finish() turns its result into an item (walking on synchronously when
// that range is drained).
__device__ __forceinline__ int queue_take(int* ctr, int q) {
  return q < XCDS ? atomicAdd(&ctr[(blockIdx.x % XCDS + q) % XCDS], 1) : 0;
}
__device__ __forceinline__ int queue_finish(int* ctr, int n, int& q, int c) {
  if (q >= XCDS) return -1;
  const int x = (blockIdx.x % XCDS + q) % XCDS;
  const int lo = (int)((int64_t)n * x / XCDS), hi = (int)((int64_t)n * (x + 1) / XCDS);
  if (c < hi - lo) return lo + c;
  ++q;
  return queue_next(ctr, n, q);
}

__global__ void clear_i32_kernel(int* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

__device__ __forceinline__ v8i fp8_operand(const u32x4& lo, const u32x4& hi) {
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
__device__ __forceinline__ v8i fp4_operand(const u32x4& b) {
  return v8i{(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
}

// =========================================================== decode path ==
constexpr int DEC_ROWS = 8;                       // gate/up: activation rows per pass
constexpr int DN_ROWS = 16;                       // down: intermediate rows per pass
constexpr int DEC_HPITCH = 64 + 4;                // LDS pitch (floats) of one pass's gate|up tile
constexpr int DEC_SPITCH = DEC_MAX_STEPS + 1;     // LDS pitch (dwords) of the staged weight scales

// Weight loads of the decode kernels are branch-free: a step past the end of
// K reloads the last step (never used), so a wavefront's loads issue back to
// back.  Whatever a pass needs besides the weights (activation rows, scales)
// is requested before the weights, so waiting for it never waits for them
// (vector-memory counters drain in issue order).

// Gate/up + SwiGLU + requant (T > 1): one workgroup per (expert, block of
// 32 intermediate columns), i.e. 64 W13 rows: wavefronts 0, 1 take gate rows
// 32 b + [0, 16) and + [16, 32), wavefronts 2, 3 the matching up rows.  Per
// pass of at most R = min(8, T) rows of the expert, the activation rows are
// gathered into LDS; each wavefront's 16 weight rows (whole K, NS >= H / 128
// steps) stay in registers for all passes and their block scales are staged
// in LDS (16 rows x H / 32 bytes, one coalesced span).  The four 16 x 16
// results meet in LDS, where one pass turns each row's 32 gate/up pairs into
// one requantized block.  Writes q, its scale, and the fp32 h = [gate | up]
// of every pair when h is non-null (diagnostics).  EXACT: H = 128 NS, so
// every address offset is a constant.
template <int NS, bool EXACT, int EPL>
__global__ __launch_bounds__(256, 2) void gu_decode_kernel(FfnArgs a, uint8_t* __restrict__ qws,
                                                           uint8_t* __restrict__ qsc_ws, float* __restrict__ h,
                                                           int Tk, int R) {
  __shared__ int tok[DEC_ROWS];
  __shared__ float hb[16 * DEC_HPITCH];
  __shared__ uint32_t bsc[4][16 * DEC_SPITCH];                 // per wavefront: [row][step] scale dwords
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int H = EXACT ? NS * KSTEP : a.H, I = a.I, nb = I / 32;
  const int nsteps = H / KSTEP, chunks = H / 16;
  const int pitch = H + 16, spitch = nsteps | 1;              // odd dword pitch: the 16 rows hit 16 banks
  uint8_t* xlds = dyn_lds;                                      // [R][H + 16]
  uint32_t* xslds = reinterpret_cast<uint32_t*>(dyn_lds + (size_t)R * pitch);   // [R][nsteps]
  u32x4 xv[DEC_ROWS];
  uint32_t xsv = 0x7F7F7F7Fu;
  // the pass's rows (tok[0, nr)): their activations and scales requested into
  // registers (one thread per 16-byte chunk / scale dword), then staged in
  // LDS; the parts past what one thread covers (H > 4096) are staged directly
  auto request_rows = [&](int nr) {
#pragma unroll
    for (int r = 0; r < DEC_ROWS; ++r) {
      const int t = r < nr ? tok[r] : -1;
      xv[r] = (t >= 0 && tid < chunks) ? ldg16(a.x + (int64_t)t * H + tid * 16) : u32x4{0u, 0u, 0u, 0u};
    }
    const int rs = tid / nsteps, ss = tid % nsteps;
    const int ts = (tid < nr * nsteps) ? tok[rs] : -1;
    xsv = ts >= 0 ? reinterpret_cast<const uint32_t*>(a.x_sc + (int64_t)ts * (H / 32))[ss] : 0x7F7F7F7Fu;
  };
  auto stage_rows = [&](int nr) {
#pragma unroll
    for (int r = 0; r < DEC_ROWS; ++r)
      if (r < nr && tid < chunks) *reinterpret_cast<u32x4*>(xlds + (size_t)r * pitch + tid * 16) = xv[r];
    if (tid < nr * nsteps) xslds[tid] = xsv;
    if (chunks > 256 || nr * nsteps > 256) {                    // H > 4096
      for (int idx = tid; idx < nr * chunks; idx += 256) {
        const int r = idx / chunks, c = idx % chunks;
        if (c < 256) continue;
        const int t = tok[r];
        *reinterpret_cast<u32x4*>(xlds + (size_t)r * pitch + c * 16) =
            t >= 0 ? ldg16(a.x + (int64_t)t * H + c * 16) : u32x4{0u, 0u, 0u, 0u};
      }
      for (int idx = tid + 256; idx < nr * nsteps; idx += 256) {
        const int t = tok[idx / nsteps];
        xslds[idx] = t >= 0 ? reinterpret_cast<const uint32_t*>(a.x_sc + (int64_t)t * (H / 32))[idx % nsteps]
                            : 0x7F7F7F7Fu;
      }
    }
  };
  auto gather_tok = [&](int p, int nr) {                       // tokens of bucket positions [p, p + nr)
    if (tid < nr) {
      const int pr = a.perm[p + tid];
      tok[tid] = (pr >= 0 && pr < Tk) ? pr / a.k : -1;
    }
  };
  WaveExperts<EPL> we;                                          // every wavefront reads the expert list itself
  wave_experts_load(a.offsets, a.E, we);
  const int nitems = wave_experts_scan(a.E, we) * nb;
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int blk = item % nb;
    int e, p0, cnt;
    wave_tile(we, a.E, item / nb, e, p0, cnt);
    if (p0 < 0 || p0 + cnt > Tk) cnt = 0;                       // malformed route: skip
    const int n0 = min(R, cnt);
    lds_barrier();                                              // the previous item's LDS reads are done
    gather_tok(p0, n0);
    lds_barrier();
    request_rows(n0);                                           // the first pass's rows: before the weights
    // this wavefront's 16 rows of scales: one contiguous span of 16 * nsteps dwords
    const int64_t wrow0 = (int64_t)e * 2 * I + (wave < 2 ? 0 : I) + blk * 32 + (wave & 1) * 16;
    const uint32_t* ssrc = reinterpret_cast<const uint32_t*>(a.w13_sc + wrow0 * (H / 32));
    constexpr int NBSV = (16 * NS + 63) / 64;                    // scale dwords per lane
    uint32_t bsv[NBSV];
#pragma unroll
    for (int i = 0; i < NBSV; ++i) {
      const int idx = lane + 64 * i;
      bsv[i] = idx < 16 * nsteps ? ssrc[idx] : 0u;
    }
    const uint8_t* wp = a.w13 + (wrow0 + col) * (H / 2) + g * 16;
    u32x4 bw[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) bw[s] = ldg16(wp + (EXACT || s < nsteps ? s : nsteps - 1) * 64);
    // stage what the first pass needs (its loads were issued before the weights)
#pragma unroll
    for (int i = 0; i < NBSV; ++i) {
      const int idx = lane + 64 * i;
      if (idx < 16 * nsteps) bsc[wave][(idx / nsteps) * spitch + idx % nsteps] = bsv[i];
    }
    stage_rows(n0);
    lds_barrier();
    const uint32_t* bsrow = &bsc[wave][col * spitch];
    // One pass over rows [r0, r0 + nrows) whose activations are in LDS.  Every
    // LDS read is unconditional: lanes of rows past nrows read row 0 again and
    // their output rows are discarded (rows of the matrix product are
    // independent), so nothing here waits behind a branch.
    auto run_pass = [&](int r0, int nrows) {
      const int ar = col < nrows ? col : 0;
      const uint8_t* arow = xlds + (size_t)ar * pitch + g * 16;
      const uint32_t* asrow = xslds + ar * nsteps;
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s < nsteps) {
          const u32x4 alo = *reinterpret_cast<const u32x4*>(arow + s * KSTEP);
          const u32x4 ahi = *reinterpret_cast<const u32x4*>(arow + s * KSTEP + 64);
          // byte g of the row's scale dword is block 4 s + g; the matrix core
          // reads only the low byte of the scale operand
          const uint32_t sb = bsrow[s] >> (8 * g);
          const uint32_t sa = asrow[s] >> (8 * g);
          acc = mfma_fp8_fp4(fp8_operand(alo, ahi), fp4_operand(bw[s]), acc, sa, sb);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) hb[(4 * g + i) * DEC_HPITCH + wave * 16 + col] = acc[i];
      lds_barrier();
      // SwiGLU + requant: 16 lanes per row, two intermediate columns each (rows < R <= 8)
      if (tid < DEC_ROWS * 16) {
        const int r = tid >> 4, c = 2 * (tid & 15);
        const float2 gg = *reinterpret_cast<const float2*>(&hb[r * DEC_HPITCH + c]);
        const float2 uu = *reinterpret_cast<const float2*>(&hb[r * DEC_HPITCH + 32 + c]);
        uint32_t sc;
        const uint32_t d = swiglu_requant2(gg.x, uu.x, gg.y, uu.y, &sc);   // rows past nrows: discarded
        if (r < nrows) {
          const int64_t p = p0 + r0 + r;
          *reinterpret_cast<uint16_t*>(qws + p * I + blk * 32 + c) = (uint16_t)d;
          if ((tid & 15) == 0) qsc_ws[p * nb + blk] = (uint8_t)sc;
          if (h != nullptr) {                                   // diagnostics only
            *reinterpret_cast<float2*>(h + p * 2 * I + blk * 32 + c) = gg;
            *reinterpret_cast<float2*>(h + p * 2 * I + I + blk * 32 + c) = uu;
          }
        }
      }
    };
    for (int r0 = 0; r0 < cnt; r0 += R) {
      const int nrows = min(R, cnt - r0);
      if (r0 > 0) {                                             // later passes: gather their rows
        lds_barrier();
        gather_tok(p0 + r0, nrows);
        lds_barrier();
        request_rows(nrows);
        stage_rows(nrows);
        lds_barrier();
      }
      run_pass(r0, nrows);
    }
  }
}

// Single row (T = 1), gate/up: one wavefront per (pair, 8 intermediate
// columns).  Its 16 weight rows are the 8 gate rows and the 8 up rows of
// those columns (each output column of the matrix core is its own dot
// product), streamed straight into registers over the whole K; the row's
// activations are in LDS.  The SwiGLU of the 8 columns, a = silu(gate) * up
// (double, rounded once to fp32), goes to abuf[j][I], row j = the pair's slot
// (so that the down kernel can request it before reading the route); the
// down kernel requantizes it (the block-32 scale needs 32 columns, four
// wavefronts).
// One-wavefront workgroups spread the 18.9 MB of a decode step's gate/up
// weights over every CU, whose outstanding-miss capacity, not HBM, bounds a
// stream this short.  RPER > 0 (single row, fused with the gate): every
// wavefront ranks the row's logits itself (the wavefront top-k with RPER
// logits per lane) instead of reading a route; item i takes the expert of
// slot i / (I / 8) (descending logit), the wavefront runs only the ranking
// rounds up to that slot before issuing the expert's weight loads and the
// remaining rounds while they are in flight, when the pair's bucket position
// (the rank of its expert among the k in ascending order) is known.
// Workgroup 0 writes the route outputs exactly as the single-row route kernel
// does, for the down kernel and the caller.  RPER = 0: the pairs come from
// the route's offsets.  SH (the routed + shared layer): the workgroups from
// groute on each run one of the shared expert's gate/up parts instead.
template <int NS, bool EXACT, int RPER, bool SH, int EPL>
__global__ __launch_bounds__(64) void gu1_kernel(FfnArgs a, float* __restrict__ abuf, float* __restrict__ h, int Tk,
                                                 FusedRoute fr, Shared1Args sh, int groute) {
  if (SH && (int)blockIdx.x >= groute) {                        // the shared expert's gate/up parts (H % 128 == 0)
    const int idx = (int)blockIdx.x - groute, nc = 2 * sh.I / 16;
    shared1_part<false>(sh, idx % nc, idx / nc);
    return;
  }
  __shared__ __attribute__((aligned(16))) uint8_t xl[NS * KSTEP];
  __shared__ uint32_t xs[NS];
  __shared__ uint32_t bsc[16 * (NS + 1)];                       // [row][step] scale dwords, odd pitch
  const int lane = threadIdx.x;
  const int col = lane & 15, g = lane >> 4;
  const int H = EXACT ? NS * KSTEP : a.H, I = a.I, ncg = I / 8;
  const int nsteps = H / KSTEP, chunks = H / 16, spitch = nsteps | 1;
  constexpr int XPT = (NS * 8 + 63) / 64;                       // 16-byte activation chunks per lane
  u32x4 xv[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int c = lane + 64 * i;
    xv[i] = (EXACT || c < chunks) ? ldg16(a.x + c * 16) : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t xsv = lane < nsteps ? reinterpret_cast<const uint32_t*>(a.x_sc)[lane] : 0x7F7F7F7Fu;
  WaveExperts<EPL> we;
  constexpr int RP = RPER > 0 ? RPER : 1;
  TopkState<RP> st;
  bool live = true;
  int nitems;
  if (RPER > 0) {
    const float sv = fr.survival != nullptr ? fr.survival[0] : 1.0f;   // in flight with the logits
    topk_begin<RP>(st, fr.logits, a.E);
    live = fr.survival == nullptr || !(sv < fr.skip_below);
    nitems = live ? a.k * ncg : 0;
  } else {
    wave_experts_load(a.offsets, a.E, we);
    nitems = wave_experts_scan(a.E, we) * ncg;
  }
  // the activation row into LDS (its loads were issued first)
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int c = lane + 64 * i;
    if (EXACT || c < chunks) *reinterpret_cast<u32x4*>(xl + c * 16) = xv[i];
  }
  if (lane < nsteps) xs[lane] = xsv;
  for (int item = blockIdx.x; item < nitems; item += SH ? groute : (int)gridDim.x) {
    const int j = item / ncg, c0 = (item % ncg) * 8;
    int e, p0 = 0, cnt = 1, slot = j;
    if (RPER > 0) {
      topk_rounds<RP>(st, j + 1);
      e = __builtin_amdgcn_readlane(st.idx, j);
    } else {
      wave_tile(we, a.E, j, e, p0, cnt);
      if (p0 < 0 || p0 >= Tk) cnt = 0;                          // malformed route: skip
      slot = cnt ? a.perm[p0] : -1;                             // T = 1: perm[p] is the pair's slot
      if (slot < 0 || slot >= a.k) cnt = 0;
    }
    // rows: lanes 0..7 the gate rows c0 + [0, 8), lanes 8..15 the up rows I + c0 + [0, 8)
    const int64_t ebase = (int64_t)e * 2 * I;
    const int64_t wrow = ebase + (col < 8 ? c0 + col : I + c0 + col - 8);
    // scales of the 16 rows: two spans of 8 rows x nsteps dwords
    constexpr int NBSV = (16 * NS + 63) / 64;
    uint32_t bsv[NBSV];
#pragma unroll
    for (int i = 0; i < NBSV; ++i) {
      const int idx = lane + 64 * i, r = idx / nsteps, sidx = idx % nsteps;
      const int64_t sr = ebase + (r < 8 ? c0 + r : I + c0 + r - 8);
      bsv[i] = idx < 16 * nsteps ? reinterpret_cast<const uint32_t*>(a.w13_sc + sr * (H / 32))[sidx] : 0u;
    }
    const uint8_t* wp = a.w13 + wrow * (H / 2) + g * 16;
    u32x4 bw[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) bw[s] = ldg16(wp + (EXACT || s < nsteps ? s : nsteps - 1) * 64);
    if (RPER > 0) {                                             // the other slots, while the weights stream in
      topk_rounds<RP>(st, a.k);
      for (int i = 0; i < a.k; ++i) p0 += __builtin_amdgcn_readlane(st.idx, i) < e ? 1 : 0;
    }
    lds_barrier();                                              // the previous item's scale reads are done
#pragma unroll
    for (int i = 0; i < NBSV; ++i) {
      const int idx = lane + 64 * i;
      if (idx < 16 * nsteps) bsc[(idx / nsteps) * spitch + idx % nsteps] = bsv[i];
    }
    lds_barrier();
    if (cnt == 0) continue;
    // every row of the A tile is the activation row (output row 0 is kept)
    const uint8_t* arow = xl + g * 16;
    const uint32_t* bsrow = &bsc[col * spitch];
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (EXACT || s < nsteps) {
        const u32x4 alo = *reinterpret_cast<const u32x4*>(arow + s * KSTEP);
        const u32x4 ahi = *reinterpret_cast<const u32x4*>(arow + s * KSTEP + 64);
        acc = mfma_fp8_fp4(fp8_operand(alo, ahi), fp4_operand(bw[s]), acc, xs[s] >> (8 * g), bsrow[s] >> (8 * g));
      }
    }
    // lanes 0..15 hold output row 0: gate values in lanes 0..7, up values in 8..15
    const float up = __shfl_down(acc[0], 8, 16);
    if (h != nullptr && lane < 16)                              // diagnostics only
      h[(int64_t)p0 * 2 * I + (col < 8 ? c0 + col : I + c0 + col - 8)] = acc[0];
    if (lane < 8) abuf[(int64_t)slot * I + c0 + lane] = swiglu(acc[0], up);
  }
  if (RPER > 0 && blockIdx.x == 0) {                            // the route outputs, as the single-row route kernel
    topk_rounds<RP>(st, a.k);
    int rrank = 0;
    for (int i = 0; i < a.k; ++i) rrank += __builtin_amdgcn_readlane(st.idx, i) < st.idx ? 1 : 0;
    const float wt = slot_weight(st.val, a.k);
    if (lane < a.k) {
      fr.ids[lane] = st.idx;
      fr.w[lane] = wt;
      fr.slot_pos[lane] = live ? rrank : -1;
      fr.perm[live ? rrank : lane] = live ? lane : -1;
    }
    for (int e = lane; e <= a.E; e += 64) {
      int below = 0;
      for (int i = 0; i < a.k; ++i) below += __builtin_amdgcn_readlane(st.idx, i) < e ? 1 : 0;
      fr.offsets[e] = live ? below : 0;
    }
  }
}

// W2 operand of one 16-row tile for NS steps, branch-free: lane (col, g)
// takes block 4 s + g of its row; blocks past I / 32 load the row's first
// bytes (in bounds) and are zeroed where the MFMA consumes them.
template <int NS>
__device__ __forceinline__ void load_w2_tile(const uint8_t* __restrict__ w2, const uint8_t* __restrict__ w2_sc,
                                             int64_t row, int I, int g, u32x4 (&bw)[NS], uint32_t (&bs)[NS]) {
  const int nb = I / 32;
  const uint8_t* wp = w2 + row * (I / 2);
  const uint8_t* wsp = w2_sc + row * nb;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const bool bv = 4 * s + g < nb;
    bw[s] = ldg16(wp + (bv ? s * 64 + g * 16 : 0));
    bs[s] = wsp[bv ? 4 * s + g : 0];
  }
}

__device__ __forceinline__ v8i fp4_operand_masked(const u32x4& b, bool valid) {
  return valid ? v8i{(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0} : v8i{0, 0, 0, 0, 0, 0, 0, 0};
}

// Stage intermediate rows [p, p + nrows) (nrows <= DN_ROWS) of the workspace in LDS.
__device__ void stage_q_rows(const uint8_t* __restrict__ qws, const uint8_t* __restrict__ qsc_ws, int64_t p, int nrows,
                             int I, uint8_t (*qlds)[MAX_I + 16], uint8_t (*slds)[MAX_I / 32]) {
  const int q16 = I / 16, nb = I / 32;
  for (int idx = threadIdx.x; idx < DN_ROWS * q16; idx += blockDim.x) {
    const int r = idx / q16, c16 = idx % q16;
    const u32x4 z = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(&qlds[r][c16 * 16]) = r < nrows ? ldg16(qws + (p + r) * I + c16 * 16) : z;
  }
  for (int idx = threadIdx.x; idx < DN_ROWS * nb; idx += blockDim.x) {
    const int r = idx / nb, b = idx % nb;
    slds[r][b] = r < nrows ? qsc_ws[(p + r) * nb + b] : (uint8_t)127;
  }
}

// Workgroups per CU of the persistent down kernel: as many as its registers
// allow, four at I <= 640 with the four-entry expert list (128 VGPRs), else
// three, or two at I > 640 (measured at the verification batch: with the
// 16-entry list three took 39 us against 43 us with two; with the four-entry
// list four took 97.2 us per FFN call against 98.4 us with three; one
// workgroup per item instead of a persistent grid: 70 us)
#define DN_WG_PER_CU(NS, EPL) ((NS) <= 5 ? ((EPL) == 4 ? 4 : 3) : 2)

// Down: one workgroup per (expert, 128 W2 rows), 32 rows (two 16-row tiles)
// per wavefront.  W2 first (NS >= I / 128 steps in registers), then the
// expert's intermediate rows, 16 per pass, from the workspace into LDS;
// writes o.
template <int NS, int EPL>
__global__ __launch_bounds__(256, DN_WG_PER_CU(NS, EPL)) void down_decode_kernel(FfnArgs a, const uint8_t* __restrict__ qws,
                                                             const uint8_t* __restrict__ qsc_ws,
                                                             float* __restrict__ o, int Tk) {
  __shared__ __attribute__((aligned(16))) uint8_t qlds[DN_ROWS][MAX_I + 16];
  __shared__ uint8_t slds[DN_ROWS][MAX_I / 32];
  WaveExperts<EPL> we;
  wave_experts_load(a.offsets, a.E, we);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int H = a.H, I = a.I, nb = I / 32;
  const int nsteps = (I + KSTEP - 1) / KSTEP;
  const int ntiles = H / 128;
  const int nitems = wave_experts_scan(a.E, we) * ntiles;
  // K past I reads zeros: the row tails are cleared once, staging never writes them
  for (int idx = threadIdx.x; idx < DN_ROWS * (NS * KSTEP - I); idx += blockDim.x)
    qlds[idx / (NS * KSTEP - I)][I + idx % (NS * KSTEP - I)] = 0;
  for (int idx = threadIdx.x; idx < DN_ROWS * (NS * 4 - nb); idx += blockDim.x)
    slds[idx / (NS * 4 - nb)][nb + idx % (NS * 4 - nb)] = 127;

  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int tile = item % ntiles;
    int e, p0, cnt;
    wave_tile(we, a.E, item / ntiles, e, p0, cnt);
    if (p0 < 0 || p0 + cnt > Tk) cnt = 0;
    const int n0 = tile * 128 + wave * 32;                      // first W2 row of this wavefront
    u32x4 bw[2][NS];
    uint32_t bs[2][NS];
#pragma unroll
    for (int n = 0; n < 2; ++n) load_w2_tile<NS>(a.w2, a.w2_sc, (int64_t)e * H + n0 + n * 16 + col, I, g, bw[n], bs[n]);
    for (int r0 = 0; r0 < cnt; r0 += DN_ROWS) {
      const int nrows = min(DN_ROWS, cnt - r0);
      lds_barrier();                                            // the previous pass's LDS reads are done
      stage_q_rows(qws, qsc_ws, p0 + r0, nrows, I, qlds, slds);
      lds_barrier();
      v4f acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s < nsteps) {
          const int klo = s * KSTEP + g * 16;
          const bool bv = 4 * s + g < nb;
          const u32x4 alo = *reinterpret_cast<const u32x4*>(&qlds[col][klo]);
          const u32x4 ahi = *reinterpret_cast<const u32x4*>(&qlds[col][klo + 64]);
          const uint32_t sa = slds[col][4 * s + g];
          const v8i av = fp8_operand(alo, ahi);
#pragma unroll
          for (int n = 0; n < 2; ++n) acc[n] = mfma_fp8_fp4(av, fp4_operand_masked(bw[n][s], bv), acc[n], sa, bs[n][s]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * g + i;
        if (row < nrows) {
          float* orow = o + (int64_t)(p0 + r0 + row) * H + n0 + col;
          orow[0] = acc[0][i];
          orow[16] = acc[1][i];
        }
      }
    }
  }
}

// Single-row decode (T = 1: every touched expert holds exactly one pair, and
// pair p belongs to the p-th touched expert): requant, down and combine in
// one kernel.  One workgroup per 16 output columns.  The k fp32 SwiGLU rows
// of the gate/up kernel are requested first, then each wavefront's W2 rows;
// while those stream in, the workgroup requantizes the k rows (block-32 E4M3,
// the routine every path uses) into LDS (workgroup 0 also writes the FP8
// intermediate to the workspace).  Wavefront w runs the down chains of slots
// w and w + 4 (then w + 8 and w + 12 when k > 8) with their W2 rows in
// registers, and the 16 columns are combined in slot order exactly as the
// combine kernel does.  SH (the routed + shared layer): workgroups H / 16 and
// on each run one of the shared expert's down tiles instead.
template <int NS, bool SH, int EPL>
__global__ __launch_bounds__(256, 2) void down_combine1_kernel(FfnArgs a, const float* __restrict__ abuf,
                                                               uint8_t* __restrict__ qws,
                                                               uint8_t* __restrict__ qsc_ws, int Tk, Shared1Args sh) {
  if (SH && (int)blockIdx.x >= a.H / 16) {                      // the shared expert's down tiles
    const int tile = (int)blockIdx.x - a.H / 16;
    if (sh.I % KSTEP) shared1_down<true>(sh, tile);
    else shared1_down<false>(sh, tile);
    return;
  }
  constexpr int QP = NS * KSTEP + 16;                           // LDS pitch of an intermediate row
  constexpr int RQP = 8;                                        // 16-byte SwiGLU chunks per thread in flight
  __shared__ int pslot[MAX_K];
  __shared__ float wslot[MAX_K];
  __shared__ float olds[MAX_K][16];
  __shared__ __attribute__((aligned(16))) uint8_t q1[MAX_K][QP];
  __shared__ uint8_t s1[MAX_K][NS * 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int H = a.H, I = a.I, nb = I / 32, k = a.k;
  const int nsteps = (I + KSTEP - 1) / KSTEP;
  const int n = blockIdx.x * 16 + col;                         // output column of this lane
  int my_p = -1;
  float my_w = 0.f;
  if (tid < k) {                                                // in flight with the offsets
    my_p = a.slot_pos[tid];
    my_w = a.topk_w[tid];
  }
  WaveExperts<EPL> we;
  wave_experts_load(a.offsets, a.E, we);
  // the k SwiGLU rows (row j = slot j), requested before any weight, as
  // 16-byte chunks: chunk ch = tid + 256 i of a round holds floats [4 c, 4 c +
  // 4) of row j (ch = j I / 4 + c); eight consecutive lanes hold the eight
  // chunks of one block of 32 (I / 4 is a multiple of 8)
  const int cpr = I / 4, nch = k * cpr;
  u32x4 av[RQP];
  auto load_round = [&](int ch0) {
    int jr = (ch0 + tid) / cpr, cr = (ch0 + tid) % cpr;
#pragma unroll
    for (int i = 0; i < RQP; ++i) {
      const bool v = jr < k;                                    // whole 8-lane blocks in or out
      av[i] = v ? *reinterpret_cast<const u32x4*>(abuf + (int64_t)jr * I + 4 * cr) : u32x4{0u, 0u, 0u, 0u};
      cr += 256;                                                // this thread's next chunk
      while (cr >= cpr) { cr -= cpr; ++jr; }
    }
  };
  load_round(0);
  if (tid < k) {
    pslot[tid] = my_p;
    wslot[tid] = my_w;
  }
  lds_barrier();
  for (int idx = tid; idx < MAX_K * (NS * KSTEP - I); idx += 256)   // K past I reads zeros
    q1[idx / (NS * KSTEP - I)][I + idx % (NS * KSTEP - I)] = 0;
  for (int idx = tid; idx < MAX_K * (NS * 4 - nb); idx += 256)
    s1[idx / (NS * 4 - nb)][nb + idx % (NS * 4 - nb)] = 127;
  auto slot_ok = [&](int j) {
    const int p = j < k ? pslot[j] : -1;
    return p >= 0 && p < Tk;
  };
  auto load_pair = [&](int j0, bool (&ok)[2], u32x4 (&bw)[2][NS], uint32_t (&bs)[2][NS]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = j0 + 4 * u;
      const int e = slot_ok(j) ? wave_owner(we, a.E, pslot[j]) : -1;
      ok[u] = e >= 0;
      load_w2_tile<NS>(a.w2, a.w2_sc, (int64_t)(ok[u] ? e : 0) * H + n, I, g, bw[u], bs[u]);
    }
  };
  auto run_pair = [&](int j0, const bool (&ok)[2], const u32x4 (&bw)[2][NS], const uint32_t (&bs)[2][NS]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = j0 + 4 * u;
      if (j >= k) continue;                                     // wavefront-uniform
      if (!ok[u]) {
        if (g == 0) olds[j][col] = 0.f;
        continue;
      }
      // every row of the A tile is the slot's one activation row (rows are
      // independent; row 0 is kept)
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s < nsteps) {
          const int klo = s * KSTEP + g * 16;
          const bool bv = 4 * s + g < nb;
          const u32x4 alo = *reinterpret_cast<const u32x4*>(&q1[j][klo]);
          const u32x4 ahi = *reinterpret_cast<const u32x4*>(&q1[j][klo + 64]);
          const uint32_t sa = s1[j][4 * s + g];
          acc = mfma_fp8_fp4(fp8_operand(alo, ahi), fp4_operand_masked(bw[u][s], bv), acc, sa, bs[u][s]);
        }
      }
      if (g == 0) olds[j][col] = acc[0];                        // row 0 of the tile
    }
  };
  bool okA[2];
  u32x4 bwA[2][NS];
  uint32_t bsA[2][NS];
  load_pair(wave, okA, bwA, bsA);
  // requant (block-32 E4M3 of each SwiGLU row) into LDS while the W2 rows stream in
  auto requant_round = [&](int ch0) {
    int jr = (ch0 + tid) / cpr, cr = (ch0 + tid) % cpr;
#pragma unroll
    for (int i = 0; i < RQP; ++i) {
      if (ch0 + i * 256 < nch) {                                // uniform over the workgroup's pass
        const float v0 = __uint_as_float(av[i][0]), v1 = __uint_as_float(av[i][1]);
        const float v2 = __uint_as_float(av[i][2]), v3 = __uint_as_float(av[i][3]);
        const float m = fmaxf(fmaxf(__builtin_fabsf(v0), __builtin_fabsf(v1)),
                              fmaxf(__builtin_fabsf(v2), __builtin_fabsf(v3)));
        const uint32_t sc = e8m0_code_for_amax(row8_max(m), 8);
        const uint32_t d = requant2_e4m3(v0, v1, sc) | (requant2_e4m3(v2, v3, sc) << 16);
        if (jr < k) {
          const int b = cr / 8;
          *reinterpret_cast<uint32_t*>(&q1[jr][4 * cr]) = d;
          if ((cr & 7) == 0) s1[jr][b] = (uint8_t)sc;
          if (blockIdx.x == 0 && slot_ok(jr)) {                 // the intermediate, for the workspace's readers
            *reinterpret_cast<uint32_t*>(qws + (int64_t)pslot[jr] * I + 4 * cr) = d;
            if ((cr & 7) == 0) qsc_ws[(int64_t)pslot[jr] * nb + b] = (uint8_t)sc;
          }
        }
      }
      cr += 256;
      while (cr >= cpr) { cr -= cpr; ++jr; }
    }
  };
  requant_round(0);
  for (int ch0 = 256 * RQP; ch0 < nch; ch0 += 256 * RQP) {     // more than 256 * RQP chunks: further rounds
    load_round(ch0);
    requant_round(ch0);
  }
  lds_barrier();
  run_pair(wave, okA, bwA, bsA);
  if (k > 8) {
    load_pair(wave + 8, okA, bwA, bsA);
    run_pair(wave + 8, okA, bwA, bsA);
  }
  lds_barrier();
  if (tid < 16) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const int pj = pslot[j];
      if (pj < 0 || pj >= Tk) continue;
      acc = fmaf(wslot[j], olds[j][tid], acc);
    }
    a.y[blockIdx.x * 16 + tid] = acc;
  }
}

// ------------------------------------------------ single-launch layer (T = 1) ==
// moe_layer_decode1 in one launch: gate/up workgroups (one per slot and block
// of 32 intermediate columns, four wavefronts of 8 columns each: the
// gu1_kernel tile per wavefront) and down + combine workgroups (L1_COLS = 16
// output columns each, two slots per wavefront) in one grid.  A gate/up workgroup
// requantizes its block itself (the block is whole in the workgroup) and
// hands the 32 E4M3 codes and the E8M0 code to every down workgroup through
// the workspace: nine 8-byte words, each four payload bytes and the call's
// 32-bit tag, written by 64-bit system-scope stores (they reach memory whole).
// A down wavefront reads a slot's words with system-scope loads (which read
// memory, never a stale cached copy) until every word carries the tag.  Tags
// are unique per call in the process, so words of earlier calls, or garbage
// in a fresh workspace, never match and
// nothing has to be cleared.  Gate/up workgroups have lower indices than down
// workgroups and never wait, so they are dispatched first; every wait is
// bounded in wall-clock time (a down workgroup whose time runs out sets bit 0
// of *status, and that call's result is undefined).
// (Handoff, next_call_tag and handoff_limit_ticks: mx_launch.hpp; here
// words = [k][l1_slot_words(I)] (payload, tag) words, nprod = k * I / 32.)
constexpr int L1_HWORDS = 9;                                    // words per block: 8 x four codes, 1 x scale code
constexpr int L1_BWORDS = 16;                                   // a block's nine words in a 128-byte line of their own
constexpr int L1_BCHUNKS = 5;                                   // 16-byte reads that cover a block's nine words
__host__ __device__ constexpr int l1_slot_words(int I) { return (I / 32) * L1_BWORDS; }

// Gate/up of one block of 32 intermediate columns of slot j: wavefront w
// computes columns [32 b + 8 w, +8) exactly as gu1_kernel's item does (the
// fused gate's top-k in every wavefront; 8 gate + 8 up weight rows per
// MFMA tile), then wavefront 0 requantizes the 32 SwiGLU values (block
// maximum, E8M0 code, E4M3 codes: the requant routine of every path) and
// publishes them; it also writes q, its scale, the fp32 SwiGLU row values
// and (workgroup 0) the route outputs, as the two-launch path does.
template <int NS, bool EXACT, int RP, bool GRAPH>
__device__ void layer1_gate_up(const FfnArgs& a, float* __restrict__ abuf, float* __restrict__ h,
                               uint8_t* __restrict__ qws, uint8_t* __restrict__ qsc_ws, const FusedRoute& fr,
                               const Handoff& ho) {
  __shared__ __attribute__((aligned(16))) uint8_t xl[NS * KSTEP];
  __shared__ uint32_t xs[NS];
  __shared__ uint32_t bsc[4][16 * (NS + 1)];                    // per wavefront: [row][step] scale dwords
  __shared__ float sw[32];
  __shared__ __attribute__((aligned(16))) uint8_t qb[32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int H = EXACT ? NS * KSTEP : a.H, I = a.I, nb = I / 32;
  const int nsteps = H / KSTEP, chunks = H / 16, spitch = nsteps | 1;
  constexpr int XPT = (NS * 8 + 63) / 64;                       // 16-byte activation chunks per lane
  u32x4 xv[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int c = lane + 64 * i;
    xv[i] = (EXACT || c < chunks) ? ldg16(a.x + c * 16) : u32x4{0u, 0u, 0u, 0u};
  }
  const uint32_t xsv = lane < nsteps ? reinterpret_cast<const uint32_t*>(a.x_sc)[lane] : 0x7F7F7F7Fu;
  const float sv = fr.survival != nullptr ? fr.survival[0] : 1.0f;   // in flight with the logits
  TopkState<RP> st;
  topk_begin<RP>(st, fr.logits, a.E);
  const uint32_t ev = handoff_epoch_issue<GRAPH>(ho);          // the graph form's call counter
  const bool live = fr.survival == nullptr || !(sv < fr.skip_below);
  const int j = (int)blockIdx.x / nb, b = (int)blockIdx.x % nb;
  const int c0 = 32 * b + 8 * wave;                             // this wavefront's first intermediate column
  int p0 = 0;                                                   // the pair's bucket position
  if (live) {                                                   // workgroup-uniform
    // every wavefront stages the whole activation row itself (the same bytes)
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int c = lane + 64 * i;
      if (EXACT || c < chunks) *reinterpret_cast<u32x4*>(xl + c * 16) = xv[i];
    }
    if (lane < nsteps) xs[lane] = xsv;
    topk_rounds<RP>(st, j + 1);
    const int e = __builtin_amdgcn_readlane(st.idx, j);
    const int64_t ebase = (int64_t)e * 2 * I;
    const int64_t wrow = ebase + (col < 8 ? c0 + col : I + c0 + col - 8);
    constexpr int NBSV = (16 * NS + 63) / 64;
    uint32_t bsv[NBSV];
#pragma unroll
    for (int i = 0; i < NBSV; ++i) {
      const int idx = lane + 64 * i, r = idx / nsteps, sidx = idx % nsteps;
      const int64_t sr = ebase + (r < 8 ? c0 + r : I + c0 + r - 8);
      bsv[i] = idx < 16 * nsteps ? reinterpret_cast<const uint32_t*>(a.w13_sc + sr * (H / 32))[sidx] : 0u;
    }
    const uint8_t* wp = a.w13 + wrow * (H / 2) + g * 16;
    u32x4 bw[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) bw[s] = ldg16(wp + (EXACT || s < nsteps ? s : nsteps - 1) * 64);
    topk_rounds<RP>(st, a.k);                                   // the other slots, while the weights stream in
    for (int i = 0; i < a.k; ++i) p0 += __builtin_amdgcn_readlane(st.idx, i) < e ? 1 : 0;
    uint32_t* bscw = bsc[wave];
#pragma unroll
    for (int i = 0; i < NBSV; ++i) {
      const int idx = lane + 64 * i;
      if (idx < 16 * nsteps) bscw[(idx / nsteps) * spitch + idx % nsteps] = bsv[i];
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);                         // lgkmcnt(0): this wavefront's LDS writes landed
    __builtin_amdgcn_wave_barrier();
    const uint8_t* arow = xl + g * 16;
    const uint32_t* bsrow = &bscw[col * spitch];
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (EXACT || s < nsteps) {
        const u32x4 alo = *reinterpret_cast<const u32x4*>(arow + s * KSTEP);
        const u32x4 ahi = *reinterpret_cast<const u32x4*>(arow + s * KSTEP + 64);
        acc = mfma_fp8_fp4(fp8_operand(alo, ahi), fp4_operand(bw[s]), acc, xs[s] >> (8 * g), bsrow[s] >> (8 * g));
      }
    }
    const float up = __shfl_down(acc[0], 8, 16);                // gate values in lanes 0..7, up values in 8..15
    if (h != nullptr && lane < 16)                              // diagnostics only
      h[(int64_t)p0 * 2 * I + (col < 8 ? c0 + col : I + c0 + col - 8)] = acc[0];
    if (lane < 8) {
      const float av = swiglu(acc[0], up);
      abuf[(int64_t)j * I + c0 + lane] = av;                    // the SwiGLU rows of the workspace's layout
      sw[8 * wave + lane] = av;
    }
    lds_barrier();
    if (wave == 0) {
      const float v = lane < 32 ? sw[lane] : 0.f;
      float m = row16_max(__builtin_fabsf(v));
      m = fmaxf(m, __shfl_xor(m, 16));                          // lanes 0..31: the block maximum
      const uint32_t sc = e8m0_code_for_amax(m, 8);
      if (lane < 32) qb[lane] = (uint8_t)(requant2_e4m3(v, 0.f, sc) & 0xFFu);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_wave_barrier();
      if (lane < L1_HWORDS) {
        const uint32_t pay = lane < 8 ? reinterpret_cast<const uint32_t*>(qb)[lane] : sc;
        __hip_atomic_store(ho.words + (int64_t)j * l1_slot_words(I) + b * L1_BWORDS + lane, (uint64_t)pay | ((uint64_t)handoff_tag<GRAPH>(ho, ev) << 32),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        if (lane < 8) reinterpret_cast<uint32_t*>(qws + (int64_t)p0 * I + 32 * b)[lane] = pay;
        else qsc_ws[(int64_t)p0 * nb + b] = (uint8_t)sc;
      }
    }
  }
  if (blockIdx.x == 0 && wave == 0) {                           // the route outputs, as the single-row route kernel
    topk_rounds<RP>(st, a.k);
    int rrank = 0;
    for (int i = 0; i < a.k; ++i) rrank += __builtin_amdgcn_readlane(st.idx, i) < st.idx ? 1 : 0;
    const float wt = slot_weight(st.val, a.k);
    if (lane < a.k) {
      fr.ids[lane] = st.idx;
      fr.w[lane] = wt;
      fr.slot_pos[lane] = live ? rrank : -1;
      fr.perm[live ? rrank : lane] = live ? lane : -1;
    }
    for (int e = lane; e <= a.E; e += 64) {
      int below = 0;
      for (int i = 0; i < a.k; ++i) below += __builtin_amdgcn_readlane(st.idx, i) < e ? 1 : 0;
      fr.offsets[e] = live ? below : 0;
    }
  }
}

// Down projection + combine of L1_COLS output columns (L1_COLS / 16 tiles):
// wavefront w takes slots w and w + 4.  It ranks the logits itself, issues
// each slot's W2 rows as soon as the slot's round has named the expert, then
// waits for the slots' codes (both slots' words in one round of reads),
// copies them into LDS and runs the slot's chains (down_combine1_kernel's
// chain: K past I zero, blocks past I / 32 scale 127).  Wavefront 0 adds the
// k products in slot order.  k <= 8, I <= NSD * 128.  (Measured at the
// decode shape: one 16-column tile per workgroup, 12.6 us per call; two
// tiles, half as many workgroups, 14.4-14.9 us.)
// SH (the routed + shared layer): the workgroup also runs the shared
// expert's down projection of the same 16 columns: wavefront 1 requests the
// shared W2 rows before anything else, every wavefront polls its share of
// the shared SwiGLU words in the same read rounds as its slots, and after
// the rounds the four wavefronts requantize the shared row while wavefront 0
// combines, then wavefront 1 runs the shared chain (shared1_down_wait's
// arithmetic: the same bits as the shared expert alone).  A dead row skips
// the routed work only.  Shared I <= NSD * 128.
constexpr int L1_COLS = 16;
template <int NSD, int RP, bool SH, bool GRAPH>
__device__ void layer1_down(const FfnArgs& a, const FusedRoute& fr, const Handoff& ho, int tile,
                            const Shared1Args& sh = Shared1Args{}, const uint64_t* swords = nullptr) {
  constexpr int QP = NSD * KSTEP + 16;
  constexpr int CT = L1_COLS / 16;
  constexpr int SN = SH ? NSD * KSTEP : 1;
  __shared__ __attribute__((aligned(16))) uint8_t q1[8][QP];
  __shared__ uint8_t s1[8][NSD * 4];
  __shared__ float olds[8][L1_COLS];
  __shared__ __attribute__((aligned(16))) float sav[SN];      // SH: the shared SwiGLU row
  __shared__ __attribute__((aligned(16))) uint8_t sq1[SN];    // SH: its E4M3 codes, K past I zero
  __shared__ uint8_t ss1[SH ? NSD * 4 : 1];                     // SH: its scale codes
  const uint64_t t0 = wall_clock64();
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int H = a.H, I = a.I, nb = I / 32, k = a.k;
  const int nsteps = (I + KSTEP - 1) / KSTEP;
  u32x4 sblo[SH ? NSD : 1], sbhi[SH ? NSD : 1];
  uint32_t sbs[SH ? NSD : 1];
  if constexpr (SH) {
    if (wave == 1) shared1_w2_rows<true, NSD>(sh, tile, sblo, sbhi, sbs);
  }
  const float sv = fr.survival != nullptr ? fr.survival[0] : 1.0f;
  TopkState<RP> st;
  topk_begin<RP>(st, fr.logits, a.E);
  const uint32_t ev = handoff_epoch_issue<GRAPH>(ho);          // the graph form's call counter
  const bool live = fr.survival == nullptr || !(sv < fr.skip_below);
  if (!live) {                                                  // no bucket: +0 (workgroup-uniform)
    if (tid < L1_COLS) a.y[tile * L1_COLS + tid] = 0.f;
    if constexpr (!SH) return;
  }
  u32x4 bw[2][CT][NSD];
  uint32_t bs[2][CT][NSD];
  if (live) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {                               // branch-free: a slot past k reloads slot k - 1's rows
      const int jj = min(wave + 4 * u, k - 1);
      topk_rounds<RP>(st, jj + 1);
      const int64_t r0 = (int64_t)__builtin_amdgcn_readlane(st.idx, jj) * H + tile * L1_COLS + col;
#pragma unroll
      for (int t = 0; t < CT; ++t) load_w2_tile<NSD>(a.w2, a.w2_sc, r0 + 16 * t, I, g, bw[u][t], bs[u][t]);
    }
  }
  topk_rounds<RP>(st, k);
  const float wt = slot_weight(st.val, k);                      // lane j: the weight of slot j
  for (int idx = lane; idx < 2 * (QP - I); idx += 64) {         // this wavefront's rows: K past I reads zeros
    const int jj = wave + 4 * (idx / (QP - I));
    q1[jj][I + idx % (QP - I)] = 0;
  }
  for (int idx = lane; idx < 2 * (NSD * 4 - nb); idx += 64)
    s1[wave + 4 * (idx / (NSD * 4 - nb))][nb + idx % (NSD * 4 - nb)] = 127;
  // the slots' words: a block's nine words sit at the start of its own
  // 128-byte line and are read as five 16-byte chunks; lane l reads chunks
  // c = l and c = 64 + l of each slot (block c / 5, parts 2 (c % 5) and
  // 2 (c % 5) + 1; part 9 is padding; parts 0..7: four codes, part 8: the
  // scale code)
  const int nchunks = nb * L1_BCHUNKS, nwp = l1_slot_words(I);
  const uint32_t tag = handoff_tag<GRAPH>(ho, ev);
  uint32_t pending = live ? (wave < k ? 1u : 0u) | (wave + 4 < k ? 2u : 0u) : 0u;
  if constexpr (SH) pending |= 4u;                              // this wavefront's share of the shared words
  while (pending) {
    u32x4 v[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t bytes = (pending >> u) & 1u ? (uint32_t)nwp * 8u : 0u;   // 0: reads nothing
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(ho.words + (int64_t)(wave + 4 * u) * nwp), (short)0, bytes, 0x00020000);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 64 * h + lane;
        v[u][h] = __builtin_amdgcn_raw_buffer_load_b128(r, (c / L1_BCHUNKS) * 128 + (c % L1_BCHUNKS) * 16, 0, 17);
      }
    }
    u32x4 sv4[2];
    if constexpr (SH) shared1_words_issue(swords, sh.I, (pending & 4u) != 0u, sv4);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if ((pending >> u) & 1u) {                                // wavefront-uniform
        bool ok = true;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 2; ++e)
            ok = ok && (64 * h + lane >= nchunks || 2 * ((64 * h + lane) % L1_BCHUNKS) + e >= L1_HWORDS ||
                        v[u][h][2 * e + 1] == tag);
        if (__ballot(ok) == ~0ull) {
          const int jj = wave + 4 * u;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int c = 64 * h + lane, blk = c / L1_BCHUNKS, part = 2 * (c % L1_BCHUNKS) + e;
              if (c < nchunks && part < L1_HWORDS) {
                if (part < 8) *reinterpret_cast<uint32_t*>(&q1[jj][32 * blk + 4 * part]) = v[u][h][2 * e];
                else s1[jj][blk] = (uint8_t)v[u][h][2 * e];
              }
            }
          __builtin_amdgcn_s_waitcnt(0xC07F);                   // lgkmcnt(0): the row is in LDS
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int t = 0; t < CT; ++t) {
            v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NSD; ++s) {
              if (s < nsteps) {
                const int klo = s * KSTEP + g * 16;
                const bool bv = 4 * s + g < nb;
                const u32x4 alo = *reinterpret_cast<const u32x4*>(&q1[jj][klo]);
                const u32x4 ahi = *reinterpret_cast<const u32x4*>(&q1[jj][klo + 64]);
                acc = mfma_fp8_fp4(fp8_operand(alo, ahi), fp4_operand_masked(bw[u][t][s], bv), acc,
                                   s1[jj][4 * s + g], bs[u][t][s]);
              }
            }
            if (g == 0) olds[jj][16 * t + col] = acc[0];        // row 0 of the tile
          }
          pending &= ~(1u << u);
        }
      }
    }
    if constexpr (SH) {
      if ((pending & 4u) && shared1_words_take(sv4, sh.I, tag, sav)) pending &= ~4u;
    }
    if (pending == 0) break;
    if ((long long)(wall_clock64() - t0) > ho.limit) {
      if (lane == 0) __hip_atomic_fetch_or(ho.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  lds_barrier();
  if (wave == 0 && live) {
    float ov[8];                                                // every slot's product read at once (k <= 8)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) ov[jj] = olds[jj][lane & (L1_COLS - 1)];
    float acc = 0.f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      if (jj < k) acc = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), jj)), ov[jj], acc);
    if (lane < L1_COLS) a.y[tile * L1_COLS + lane] = acc;
  }
  if constexpr (SH) {
    shared1_requant<NSD>(sh, sav, sq1, ss1, tile == 0);
    lds_barrier();
    if (wave == 1) shared1_chain<NSD>(sh, tile, sq1, ss1, sblo, sbhi, sbs);
  }
}

// Workgroups [0, k I / 32): routed gate/up; SH: [k I / 32, ho.nprod) the
// shared expert's gate/up (8 intermediate columns each, its words in the
// shared workspace's parts region); then H / 16 down workgroups.
template <int NS, bool EXACT, int RP, int NSD, bool SH, bool GRAPH>
__global__ __launch_bounds__(256) void layer1_kernel(FfnArgs a, float* __restrict__ abuf, float* __restrict__ h,
                                                     uint8_t* __restrict__ qws, uint8_t* __restrict__ qsc_ws,
                                                     FusedRoute fr, Handoff ho, Shared1Args sh) {
  const int nr = a.k * (a.I / 32);
  if ((int)blockIdx.x >= ho.nprod)
    layer1_down<NSD, RP, SH, GRAPH>(a, fr, ho, (int)blockIdx.x - ho.nprod, sh, reinterpret_cast<const uint64_t*>(sh.pbuf));
  else if (SH && (int)blockIdx.x >= nr)
    shared1_gate_up8<GRAPH>(sh, reinterpret_cast<uint64_t*>(sh.pbuf), ho, (int)blockIdx.x - nr);
  else
    layer1_gate_up<NS, EXACT, RP, GRAPH>(a, abuf, h, qws, qsc_ws, fr, ho);
}

// ========================================================== prefill path ==
// (measured: 256-row tiles, eight wavefronts and one workgroup per CU, which
// halve the weight re-reads, ran at 505-539 us against 474 us, bitwise equal)
constexpr int GU_BM = 128;                        // expert tile rows
constexpr int GU_BN = 256;                        // W13 rows per tile (128 intermediate columns)
constexpr int GU_ICOLS = GU_BN / 2;
constexpr int GU_STAGES = 2;                      // LDS stages per workgroup
constexpr int GU_NT = 2 * GU_BM;                  // threads: one wavefront per 64 rows x 64 columns
constexpr int GU_WG_PER_CU = GU_BM == 128 ? 4 / GU_STAGES : 1;   // workgroups resident per CU (LDS-bound)

// LDS slot (16-byte chunk) of chunk c of tile row r.  A 16-byte LDS read is
// served eight lanes at a time, and the eight lanes of an operand read are
// eight consecutive rows at one chunk: the swizzles put those eight chunks
// at eight distinct 16-byte positions of a 128-byte bank sweep.  Activation
// rows are 128 bytes (8 chunks): position c ^ (r mod 8).  Weight rows are 64
// bytes (4 chunks, two rows per sweep): position 4 (r mod 2) + (c ^ (r / 2
// mod 4)).
__device__ __forceinline__ int a_swz(int r) { return r & 7; }
__device__ __forceinline__ int b_swz(int r) { return (r >> 1) & 3; }
__device__ __forceinline__ int a_phys(int r, int c) { return r * 8 + (c ^ a_swz(r)); }
__device__ __forceinline__ int b_phys(int r, int c) { return r * 4 + (c ^ b_swz(r)); }

struct GuStage {
  u32x4 a[GU_BM * 8];                             // [row][8 chunks] swizzled
  u32x4 b[GU_BN * 4];                             // [row][4 chunks] swizzled
  uint32_t as[GU_BM];
  uint32_t bs[GU_BN];
};

// Gate/up over an expert tile of up to 128 rows and 128 intermediate columns
// (256 W13 rows: the 128 gate rows, then the 128 up rows).  Wavefront (wm,
// wn) computes rows [64 wm, 64 wm + 64) x intermediate columns [64 wn, 64 wn
// + 64): four 16-row A tiles against eight 16-row B tiles (4 gate + 4 up).
// One MFMA step (K = 128) per stage; the gathered activation rows (16 KB),
// the weight rows (16 KB) and their scale dwords go straight from global
// memory into one of NSTG LDS buffers (no registers), NSTG - 1 stages ahead
// of the matrix cores; within a stage each activation fragment is read from LDS
// while the previous one is multiplied.  Each lane fetches the global chunk that belongs at its
// LDS slot, so the buffers come out XOR-swizzled by 16-byte chunk and the 16
// rows one MFMA operand read touches fall in distinct banks.
template <int NSTG>
__global__ __launch_bounds__(GU_NT, GU_WG_PER_CU) void gu_prefill_kernel(FfnArgs a, uint8_t* __restrict__ qws,
                                                                         uint8_t* __restrict__ qsc_ws,
                                                                         float* __restrict__ h, int Tk,
                                                                         int* __restrict__ queue) {
  constexpr int NBD = GU_BN * 4 / GU_NT;          // B chunk DMAs per thread per stage
  constexpr int DMA_PER_STAGE = 4 + NBD + 2;      // per thread: 4 A + NBD B chunks, 1 A + 1 B scale dword
  __shared__ int tile_start[MAX_E + 1];
  __shared__ int tok[GU_BM];
  __shared__ GuStage st[NSTG];
  build_tiles(a.offsets, a.E, GU_BM, tile_start);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int H = a.H, I = a.I, nb = I / 32;
  const int nsteps = H / KSTEP;
  const uint32_t st_lds = __builtin_amdgcn_readfirstlane(lds_addr(&st[0]));   // LDS byte address of stage 0
  const int nct = (I + GU_ICOLS - 1) / GU_ICOLS;
  const int nitems = tile_start[a.E] * nct;
  __shared__ int s_item;
  int qpos = 0;                                                 // queue position (thread 0)

  for (;;) {
    lds_barrier();                                              // previous item's LDS reads are done
    if (tid == 0) s_item = queue_next(queue, nitems, qpos);
    lds_barrier();
    const int item = s_item;
    if (item < 0) break;
    const int tile = item / nct, ct = item % nct;
    const int e = tile_expert(tile_start, a.E, tile);
    const int p0 = a.offsets[e] + (tile - tile_start[e]) * GU_BM;
    int nrows = a.offsets[e + 1] - p0;
    nrows = nrows > GU_BM ? GU_BM : nrows;
    if (p0 < 0 || p0 + nrows > Tk) nrows = 0;
    const int c0 = ct * GU_ICOLS;                               // first intermediate column of the tile
    const int ncols = min(GU_ICOLS, I - c0);
    if (tid < GU_BM) {
      int t = -1;
      if (tid < nrows) {
        const int pr = a.perm[p0 + tid];
        t = (pr >= 0 && pr < Tk) ? pr / a.k : -1;
      }
      tok[tid] = t;
    }
    lds_barrier();

    // sources of this thread's LDS slots (rows past the tile read a valid
    // row whose results are discarded: rows and columns are independent)
    // (byte offsets from wavefront-uniform bases: the activations, and this
    // expert's weights and scales; T * H < 2^32 is checked at the boundary)
    uint32_t aoff[4], boff[NBD];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p = j * GU_NT + tid;
      const int r = p >> 3, c = (p & 7) ^ a_swz(r);
      const int t = tok[r];
      aoff[j] = (uint32_t)(t < 0 ? 0 : t) * (uint32_t)H + c * 16;
    }
#pragma unroll
    for (int j = 0; j < NBD; ++j) {
      const int p = j * GU_NT + tid;
      const int rb = p >> 2, cb = (p & 3) ^ b_swz(rb);
      const int icol = rb & 127;
      const int r13 = (rb < 128 ? 0 : I) + c0 + (icol < ncols ? icol : 0);
      boff[j] = (uint32_t)r13 * (uint32_t)(H / 2) + cb * 16;
    }
    const int ra = wave * 32 + (lane & 31);                     // A scale row of this lane (lanes < 32)
    const int tas = tok[ra];
    const uint32_t asoff = (uint32_t)(tas < 0 ? 0 : tas) * (uint32_t)(H / 32);
    // B scale row of this lane; with more than four wavefronts the others
    // repeat the first four's transfers (same source, same LDS slot)
    const int rbs = (wave & 3) * 64 + lane, icol_s = rbs & 127;
    const uint32_t bsoff = (uint32_t)((rbs < 128 ? 0 : I) + c0 + (icol_s < ncols ? icol_s : 0)) * (uint32_t)(H / 32);
    const uint8_t* w13e = a.w13 + (int64_t)e * 2 * I * (H / 2);
    const uint8_t* w13se = a.w13_sc + (int64_t)e * 2 * I * (H / 32);

    auto issue = [&](int s, int buf) {
      const uint32_t d = st_lds + buf * (uint32_t)sizeof(GuStage);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dma16_to_lds(a.x + s * KSTEP, aoff[j], d + (uint32_t)offsetof(GuStage, a) + (j * GU_NT + wave * 64) * 16);
#pragma unroll
      for (int j = 0; j < NBD; ++j)
        dma16_to_lds(w13e + s * 64, boff[j], d + (uint32_t)offsetof(GuStage, b) + (j * GU_NT + wave * 64) * 16);
      if (lane < 32) dma4_to_lds(a.x_sc + s * 4, asoff, d + (uint32_t)offsetof(GuStage, as) + wave * 32 * 4);
      dma4_to_lds(w13se + s * 4, bsoff, d + (uint32_t)offsetof(GuStage, bs) + (wave & 3) * 64 * 4);
    };

    v4f acc[4][8];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 8; ++n) acc[m][n] = v4f{0.f, 0.f, 0.f, 0.f};
    // waves whose rows or columns fall outside the tile skip the matrix work,
    // and 16-row subtiles past the tile's rows are skipped
    const bool wact = wm * 64 < nrows && wn * 64 < ncols;
    const int msub = min(4, (nrows - wm * 64 + 15) / 16);

    // one stage: the eight weight fragments and the first activation
    // fragment are read, then each group of eight MFMAs runs while the next
    // activation fragment is on its way from LDS
    // one stage: the eight weight fragments and the first activation
    // fragment are read, then each group of eight MFMAs runs while the next
    // activation fragment is on its way from LDS; the groups of 16-row
    // subtiles past the tile's rows are skipped (wavefront-uniform branches)
    // lane parts of the swizzled LDS indices (row bases are multiples of 16,
    // so the swizzle depends on the lane alone)
    const int bl = b_phys(col, g), al0 = a_phys(col, g), al1 = a_phys(col, 4 + g);
    auto compute = [&](const GuStage& S) {
      if (!wact) return;
      v8i bf[8];
      uint32_t bsv[8];
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const int rb = (n < 4 ? 0 : 128) + wn * 64 + (n & 3) * 16;
        bf[n] = fp4_operand(S.b[rb * 4 + bl]);
        bsv[n] = S.bs[rb + col];
      }
      const int ra0 = wm * 64;
      v8i af = fp8_operand(S.a[ra0 * 8 + al0], S.a[ra0 * 8 + al1]);
      uint32_t sa = S.as[ra0 + col];
      __builtin_amdgcn_sched_barrier(0);                        // all of the stage's first reads in flight at once
#pragma unroll
      for (int n = 0; n < 8; ++n) bsv[n] >>= 8 * g;
      sa >>= 8 * g;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        v8i an;
        uint32_t san = 0;
        if (m < 3) {
          const int ra = wm * 64 + (m + 1) * 16;
          an = fp8_operand(S.a[ra * 8 + al0], S.a[ra * 8 + al1]);
          san = S.as[ra + col];
        }
        __builtin_amdgcn_sched_barrier(0);                      // the next fragment's reads stay ahead of these MFMAs
        if (m < msub) {
#pragma unroll
          for (int n = 0; n < 8; ++n) acc[m][n] = mfma_fp8_fp4(af, bf[n], acc[m][n], sa, bsv[n]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (m < 3) {
          af = an;
          sa = san >> (8 * g);
        }
      }
    };
    // stage s: wait for its own DMA (later stages stay in flight), make every
    // wavefront's part visible, refill the buffer freed by stage s - 1, multiply
    auto step = [&](int s, const GuStage& S, int refill) {
      const int later = min(NSTG - 2, nsteps - 1 - s);          // stages after s already in flight
      if (later >= 2) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * DMA_PER_STAGE) : "memory");
      else if (later == 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(DMA_PER_STAGE) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
      if (s + NSTG - 1 < nsteps) issue(s + NSTG - 1, refill);
      compute(S);
    };
#pragma unroll
    for (int j = 0; j < NSTG - 1; ++j)
      if (j < nsteps) issue(j, j);
    for (int s = 0; s < nsteps; s += NSTG) {
#pragma unroll
      for (int j = 0; j < NSTG; ++j)
        if (s + j < nsteps) step(s + j, st[j], (j + NSTG - 1) % NSTG);
    }

    // epilogue: SwiGLU + requant; one block of 32 = two 16-column subtiles of one row
    if (wact) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint32_t sc;
            const uint32_t d = swiglu_requant2(acc[m][2 * blk][i], acc[m][4 + 2 * blk][i], acc[m][2 * blk + 1][i],
                                               acc[m][5 + 2 * blk][i], &sc);
            const int row = wm * 64 + m * 16 + 4 * g + i;
            const int cb = c0 + wn * 64 + blk * 32;           // first column of the block
            if (row < nrows && cb < I) {
              uint8_t* qrow = qws + (int64_t)(p0 + row) * I;
              qrow[cb + col] = (uint8_t)d;
              qrow[cb + 16 + col] = (uint8_t)(d >> 8);
              if (col == 0) qsc_ws[(int64_t)(p0 + row) * nb + cb / 32] = (uint8_t)sc;
              if (h != nullptr) {                               // diagnostics only: the fp32 gate/up values
                float* hrow = h + (int64_t)(p0 + row) * 2 * I;
                hrow[cb + col] = acc[m][2 * blk][i];
                hrow[cb + 16 + col] = acc[m][2 * blk + 1][i];
                hrow[I + cb + col] = acc[m][4 + 2 * blk][i];
                hrow[I + cb + 16 + col] = acc[m][5 + 2 * blk][i];
              }
            }
          }
        }
      }
    }
  }
}

// Down, weight-stationary, one workgroup of eight wavefronts per CU taking
// (expert, 256 W2 rows) items from the work queue: each wavefront keeps its
// 32 W2 rows (two 16-row B tiles, whole K = I) in registers and walks all of
// the expert's 32-row tiles.  Every global -> LDS transfer is an LDS DMA
// issued well ahead of its use, and the kernel counts them itself (vmcnt):
//  - the next tile's intermediate rows and scale bytes (this tile's MFMAs
//    read the other of two buffers);
//  - the next item's W2 slice (rows and scales, into one LDS buffer, read
//    into registers at the item's first tile), requested at this item's first
//    tile: the queue runs two items ahead, so the next item is known.
// Results leave through a per-wavefront LDS transpose, 8 rows x 128 bytes per
// store; every wavefront issues the same number of memory instructions per
// tile (rows past the tile go to a scratch row of the workspace), so the
// counts are exact.
constexpr int DN_WAVES = 8;
constexpr int DN_NT = 64 * DN_WAVES;
constexpr int DN_ROWS_T = 32;                     // intermediate rows per tile
constexpr int DN_NCOLS = 256;                     // W2 rows per item
constexpr int DN_QPITCH = 5 * KSTEP + 16;         // LDS pitch of an intermediate row (K past I zero)
constexpr int DN_TPITCH = 36;                     // transpose rows: 32 floats + 4 (bank spread)
constexpr int DN_W2_DMA = 10;                     // W2 row DMAs per wavefront per item (256 rows x <= 20 chunks)
constexpr int DN_W2S_DMA = 3;                     // W2 scale dword DMAs per wavefront per item
constexpr int DN_TILE_ST = 4;                     // per tile: stores (2 subtiles x 2 halves)
struct DnLds {
  uint8_t q[2][DN_ROWS_T][DN_QPITCH];             // intermediate rows, two buffers
  uint8_t qs[2][DN_WAVES * 256];                  // their scale bytes (DMA'd as dwords; waves 3.. fill slack)
  u32x4 w2[DN_WAVES * DN_W2_DMA * 64];            // W2 slice: row r, 16-byte chunk c at r * (nb + 1) + c
  uint32_t w2s[DN_WAVES * DN_W2S_DMA * 64];       // its scale bytes, row-major [256][nb]
  float tr[DN_WAVES][16][DN_TPITCH];
};

template <int NS>
__global__ __launch_bounds__(DN_NT, 1) void down_prefill_kernel(FfnArgs a, const uint8_t* __restrict__ qws,
                                                                const uint8_t* __restrict__ qsc_ws,
                                                                float* __restrict__ o, float* __restrict__ junk, int Tk,
                                                                int* __restrict__ queue) {
  __shared__ int tile_start[MAX_E + 1];
  __shared__ int s_slot[2];
  __shared__ __attribute__((aligned(16))) DnLds L;
  build_tiles(a.offsets, a.E, 0, tile_start);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int H = a.H, I = a.I, nb = I / 32, nch = nb + 1;        // W2 row: nb 16-byte chunks + 1 pad
  const int nsteps = (I + KSTEP - 1) / KSTEP;                   // <= NS
  const int q16 = I / 16;
  const int nnt = H / DN_NCOLS;
  const int nitems = tile_start[a.E] * nnt;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(&L));
  // K past I of the intermediate rows reads zeros: staging never writes there
  for (int idx = tid; idx < 2 * DN_ROWS_T * (NS * KSTEP - I); idx += DN_NT) {
    const int bf = idx / (DN_ROWS_T * (NS * KSTEP - I)), rem = idx % (DN_ROWS_T * (NS * KSTEP - I));
    L.q[bf][rem / (NS * KSTEP - I)][I + rem % (NS * KSTEP - I)] = 0;
  }

  struct Item { int e, pbeg, cnt, ntiles, nt; };
  auto describe = [&](int item) {
    Item it;
    it.e = __builtin_amdgcn_readfirstlane(tile_expert(tile_start, a.E, item / nnt));
    it.pbeg = a.offsets[it.e];
    it.cnt = a.offsets[it.e + 1] - it.pbeg;
    if (it.pbeg < 0 || it.pbeg + it.cnt > Tk) it.cnt = 0;
    it.ntiles = (it.cnt + DN_ROWS_T - 1) / DN_ROWS_T;
    it.nt = item % nnt;
    return it;
  };
  // one tile's rows and scale bytes into buffer bf: 4 row DMAs and one scale
  // DMA per wavefront (rows past the tile repeat its last row; waves past the
  // tile's scale dwords load a valid dword into slack)
  auto stage = [&](const Item& it, int t, int bf) {
    const int p0 = min(it.pbeg + t * DN_ROWS_T, Tk - 1);
    const int nrows = max(1, min(DN_ROWS_T, it.cnt - t * DN_ROWS_T));   // (an item without rows stages row p0)
#pragma unroll
    for (int i = 0; i < DN_ROWS_T / DN_WAVES; ++i) {
      const int r = wave + DN_WAVES * i;
      if (lane < q16)
        dma16_to_lds(qws, (uint32_t)(min(p0 + min(r, nrows - 1), Tk - 1) * I + lane * 16),
                     lds0 + (uint32_t)offsetof(DnLds, q) + (bf * DN_ROWS_T + r) * DN_QPITCH);
    }
    const uint32_t sb = (uint32_t)p0 * nb & ~3u;               // first scale dword of the tile
    const uint32_t ndw = ((uint32_t)(p0 * nb & 3) + DN_ROWS_T * nb + 3) / 4;
    const uint32_t d = wave * 64 + lane;
    dma4_to_lds(qsc_ws, sb + 4 * (d < ndw ? d : 0), lds0 + (uint32_t)offsetof(DnLds, qs) + bf * DN_WAVES * 256 + wave * 256);
  };
  // the item's W2 slice: rows [nt * 256, nt * 256 + 256) of expert e
  auto stage_w2 = [&](const Item& it) {
    const uint8_t* w2e = a.w2 + (int64_t)it.e * H * (I / 2) + (int64_t)it.nt * DN_NCOLS * (I / 2);
#pragma unroll
    for (int i = 0; i < DN_W2_DMA; ++i) {
      const int slot = (wave * DN_W2_DMA + i) * 64 + lane;       // 16-byte slot of the LDS slice
      const int r = slot / nch, c = slot % nch;
      const bool ok = r < DN_NCOLS && c < nb;
      dma16_to_lds(w2e, ok ? (uint32_t)(r * (I / 2) + c * 16) : 0u,
                   lds0 + (uint32_t)offsetof(DnLds, w2) + (wave * DN_W2_DMA + i) * 1024);
    }
    const uint8_t* w2se = a.w2_sc + ((int64_t)it.e * H + (int64_t)it.nt * DN_NCOLS) * nb;
#pragma unroll
    for (int i = 0; i < DN_W2S_DMA; ++i) {
      const int dw = (wave * DN_W2S_DMA + i) * 64 + lane;
      dma4_to_lds(w2se, dw < DN_NCOLS * nb / 4 ? 4u * dw : 0u,
                  lds0 + (uint32_t)offsetof(DnLds, w2s) + (wave * DN_W2S_DMA + i) * 256);
    }
  };

  // the workgroup's items, two ahead: its k-th item sits in s_slot[k & 1]
  int qpos = 0;                                                 // queue position (thread 0)
  if (tid == 0) {
    const int i0 = queue_next(queue, nitems, qpos);
    s_slot[0] = i0;
    s_slot[1] = i0 < 0 ? -1 : queue_next(queue, nitems, qpos);
  }
  lds_barrier();
  int cur = __builtin_amdgcn_readfirstlane(s_slot[0]);
  if (cur < 0) return;
  Item C = describe(cur);
  stage_w2(C);
  if (C.ntiles > 0) stage(C, 0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  u32x4 bw[2][NS];
  uint32_t bs[2][NS];
  int buf = 0;
  for (int k = 0;; ++k) {
    const int n0 = C.nt * DN_NCOLS + wave * 32;                 // this wavefront's first W2 row (= output column)
    int raw = 0;
    int nxt = -1;
    Item N = C;
    const int ntl = C.ntiles > 0 ? C.ntiles : 1;                // an item without rows only passes the queue on
    for (int t = 0; t < ntl; ++t) {
      const bool last = t + 1 == ntl;
      lds_barrier();                                            // tile t (and at t = 0 the W2 slice) in LDS
      if (t == 0) {
        // the next item (published at the previous item's last tile, before this barrier)
        nxt = __builtin_amdgcn_readfirstlane(s_slot[(k + 1) & 1]);
        N = describe(nxt < 0 ? cur : nxt);
        if (tid == 0) raw = queue_take(queue, qpos);           // item k + 2; consumed after the last tile
        // this wavefront's W2 rows into registers, then the slice is free
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int r = wave * 32 + n * 16 + col;
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            const int c = 4 * s + g;
            const u32x4 v = L.w2[r * nch + (c < nb ? c : 0)];
            bw[n][s] = c < nb ? v : u32x4{0u, 0u, 0u, 0u};      // K past I multiplies zeros
            bs[n][s] = reinterpret_cast<const uint8_t*>(L.w2s)[r * nb + (c < nb ? c : 0)];
          }
        }
        lds_barrier();
        // next: the following tile (or the next item's first), then the next item's W2
        if (!last) stage(C, t + 1, buf ^ 1);
        else stage(N, 0, buf ^ 1);
        stage_w2(N);
      } else {
        if (!last) stage(C, t + 1, buf ^ 1);
        else stage(N, 0, buf ^ 1);
      }

      if (C.ntiles > 0) {
        const int p0 = C.pbeg + t * DN_ROWS_T, nrows = min(DN_ROWS_T, C.cnt - t * DN_ROWS_T);
        const uint8_t* qsb = L.qs[buf] + ((uint32_t)p0 * nb & 3u);
        v4f acc[2][2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int n = 0; n < 2; ++n) acc[m][n] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          if (s < nsteps) {
            const int klo = s * KSTEP + g * 16, c = 4 * s + g;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              const int r = m * 16 + col;
              const v8i av = fp8_operand(*reinterpret_cast<const u32x4*>(&L.q[buf][r][klo]),
                                         *reinterpret_cast<const u32x4*>(&L.q[buf][r][klo + 64]));
              const uint32_t sa = c < nb ? (uint32_t)qsb[r * nb + c] : 127u;
#pragma unroll
              for (int n = 0; n < 2; ++n)
                acc[m][n] = mfma_fp8_fp4(av, fp4_operand(bw[n][s]), acc[m][n], sa, bs[n][s]);
            }
          }
        }
        // results: 16 rows x 32 columns per subtile through the transpose,
        // 8 rows x 128 bytes per store (rows past the tile: the scratch row)
        float(*Tt)[DN_TPITCH] = L.tr[wave];
        const int rr = lane >> 3, c4 = (lane & 7) * 4;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int n = 0; n < 2; ++n) Tt[4 * g + i][n * 16 + col] = acc[m][n][i];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int row = m * 16 + h * 8 + rr;
            const v4f v = *reinterpret_cast<const v4f*>(&Tt[h * 8 + rr][c4]);
            float* dst = row < nrows ? o + (int64_t)(p0 + row) * H + n0 + c4 : junk + c4;
            __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(dst));   // read once, by the combine
          }
        }
      } else {
        // keep the per-tile store count: four stores to the scratch row
#pragma unroll
        for (int i = 0; i < DN_TILE_ST; ++i)
          __builtin_nontemporal_store(v4f{0.f, 0.f, 0.f, 0.f}, reinterpret_cast<v4f*>(junk + (lane & 7) * 4));
      }
      if (last && tid == 0) s_slot[k & 1] = queue_finish(queue, nitems, qpos, raw);
      // the next tile's DMAs have landed once at most the newer operations
      // (the W2 slice at t = 0, then this tile's stores) are outstanding
      // (at an item's only tile the next W2 slice must have landed as well)
      if (t == 0 && !last) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(DN_W2_DMA + DN_W2S_DMA + DN_TILE_ST) : "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(DN_TILE_ST) : "memory");
      buf ^= 1;
    }
    if (nxt < 0) break;
    cur = nxt;
    C = N;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ============================================================== combine ===
// y_t = sum_j w_tj * o[slot_pos[t][j]], j = 0..k-1 in order; 4 columns per
// thread.  Every slot's position, weight and output are requested before the
// first add (a dead slot reads row 0 and is skipped by a select).  o is read
// once and y written once: both bypass the caches' retention (nontemporal).
template <int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o, const float* __restrict__ w,
                                                      const int32_t* __restrict__ slot_pos, int T, int H, int k, int Tk,
                                                      float* __restrict__ y) {
  const int n = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (n >= H) return;
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
    int p[KMAX];
    float wj[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int jj = j < k ? j : 0;
      p[j] = slot_pos[(int64_t)t * k + jj];
      wj[j] = w[(int64_t)t * k + jj];
    }
    v4f v[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const bool ok = j < k && p[j] >= 0 && p[j] < Tk;
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(o + (int64_t)(ok ? p[j] : 0) * H + n));
    }
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const bool ok = j < k && p[j] >= 0 && p[j] < Tk;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = ok ? fmaf(wj[j], v[j][c], acc[c]) : acc[c];
    }
    __builtin_nontemporal_store(acc, reinterpret_cast<v4f*>(y + (int64_t)t * H + n));
  }
}

// ================================================================= host ===
static size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// workspace: [q: Tk*I][q_sc: Tk*I/32][o: Tk*H fp32][queue counters][scratch row][T = 1: handoff words],
// each 256-byte aligned
void ffn_ws_layout(int T, int H, int I, int k, size_t* off_q, size_t* off_q_sc, size_t* off_o) {
  const size_t Tk = (size_t)T * k;
  *off_q = 0;
  *off_q_sc = align256(Tk * I);
  *off_o = *off_q_sc + align256(Tk * (I / 32));
  (void)H;
}

size_t ffn_ws_bytes(int T, int H, int E, int I, int k) {
  (void)E;
  size_t q, qs, o;
  ffn_ws_layout(T, H, I, k, &q, &qs, &o);
  // o holds T*k rows of H floats (per-slot outputs) or, at T = 1, of I floats (the SwiGLU rows);
  // then the work-queue counters (at T = 1: the handoff status word), a scratch row and, at T = 1,
  // the single-launch layer's handoff words (nine 8-byte words per block of 32 intermediate values)
  return o + align256((size_t)T * k * (H > I ? H : I) * 4) + 256 + 256 +
         (T == 1 ? align256((size_t)k * l1_slot_words(I) * 8) : 0);
}

// Row pairs at or below which the decode kernels are chosen.
constexpr int DECODE_MAX_PAIRS = 1024;

static bool decode_path_ok(int H, int I) { return H % KSTEP == 0 && H <= KSTEP * DEC_MAX_STEPS && I <= MAX_I; }
static bool prefill_path_ok(int H, int I) { return H % PF_NCOLS == 0 && I <= PF_MAX_I; }

int ffn_resolve_path(int path, int64_t Tk, int H, int I) {
  const bool dec = decode_path_ok(H, I), pre = prefill_path_ok(H, I);
  if (path == 1) return dec ? 1 : 0;
  if (path == 2) return pre ? 2 : 0;
  if (dec && (Tk <= DECODE_MAX_PAIRS || !pre)) return 1;
  return pre ? 2 : 0;
}

// Diagnostic phase events of this thread's FFN calls (set_ffn_phase_events).
static thread_local hipEvent_t g_phase_ev[4];
static thread_local bool g_phase_on = false;
void set_ffn_phase_events(const hipEvent_t* ev, int n) {
  g_phase_on = n == 4;
  for (int i = 0; i < 4; ++i) g_phase_ev[i] = g_phase_on ? ev[i] : nullptr;
}
static inline void phase(int i, hipStream_t stream) {
  if (g_phase_on) (void)hipEventRecord(g_phase_ev[i], stream);
}

// gate/up of one row: the NS / EXACT variant for H = 128 hs
template <int RP, bool SH, int EPL>
static void launch_gu1(int hs, int groute, int gshared, hipStream_t stream, const FfnArgs& a, float* abuf, float* h,
                       int Tk, const FusedRoute& fr, const Shared1Args& sh) {
  const dim3 grid(groute + gshared);
#define MX_GU1(NS_, EX_) \
  hipLaunchKernelGGL((gu1_kernel<NS_, EX_, RP, SH, EPL>), grid, dim3(64), 0, stream, a, abuf, h, Tk, fr, sh, groute)
  if (hs == 32) MX_GU1(32, true);
  else if (hs == 40) MX_GU1(40, true);
  else if (hs == 16) MX_GU1(16, true);
  else if (hs == 8) MX_GU1(8, true);
  else if (hs <= 4) MX_GU1(4, false);
  else if (hs <= 8) MX_GU1(8, false);
  else if (hs <= 16) MX_GU1(16, false);
  else if (hs <= 32) MX_GU1(32, false);
  else MX_GU1(40, false);
#undef MX_GU1
}

// The single-launch layer of one row: k * I / 32 gate/up workgroups and
// H / 32 down + combine workgroups in one grid.
template <int RP, int NSD, bool SH = false, bool GRAPH = false>
static void launch_layer1(int hs, hipStream_t stream, const FfnArgs& a, float* abuf, float* h, uint8_t* qws,
                          uint8_t* qsc, const FusedRoute& fr, const Handoff& ho, const Shared1Args& sh) {
  const dim3 grid(ho.nprod + a.H / L1_COLS);
#define MX_L1(NS_, EX_)                                                                                            \
  hipLaunchKernelGGL((layer1_kernel<NS_, EX_, RP, NSD, SH, GRAPH>), grid, dim3(256), 0, stream, a, abuf, h, qws, qsc, fr, \
                     ho, sh)
  if (hs == 32) MX_L1(32, true);
  else if (hs == 40) MX_L1(40, true);
  else if (hs == 16) MX_L1(16, true);
  else if (hs == 8) MX_L1(8, true);
  else if (hs <= 4) MX_L1(4, false);
  else if (hs <= 8) MX_L1(8, false);
  else if (hs <= 16) MX_L1(16, false);
  else if (hs <= 32) MX_L1(32, false);
  else MX_L1(40, false);
#undef MX_L1
}

static std::atomic<bool> g_layer1_onepass{true};
void set_layer1_onepass(bool on) { g_layer1_onepass.store(on); }
bool single_launch_on() { return g_layer1_onepass.load(); }

// A tag no earlier call of this process used (a random start, then +1 per
// call; unique over 2^32 calls).
__global__ void handoff_epoch_kernel(uint32_t* epoch) {
  if (threadIdx.x == 0)
    __hip_atomic_store(epoch, __hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) + 1u,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
hipError_t launch_handoff_epoch(uint32_t* epoch, hipStream_t stream) {
  hipLaunchKernelGGL(handoff_epoch_kernel, dim3(1), dim3(64), 0, stream, epoch);
  return hipGetLastError();
}

uint32_t next_call_tag() {
  static std::atomic<uint32_t> next{[] {
    uint64_t z = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() ^ (uint64_t)(uintptr_t)&next;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;               // splitmix64 finalizer
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return (uint32_t)(z ^ (z >> 31));
  }()};
  return next.fetch_add(1) & 0x7FFFFFFFu;                      // bit 31 marks the graph form's tags
}

// Wall-clock ticks in 20 ms on the current device (the limit of one consumer's waits).
long long handoff_limit_ticks() {
  static std::atomic<long long> ticks_per_ms[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  long long t = ticks_per_ms[dev].load();
  if (t == 0) {
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) khz = 100000;
    t = khz;
    ticks_per_ms[dev].store(t);
  }
  return 20 * t;
}

// gate/up for T > 1 and the down projection for T > 1 and T = 1, with the
// expert list's capacity chosen from E
template <int NS, bool EX>
static void launch_gu_decode(dim3 grid, size_t lds, hipStream_t stream, const FfnArgs& a, uint8_t* qws, uint8_t* qsc,
                             float* h, int Tk, int R) {
  if (epl_for(a.E) == 4) hipLaunchKernelGGL((gu_decode_kernel<NS, EX, 4>), grid, dim3(256), lds, stream, a, qws, qsc, h, Tk, R);
  else hipLaunchKernelGGL((gu_decode_kernel<NS, EX, 16>), grid, dim3(256), lds, stream, a, qws, qsc, h, Tk, R);
}
template <int NS>
static void launch_down_decode(dim3 grid, hipStream_t stream, const FfnArgs& a, const uint8_t* qws,
                               const uint8_t* qsc, float* o, int Tk) {
  if (epl_for(a.E) == 4) hipLaunchKernelGGL((down_decode_kernel<NS, 4>), grid, dim3(256), 0, stream, a, qws, qsc, o, Tk);
  else hipLaunchKernelGGL((down_decode_kernel<NS, 16>), grid, dim3(256), 0, stream, a, qws, qsc, o, Tk);
}
template <int NS>
static void launch_down_combine1(dim3 grid, hipStream_t stream, const FfnArgs& a, const float* abuf, uint8_t* qws,
                                 uint8_t* qsc, int Tk, const Shared1Args& sh, bool with_shared) {
  if (with_shared) {
    if (epl_for(a.E) == 4) hipLaunchKernelGGL((down_combine1_kernel<NS, true, 4>), grid, dim3(256), 0, stream, a, abuf, qws, qsc, Tk, sh);
    else hipLaunchKernelGGL((down_combine1_kernel<NS, true, 16>), grid, dim3(256), 0, stream, a, abuf, qws, qsc, Tk, sh);
  } else {
    if (epl_for(a.E) == 4) hipLaunchKernelGGL((down_combine1_kernel<NS, false, 4>), grid, dim3(256), 0, stream, a, abuf, qws, qsc, Tk, sh);
    else hipLaunchKernelGGL((down_combine1_kernel<NS, false, 16>), grid, dim3(256), 0, stream, a, abuf, qws, qsc, Tk, sh);
  }
}

hipError_t launch_ffn(const FfnArgs& a, void* ws, int path, hipStream_t stream, const char** variant,
                      const FusedRoute* fr, float* h, const Shared1Args* sh) {
  const int Tk = a.T * a.k;
  // the caller validated the shape; a path that cannot run it is never launched
  path = ffn_resolve_path(path, Tk, a.H, a.I);
  if (path == 0) return hipErrorInvalidValue;
  uint8_t* base = static_cast<uint8_t*>(ws);
  size_t oq, oqs, oo;
  ffn_ws_layout(a.T, a.H, a.I, a.k, &oq, &oqs, &oo);
  uint8_t* qws = base + oq;
  uint8_t* qsc = base + oqs;
  float* o = reinterpret_cast<float*>(base + oo);
  const size_t obytes = align256((size_t)Tk * (a.H > a.I ? a.H : a.I) * 4);
  int* queue = reinterpret_cast<int*>(base + oo + obytes);                 // work-queue counters
  float* junk = reinterpret_cast<float*>(base + oo + obytes + 256);        // scratch row
  const int cus = num_cus();
  const int max_active = a.E < Tk ? a.E : Tk;
  phase(0, stream);
  if (path == 1) {
    const int R = a.T < DEC_ROWS ? a.T : DEC_ROWS;               // rows of one expert never exceed T
    const size_t lds = (size_t)R * (a.H + 16) + (size_t)R * (a.H / KSTEP) * 4;
    const int gu_items = max_active * (a.I / 32);
    const int gu_grid = gu_items < cus * 2 ? gu_items : cus * 2;
    const int hs = a.H / KSTEP, is = (a.I + KSTEP - 1) / KSTEP;
    if (hs > DEC_MAX_STEPS || is > DOWN_MAX_STEPS) return hipErrorInvalidValue;   // the kernels' register arrays hold every step
    const dim3 g0(gu_grid);
#define MX_GU(NS_, EX_) launch_gu_decode<NS_, EX_>(g0, lds, stream, a, qws, qsc, h, Tk, R)
    const Shared1Args shv = sh ? *sh : Shared1Args{};
    if (a.T == 1) {
      // one wavefront per (pair, 8 intermediate columns); the SwiGLU rows go
      // to the o region; then the shared expert's gate/up parts, if any
      const int items = a.k * (a.I / 8);
      const int gr = items < cus * 8 ? items : cus * 8;
      const int gs = sh ? 2 * sh->I / 16 * shared1_nparts(a.H) : 0;
      // (the fused gate ranks the logits itself: the expert list is unused there)
      // One launch when the down projection fits a consumer wavefront (k <= 8,
      // I <= 640) and the stream is not being captured (a graph would replay
      // one tag; the two-launch path below has no tags).
      // With the shared expert (its I <= 640): its gate/up workgroups after
      // the routed ones, its down projection inside the down workgroups.
      // Under graph capture the same launch, preceded by the one-thread
      // kernel that advances the workspace's call counter (the tag source).
      hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
      if (fr && (!sh || sh->I <= 5 * KSTEP) && a.k <= 8 && is <= 5 && g_layer1_onepass.load() &&
          hipStreamIsCapturing(stream, &cap) == hipSuccess &&
          (cap == hipStreamCaptureStatusNone || cap == hipStreamCaptureStatusActive)) {
        uint32_t* status = reinterpret_cast<uint32_t*>(queue);     // then the call counter
        const bool graph = cap == hipStreamCaptureStatusActive;
        if (graph) {
          const hipError_t e = launch_handoff_epoch(status + 1, stream);
          if (e != hipSuccess) return e;
        }
        const Handoff ho{reinterpret_cast<uint64_t*>(base + oo + obytes + 512), status, graph ? 0u : next_call_tag(),
                         handoff_limit_ticks(), a.k * (a.I / 32) + (sh ? sh->I / 8 : 0), status + 1, graph ? 1 : 0};
        if (graph) {                                            // the graph form: one down-step count, NSD = 5
          if (sh && a.E <= 256) launch_layer1<4, 5, true, true>(hs, stream, a, o, h, qws, qsc, *fr, ho, *sh);
          else if (sh) launch_layer1<16, 5, true, true>(hs, stream, a, o, h, qws, qsc, *fr, ho, *sh);
          else if (a.E <= 256) launch_layer1<4, 5, false, true>(hs, stream, a, o, h, qws, qsc, *fr, ho, shv);
          else launch_layer1<16, 5, false, true>(hs, stream, a, o, h, qws, qsc, *fr, ho, shv);
        } else if (sh) {
          if (a.E <= 256) launch_layer1<4, 5, true>(hs, stream, a, o, h, qws, qsc, *fr, ho, *sh);
          else launch_layer1<16, 5, true>(hs, stream, a, o, h, qws, qsc, *fr, ho, *sh);
        } else if (is <= 2) {
          if (a.E <= 256) launch_layer1<4, 2>(hs, stream, a, o, h, qws, qsc, *fr, ho, shv);
          else launch_layer1<16, 2>(hs, stream, a, o, h, qws, qsc, *fr, ho, shv);
        } else {
          if (a.E <= 256) launch_layer1<4, 5>(hs, stream, a, o, h, qws, qsc, *fr, ho, shv);
          else launch_layer1<16, 5>(hs, stream, a, o, h, qws, qsc, *fr, ho, shv);
        }
        *variant = sh ? "layer1_shared:gate_up_topk+shared_gate_up+down_combine+shared_down (one launch)"
                      : "layer1:gate_up_topk+down_combine (one launch)";
        phase(1, stream);
        phase(2, stream);
        phase(3, stream);
        return hipGetLastError();
      }
      if (!fr && epl_for(a.E) == 4) launch_gu1<0, false, 4>(hs, gr, 0, stream, a, o, h, Tk, FusedRoute{}, shv);
      else if (!fr) launch_gu1<0, false, 16>(hs, gr, 0, stream, a, o, h, Tk, FusedRoute{}, shv);
      else if (sh && a.E <= 256) launch_gu1<4, true, 4>(hs, gr, gs, stream, a, o, h, Tk, *fr, shv);
      else if (sh) launch_gu1<16, true, 4>(hs, gr, gs, stream, a, o, h, Tk, *fr, shv);
      else if (a.E <= 256) launch_gu1<4, false, 4>(hs, gr, 0, stream, a, o, h, Tk, *fr, shv);
      else launch_gu1<16, false, 4>(hs, gr, 0, stream, a, o, h, Tk, *fr, shv);
    } else {
      if (hs == 32) MX_GU(32, true);
      else if (hs == 40) MX_GU(40, true);
      else if (hs == 16) MX_GU(16, true);
      else if (hs == 8) MX_GU(8, true);
      else if (hs <= 4) MX_GU(4, false);
      else if (hs <= 8) MX_GU(8, false);
      else if (hs <= 16) MX_GU(16, false);
      else if (hs <= 32) MX_GU(32, false);
      else MX_GU(40, false);
    }
#undef MX_GU
    phase(1, stream);
    if (a.T == 1) {
      const dim3 g1(a.H / 16 * (sh ? 2 : 1));                   // the shared expert's down tiles after the routed ones
#define MX_DC1(NS_) launch_down_combine1<NS_>(g1, stream, a, o, qws, qsc, Tk, shv, sh != nullptr)
      if (is <= 2) { MX_DC1(2); }
      else if (is <= 5) { MX_DC1(5); }
      else if (is <= 8) { MX_DC1(8); }
      else { MX_DC1(16); }
#undef MX_DC1
      *variant = sh ? "layer1_shared:gu1_decode_topk+shared_parts+down_combine1+shared_down"
                    : fr ? "layer1:gu1_decode_topk+down_combine1" : "ffn:gu1_decode+down_combine1";
      phase(2, stream);                                         // the down kernel also combines
      phase(3, stream);
      return hipGetLastError();
    }
    const int dn_items = max_active * (a.H / 128);
    const int dn_occ = DN_WG_PER_CU(is <= 2 ? 2 : is <= 5 ? 5 : is <= 8 ? 8 : 16, epl_for(a.E));
    const dim3 g2(dn_items < cus * dn_occ ? dn_items : cus * dn_occ);
    if (is <= 2) launch_down_decode<2>(g2, stream, a, qws, qsc, o, Tk);
    else if (is <= 5) launch_down_decode<5>(g2, stream, a, qws, qsc, o, Tk);
    else if (is <= 8) launch_down_decode<8>(g2, stream, a, qws, qsc, o, Tk);
    else launch_down_decode<16>(g2, stream, a, qws, qsc, o, Tk);
    *variant = "ffn:gu_decode+down_decode+combine";
    phase(2, stream);
  } else {
    const int gu_items = (Tk / GU_BM + max_active) * ((a.I + GU_ICOLS - 1) / GU_ICOLS);
    const int dn_items = max_active * (a.H / DN_NCOLS);
    int gu_grid = gu_items < cus * GU_WG_PER_CU ? gu_items : cus * GU_WG_PER_CU;
    int dn_grid = dn_items < cus ? dn_items : cus;             // one 8-wavefront workgroup per CU
    gu_grid = (gu_grid + XCDS - 1) / XCDS * XCDS;
    dn_grid = (dn_grid + XCDS - 1) / XCDS * XCDS;
    hipLaunchKernelGGL(clear_i32_kernel, dim3(1), dim3(64), 0, stream, queue, 64);
    hipLaunchKernelGGL(gu_prefill_kernel<GU_STAGES>, dim3(gu_grid), dim3(GU_NT), 0, stream, a, qws, qsc, h, Tk, queue);
    phase(1, stream);
    if (a.I <= 2 * KSTEP)
      hipLaunchKernelGGL(down_prefill_kernel<2>, dim3(dn_grid), dim3(DN_NT), 0, stream, a, qws, qsc, o, junk, Tk, queue + 32);
    else
      hipLaunchKernelGGL(down_prefill_kernel<5>, dim3(dn_grid), dim3(DN_NT), 0, stream, a, qws, qsc, o, junk, Tk, queue + 32);
    *variant = "ffn:gu_prefill128+down_prefill32+combine";
    phase(2, stream);
  }
  const dim3 cgrid((a.H / 4 + 255) / 256, a.T < 65535 ? a.T : 65535);
  if (a.k <= 8) hipLaunchKernelGGL(combine_kernel<8>, cgrid, dim3(256), 0, stream, o, a.topk_w, a.slot_pos, a.T, a.H, a.k, Tk, a.y);
  else hipLaunchKernelGGL(combine_kernel<MAX_K>, cgrid, dim3(256), 0, stream, o, a.topk_w, a.slot_pos, a.T, a.H, a.k, Tk, a.y);
  phase(3, stream);
  return hipGetLastError();
}

// ---------------------------------------------------- allocation-free entry ==
// The FFN workspace of moe_expert_ffn_noalloc: a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): its device address is looked up once per device with
// hipGetSymbolAddress and cached.
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

static constexpr int NOALLOC_MAX_DEVICES = 64;
static std::atomic<void*> g_scratch_ptr[NOALLOC_MAX_DEVICES];

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {                           // first call on this device (it is current): look the copy up
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace mx
