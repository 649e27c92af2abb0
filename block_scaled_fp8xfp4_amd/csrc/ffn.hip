// Routed-expert FFN kernels: gate/up GEMM, SwiGLU + FP8 requant, down GEMM
// and the fixed-order weighted combine ("New Deepseek 4.1 flash recipe"
// thread, post #6, "How it works": routed experts with FP8 activations x FP4
// weights, decode rows on small tiles; "Why TileLang": SwiGLU, per-block FP8
// quantization, reductions in a fixed order; DeepSeek-V4.1-Flash-4x-DGX-
// Spark-TP4 README, settings table, row "Experts": per-slot buffer and a
// fixed-order sum instead of atomics).
//
// Decode path (few rows per expert): a work item is (expert with live pairs,
// 16-wide tile of weight rows).  A workgroup's four wavefronts split K into
// the canonical parts and stream their share of the weight tile straight
// from HBM into registers; the parts meet in LDS and are added in part order.
// Gate/up writes h = [gate | up] in fp32 per bucket position; the down kernel
// stages SwiGLU + requant of its rows in LDS (every down workgroup of an
// expert recomputes the same values with the same device routine), then
// streams W2 the same way and writes the per-slot output o.
// The combine adds w_tj * o_tj over the slots in order j = 0..k-1.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mx {

// Experts that own at least one live pair, ascending, listed by wavefront 0.
__device__ void list_active_experts(const int32_t* __restrict__ offsets, int E, int* list, int* n_out) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int base = 0;
    for (int c = 0; c < E; c += 64) {
      const int e = c + lane;
      const bool nz = e < E && offsets[e + 1] > offsets[e];
      const unsigned long long m = __ballot(nz);
      if (nz) list[base + __popcll(m & ((1ull << lane) - 1ull))] = e;
      base += __popcll(m);
    }
    if (lane == 0) *n_out = base;
  }
  __syncthreads();
}

__device__ __forceinline__ v8i fp8_operand(const u32x4& lo, const u32x4& hi) {
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
__device__ __forceinline__ v8i fp4_operand(const u32x4& b) {
  return v8i{(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
}

// --------------------------------------------------------------------------
// Gate/up, decode tiles.  h[p][n] for the expert's pairs p and W13 rows n.
__global__ __launch_bounds__(256) void gu_decode_kernel(FfnArgs a, float* __restrict__ h, int Tk) {
  __shared__ int active[MAX_E];
  __shared__ int n_active;
  __shared__ float red[MAX_PARTS][16][16];
  list_active_experts(a.offsets, a.E, active, &n_active);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int H = a.H, twoI = 2 * a.I;
  const int nsteps = H / KSTEP, nparts = (nsteps + KPART_STEPS - 1) / KPART_STEPS;
  const int ntiles = twoI / 16;
  const int nitems = n_active * ntiles;

  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int e = active[item / ntiles], nt = item % ntiles;
    const int p0 = a.offsets[e];
    int cnt = a.offsets[e + 1] - p0;
    if (p0 < 0 || p0 + cnt > Tk) cnt = 0;                       // malformed route: skip
    const int64_t wrow = (int64_t)e * twoI + nt * 16 + col;     // B column served by this lane
    const uint8_t* wp = a.w13 + wrow * (H / 2);
    const uint32_t* wsp = reinterpret_cast<const uint32_t*>(a.w13_sc + wrow * (H / 32));
    for (int rt = 0; rt * 16 < cnt; ++rt) {
      const int r = rt * 16 + col;                               // A row served by this lane
      int tok = 0;
      bool rv = r < cnt;
      if (rv) {
        const int pr = a.perm[p0 + r];
        rv = pr >= 0 && pr < Tk;
        tok = rv ? pr / a.k : 0;
      }
      const uint8_t* xp = a.x + (int64_t)tok * H;
      const uint32_t* xsp = reinterpret_cast<const uint32_t*>(a.x_sc + (int64_t)tok * (H / 32));
      for (int q = wave; q < nparts; q += 4) {
        const int s0 = q * KPART_STEPS;
        u32x4 bw[KPART_STEPS], alo[KPART_STEPS], ahi[KPART_STEPS];
        uint32_t bs[KPART_STEPS], as[KPART_STEPS];
#pragma unroll
        for (int m = 0; m < KPART_STEPS; ++m) {
          const int s = s0 + m;
          if (s < nsteps) {
            bw[m] = ldg16(wp + s * 64 + g * 16);
            bs[m] = wsp[s] >> (8 * g);
          }
        }
#pragma unroll
        for (int m = 0; m < KPART_STEPS; ++m) {
          const int s = s0 + m;
          if (s < nsteps) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            alo[m] = rv ? ldg16(xp + s * KSTEP + g * 16) : z;
            ahi[m] = rv ? ldg16(xp + s * KSTEP + 64 + g * 16) : z;
            as[m] = rv ? (xsp[s] >> (8 * g)) : bs[m];
          }
        }
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < KPART_STEPS; ++m) {
          if (s0 + m < nsteps) acc = mfma_fp8_fp4(fp8_operand(alo[m], ahi[m]), fp4_operand(bw[m]), acc, as[m], bs[m]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) red[q][4 * g + i][col] = acc[i];
      }
      __syncthreads();
      {
        const int row = threadIdx.x >> 4, c = threadIdx.x & 15;
        float v = red[0][row][c];
        for (int q = 1; q < nparts; ++q) v = v + red[q][row][c];
        if (rt * 16 + row < cnt) h[(int64_t)(p0 + rt * 16 + row) * twoI + nt * 16 + c] = v;
      }
      __syncthreads();
    }
  }
}

// --------------------------------------------------------------------------
// SwiGLU + FP8 requant of pair rows [p0, p0 + n) (n <= 16) into LDS (and the
// workspace copy when `publish`).  Block-wide.
__device__ void stage_intermediate(const float* __restrict__ h, int p0, int n, int I, uint8_t (*qlds)[MAX_I + 16],
                                   uint8_t (*slds)[MAX_I / 32], uint8_t* __restrict__ qws, uint8_t* __restrict__ qsc_ws,
                                   bool publish) {
  const int nb = I / 32;
  for (int idx = threadIdx.x; idx < 16 * nb; idx += blockDim.x) {
    const int r = idx / nb, b = idx % nb;
    if (r >= n) continue;
    const float* hp = h + (int64_t)(p0 + r) * 2 * I + b * 32;
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const float4 gg = *reinterpret_cast<const float4*>(hp + i);
      const float4 uu = *reinterpret_cast<const float4*>(hp + I + i);
      v[i] = swiglu(gg.x, uu.x);
      v[i + 1] = swiglu(gg.y, uu.y);
      v[i + 2] = swiglu(gg.z, uu.z);
      v[i + 3] = swiglu(gg.w, uu.w);
    }
    uint32_t out[8];
    const uint32_t sc = quantize32_e4m3(v, out);
    u32x4* dst = reinterpret_cast<u32x4*>(&qlds[r][b * 32]);
    dst[0] = u32x4{out[0], out[1], out[2], out[3]};
    dst[1] = u32x4{out[4], out[5], out[6], out[7]};
    slds[r][b] = (uint8_t)sc;
    if (publish) {
      u32x4* gdst = reinterpret_cast<u32x4*>(qws + (int64_t)(p0 + r) * I + b * 32);
      gdst[0] = u32x4{out[0], out[1], out[2], out[3]};
      gdst[1] = u32x4{out[4], out[5], out[6], out[7]};
      qsc_ws[(int64_t)(p0 + r) * nb + b] = (uint8_t)sc;
    }
  }
}

constexpr int DOWN_MAX_STEPS = MAX_I / KSTEP;   // 16

// Down projection, decode tiles: o[p][n] for the expert's pairs and a 64-row
// tile of W2 (16 rows per wavefront, full K = I per wavefront).
__global__ __launch_bounds__(256) void down_decode_kernel(FfnArgs a, const float* __restrict__ h,
                                                          uint8_t* __restrict__ qws, uint8_t* __restrict__ qsc_ws,
                                                          float* __restrict__ o, int Tk) {
  __shared__ int active[MAX_E];
  __shared__ int n_active;
  __shared__ __attribute__((aligned(16))) uint8_t qlds[16][MAX_I + 16];   // padded rows: fewer bank conflicts
  __shared__ uint8_t slds[16][MAX_I / 32];
  list_active_experts(a.offsets, a.E, active, &n_active);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int H = a.H, I = a.I, nb = I / 32;
  const int nsteps = (I + KSTEP - 1) / KSTEP;
  const int ntiles = H / 64;
  const int nitems = n_active * ntiles;

  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int e = active[item / ntiles], tile = item % ntiles;
    const int p0 = a.offsets[e];
    int cnt = a.offsets[e + 1] - p0;
    if (p0 < 0 || p0 + cnt > Tk) cnt = 0;
    const int n = tile * 64 + wave * 16 + col;                  // W2 row = output column of this lane
    const uint8_t* wp = a.w2 + ((int64_t)e * H + n) * (I / 2);
    const uint8_t* wsp = a.w2_sc + ((int64_t)e * H + n) * nb;
    // weights first: the whole K = I of this lane's column stays in registers
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
      __syncthreads();
      const bool rv = col < nrows;
      v4f total = {0.f, 0.f, 0.f, 0.f};
      for (int q = 0; q * KPART_STEPS < nsteps; ++q) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < KPART_STEPS; ++m) {
          const int s = q * KPART_STEPS + m;
          if (s < nsteps && s < DOWN_MAX_STEPS) {
            const int klo = s * KSTEP + g * 16, khi = klo + 64;
            const u32x4 z = {0u, 0u, 0u, 0u};
            const u32x4 alo = (rv && klo < I) ? *reinterpret_cast<const u32x4*>(&qlds[col][klo]) : z;
            const u32x4 ahi = (rv && khi < I) ? *reinterpret_cast<const u32x4*>(&qlds[col][khi]) : z;
            const uint32_t sa = (rv && 4 * s + g < nb) ? (uint32_t)slds[col][4 * s + g] : bs[s];
            acc = mfma_fp8_fp4(fp8_operand(alo, ahi), fp4_operand(bw[s]), acc, sa, bs[s]);
          }
        }
        if (q == 0) total = acc;
        else total = total + acc;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * g + i;
        if (row < nrows) o[(int64_t)(p0 + rt * 16 + row) * H + n] = total[i];
      }
      __syncthreads();
    }
  }
}

// --------------------------------------------------------------------------
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

// --------------------------------------------------------------------------
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

hipError_t launch_ffn(const FfnArgs& a, void* ws, int path, hipStream_t stream, const char** variant) {
  const int Tk = a.T * a.k;
  uint8_t* base = static_cast<uint8_t*>(ws);
  size_t oq, oqs, oh, oo;
  ffn_ws_layout(a.T, a.H, a.I, a.k, &oq, &oqs, &oh, &oo);
  uint8_t* qws = base + oq;
  uint8_t* qsc = base + oqs;
  float* h = reinterpret_cast<float*>(base + oh);
  float* o = reinterpret_cast<float*>(base + oo);
  (void)path;
  const int cap = num_cus() * 4;
  const int max_active = a.E < Tk ? a.E : Tk;
  const int gu_items = max_active * (2 * a.I / 16);
  const int dn_items = max_active * (a.H / 64);
  const int gu_grid = gu_items < cap ? gu_items : cap;
  const int dn_grid = dn_items < cap ? dn_items : cap;
  if (gu_grid > 0) hipLaunchKernelGGL(gu_decode_kernel, dim3(gu_grid), dim3(256), 0, stream, a, h, Tk);
  if (dn_grid > 0) hipLaunchKernelGGL(down_decode_kernel, dim3(dn_grid), dim3(256), 0, stream, a, h, qws, qsc, o, Tk);
  const dim3 cgrid((a.H / 4 + 255) / 256, a.T < 65535 ? a.T : 65535);
  hipLaunchKernelGGL(combine_kernel, cgrid, dim3(256), 0, stream, o, a.topk_w, a.slot_pos, a.T, a.H, a.k, Tk, a.y);
  *variant = "ffn:gu_decode16+down_decode16+combine";
  return hipGetLastError();
}

}  // namespace mx
