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

// ------------------------------------------- one row in one launch: pieces --
// The single-launch forms (the shared expert alone, and beside the routed
// experts) hand the SwiGLU row from gate/up workgroups to down workgroups as
// tagged 8-byte words (payload: the fp32 SwiGLU value; tag: the call's),
// written with system-scope stores and read with system-scope loads, every
// wait bounded.  Columns [8 i, 8 i + 8) sit in the first 64 bytes of their
// own 128-byte line i (words 16 i + 0..7), so no line takes two gate/up
// workgroups' stores.
__host__ __device__ constexpr size_t shared1_words_bytes(int I) { return (size_t)(I / 8) * 128; }

// Gate/up of intermediate columns [8 item, 8 item + 8) over the whole K (256
// threads): the W13 rows of those 8 gate and 8 up columns, wavefront w
// running K parts w, w + 4, ... (each part's chain from zero, exactly
// shared1_part's); wavefront 0 adds the parts in part order (shared1_down's
// sum), writes the 16 h values, and publishes the 8 SwiGLU values as words[c].
// H % 128 == 0, H <= 16384.
template <bool GRAPH>
__device__ __forceinline__ void shared1_gate_up8(const Shared1Args& sh, uint64_t* __restrict__ words, const Handoff& ho,
                                                 int item) {
  constexpr int MAXP = 16;                                      // K parts: H <= 16384
  __shared__ float ps[MAXP][16];
  const uint32_t ev = handoff_epoch_issue<GRAPH>(ho);           // the graph form's call counter
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
    __hip_atomic_store(words + 16 * item + lane,
                       (uint64_t)__float_as_uint(swiglu(v, up)) | ((uint64_t)handoff_tag<GRAPH>(ho, ev) << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// The 16 W2 rows of output columns [16 tile, 16 tile + 16), NSD steps of K = I
// (a step past K reloads the last one; TAIL: chunks past K zero, scale blocks
// past K 127), as shared1_down loads them.
template <bool TAIL, int NSD>
__device__ __forceinline__ void shared1_w2_rows(const Shared1Args& sh, int tile, u32x4 (&blo)[NSD], u32x4 (&bhi)[NSD],
                                                uint32_t (&bs)[NSD]) {
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  const int I = sh.I, nsteps = (I + KSTEP - 1) / KSTEP, nblk = I / 32;
  const int64_t n = (int64_t)tile * 16 + col;
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

// One read round of the SwiGLU words by one wavefront w (of four): lane l
// reads 16-byte chunks c = 64 w + l and 256 + 64 w + l (chunk c: line c / 4,
// columns 8 (c / 4) + 2 (c % 4) + {0, 1}; reads past the I / 8 lines, and
// every read when `on` is false, return zeros).
// shared1_words_take is true when every word of the wavefront's share
// carries the tag; the values are then in av.  I <= 1024.
__device__ __forceinline__ void shared1_words_issue(const uint64_t* words, int I, bool on, u32x4 (&v)[2]) {
  const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) & 3;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)words, (short)0, on ? (uint32_t)shared1_words_bytes(I) : 0u, 0x00020000);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = 256 * h + 64 * wave + lane;
    v[h] = __builtin_amdgcn_raw_buffer_load_b128(r, (c >> 2) * 128 + (c & 3) * 16, 0, 17);
  }
}
__device__ __forceinline__ bool shared1_words_take(const u32x4 (&v)[2], int I, uint32_t tag, float* av) {
  const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) & 3;
  bool ok = true;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = 256 * h + 64 * wave + lane;
      ok = ok && (c >= I / 2 || v[h][2 * e + 1] == tag);        // chunks of lines past I / 8 hold nothing
    }
  if (__ballot(ok) != ~0ull) return false;                      // wavefront-uniform
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = 256 * h + 64 * wave + lane;
      if (c < I / 2) av[8 * (c >> 2) + 2 * (c & 3) + e] = __uint_as_float(v[h][2 * e]);
    }
  return true;
}
__device__ __forceinline__ bool shared1_words_round(const uint64_t* words, int I, uint32_t tag, float* av) {
  u32x4 v[2];
  shared1_words_issue(words, I, true, v);
  return shared1_words_take(v, I, tag, av);
}

// Requant of the SwiGLU row av into q1 / s1 (LDS) by 256 threads: 16 lanes
// per block of 32, columns c and c + 16 (swiglu_requant2 past its SwiGLU:
// the amax over the DPP row, the E8M0 code, the E4M3 pairs); K past I zero
// elements and unit scales up to NSD steps; wq != 0 also writes q and q_sc.
template <int NSD>
__device__ __forceinline__ void shared1_requant(const Shared1Args& sh, const float* av, uint8_t* q1, uint8_t* s1,
                                                bool wq) {
  const int tid = threadIdx.x, I = sh.I, nblk = I / 32;
  for (int idx = tid; idx < NSD * KSTEP - I; idx += 256) q1[I + idx] = 0;
  for (int idx = tid; idx < NSD * 4 - nblk; idx += 256) s1[nblk + idx] = 127;
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
      if (wq) {
        sh.q[cb + c] = (uint8_t)d;
        sh.q[cb + 16 + c] = (uint8_t)(d >> 8);
        if (c == 0) sh.q_sc[b] = (uint8_t)sc;
      }
    }
  }
}

// The down chain of output columns [16 tile, 16 tile + 16) from q1 / s1 (one
// wavefront, shared1_down's): y written by lanes 0..15.
template <int NSD>
__device__ __forceinline__ void shared1_chain(const Shared1Args& sh, int tile, const uint8_t* q1, const uint8_t* s1,
                                              const u32x4 (&blo)[NSD], const u32x4 (&bhi)[NSD],
                                              const uint32_t (&bs)[NSD]) {
  const int lane = threadIdx.x & 63, col = lane & 15, g = lane >> 4;
  const int nsteps = (sh.I + KSTEP - 1) / KSTEP;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NSD; ++s)
    if (s < nsteps) {
      const u32x4 alo = *reinterpret_cast<const u32x4*>(&q1[s * KSTEP + g * 16]);
      const u32x4 ahi = *reinterpret_cast<const u32x4*>(&q1[s * KSTEP + 64 + g * 16]);
      const uint32_t sa = (uint32_t)s1[4 * s + g] << (8 * g);
      acc = mfma_fp8_fp8(fp8_pair(alo, ahi), fp8_pair(blo[s], bhi[s]), acc, sa >> (8 * g), bs[s] >> (8 * g));
    }
  if (g == 0) sh.y[(int64_t)tile * 16 + col] = acc[0];
}

// Down projection of output columns [16 tile, 16 tile + 16) in the shared
// expert's own single launch: wavefront 0 requests its 16 W2 rows first; the
// four wavefronts wait for their shares of the I words, then the requant
// (tile 0 writes q and q_sc) and wavefront 0's chain.  I <= 1024.
template <bool TAIL, bool GRAPH>
__device__ void shared1_down_wait(const Shared1Args& sh, const Handoff& ho, int tile) {
  constexpr int NSD = KPART_STEPS;                              // steps of K = I <= 1024
  __shared__ __attribute__((aligned(16))) float av[NSD * KSTEP];
  __shared__ __attribute__((aligned(16))) uint8_t q1[NSD * KSTEP];
  __shared__ uint8_t s1[NSD * 4];
  const uint64_t t0 = wall_clock64();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t ev = handoff_epoch_issue<GRAPH>(ho);           // the graph form's call counter
  u32x4 blo[NSD], bhi[NSD];
  uint32_t bs[NSD];
  if (wave == 0) shared1_w2_rows<TAIL, NSD>(sh, tile, blo, bhi, bs);
  const uint32_t tag = handoff_tag<GRAPH>(ho, ev);
  while (!shared1_words_round(ho.words, sh.I, tag, av)) {
    if ((long long)(wall_clock64() - t0) > ho.limit) {
      if (lane == 0) __hip_atomic_fetch_or(ho.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  lds_barrier();
  shared1_requant<NSD>(sh, av, q1, s1, tile == 0);
  lds_barrier();
  if (wave == 0) shared1_chain<NSD>(sh, tile, q1, s1, blo, bhi, bs);
}

}  // namespace mx
