// Device-side building blocks shared by the HIP kernels of this library.
//
// Scaled matrix-core step (gfx950 V_MFMA_SCALE_F32_16X16X128_F8F6F4), as
// measured on MI355X with a one-tile probe against the definition:
//   - A is 16 rows x 128 K, B is 128 K x 16 columns, C/D 16 x 16 fp32.
//   - Lane l serves row (A) / column (B) l % 16 and lane group g = l / 16.
//   - FP8 operand (8 dwords per lane): bytes 0..15 hold K = 16g + [0,16),
//     bytes 16..31 hold K = 64 + 16g + [0,16).
//   - FP4 operand (low 4 dwords per lane): 32 nibbles = K = 32g + [0,32),
//     element 2i in the low nibble of byte i.
//   - Scale operand: byte 0 of the lane's scale dword is the E8M0 scale of
//     K block g (K = 32g + [0,32)) of that lane's row / column; 127 = 1.0.
//   - D: lane l holds column l % 16, rows 4g + r in register r.
// The FP8 encoding is OCP E4M3 (bias 7, max 448).
//
// Canonical reduction orders (one per GEMM, the same for every batch size
// and every path, so that a row's result never depends on either):
//   K is cut into steps of 128 (step m covers K blocks 4m..4m+3 of 32); a
//   step whose blocks run past K is padded with zero elements in registers.
//   - Routed-expert gate/up and down: one MFMA chain over all steps in
//     order, accumulator started from zero and carried through C.
//   - Dense projection: steps grouped in parts of KPART_STEPS; each part is
//     a chain started from zero, and the parts are added left to right in
//     fp32: total = ((p0 + p1) + p2) + ...  (lets four wavefronts split K).
// The scaled MFMA does not round its 128-product sum exactly (measured on
// MI355X: a few 1e-6 relative), identically for every chaining tried, so the
// chain choice is about parallelism, not accuracy.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

constexpr int KSTEP = 128;        // K per MFMA step
constexpr int KPART_STEPS = 8;    // steps per part (K = 1024)
constexpr int KPART = KSTEP * KPART_STEPS;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// E4M3 (A) x E2M1 (B) step.
__device__ __forceinline__ v4f mfma_fp8_fp4(const v8i& a, const v8i& b, v4f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, (int)sa, 0, (int)sb);
}
// E4M3 (A) x E4M3 (B) step.
__device__ __forceinline__ v4f mfma_fp8_fp8(const v8i& a, const v8i& b, v4f c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, (int)sa, 0, (int)sb);
}

__device__ __forceinline__ u32x4 ldg16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Workgroup barrier for LDS hand-offs only.  __syncthreads() also releases
// global memory, which on gfx9-class hardware waits for every outstanding
// global load (vmcnt(0)) and would drain the prefetches that are meant to
// stay in flight across the barrier; this one waits for LDS operations only.
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

// Global -> LDS without registers (gfx950 LDS DMA): lane l's 16 (4) bytes
// land at dst + 16 l (4 l); dst is the same for the whole wavefront.  Issued
// as inline assembly so that the compiler neither tracks nor waits for these
// writes: the kernel orders them itself with explicit vmcnt waits and LDS
// barriers.  Extra operations outside the compiler's count only make its own
// vmcnt waits stricter (vector-memory loads complete in issue order).
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(size_t)(lds_void*)p; }
__device__ __forceinline__ void dma16_to_lds(const void* src, void* dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_addr(dst))) : "m0");
}
__device__ __forceinline__ void dma4_to_lds(const void* src, void* dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_addr(dst))) : "m0");
}
// The same from a wavefront-uniform base plus a 32-bit per-lane byte offset,
// to the wavefront-uniform LDS byte address dst.
__device__ __forceinline__ void dma16_to_lds(const void* base, uint32_t off, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(dst) : "m0");
}
__device__ __forceinline__ void dma4_to_lds(const void* base, uint32_t off, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(off), "s"(base), "s"(dst) : "m0");
}

// ---------------------------------------------------------------------------
// Block-32 quantization (OCP MX v1.0 conversion): shared scale
// X = 2^(floor(log2 amax) - emax) as an E8M0 code clamped to [0, 254]
// (amax == 0 -> 0); elements round to nearest even, saturate, keep the sign.
__device__ __forceinline__ uint32_t e8m0_code_for_amax(float amax, int emax) {
  const int be = (int)((__float_as_uint(amax) >> 23) & 0xFF);   // 0 for zero / subnormal
  int c = be - emax;
  c = c < 0 ? 0 : c;
  return (uint32_t)(c > 254 ? 254 : c);
}

// fp32 -> E4M3 code under scale code sc.
__device__ __forceinline__ uint32_t encode_e4m3(float v, uint32_t sc) {
  const float t = __builtin_ldexpf(v, 127 - (int)sc);           // exact power-of-two scaling
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80;
  const float a = __builtin_fabsf(t);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7E;                                                 // saturate
  } else if (a < 0.015625f) {                                    // below 2^-6: subnormal grid of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);                 // 8 -> 0x08 = 2^-6
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);                            // round mantissa to 3 bits, ties even
    const uint32_t e = (b >> 23) - 127u + 7u;
    code = (e << 3) | ((b >> 20) & 7u);
  }
  return code | sign;
}

// fp32 -> E2M1 code (0..15) under scale code sc.
__device__ __forceinline__ uint32_t encode_e2m1(float v, uint32_t sc) {
  const float t = __builtin_ldexpf(v, 127 - (int)sc);
  const uint32_t sign = (__float_as_uint(v) >> 28) & 0x8;
  const float a = __builtin_fabsf(t);
  uint32_t code;
  if (a >= 6.0f) {
    code = 7;
  } else if (a < 1.0f) {                                         // subnormal grid of 0.5
    code = (uint32_t)__builtin_rintf(a * 2.0f);                   // 2 -> code 2 = 1.0
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x1FFFFFu + ((b >> 22) & 1u);                           // round mantissa to 1 bit, ties even
    const uint32_t e = (b >> 23) - 127u + 1u;
    code = (e << 1) | ((b >> 22) & 1u);
  }
  return code | sign;
}

// SwiGLU of one gate/up pair: silu(g) * u, silu(g) = g / (1 + e^-g),
// evaluated in double (exponential of the device math library, IEEE
// division) and rounded once to fp32.  The rounding of a into the FP8
// requant that follows then depends on the fp32 gate/up values alone, not on
// the precision of a short fp32 evaluation (with the hardware exponential and
// reciprocal, a few results per 10^5 landed on the other side of an E4M3
// rounding midpoint).  Contraction is off so every kernel that inlines it
// rounds identically.
__device__ __forceinline__ float swiglu(float g, float u) {
#pragma clang fp contract(off)
  const double gd = (double)g;
  const double s = gd / (1.0 + exp(-gd));
  return (float)(s * (double)u);
}

// Maximum over the 16 lanes of a DPP row (lanes 16 r .. 16 r + 15), in
// registers: quad butterflies, then rotations by 4 and 8 within the row.
__device__ __forceinline__ float row16_max(float m) {
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1, 0xF, 0xF, false)));   // quad [1,0,3,2]
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x4E, 0xF, 0xF, false)));   // quad [2,3,0,1]
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x124, 0xF, 0xF, false)));  // row_ror:4
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x128, 0xF, 0xF, false)));  // row_ror:8
  return m;
}

// Maximum over each group of 8 lanes (lanes 8 r .. 8 r + 7), in registers:
// quad butterflies, then the mirror within the half row.
__device__ __forceinline__ float row8_max(float m) {
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1, 0xF, 0xF, false)));   // quad [1,0,3,2]
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x4E, 0xF, 0xF, false)));   // quad [2,3,0,1]
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x141, 0xF, 0xF, false)));  // row_half_mirror
  return m;
}

// E4M3 codes of two elements of a block whose shared scale code is sc (the
// requant of the intermediate), first element in bits 0..7, second in 8..15:
// identical in every kernel that uses it.  The value is scaled by 2^(127 - sc)
// (exact), clamped to +-448 and converted by the hardware (round to nearest
// even, OCP E4M3, subnormals kept).  Inputs are finite and the scaled value
// is below 512 in magnitude (the scale comes from the block's amax); on that
// whole domain this equals encode_e4m3 bit for bit, every float compared.
__device__ __forceinline__ uint32_t requant2_e4m3(float a, float b, uint32_t sc) {
  const int k = 127 - (int)sc;
  const float ta = __builtin_amdgcn_fmed3f(__builtin_ldexpf(a, k), -448.0f, 448.0f);
  const float tb = __builtin_amdgcn_fmed3f(__builtin_ldexpf(b, k), -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ta, tb, 0, false) & 0xFFFFu;
}

// SwiGLU + E4M3 requant of this lane's two elements of a block of 32 that is
// spread over the 16 lanes of a DPP row (element 0 of lane c is column c of
// the block, element 1 column c + 16): a = swiglu(g, u) (double, rounded
// once), the block's scale code from max |a| (into *sc_out), and the two
// codes (bits 0..7 and 8..15).  The same routine in every kernel that
// requantizes an intermediate.
__device__ __forceinline__ uint32_t swiglu_requant2(float g0, float u0, float g1, float u1, uint32_t* sc_out) {
  const float a0 = swiglu(g0, u0), a1 = swiglu(g1, u1);
  const uint32_t sc = e8m0_code_for_amax(row16_max(fmaxf(__builtin_fabsf(a0), __builtin_fabsf(a1))), 8);
  *sc_out = sc;
  return requant2_e4m3(a0, a1, sc);
}

// Quantize 32 fp32 values to E4M3: writes 32 code bytes as 8 dwords, returns the scale code.
__device__ __forceinline__ uint32_t quantize32_e4m3(const float* v, uint32_t* out8) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, __builtin_fabsf(v[i]));
  const uint32_t sc = e8m0_code_for_amax(amax, 8);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t d = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) d |= encode_e4m3(v[4 * w + i], sc) << (8 * i);
    out8[w] = d;
  }
  return sc;
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace mx
