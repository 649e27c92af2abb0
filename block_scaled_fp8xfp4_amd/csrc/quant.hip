// Block-32 quantizer kernel: fp32 or bf16 rows -> E4M3 bytes or packed E2M1
// nibbles plus one E8M0 scale per 32 values (the per-block FP8/FP4 casts of
// the "New Deepseek 4.1 flash recipe" thread, post #6, "Why TileLang"; the
// conversion rule is OCP MX v1.0's).  One thread per block of 32: a thread
// reads 64-128 contiguous bytes and its neighbours the next ones, so a wave
// streams a contiguous span of the row-major source.
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mx {

template <bool BF16, bool FP4>
__global__ __launch_bounds__(256) void quantize_kernel(const void* __restrict__ src, int64_t nblocks,
                                                       uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  float v[32];
  if (BF16) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + b * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 d = p[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __uint_as_float(d[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
      }
    }
  } else {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(src) + b * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 d = p[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * i + j] = __uint_as_float(d[j]);
    }
  }
  if (FP4) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, __builtin_fabsf(v[i]));
    const uint32_t s = e8m0_code_for_amax(amax, 2);
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t d = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) d |= encode_e2m1(v[8 * w + i], s) << (4 * i);
      out[w] = d;
    }
    *reinterpret_cast<u32x4*>(q + b * 16) = out;
    sc[b] = (uint8_t)s;
  } else {
    uint32_t out[8];
    const uint32_t s = quantize32_e4m3(v, out);
    u32x4* dst = reinterpret_cast<u32x4*>(q + b * 32);
    dst[0] = u32x4{out[0], out[1], out[2], out[3]};
    dst[1] = u32x4{out[4], out[5], out[6], out[7]};
    sc[b] = (uint8_t)s;
  }
}

hipError_t launch_quantize(const void* src, bool bf16, int64_t rows, int64_t cols, bool fp4,
                           uint8_t* q, uint8_t* sc, hipStream_t stream) {
  const int64_t nblocks = rows * (cols / 32);
  if (nblocks == 0) return hipSuccess;
  const dim3 block(256), grid((unsigned)((nblocks + 255) / 256));
  if (bf16 && fp4) hipLaunchKernelGGL((quantize_kernel<true, true>), grid, block, 0, stream, src, nblocks, q, sc);
  else if (bf16) hipLaunchKernelGGL((quantize_kernel<true, false>), grid, block, 0, stream, src, nblocks, q, sc);
  else if (fp4) hipLaunchKernelGGL((quantize_kernel<false, true>), grid, block, 0, stream, src, nblocks, q, sc);
  else hipLaunchKernelGGL((quantize_kernel<false, false>), grid, block, 0, stream, src, nblocks, q, sc);
  return hipGetLastError();
}

// Diagnostic: the finite floats whose magnitude bits lie in [lo, hi), with
// both signs, through both E4M3 encoders of the intermediate: the hardware
// conversion of requant2_e4m3 and the integer rounding of encode_e4m3 (scale
// code 127: the value itself is encoded).  Mismatches are added to *nbad.
__global__ __launch_bounds__(256) void check_requant_kernel(uint32_t lo, uint32_t hi, unsigned long long* nbad) {
  unsigned long long bad = 0;
  for (uint64_t i = lo + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < hi; i += (uint64_t)gridDim.x * blockDim.x) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float v = __uint_as_float((uint32_t)i | (s ? 0x80000000u : 0u));
      bad += (requant2_e4m3(v, 0.0f, 127) & 0xFFu) != encode_e4m3(v, 127);
    }
  }
  if (bad) atomicAdd(nbad, bad);
}

hipError_t launch_check_requant(uint32_t lo, uint32_t hi, unsigned long long* nbad, hipStream_t stream) {
  if (lo >= hi) return hipSuccess;
  hipLaunchKernelGGL(check_requant_kernel, dim3(2048), dim3(256), 0, stream, lo, hi, nbad);
  return hipGetLastError();
}

}  // namespace mx

namespace mx {

// Weight prefetch (spark-ds41f README, "Current baseline": L2 weight prefetch
// during decode, the next layer's weights and scale words streamed in while
// latency-bound kernels run; TP4 README, settings table, row "L2 prefetch": a
// side-stream kernel during idle phases, data untouched).  Workgroup i reads
// chunk i of the range, so the chunk lands in the L2 of the XCD that runs
// workgroup i and in the memory-side cache (MALL) shared by every XCD.  The
// reads are LDS DMA into a scratch row per wavefront (no register ever holds
// them, nothing is kept); the workgroup waits for all of them before it ends.
// Whole 16-byte units only (p 16-byte aligned, chunk a multiple of 16).
__global__ __launch_bounds__(256) void prefetch_kernel(const uint8_t* __restrict__ p, uint64_t bytes, uint64_t chunk) {
  __shared__ u32x4 scratch[256];
  const int wave = threadIdx.x >> 6;
  const uint64_t c0 = (uint64_t)blockIdx.x * chunk;
  const uint64_t c1 = c0 + chunk < bytes ? c0 + chunk : bytes;
  for (uint64_t off = c0 + (uint64_t)threadIdx.x * 16; off + 16 <= c1; off += 256 * 16)
    dma16_to_lds(p + off, &scratch[wave * 64]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

hipError_t launch_prefetch(const void* p, uint64_t bytes, uint64_t chunk, hipStream_t stream) {
  const uint64_t n = (bytes + chunk - 1) / chunk;
  hipLaunchKernelGGL(prefetch_kernel, dim3((unsigned)n), dim3(256), 0, stream, static_cast<const uint8_t*>(p), bytes,
                     chunk);
  return hipGetLastError();
}

}  // namespace mx
