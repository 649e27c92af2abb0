// Top-k gate and bucketing (the MoE top-k gate of the "New Deepseek 4.1
// flash recipe" thread, post #6, "How it works"; dead verification rows of
// post #2, "What changed"; the route planner and per-slot buffer of the
// DeepSeek-V4.1-Flash-4x-DGX-Spark-TP4 README, settings table, row "Experts").
//
// topk_kernel: one wavefront per row.  Each lane holds E/64 logits in
//   registers; k rounds of a butterfly arg-max over (logit desc, index asc)
//   pick the slots.  Weights are the softmax over the picked logits,
//   evaluated in double and rounded to fp32.
// Bucketing is a counting sort of the live (row, slot) pairs by expert with
//   the canonical order (expert, row): per chunk of 256 rows, each row ORs
//   its bit into a per-expert row bitmask in LDS; a pair's rank among the
//   chunk's rows that picked the same expert is a population count of the
//   lower bits, so no atomic ordering ever decides a position.
#include <climits>
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mx {

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   const float* __restrict__ survival, float skip_below,
                                                   int32_t* __restrict__ ids, float* __restrict__ w,
                                                   int32_t* __restrict__ slot_pos) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + (int64_t)t * E;
  float v[16];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    const bool ok = e < E;
    v[i] = ok ? l[e] : 0.0f;
    avail |= (ok ? 1u : 0u) << i;
  }
  float my_val = 0.0f;
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    float best = 0.0f;
    int be = INT_MAX;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((avail >> i) & 1u) {
        if (be == INT_MAX || v[i] > best) { best = v[i]; be = lane + 64 * i; }   // ties keep the lower index
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(best, off);
      const int oe = __shfl_xor(be, off);
      const bool take = oe != INT_MAX && (be == INT_MAX || ov > best || (ov == best && oe < be));
      if (take) { best = ov; be = oe; }
    }
    if ((be & 63) == lane) avail &= ~(1u << (be >> 6));
    if (lane == j) { my_val = best; my_idx = be; }
  }
  // softmax over the k picked logits: w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0)
  const double l0 = (double)__shfl(my_val, 0);
  const double ex = lane < k ? exp((double)my_val - l0) : 0.0;
  double den = 0.0;
  for (int j = 0; j < k; ++j) den += __shfl(ex, j);
  const bool live = survival == nullptr || !(survival[t] < skip_below);
  if (lane < k) {
    ids[(int64_t)t * k + lane] = my_idx;
    w[(int64_t)t * k + lane] = (float)(ex / den);
    if (!live) slot_pos[(int64_t)t * k + lane] = -1;
  }
}

// LDS bitmask of the rows (within a chunk of 256) that picked each expert.
struct ChunkMasks {
  unsigned long long m[MAX_E][4];
};

__device__ __forceinline__ bool row_live(const float* survival, float skip_below, int t) {
  return survival == nullptr || !(survival[t] < skip_below);
}

// Build the masks of chunk c (rows c*256 .. c*256+255); block of 256 threads.
__device__ void fill_masks(ChunkMasks& cm, const int32_t* __restrict__ ids, int T, int E, int k,
                           const float* __restrict__ survival, float skip_below, int c) {
  for (int i = threadIdx.x; i < E * 4; i += blockDim.x) (&cm.m[0][0])[i] = 0ull;
  __syncthreads();
  const int r = threadIdx.x, t = c * ROUTE_CHUNK + r;
  if (t < T && row_live(survival, skip_below, t)) {
    for (int j = 0; j < k; ++j) {
      const int e = ids[(int64_t)t * k + j];
      if (e >= 0 && e < E) atomicOr(&cm.m[e][r >> 6], 1ull << (r & 63));
    }
  }
  __syncthreads();
}

__device__ __forceinline__ int mask_count(const ChunkMasks& cm, int e) {
  return __popcll(cm.m[e][0]) + __popcll(cm.m[e][1]) + __popcll(cm.m[e][2]) + __popcll(cm.m[e][3]);
}

// rank of row r among the chunk rows that picked e
__device__ __forceinline__ int mask_rank(const ChunkMasks& cm, int e, int r) {
  int n = 0;
  for (int w = 0; w < (r >> 6); ++w) n += __popcll(cm.m[e][w]);
  const unsigned long long below = (r & 63) ? (cm.m[e][r >> 6] & ((1ull << (r & 63)) - 1ull)) : 0ull;
  return n + __popcll(below);
}

__device__ void scatter_chunk(const ChunkMasks& cm, const int32_t* __restrict__ ids, int T, int E, int k,
                              const float* __restrict__ survival, float skip_below, int c,
                              const int32_t* base /* [E], LDS or global */, int32_t* __restrict__ perm,
                              int32_t* __restrict__ slot_pos) {
  const int r = threadIdx.x, t = c * ROUTE_CHUNK + r;
  if (t < T && row_live(survival, skip_below, t)) {
    for (int j = 0; j < k; ++j) {
      const int e = ids[(int64_t)t * k + j];
      if (e < 0 || e >= E) continue;
      const int p = base[e] + mask_rank(cm, e, r);
      perm[p] = t * k + j;
      slot_pos[(int64_t)t * k + j] = p;
    }
  }
}

// Exclusive scan of n <= MAX_E ints in LDS by a block of 256 threads (4 per thread).
__device__ void block_exclusive_scan(int32_t* vals, int n) {
  __shared__ int32_t partial[256];
  const int tid = threadIdx.x;
  int local[4], s = 0;
  for (int i = 0; i < 4; ++i) {
    const int idx = tid * 4 + i;
    local[i] = idx < n ? vals[idx] : 0;
    s += local[i];
  }
  partial[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < 256; ++i) { const int v = partial[i]; partial[i] = run; run += v; }
  }
  __syncthreads();
  int run = partial[tid];
  for (int i = 0; i < 4; ++i) {
    const int idx = tid * 4 + i;
    if (idx < n) vals[idx] = run;
    run += local[i];
  }
  __syncthreads();
}

// One chunk: count, scan, scatter in a single block (T <= 256).
__global__ __launch_bounds__(256) void bucket_single_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                            const float* __restrict__ survival, float skip_below,
                                                            int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                            int32_t* __restrict__ slot_pos) {
  __shared__ ChunkMasks cm;
  __shared__ int32_t base[MAX_E];
  __shared__ int32_t total;
  fill_masks(cm, ids, T, E, k, survival, skip_below, 0);
  for (int e = threadIdx.x; e < E; e += blockDim.x) base[e] = mask_count(cm, e);
  __syncthreads();
  const int last_count = base[E - 1];
  __syncthreads();
  block_exclusive_scan(base, E);
  if (threadIdx.x == 0) total = base[E - 1] + last_count;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) offsets[e] = base[e];
  if (threadIdx.x == 0) offsets[E] = total;
  for (int p = total + threadIdx.x; p < T * k; p += blockDim.x) perm[p] = -1;
  scatter_chunk(cm, ids, T, E, k, survival, skip_below, 0, base, perm, slot_pos);
}

// Multi-chunk path, step 1: per-chunk counts -> counts[c][e].
__global__ __launch_bounds__(256) void bucket_count_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                           const float* __restrict__ survival, float skip_below,
                                                           int32_t* __restrict__ counts) {
  __shared__ ChunkMasks cm;
  const int c = blockIdx.x;
  fill_masks(cm, ids, T, E, k, survival, skip_below, c);
  for (int e = threadIdx.x; e < E; e += blockDim.x) counts[(int64_t)c * E + e] = mask_count(cm, e);
}

// Step 2 (one block): expert offsets and per-chunk bases (written over counts).
__global__ __launch_bounds__(256) void bucket_scan_kernel(int32_t* __restrict__ counts, int nchunks, int T, int E, int k,
                                                          int32_t* __restrict__ offsets, int32_t* __restrict__ perm) {
  __shared__ int32_t tot[MAX_E];
  __shared__ int32_t total;
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int s = 0;
    for (int c = 0; c < nchunks; ++c) s += counts[(int64_t)c * E + e];
    tot[e] = s;
  }
  __syncthreads();
  const int last_count = tot[E - 1];
  __syncthreads();
  block_exclusive_scan(tot, E);
  if (threadIdx.x == 0) total = tot[E - 1] + last_count;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    offsets[e] = tot[e];
    int run = tot[e];
    for (int c = 0; c < nchunks; ++c) {
      const int n = counts[(int64_t)c * E + e];
      counts[(int64_t)c * E + e] = run;
      run += n;
    }
  }
  if (threadIdx.x == 0) offsets[E] = total;
  for (int p = total + threadIdx.x; p < T * k; p += blockDim.x) perm[p] = -1;
}

// Step 3: scatter each chunk at its bases.
__global__ __launch_bounds__(256) void bucket_scatter_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                             const float* __restrict__ survival, float skip_below,
                                                             const int32_t* __restrict__ bases,
                                                             int32_t* __restrict__ perm, int32_t* __restrict__ slot_pos) {
  __shared__ ChunkMasks cm;
  const int c = blockIdx.x;
  fill_masks(cm, ids, T, E, k, survival, skip_below, c);
  scatter_chunk(cm, ids, T, E, k, survival, skip_below, c, bases + (int64_t)c * E, perm, slot_pos);
}

size_t route_ws_bytes(int T, int E) {
  const size_t nchunks = ((size_t)T + ROUTE_CHUNK - 1) / ROUTE_CHUNK;
  const size_t b = nchunks * (size_t)E * 4;
  return ((b + 255) / 256) * 256 + 256;
}

hipError_t launch_route(const float* logits, int T, int E, int k, const float* survival, float skip_below,
                        int32_t* ids, float* w, int32_t* offsets, int32_t* perm, int32_t* slot_pos,
                        void* ws, hipStream_t stream, const char** variant) {
  const int nchunks = (T + ROUTE_CHUNK - 1) / ROUTE_CHUNK;
  if (T > 0)
    hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, logits, T, E, k, survival, skip_below,
                       ids, w, slot_pos);
  if (nchunks <= 1) {
    hipLaunchKernelGGL(bucket_single_kernel, dim3(1), dim3(256), 0, stream, ids, T, E, k, survival, skip_below,
                       offsets, perm, slot_pos);
    *variant = "route:topk_wave+bucket_single";
  } else {
    int32_t* counts = static_cast<int32_t*>(ws);
    hipLaunchKernelGGL(bucket_count_kernel, dim3(nchunks), dim3(256), 0, stream, ids, T, E, k, survival, skip_below,
                       counts);
    hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(256), 0, stream, counts, nchunks, T, E, k, offsets, perm);
    hipLaunchKernelGGL(bucket_scatter_kernel, dim3(nchunks), dim3(256), 0, stream, ids, T, E, k, survival,
                       skip_below, counts, perm, slot_pos);
    *variant = "route:topk_wave+bucket_count/scan/scatter";
  }
  return hipGetLastError();
}

}  // namespace mx
