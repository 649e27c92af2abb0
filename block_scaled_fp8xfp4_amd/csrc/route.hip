// Top-k gate and bucketing (the MoE top-k gate of the "New Deepseek 4.1
// flash recipe" thread, post #6, "How it works"; exact ties by lowest
// position, post #4, "Exact indexer selections"; dead verification rows of
// post #2, "What changed"; the route planner and per-slot buffer of the
// DeepSeek-V4.1-Flash-4x-DGX-Spark-TP4 README, settings table, row "Experts").
//
// Top-k of one row, one wavefront: each lane holds E/64 logits as order-
// preserving 32-bit keys (-0 folded into +0, so it ties with +0).  The k-th
// largest key is found by a 32-round radix select in which every round is
// one wavefront ballot per register (no LDS traffic); the rows picked are
// all keys above it plus, among keys equal to it, the lowest expert indices.
// The k winners are ranked by (logit descending, index ascending) inside the
// wavefront.  Weights are the softmax over the picked logits, evaluated in
// double and rounded to fp32.
//
// Bucketing is a counting sort of the live (row, slot) pairs by expert with
// the canonical order (expert, row): per chunk of 256 rows, each row ORs its
// bit into a per-expert row bitmask in LDS; a pair's rank among the chunk's
// rows that picked the same expert is a population count of the lower bits,
// so no atomic ordering ever decides a position.  Up to 256 rows the whole
// route is one workgroup and one launch.
#include <climits>
#include "mx_device.hpp"
#include "mx_launch.hpp"

namespace mx {


__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int ballot_count(bool p) { return __popcll(__ballot(p)); }

// One wavefront ranks row t.  PER = logits per lane (E <= 64 * PER); lanes
// j < k end with (idx, logit) of slot j.
template <int PER>
__device__ void wave_topk(const float* __restrict__ l, int E, int k, int* sel_idx /* LDS [16] */,
                          float* sel_val /* LDS [16] */, uint32_t* sel_key /* LDS [16] */, int& out_idx,
                          float& out_val) {
  const int lane = threadIdx.x & 63;
  float v[PER];
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? l[e] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) key[i] = (lane + 64 * i < E) ? order_key(v[i]) : 0u;   // 0: never selected
  // k-th largest key: the largest x with #(key >= x) >= k.  Each lane counts
  // its own keys; the wavefront total is assembled bit by bit from ballots.
  constexpr int CBITS = PER <= 1 ? 1 : PER <= 3 ? 2 : PER <= 7 ? 3 : PER <= 15 ? 4 : 5;
  uint32_t x = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t t = x | (1u << b);
    int c = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) c += key[i] >= t ? 1 : 0;
    int total = 0;
#pragma unroll
    for (int q = 0; q < CBITS; ++q) total += __popcll(__ballot((c >> q) & 1)) << q;
    if (total >= k) x = t;
  }
  int gtl = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) gtl += key[i] > x ? 1 : 0;
  int gt = 0;
#pragma unroll
  for (int q = 0; q < CBITS; ++q) gt += __popcll(__ballot((gtl >> q) & 1)) << q;
  const int need = k - gt;                                       // ties at x to take, lowest index first
  const unsigned long long below = lane ? ((1ull << lane) - 1ull) : 0ull;
  int ties_before = 0, placed = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool eq = key[i] == x && lane + 64 * i < E;
    const unsigned long long me = __ballot(eq);
    const bool take = key[i] > x || (eq && ties_before + __popcll(me & below) < need);
    const unsigned long long ms = __ballot(take);
    if (take) {
      const int pos = placed + __popcll(ms & below);
      sel_idx[pos] = lane + 64 * i;
      sel_val[pos] = v[i];
      sel_key[pos] = key[i];
    }
    ties_before += __popcll(me);
    placed += __popcll(ms);
  }
  __builtin_amdgcn_wave_barrier();
  // rank the k winners by (key descending, index ascending)
  int my_rank = 0;
  int mi = 0;
  float mv = 0.0f;
  if (lane < k) {
    mi = sel_idx[lane];
    mv = sel_val[lane];
    const uint32_t mk = sel_key[lane];
    for (int m = 0; m < k; ++m) {
      const uint32_t ok2 = sel_key[m];
      my_rank += (ok2 > mk || (ok2 == mk && sel_idx[m] < mi)) ? 1 : 0;
    }
  }
  __builtin_amdgcn_wave_barrier();
  if (lane < k) {
    sel_idx[my_rank] = mi;
    sel_val[my_rank] = mv;
  }
  __builtin_amdgcn_wave_barrier();
  out_idx = lane < k ? sel_idx[lane] : 0;
  out_val = lane < k ? sel_val[lane] : 0.0f;
}

// softmax over the k picked logits: w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), in double
__device__ __forceinline__ float slot_weight(float val, int k) {
  const int lane = threadIdx.x & 63;
  const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(val), 0));   // slot 0's logit
  const double ex = lane < k ? exp((double)val - (double)v0) : 0.0;
  double den = 0.0;
  for (int j = 0; j < k; ++j) {
    const long long bits = __double_as_longlong(ex);
    const int lo = __builtin_amdgcn_readlane((int)(bits & 0xFFFFFFFFll), j);
    const int hi = __builtin_amdgcn_readlane((int)(bits >> 32), j);
    den += __longlong_as_double(((long long)(unsigned)hi << 32) | (unsigned)lo);
  }
  return (float)(ex / den);
}

__device__ __forceinline__ bool row_live(const float* survival, float skip_below, int t) {
  return survival == nullptr || !(survival[t] < skip_below);
}

struct TopkScratch {
  int idx[4][16];
  float val[4][16];
  uint32_t key[4][16];
};

// Top-k of rows t = row0 + wave, + 4, ... (< T) by the four wavefronts of a block.
template <int PER>
__device__ void topk_rows(const float* __restrict__ logits, int T, int E, int k, const float* __restrict__ survival,
                          float skip_below, int32_t* __restrict__ ids, float* __restrict__ w,
                          int32_t* __restrict__ slot_pos, int row0, int row_stride, TopkScratch& sc,
                          int32_t* ids_lds /* optional [T][k] copy */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int t = row0 + wave; t < T; t += row_stride) {
    int idx;
    float val;
    wave_topk<PER>(logits + (int64_t)t * E, E, k, sc.idx[wave], sc.val[wave], sc.key[wave], idx, val);
    const float wt = slot_weight(val, k);
    if (lane < k) {
      ids[(int64_t)t * k + lane] = idx;
      w[(int64_t)t * k + lane] = wt;
      if (!row_live(survival, skip_below, t)) slot_pos[(int64_t)t * k + lane] = -1;
      if (ids_lds) ids_lds[t * k + lane] = idx;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int PER>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   const float* __restrict__ survival, float skip_below,
                                                   int32_t* __restrict__ ids, float* __restrict__ w,
                                                   int32_t* __restrict__ slot_pos) {
  __shared__ TopkScratch sc;
  topk_rows<PER>(logits, T, E, k, survival, skip_below, ids, w, slot_pos, blockIdx.x * 4, 1 << 30, sc, nullptr);
}

// ------------------------------------------------------------------ buckets
// LDS bitmask of the rows (within a chunk of 256) that picked each expert.
struct ChunkMasks {
  unsigned long long m[MAX_E][4];
};

// Build the masks of chunk c (rows c*256 .. c*256+255); block of 256 threads.
// ids come from `ids` (global) or, when ids_lds is set, from LDS.
__device__ void fill_masks(ChunkMasks& cm, const int32_t* __restrict__ ids, const int32_t* ids_lds, int T, int E, int k,
                           const float* __restrict__ survival, float skip_below, int c) {
  for (int i = threadIdx.x; i < E * 4; i += blockDim.x) (&cm.m[0][0])[i] = 0ull;
  lds_barrier();
  const int r = threadIdx.x, t = c * ROUTE_CHUNK + r;
  if (t < T && row_live(survival, skip_below, t)) {
    for (int j = 0; j < k; ++j) {
      const int e = ids_lds ? ids_lds[r * k + j] : ids[(int64_t)t * k + j];
      if (e >= 0 && e < E) atomicOr(&cm.m[e][r >> 6], 1ull << (r & 63));
    }
  }
  lds_barrier();
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

__device__ void scatter_chunk(const ChunkMasks& cm, const int32_t* __restrict__ ids, const int32_t* ids_lds, int T,
                              int E, int k, const float* __restrict__ survival, float skip_below, int c,
                              const int32_t* base /* [E], LDS or global */, int32_t* __restrict__ perm,
                              int32_t* __restrict__ slot_pos) {
  const int r = threadIdx.x, t = c * ROUTE_CHUNK + r;
  if (t < T && row_live(survival, skip_below, t)) {
    for (int j = 0; j < k; ++j) {
      const int e = ids_lds ? ids_lds[r * k + j] : ids[(int64_t)t * k + j];
      if (e < 0 || e >= E) continue;
      const int p = base[e] + mask_rank(cm, e, r);
      perm[p] = t * k + j;
      slot_pos[(int64_t)t * k + j] = p;
    }
  }
}

// Exclusive scan of n <= MAX_E ints in LDS (4 per thread, block of 256, one
// wavefront scan of the per-thread sums); returns the total to every thread.
__device__ int block_exclusive_scan(int32_t* vals, int n) {
  __shared__ int32_t partial[256];
  __shared__ int32_t total;
  const int tid = threadIdx.x;
  int local[4], s = 0;
  for (int i = 0; i < 4; ++i) {
    const int idx = tid * 4 + i;
    local[i] = idx < n ? vals[idx] : 0;
    s += local[i];
  }
  partial[tid] = s;
  lds_barrier();
  if (tid < 64) {
    int q[4], run = 0;
    for (int i = 0; i < 4; ++i) { q[i] = partial[tid * 4 + i]; run += q[i]; }
    int x = run;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (tid >= off) x += y;
    }
    int excl = x - run;
    for (int i = 0; i < 4; ++i) { partial[tid * 4 + i] = excl; excl += q[i]; }
    if (tid == 63) total = x;
  }
  lds_barrier();
  int run = partial[tid];
  for (int i = 0; i < 4; ++i) {
    const int idx = tid * 4 + i;
    if (idx < n) vals[idx] = run;
    run += local[i];
  }
  lds_barrier();
  return total;
}

// The whole route for T <= 256 in one workgroup and one launch.
template <int PER>
__global__ __launch_bounds__(256) void route_small_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                          const float* __restrict__ survival, float skip_below,
                                                          int32_t* __restrict__ ids, float* __restrict__ w,
                                                          int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ slot_pos) {
  __shared__ TopkScratch sc;
  __shared__ int32_t ids_lds[ROUTE_CHUNK * MAX_K];
  __shared__ ChunkMasks cm;
  __shared__ int32_t base[MAX_E];
  topk_rows<PER>(logits, T, E, k, survival, skip_below, ids, w, slot_pos, 0, 4, sc, ids_lds);
  lds_barrier();
  fill_masks(cm, ids, ids_lds, T, E, k, survival, skip_below, 0);
  for (int e = threadIdx.x; e < E; e += blockDim.x) base[e] = mask_count(cm, e);
  lds_barrier();
  const int total = block_exclusive_scan(base, E);
  for (int e = threadIdx.x; e < E; e += blockDim.x) offsets[e] = base[e];
  if (threadIdx.x == 0) offsets[E] = total;
  for (int p = total + threadIdx.x; p < T * k; p += blockDim.x) perm[p] = -1;
  scatter_chunk(cm, ids, ids_lds, T, E, k, survival, skip_below, 0, base, perm, slot_pos);
}

// Multi-chunk path, step 1: per-chunk counts -> counts[c][e].
__global__ __launch_bounds__(256) void bucket_count_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                           const float* __restrict__ survival, float skip_below,
                                                           int32_t* __restrict__ counts) {
  __shared__ ChunkMasks cm;
  const int c = blockIdx.x;
  fill_masks(cm, ids, nullptr, T, E, k, survival, skip_below, c);
  for (int e = threadIdx.x; e < E; e += blockDim.x) counts[(int64_t)c * E + e] = mask_count(cm, e);
}

// Step 2 (one block): expert offsets and per-chunk bases (written over counts).
__global__ __launch_bounds__(256) void bucket_scan_kernel(int32_t* __restrict__ counts, int nchunks, int T, int E, int k,
                                                          int32_t* __restrict__ offsets, int32_t* __restrict__ perm) {
  __shared__ int32_t tot[MAX_E];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int s = 0;
    for (int c = 0; c < nchunks; ++c) s += counts[(int64_t)c * E + e];
    tot[e] = s;
  }
  __syncthreads();
  const int total = block_exclusive_scan(tot, E);
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
  fill_masks(cm, ids, nullptr, T, E, k, survival, skip_below, c);
  scatter_chunk(cm, ids, nullptr, T, E, k, survival, skip_below, c, bases + (int64_t)c * E, perm, slot_pos);
}

size_t route_ws_bytes(int T, int E) {
  const size_t nchunks = ((size_t)T + ROUTE_CHUNK - 1) / ROUTE_CHUNK;
  const size_t b = nchunks * (size_t)E * 4;
  return ((b + 255) / 256) * 256 + 256;
}

template <int PER>
static void launch_route_per(const float* logits, int T, int E, int k, const float* survival, float skip_below,
                             int32_t* ids, float* w, int32_t* offsets, int32_t* perm, int32_t* slot_pos, void* ws,
                             hipStream_t stream, const char** variant) {
  const int nchunks = (T + ROUTE_CHUNK - 1) / ROUTE_CHUNK;
  if (nchunks <= 1) {
    hipLaunchKernelGGL((route_small_kernel<PER>), dim3(1), dim3(256), 0, stream, logits, T, E, k, survival,
                       skip_below, ids, w, offsets, perm, slot_pos);
    *variant = "route:fused_single_workgroup";
  } else {
    int32_t* counts = static_cast<int32_t*>(ws);
    hipLaunchKernelGGL((topk_kernel<PER>), dim3((T + 3) / 4), dim3(256), 0, stream, logits, T, E, k, survival,
                       skip_below, ids, w, slot_pos);
    hipLaunchKernelGGL(bucket_count_kernel, dim3(nchunks), dim3(256), 0, stream, ids, T, E, k, survival, skip_below,
                       counts);
    hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(256), 0, stream, counts, nchunks, T, E, k, offsets, perm);
    hipLaunchKernelGGL(bucket_scatter_kernel, dim3(nchunks), dim3(256), 0, stream, ids, T, E, k, survival,
                       skip_below, counts, perm, slot_pos);
    *variant = "route:topk_wave+bucket_count/scan/scatter";
  }
}

hipError_t launch_route(const float* logits, int T, int E, int k, const float* survival, float skip_below,
                        int32_t* ids, float* w, int32_t* offsets, int32_t* perm, int32_t* slot_pos,
                        void* ws, hipStream_t stream, const char** variant) {
  if (E <= 64) launch_route_per<1>(logits, T, E, k, survival, skip_below, ids, w, offsets, perm, slot_pos, ws, stream, variant);
  else if (E <= 128) launch_route_per<2>(logits, T, E, k, survival, skip_below, ids, w, offsets, perm, slot_pos, ws, stream, variant);
  else if (E <= 256) launch_route_per<4>(logits, T, E, k, survival, skip_below, ids, w, offsets, perm, slot_pos, ws, stream, variant);
  else if (E <= 512) launch_route_per<8>(logits, T, E, k, survival, skip_below, ids, w, offsets, perm, slot_pos, ws, stream, variant);
  else launch_route_per<16>(logits, T, E, k, survival, skip_below, ids, w, offsets, perm, slot_pos, ws, stream, variant);
  return hipGetLastError();
}

}  // namespace mx
