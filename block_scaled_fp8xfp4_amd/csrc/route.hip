// Top-k gate and bucketing (the MoE top-k gate of the "New Deepseek 4.1
// flash recipe" thread, post #6, "How it works"; exact ties by lowest
// position, post #4, "Exact indexer selections"; dead verification rows of
// post #2, "What changed"; the route planner and per-slot buffer of the
// DeepSeek-V4.1-Flash-4x-DGX-Spark-TP4 README, settings table, row "Experts";
// router-live verification rows, same table, row "Verify length").
//
// Top-k of one row, one wavefront: each lane holds E/64 logits as order-
// preserving 32-bit keys (-0 folded into +0, so it ties with +0).  k rounds
// of a wavefront maximum (cross-lane reduction in registers) pick the slots
// in order: the largest remaining key, and among equal keys the lowest
// expert index, which is exactly slot order (logit descending, ties to the
// lower index).  Weights are the softmax over the picked logits, evaluated
// in double and rounded to fp32.
//
// Bucketing is a counting sort of the live (row, slot) pairs by expert with
// the canonical order (expert, row): each row ORs its bit into a per-expert
// row bitmask in LDS; a pair's rank among the rows that picked the same
// expert is a population count of the lower bits, so no atomic ordering ever
// decides a position.  One row: the wavefront that ranked it also buckets it
// in registers.  Up to 256 rows: one workgroup, one wavefront per row at a
// time.  More rows: chunks of 256 rows over several launches.
//
// Router-live mode (an anchor per row): a verification row below the
// survival threshold does not skip the experts but takes its anchor row's
// top-k, found by its own wavefront from the anchor's logits (no dependence
// between rows), weighted by the softmax of its own logits over those
// experts; every row joins the buckets.
#include <climits>
#include "mx_device.hpp"
#include "mx_launch.hpp"
#include "route_device.hpp"

namespace mx {

// softmax over k logits of another row's picks, w_j = exp(l_j - m) / sum_i
// exp(l_i - m) with m the largest of them, in double
__device__ __forceinline__ float slot_weight_max(float val, int k) {
  const int lane = threadIdx.x & 63;
  float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(val), 0));
  for (int j = 1; j < k; ++j) m = fmaxf(m, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(val), j)));
  const double ex = lane < k ? exp((double)val - (double)m) : 0.0;
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

// How row t is routed.  Skip mode (anchor == NULL): its own experts, in the
// buckets only when live.  Router-live mode: every row is bucketed; a row
// below the threshold with a valid anchor a != t takes row a's experts.
__device__ __forceinline__ void row_mode(const float* survival, float thr, const int32_t* anchor, int T, int t,
                                         bool& live, int& src) {
  src = t;
  if (!anchor) {
    live = row_live(survival, thr, t);
    return;
  }
  live = true;
  if (survival && survival[t] < thr) {
    const int a = anchor[t];
    if (a >= 0 && a < T) src = a;
  }
}

// Top-k + weights of row t by one wavefront; writes ids and weights (and -1
// slot positions for a dead row); returns the row's expert in lanes < k.
// The experts are row src's top-k (src = t, or a router-live row's anchor);
// the weights always come from row t's own logits.
template <int PER>
__device__ int topk_row(const float* __restrict__ logits, int t, int src, int E, int k, bool live,
                        int32_t* __restrict__ ids, float* __restrict__ w, int32_t* __restrict__ slot_pos) {
  const int lane = threadIdx.x & 63;
  int idx;
  float val;
  wave_topk<PER>(logits + (int64_t)src * E, E, k, idx, val);
  float wt;
  if (src == t) {
    wt = slot_weight(val, k);
  } else {
    val = lane < k ? logits[(int64_t)t * E + idx] : 0.0f;
    wt = slot_weight_max(val, k);
  }
  if (lane < k) {
    ids[(int64_t)t * k + lane] = idx;
    w[(int64_t)t * k + lane] = wt;
    if (!live) slot_pos[(int64_t)t * k + lane] = -1;
  }
  return idx;
}

// ------------------------------------------------------------------ one row
// T = 1: a live row's k experts are distinct, so its pair for slot j sits at
// the rank of expert j among the row's experts, and offsets[e] counts the
// row's experts below e.  One wavefront, no LDS.
template <int PER>
__global__ __launch_bounds__(64) void route1_kernel(const float* __restrict__ logits, int E, int k,
                                                    const float* __restrict__ survival, float skip_below,
                                                    const int32_t* __restrict__ anchor,
                                                    int32_t* __restrict__ ids, float* __restrict__ w,
                                                    int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                    int32_t* __restrict__ slot_pos) {
  const int lane = threadIdx.x;
  bool live;
  int src;
  row_mode(survival, skip_below, anchor, 1, 0, live, src);
  const int idx = topk_row<PER>(logits, 0, src, E, k, live, ids, w, slot_pos);
  int rank = 0;
  for (int i = 0; i < k; ++i) rank += __builtin_amdgcn_readlane(idx, i) < idx ? 1 : 0;
  if (lane < k) {
    if (live) {
      slot_pos[lane] = rank;
      perm[rank] = lane;
    } else {
      perm[lane] = -1;
    }
  }
  for (int e = lane; e <= E; e += 64) {
    int below = 0;
    for (int i = 0; i < k; ++i) below += __builtin_amdgcn_readlane(idx, i) < e ? 1 : 0;
    offsets[e] = live ? below : 0;
  }
}

// Gather chunk c's experts (-1 for dead rows) into LDS.
__device__ int load_chunk_ids(const int32_t* __restrict__ ids, int T, int k, const float* __restrict__ survival,
                              float skip_below, int c, int32_t* ids_lds) {
  const int c0 = c * ROUTE_CHUNK, nrows = min(ROUTE_CHUNK, T - c0);
  for (int p = threadIdx.x; p < nrows * k; p += blockDim.x) {
    const int t = c0 + p / k;
    ids_lds[p] = row_live(survival, skip_below, t) ? ids[(int64_t)c0 * k + p] : -1;
  }
  return nrows;
}

// ----------------------------------------------------------- up to 256 rows
// Exclusive scan of v over the threads of the block (any multiple of 64 up to
// 1024 threads); every thread gets its prefix, and the total.
__device__ int block_excl_scan(int v, int& total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  lds_barrier();
  int before = 0;
  total = 0;
  for (int i = 0; i < nw; ++i) {
    const int s = wsum[i];
    before += i < wave ? s : 0;
    total += s;
  }
  lds_barrier();                                                // wsum may be reused by the caller
  return before + x - v;
}

// Bitmasks of the rows (< 256) that picked each expert.
struct RowMasks {
  unsigned long long m[MAX_E][4];
};

__device__ __forceinline__ int mask_rank(const RowMasks& cm, int e, int r) {
  int n = 0;
  for (int q = 0; q < (r >> 6); ++q) n += __popcll(cm.m[e][q]);
  const unsigned long long below = (r & 63) ? (cm.m[e][r >> 6] & ((1ull << (r & 63)) - 1ull)) : 0ull;
  return n + __popcll(below);
}

// Bucket the pairs of chunk rows [c0, c0 + nrows) (nrows <= 256) whose
// experts are in ids_lds[(t - c0) * k + j] (-1: dead row).  base[e] (LDS or
// global) is where the chunk's first pair of expert e goes.
__device__ void fill_chunk_masks(RowMasks& cm, const int32_t* ids_lds, int nrows, int E, int k) {
  for (int i = threadIdx.x; i < E * 4; i += blockDim.x) (&cm.m[0][0])[i] = 0ull;
  lds_barrier();
  for (int p = threadIdx.x; p < nrows * k; p += blockDim.x) {
    const int r = p / k, e = ids_lds[p];
    if (e >= 0 && e < E) atomicOr(&cm.m[e][r >> 6], 1ull << (r & 63));
  }
  lds_barrier();
}

__device__ void scatter_chunk(const RowMasks& cm, const int32_t* ids_lds, int c0, int nrows, int E, int k,
                              const int32_t* base, int32_t* __restrict__ perm, int32_t* __restrict__ slot_pos) {
  for (int p = threadIdx.x; p < nrows * k; p += blockDim.x) {
    const int r = p / k, j = p % k, e = ids_lds[p];
    if (e < 0 || e >= E) continue;
    const int pos = base[e] + mask_rank(cm, e, r);
    const int t = c0 + r;
    perm[pos] = t * k + j;
    slot_pos[(int64_t)t * k + j] = pos;
  }
}

// The whole route for 1 < T <= 256 in one workgroup: one wavefront per row
// for the top-k, then the bitmask counting sort over all the block's threads.
// TOPK false: the rows were ranked by topk_kernel (one wavefront per row over
// many CUs: one CU ranking more than a few rows is bound by its own issue
// rate), and this workgroup only buckets ids (bucket_survival: the rows that
// join the buckets, NULL for all).
template <int PER, bool TOPK>
__global__ __launch_bounds__(1024) void route_small_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                           const float* __restrict__ survival, float skip_below,
                                                           const int32_t* __restrict__ anchor,
                                                           int32_t* __restrict__ ids, float* __restrict__ w,
                                                           int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ slot_pos) {
  __shared__ int32_t ids_lds[ROUTE_CHUNK * MAX_K];
  __shared__ RowMasks cm;
  __shared__ int32_t base[MAX_E];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int i = threadIdx.x; i < E * 4; i += blockDim.x) (&cm.m[0][0])[i] = 0ull;
  if (TOPK) {
    for (int t = wave; t < T; t += nw) {
      bool live;
      int src;
      row_mode(survival, skip_below, anchor, T, t, live, src);
      const int idx = topk_row<PER>(logits, t, src, E, k, live, ids, w, slot_pos);
      if (lane < k) ids_lds[t * k + lane] = live ? idx : -1;
    }
  } else {
    load_chunk_ids(ids, T, k, survival, skip_below, 0, ids_lds);
  }
  lds_barrier();
  for (int p = threadIdx.x; p < T * k; p += blockDim.x) {
    const int r = p / k, e = ids_lds[p];
    if (e >= 0 && e < E) atomicOr(&cm.m[e][r >> 6], 1ull << (r & 63));
  }
  lds_barrier();
  int total = 0;
  for (int e0 = 0; e0 < E; e0 += blockDim.x) {                  // experts in rounds of blockDim
    const int e = e0 + threadIdx.x;
    const int n = e < E ? __popcll(cm.m[e][0]) + __popcll(cm.m[e][1]) + __popcll(cm.m[e][2]) + __popcll(cm.m[e][3]) : 0;
    int round_total;
    const int before = block_excl_scan(n, round_total);
    if (e < E) {
      base[e] = total + before;
      offsets[e] = total + before;
    }
    total += round_total;
  }
  if (threadIdx.x == 0) offsets[E] = total;
  for (int p = total + threadIdx.x; p < T * k; p += blockDim.x) perm[p] = -1;
  lds_barrier();
  scatter_chunk(cm, ids_lds, 0, T, E, k, base, perm, slot_pos);
}

// ------------------------------------------------------------ more rows
// Top-k of rows blockIdx.x * 4 + wave.
template <int PER>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   const float* __restrict__ survival, float skip_below,
                                                   const int32_t* __restrict__ anchor,
                                                   int32_t* __restrict__ ids, float* __restrict__ w,
                                                   int32_t* __restrict__ slot_pos) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  bool live;
  int src;
  row_mode(survival, skip_below, anchor, T, t, live, src);
  topk_row<PER>(logits, t, src, E, k, live, ids, w, slot_pos);
}

// Multi-chunk path, step 1: per-chunk counts -> counts[c][e].
__global__ __launch_bounds__(256) void bucket_count_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                           const float* __restrict__ survival, float skip_below,
                                                           int32_t* __restrict__ counts) {
  __shared__ int32_t ids_lds[ROUTE_CHUNK * MAX_K];
  __shared__ RowMasks cm;
  const int c = blockIdx.x;
  const int nrows = load_chunk_ids(ids, T, k, survival, skip_below, c, ids_lds);
  fill_chunk_masks(cm, ids_lds, nrows, E, k);
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    counts[(int64_t)c * E + e] = __popcll(cm.m[e][0]) + __popcll(cm.m[e][1]) + __popcll(cm.m[e][2]) + __popcll(cm.m[e][3]);
}

// Step 2 (one block): expert offsets and per-chunk bases (written over counts).
__global__ __launch_bounds__(256) void bucket_scan_kernel(int32_t* __restrict__ counts, int nchunks, int T, int E, int k,
                                                          int32_t* __restrict__ offsets, int32_t* __restrict__ perm) {
  int total = 0;
  for (int e0 = 0; e0 < E; e0 += blockDim.x) {
    const int e = e0 + threadIdx.x;
    int s = 0;
    if (e < E)
      for (int c = 0; c < nchunks; ++c) s += counts[(int64_t)c * E + e];
    int round_total;
    const int before = block_excl_scan(s, round_total);
    if (e < E) {
      int run = total + before;
      offsets[e] = run;
      for (int c = 0; c < nchunks; ++c) {
        const int n = counts[(int64_t)c * E + e];
        counts[(int64_t)c * E + e] = run;
        run += n;
      }
    }
    total += round_total;
  }
  if (threadIdx.x == 0) offsets[E] = total;
  for (int p = total + threadIdx.x; p < T * k; p += blockDim.x) perm[p] = -1;
}

// Step 3: scatter each chunk at its bases.
__global__ __launch_bounds__(256) void bucket_scatter_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                             const float* __restrict__ survival, float skip_below,
                                                             const int32_t* __restrict__ bases,
                                                             int32_t* __restrict__ perm, int32_t* __restrict__ slot_pos) {
  __shared__ int32_t ids_lds[ROUTE_CHUNK * MAX_K];
  __shared__ RowMasks cm;
  const int c = blockIdx.x;
  const int nrows = load_chunk_ids(ids, T, k, survival, skip_below, c, ids_lds);
  fill_chunk_masks(cm, ids_lds, nrows, E, k);
  scatter_chunk(cm, ids_lds, c * ROUTE_CHUNK, nrows, E, k, bases + (int64_t)c * E, perm, slot_pos);
}

// T = 0: no pairs, every bucket offset is 0
__global__ __launch_bounds__(256) void zero_offsets_kernel(int32_t* __restrict__ offsets, int n) {
  for (int i = threadIdx.x; i < n; i += 256) offsets[i] = 0;
}

size_t route_ws_bytes(int T, int E) {
  const size_t nchunks = ((size_t)T + ROUTE_CHUNK - 1) / ROUTE_CHUNK;
  const size_t b = nchunks * (size_t)E * 4;
  return ((b + 255) / 256) * 256 + 256;
}

template <int PER>
static void launch_route_per(const float* logits, int T, int E, int k, const float* survival, float skip_below,
                             const int32_t* anchor, int32_t* ids, float* w, int32_t* offsets, int32_t* perm,
                             int32_t* slot_pos, void* ws, hipStream_t stream, const char** variant) {
  const int nchunks = (T + ROUTE_CHUNK - 1) / ROUTE_CHUNK;
  const float* bucket_survival = anchor ? nullptr : survival;   // router-live: every row is bucketed
  if (T == 0) {
    hipLaunchKernelGGL(zero_offsets_kernel, dim3(1), dim3(256), 0, stream, offsets, E + 1);
    *variant = "route:empty";
  } else if (T == 1) {
    hipLaunchKernelGGL((route1_kernel<PER>), dim3(1), dim3(64), 0, stream, logits, E, k, survival, skip_below, anchor,
                       ids, w, offsets, perm, slot_pos);
    *variant = anchor ? "route_live:one_row_wavefront" : "route:one_row_wavefront";
  } else if (T <= ROUTE_FUSED_MAX_T) {
    const int threads = 64 * (T < 16 ? T : 16);
    hipLaunchKernelGGL((route_small_kernel<PER, true>), dim3(1), dim3(threads), 0, stream, logits, T, E, k, survival,
                       skip_below, anchor, ids, w, offsets, perm, slot_pos);
    *variant = anchor ? "route_live:fused_single_workgroup" : "route:fused_single_workgroup";
  } else if (nchunks <= 1) {
    hipLaunchKernelGGL((topk_kernel<PER>), dim3((T + 3) / 4), dim3(256), 0, stream, logits, T, E, k, survival,
                       skip_below, anchor, ids, w, slot_pos);
    hipLaunchKernelGGL((route_small_kernel<PER, false>), dim3(1), dim3(1024), 0, stream, logits, T, E, k,
                       bucket_survival, skip_below, anchor, ids, w, offsets, perm, slot_pos);
    *variant = anchor ? "route_live:topk_wave+bucket_single_workgroup" : "route:topk_wave+bucket_single_workgroup";
  } else {
    int32_t* counts = static_cast<int32_t*>(ws);
    hipLaunchKernelGGL((topk_kernel<PER>), dim3((T + 3) / 4), dim3(256), 0, stream, logits, T, E, k, survival,
                       skip_below, anchor, ids, w, slot_pos);
    hipLaunchKernelGGL(bucket_count_kernel, dim3(nchunks), dim3(256), 0, stream, ids, T, E, k, bucket_survival,
                       skip_below, counts);
    hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(256), 0, stream, counts, nchunks, T, E, k, offsets, perm);
    hipLaunchKernelGGL(bucket_scatter_kernel, dim3(nchunks), dim3(256), 0, stream, ids, T, E, k, bucket_survival,
                       skip_below, counts, perm, slot_pos);
    *variant = anchor ? "route_live:topk_wave+bucket_count/scan/scatter" : "route:topk_wave+bucket_count/scan/scatter";
  }
}

hipError_t launch_route(const float* logits, int T, int E, int k, const float* survival, float skip_below,
                        const int32_t* anchor, int32_t* ids, float* w, int32_t* offsets, int32_t* perm,
                        int32_t* slot_pos, void* ws, hipStream_t stream, const char** variant) {
#define MX_ROUTE(P) launch_route_per<P>(logits, T, E, k, survival, skip_below, anchor, ids, w, offsets, perm, \
                                        slot_pos, ws, stream, variant)
  if (E <= 64) MX_ROUTE(1);
  else if (E <= 128) MX_ROUTE(2);
  else if (E <= 256) MX_ROUTE(4);
  else if (E <= 512) MX_ROUTE(8);
  else MX_ROUTE(16);
#undef MX_ROUTE
  return hipGetLastError();
}

}  // namespace mx
