// Top-k of one row by one wavefront and the softmax over the picks, shared
// by the route kernels and the fused single-row layer (the MoE top-k gate of
// the "New Deepseek 4.1 flash recipe" thread, post #6, "How it works"; exact
// ties by lowest position, post #4, "Exact indexer selections").
#pragma once
#include "mx_device.hpp"

extern "C" __device__ unsigned int __ockl_wfred_max_u32(unsigned int);
extern "C" __device__ unsigned int __ockl_wfred_min_u32(unsigned int);

namespace mx {

__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// One wavefront ranks the row at l.  PER = logits per lane (E <= 64 * PER);
// after round j, lane j holds (expert, logit) of slot j.  Lane l holds the
// block of logits [PER l, PER l + PER), so lane order is index order: of the
// lanes whose best key equals the round's maximum, the lowest one holds the
// lowest index, and within a lane a strict comparison keeps the lowest
// position.  Each round is branch-free: one wavefront maximum, one ballot,
// one readlane.  The rounds can be run in installments (topk_rounds), so a
// caller that needs slot j only waits for j + 1 rounds before using it and
// runs the rest later (e.g. while its loads are in flight).
template <int PER>
struct TopkState {
  uint32_t key[PER];
  int idx;                                                      // lane j: expert of slot j (after round j)
  float val;                                                    // lane j: its logit
  int done;                                                     // rounds run so far
};

template <int PER>
__device__ __forceinline__ void topk_begin(TopkState<PER>& st, const float* __restrict__ l, int E) {
  const int lane = threadIdx.x & 63;
  float v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = l[min(PER * lane + i, E - 1)];   // all loads in flight together
#pragma unroll
  for (int i = 0; i < PER; ++i) st.key[i] = PER * lane + i < E ? order_key(v[i]) : 0u;   // 0: below every logit
  st.idx = 0;
  st.val = 0.0f;
  st.done = 0;
}

template <int PER>
__device__ __forceinline__ void topk_rounds(TopkState<PER>& st, int upto) {
  const int lane = threadIdx.x & 63;
  for (int j = st.done; j < upto; ++j) {
    uint32_t bk = st.key[0];                                    // this lane's best: ties keep the lower index
    int bi = 0;
#pragma unroll
    for (int i = 1; i < PER; ++i) {
      const bool gt = st.key[i] > bk;
      bk = gt ? st.key[i] : bk;
      bi = gt ? i : bi;
    }
    const uint32_t m = __ockl_wfred_max_u32(bk);
    const int wl = (int)__builtin_ctzll(__ballot(bk == m));    // lowest lane holding the maximum
    const int wbi = __builtin_amdgcn_readlane(bi, wl);
    const bool mine = lane == wl;
#pragma unroll
    for (int i = 0; i < PER; ++i) st.key[i] = (mine && i == wbi) ? 0u : st.key[i];
    st.idx = lane == j ? PER * wl + wbi : st.idx;
    st.val = lane == j ? key_value(m) : st.val;
  }
  st.done = upto > st.done ? upto : st.done;
}

// All k rounds at once: lanes j < k end with (expert, logit) of slot j.
template <int PER>
__device__ void wave_topk(const float* __restrict__ l, int E, int k, int& out_idx, float& out_val) {
  TopkState<PER> st;
  topk_begin<PER>(st, l, E);
  topk_rounds<PER>(st, k);
  out_idx = st.idx;
  out_val = st.val;
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

}  // namespace mx
