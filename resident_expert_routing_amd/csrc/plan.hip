// moe_hot_pick: the hot-read decision (TideLM README, "How adaptive expert
// loading works", item 3, GLM-5.3 bullet): the heaviest miss carrying at least
// a threshold share of a token's routing weight, and the coldest expert held
// in an arena slot (hot-ring slots are never evicted).
#include "common.hpp"

namespace moe {

// Candidate miss: larger share first, then lower expert id, then lower token.
struct Miss {
  double share;
  int e, t;
};

__device__ __forceinline__ bool better(const Miss& a, const Miss& b) {
  if (a.share != b.share) return a.share > b.share;
  if (a.e != b.e) return a.e < b.e;
  return a.t < b.t;
}

// Resident candidate: smaller history first, then lower expert id.
struct Cold {
  double hist;
  int e;
};

__device__ __forceinline__ bool colder(const Cold& a, const Cold& b) {
  if (a.hist != b.hist) return a.hist < b.hist;
  return a.e < b.e;
}

__global__ __launch_bounds__(1024) void hot_pick_kernel(
    const int32_t* __restrict__ te, const float* __restrict__ ts, int T, int k, int E,
    const int32_t* __restrict__ expert_slot, int S, int n_arena, const double* __restrict__ hist,
    double threshold, int32_t* __restrict__ out) {
  __shared__ Miss wm[16];
  __shared__ Cold wc[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  Miss best{-1.0, 0x7FFFFFFF, 0x7FFFFFFF};
  for (int t = tid; t < T; t += 1024) {
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += (double)ts[(size_t)t * k + j];
    for (int j = 0; j < k; ++j) {
      const int e = te[(size_t)t * k + j];
      if (e < 0 || e >= E) continue;
      const int s = expert_slot[e];
      if (s >= 0 && s < S) continue;  // routable: not a miss
      const double share = (double)ts[(size_t)t * k + j] / sum;
      if (share >= threshold) {
        const Miss m{share, e, t};
        if (better(m, best)) best = m;
      }
    }
  }
  Cold cold{INFINITY, 0x7FFFFFFF};
  for (int e = tid; e < E; e += 1024) {
    const int s = expert_slot[e];
    if (s >= 0 && s < n_arena && s < S) {
      const Cold c{hist[e], e};
      if (colder(c, cold)) cold = c;
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const Miss o{__shfl_xor(best.share, d, kWave), __shfl_xor(best.e, d, kWave),
                 __shfl_xor(best.t, d, kWave)};
    if (better(o, best)) best = o;
    const Cold oc{__shfl_xor(cold.hist, d, kWave), __shfl_xor(cold.e, d, kWave)};
    if (colder(oc, cold)) cold = oc;
  }
  if (lane == 0) {
    wm[wv] = best;
    wc[wv] = cold;
  }
  __syncthreads();
  if (tid == 0) {
    Miss b = wm[0];
    Cold c = wc[0];
    for (int i = 1; i < 16; ++i) {
      if (better(wm[i], b)) b = wm[i];
      if (colder(wc[i], c)) c = wc[i];
    }
    out[0] = b.share >= 0.0 ? b.e : -1;
    out[1] = c.e != 0x7FFFFFFF ? c.e : -1;
  }
}

}  // namespace moe

using namespace moe;

extern "C" MOE_EXPORT int moe_hot_pick(const int32_t* topk_expert, const float* topk_score, int T,
                                       int k, int E, const int32_t* expert_slot, int S,
                                       int n_arena, const double* hist_row, double threshold,
                                       int32_t* out, hipStream_t stream) {
  if (T < 0 || k <= 0 || E <= 0 || S < 0 || n_arena < 0) return MOE_EINVAL;
  if (k > MOE_MAX_K || E > MOE_MAX_E || S > MOE_MAX_S) return MOE_EUNSUPPORTED;
  if (!expert_slot || !hist_row || !out) return MOE_EINVAL;
  if (T > 0 && (!topk_expert || !topk_score)) return MOE_EINVAL;
  if (!aligned(hist_row, 8) || !aligned(out, 4)) return MOE_EINVAL;
  if (!(threshold >= 0.0)) return MOE_EINVAL;  // also rejects NaN
  hot_pick_kernel<<<1, 1024, 0, stream>>>(topk_expert, topk_score, T, k, E, expert_slot, S,
                                          n_arena, hist_row, threshold, out);
  return hip_status();
}
