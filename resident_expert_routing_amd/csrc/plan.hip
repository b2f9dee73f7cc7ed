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

// Token pass: workgroup b takes tokens b*256 + tid, + grid*256, ...; its best
// miss goes to part[b].  The score sum of a token is added in pick order, its
// loads issued 8 at a time; the routable table is read once into LDS.
constexpr int kHotTokenWg = 256;
constexpr int kHotMaxWgs = 256;

__host__ __device__ inline int hot_pick_wgs(int T) {
  const int n = (T + kHotTokenWg - 1) / kHotTokenWg;
  return n < kHotMaxWgs ? n : kHotMaxWgs;
}

__global__ __launch_bounds__(kHotTokenWg) void hot_pick_tokens(
    const int32_t* __restrict__ te, const float* __restrict__ ts, int T, int k, int E,
    const int32_t* __restrict__ expert_slot, int S, double threshold, Miss* __restrict__ part) {
  __shared__ int slot_of[MOE_MAX_E];
  __shared__ Miss wm[kHotTokenWg / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < E; e += kHotTokenWg) slot_of[e] = expert_slot[e];
  __syncthreads();
  Miss best{-1.0, 0x7FFFFFFF, 0x7FFFFFFF};
  for (int t = blockIdx.x * kHotTokenWg + tid; t < T; t += gridDim.x * kHotTokenWg) {
    const float* tsr = ts + (size_t)t * k;
    const int32_t* ter = te + (size_t)t * k;
    double sum = 0.0;
    for (int j0 = 0; j0 < k; j0 += 8) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = tsr[min(j0 + q, k - 1)];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (j0 + q < k) sum += (double)v[q];
    }
    for (int j = 0; j < k; ++j) {  // the rows are in cache now
      const int e = ter[j];
      if (e < 0 || e >= E) continue;
      const int s = slot_of[e];
      if (s >= 0 && s < S) continue;  // routable: not a miss
      const double share = (double)tsr[j] / sum;
      if (share >= threshold) {
        const Miss m{share, e, t};
        if (better(m, best)) best = m;
      }
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const Miss o{__shfl_xor(best.share, d, kWave), __shfl_xor(best.e, d, kWave),
                 __shfl_xor(best.t, d, kWave)};
    if (better(o, best)) best = o;
  }
  if (lane == 0) wm[wv] = best;
  __syncthreads();
  if (tid == 0) {
    Miss b = wm[0];
    for (int i = 1; i < kHotTokenWg / 64; ++i)
      if (better(wm[i], b)) b = wm[i];
    part[blockIdx.x] = b;
  }
}

// Final pass (one workgroup): the best of the nparts token-pass results and
// the coldest arena expert.
__global__ __launch_bounds__(1024) void hot_pick_final(
    const Miss* __restrict__ part, int nparts, int E, const int32_t* __restrict__ expert_slot,
    int S, int n_arena, const double* __restrict__ hist, int32_t* __restrict__ out) {
  __shared__ Miss wm[16];
  __shared__ Cold wc[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  Miss best{-1.0, 0x7FFFFFFF, 0x7FFFFFFF};
  for (int i = tid; i < nparts; i += 1024)
    if (better(part[i], best)) best = part[i];
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

size_t moe_hot_pick_ws_bytes_internal(int T) {
  return up_to((size_t)hot_pick_wgs(T) * sizeof(Miss), 256);
}

extern "C" MOE_EXPORT int moe_hot_pick(const int32_t* topk_expert, const float* topk_score, int T,
                                       int k, int E, const int32_t* expert_slot, int S,
                                       int n_arena, const double* hist_row, double threshold,
                                       int32_t* out, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
  if (T < 0 || k <= 0 || E <= 0 || S < 0 || n_arena < 0) return MOE_EINVAL;
  if (k > MOE_MAX_K || E > MOE_MAX_E || S > MOE_MAX_S) return MOE_EUNSUPPORTED;
  if (!expert_slot || !hist_row || !out) return MOE_EINVAL;
  if (T > 0 && (!topk_expert || !topk_score)) return MOE_EINVAL;
  if (!aligned(hist_row, 8) || !aligned(out, 4) || !aligned(expert_slot, 4)) return MOE_EINVAL;
  if (T > 0 && (!aligned(topk_expert, 4) || !aligned(topk_score, 4))) return MOE_EINVAL;
  if (!(threshold >= 0.0)) return MOE_EINVAL;  // also rejects NaN
  const size_t need = moe_hot_pick_ws_bytes_internal(T);
  if (ws_bytes < need) return MOE_EWORKSPACE;
  if (need > 0 && (!ws || !aligned(ws, 256))) return MOE_EINVAL;
  Miss* part = static_cast<Miss*>(ws);
  const int nb = hot_pick_wgs(T);
  if (nb > 0)
    hot_pick_tokens<<<nb, kHotTokenWg, 0, stream>>>(topk_expert, topk_score, T, k, E,
                                                    expert_slot, S, threshold, part);
  hot_pick_final<<<1, 1024, 0, stream>>>(part, nb, E, expert_slot, S, n_arena, hist_row, out);
  return hip_status();
}
