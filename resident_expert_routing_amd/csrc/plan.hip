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

// Applies a hot-read decision to the slot table on the device: the loaded
// expert takes the evicted expert's arena slot.  One thread; the decision is
// applied only when e* is a miss and c holds an arena slot, so a stale or
// empty decision leaves the table as it is.
__global__ __launch_bounds__(64) void hot_install_kernel(const int32_t* __restrict__ pick,
                                                         int32_t* __restrict__ expert_slot, int E,
                                                         int S, int n_arena,
                                                         int32_t* __restrict__ slot_out) {
  if (threadIdx.x != 0) return;
  const int e = pick[0], c = pick[1];
  int slot = -1;
  if (e >= 0 && e < E && c >= 0 && c < E && e != c) {
    const int se = expert_slot[e], sc = expert_slot[c];
    if (!(se >= 0 && se < S) && sc >= 0 && sc < n_arena && sc < S) {
      expert_slot[e] = sc;
      expert_slot[c] = -1;
      slot = sc;
    }
  }
  if (slot_out) slot_out[0] = slot;
}

// ---------------------------------------------------------------------------
// Hot ring (TideLM README, "How adaptive expert loading works", item 3,
// DeepSeek bullet): after each step the step's heaviest misses take ring
// entries in round-robin order.  One workgroup; a pair's key packs its weight
// and its id in 64 bits (larger weight first, then lower id) so that one
// unsigned maximum orders candidates.  Each pick is one workgroup maximum over
// a fresh scan of the pairs (weights and table stay in L2 after the first
// round); pairs held by the ring or already picked are marked in an LDS bitmap.
// ---------------------------------------------------------------------------
constexpr int kRingThreads = 1024;

__device__ __forceinline__ uint64_t ring_key(float w, int p) {
  // w > 0 and finite: its bits order like its value
  return ((uint64_t)__float_as_uint(w) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)p);
}

__global__ __launch_bounds__(kRingThreads) void ring_plan_kernel(
    const float* __restrict__ w, int32_t* __restrict__ table, int n, int E,
    int32_t* __restrict__ ring, int R, int slot0, int per_step, int32_t* __restrict__ plan) {
  __shared__ uint32_t taken[MOE_MAX_RING_PAIRS / 32];  // in the ring, or picked this call
  __shared__ uint64_t part[kRingThreads / 64];
  __shared__ int32_t chosen[MOE_MAX_RING_PER_STEP];
  __shared__ uint64_t winner;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < (n + 31) / 32; i += kRingThreads) taken[i] = 0u;
  __syncthreads();
  for (int r = tid; r < R; r += kRingThreads) {
    const int p = ring[1 + r];
    if (p >= 0 && p < n) atomicOr(&taken[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  const int m = per_step < R ? per_step : R;
  int count = 0;
  for (; count < m; ++count) {
    uint64_t best = 0ull;
    for (int p = tid; p < n; p += kRingThreads) {
      if ((taken[p >> 5] >> (p & 31)) & 1u) continue;
      if (table[p] >= 0) continue;  // routable: not a miss
      const float v = w[p];
      if (v > 0.f && v <= 3.402823466e38f) {  // NaN and inf never win
        const uint64_t key = ring_key(v, p);
        best = key > best ? key : best;
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const uint64_t o = __shfl_xor(best, d, kWave);
      best = o > best ? o : best;
    }
    if (lane == 0) part[wv] = best;
    __syncthreads();
    if (tid == 0) {
      uint64_t b = part[0];
      for (int i = 1; i < kRingThreads / 64; ++i) b = part[i] > b ? part[i] : b;
      winner = b;
      if (b != 0ull) {
        const int p = (int)(0xFFFFFFFFu - (uint32_t)b);
        chosen[count] = p;
        taken[p >> 5] |= 1u << (p & 31);
      }
    }
    __syncthreads();
    if (winner == 0ull) break;  // no candidate left (uniform)
    __syncthreads();            // part[] and winner are rewritten by the next pick
  }
  if (tid == 0) {
    const int head = ring[0];
    for (int i = 0; i < count; ++i) {
      const int r = (head + i) % R;
      const int old = ring[1 + r];
      if (old >= 0 && old < n && table[old] == slot0 + r) table[old] = -1;  // evicted
      const int p = chosen[i];
      ring[1 + r] = p;
      plan[1 + 3 * i] = r;
      plan[2 + 3 * i] = p / E;
      plan[3 + 3 * i] = p % E;
    }
    ring[0] = (head + count) % R;
    plan[0] = count;
  }
}

// Install a plan's pairs whose ring entries still hold them.
__global__ __launch_bounds__(64) void ring_install_kernel(const int32_t* __restrict__ plan,
                                                         int32_t* __restrict__ table, int n,
                                                         int E, const int32_t* __restrict__ ring,
                                                         int R, int slot0, int max_count) {
  const int count = min(plan[0], max_count);
  for (int i = threadIdx.x; i < count; i += 64) {
    const int r = plan[1 + 3 * i], l = plan[2 + 3 * i], e = plan[3 + 3 * i];
    if (r < 0 || r >= R || e < 0 || e >= E) continue;
    const int p = l * E + e;
    if (p >= 0 && p < n && ring[1 + r] == p) table[p] = slot0 + r;
  }
}

}  // namespace moe

using namespace moe;

static int ring_args_ok(int L, int E, int R, int ring_slot0, const void* table, const void* ring) {
  if (L <= 0 || E <= 0 || R <= 0 || ring_slot0 < 0) return MOE_EINVAL;
  if ((size_t)L * E > (size_t)MOE_MAX_RING_PAIRS || R > MOE_MAX_RING) return MOE_EUNSUPPORTED;
  if ((size_t)ring_slot0 + R > (size_t)MOE_MAX_S) return MOE_EUNSUPPORTED;
  if (!table || !ring || !aligned(table, 4) || !aligned(ring, 4)) return MOE_EINVAL;
  return MOE_OK;
}

extern "C" MOE_EXPORT int moe_ring_plan(const float* miss_weight, int32_t* expert_slot, int L,
                                        int E, int32_t* ring, int R, int ring_slot0,
                                        int per_step, int32_t* plan, hipStream_t stream) {
  const int r = ring_args_ok(L, E, R, ring_slot0, expert_slot, ring);
  if (r != MOE_OK) return r;
  if (per_step <= 0) return MOE_EINVAL;
  if (per_step > MOE_MAX_RING_PER_STEP) return MOE_EUNSUPPORTED;
  if (!miss_weight || !plan || !aligned(miss_weight, 4) || !aligned(plan, 4)) return MOE_EINVAL;
  ring_plan_kernel<<<1, kRingThreads, 0, stream>>>(miss_weight, expert_slot, L * E, E, ring, R,
                                                   ring_slot0, per_step, plan);
  return hip_status();
}

extern "C" MOE_EXPORT int moe_ring_install(const int32_t* plan, int32_t* expert_slot, int L,
                                           int E, const int32_t* ring, int R, int ring_slot0,
                                           hipStream_t stream) {
  const int r = ring_args_ok(L, E, R, ring_slot0, expert_slot, ring);
  if (r != MOE_OK) return r;
  if (!plan || !aligned(plan, 4)) return MOE_EINVAL;
  ring_install_kernel<<<1, 64, 0, stream>>>(plan, expert_slot, L * E, E, ring, R, ring_slot0,
                                            MOE_MAX_RING_PER_STEP);
  return hip_status();
}

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

extern "C" MOE_EXPORT int moe_hot_install(const int32_t* pick, int32_t* expert_slot, int E, int S,
                                          int n_arena, int32_t* slot_out, hipStream_t stream) {
  if (E <= 0 || S < 0 || n_arena < 0) return MOE_EINVAL;
  if (E > MOE_MAX_E || S > MOE_MAX_S) return MOE_EUNSUPPORTED;
  if (!pick || !expert_slot || !aligned(pick, 4) || !aligned(expert_slot, 4)) return MOE_EINVAL;
  if (slot_out && !aligned(slot_out, 4)) return MOE_EINVAL;
  hot_install_kernel<<<1, 64, 0, stream>>>(pick, expert_slot, E, S, n_arena, slot_out);
  return hip_status();
}
