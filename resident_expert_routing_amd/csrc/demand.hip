// moe_demand_accumulate: score-weighted demand per expert over the router's
// unrestricted picks (TideLM README, "How adaptive expert loading works",
// item 1: every routed pick the router wants, resident or not, is recorded per
// (layer, expert), weighted by its routing score).
//
// Deterministic: per chunk of 64 tokens each expert's sum runs over ascending
// tokens; chunk sums are added in ascending chunk order, in float64.
#include <algorithm>

#include "common.hpp"
#include "demand_sums.hpp"

namespace moe {

// Partial (or, with part == null, final) demand of chunk blockIdx.x.  With
// E <= kDemandTableE the chunk goes through the LDS score table; above it each
// expert's sum scans the chunk's picks in order (still ascending tokens).
__global__ __launch_bounds__(1024) void demand_chunks(const int32_t* __restrict__ te,
                                                      const float* __restrict__ ts, int T, int k,
                                                      int E, double* __restrict__ part,
                                                      double* __restrict__ hist,
                                                      float* __restrict__ delta) {
  const int c = blockIdx.x;
  if (E <= kDemandTableE) {
    __shared__ float table[kDemandChunk][kDemandTableE];
    demand_chunk_table(te, ts, T, k, E, c, table, part, hist, delta);
    return;
  }
  __shared__ int se[kDemandChunk * MOE_MAX_K];
  __shared__ float ss[kDemandChunk * MOE_MAX_K];
  const int t0 = c * kDemandChunk;
  const int n = min(kDemandChunk, T - t0) * k;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    se[i] = te[(size_t)t0 * k + i];
    ss[i] = ts[(size_t)t0 * k + i];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    double acc = 0.0;
    for (int i = 0; i < n; ++i)
      if (se[i] == e) acc += (double)ss[i];
    if (part) {
      part[(size_t)c * E + e] = acc;
    } else {
      hist[e] += acc;
      if (delta) delta[e] = (float)acc;
    }
  }
}

__global__ __launch_bounds__(1024) void demand_finalize(const double* __restrict__ part, int nchunk,
                                                        int E, double* __restrict__ hist,
                                                        float* __restrict__ delta) {
  demand_finalize_sums(part, nchunk, E, hist, delta);
}

// hist[i] *= factor for every entry (the history's forgetting before a re-plan).
__global__ __launch_bounds__(256) void history_scale_kernel(double* __restrict__ hist, size_t n,
                                                           double factor) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    hist[i] *= factor;
}

}  // namespace moe

using namespace moe;

extern "C" MOE_EXPORT int moe_history_scale(double* hist, size_t n, double factor,
                                            hipStream_t stream) {
  if (!hist || !aligned(hist, 8)) return MOE_EINVAL;
  if (!(factor >= 0.0 && factor <= 1.0)) return MOE_EINVAL;  // also rejects NaN
  if (n == 0) return MOE_OK;
  const size_t blocks = std::min<size_t>((n + 255) / 256, 1024);
  history_scale_kernel<<<(unsigned)blocks, 256, 0, stream>>>(hist, n, factor);
  return hip_status();
}

size_t moe_demand_ws_bytes_internal(int T, int E) {
  if (T <= kDemandChunk) return 0;
  const size_t nchunk = (size_t)(T + kDemandChunk - 1) / kDemandChunk;
  return up_to(nchunk * E * sizeof(double), 256);
}

// Enqueues the demand kernels (arguments already validated; ws holds
// moe_demand_ws_bytes_internal(T, E) bytes).
int moe_demand_launch_internal(const int32_t* te, const float* ts, int T, int k, int E,
                               double* hist, float* delta, void* ws, hipStream_t stream) {
  const int threads = E <= 256 ? 256 : 1024;
  if (T <= kDemandChunk) {
    demand_chunks<<<1, threads, 0, stream>>>(te, ts, T, k, E, nullptr, hist, delta);
    return hip_status();
  }
  const int nchunk = (T + kDemandChunk - 1) / kDemandChunk;
  double* part = static_cast<double*>(ws);
  demand_chunks<<<nchunk, threads, 0, stream>>>(te, ts, T, k, E, part, hist, delta);
  demand_finalize<<<1, threads, 0, stream>>>(part, nchunk, E, hist, delta);
  return hip_status();
}

extern "C" MOE_EXPORT int moe_demand_accumulate(const int32_t* topk_expert,
                                                const float* topk_score, int T, int k, int E,
                                                double* hist_row, float* delta, void* ws,
                                                size_t ws_bytes, hipStream_t stream) {
  if (T < 0 || k <= 0 || E <= 0) return MOE_EINVAL;
  if (k > MOE_MAX_K || E > MOE_MAX_E) return MOE_EUNSUPPORTED;
  if (!hist_row) return MOE_EINVAL;
  if (T > 0 && (!topk_expert || !topk_score)) return MOE_EINVAL;
  if (!aligned(hist_row, 8)) return MOE_EINVAL;
  const size_t need = moe_demand_ws_bytes_internal(T, E);
  if (ws_bytes < need) return MOE_EWORKSPACE;
  if (need > 0 && (!ws || !aligned(ws, 256))) return MOE_EINVAL;
  return moe_demand_launch_internal(topk_expert, topk_score, T, k, E, hist_row, delta, ws, stream);
}
