// Device steps of the score-weighted demand per expert (TideLM README, "How
// adaptive expert loading works", item 1), shared by the demand kernels and by
// the larger-batch routing kernels that run them beside the bucket counting.
//
// Order of the float64 sums, the same wherever they run: within a chunk of
// kDemandChunk tokens each expert's sum runs over ascending tokens; chunk sums
// are added in ascending chunk order.
#pragma once

#include "common.hpp"

namespace moe {

// Experts up to which a chunk's picks are spread into an LDS [token][expert]
// score table (64 KB of float).
constexpr int kDemandTableE = 256;
constexpr size_t kDemandTableBytes = (size_t)kDemandChunk * kDemandTableE * sizeof(float);

// Demand of chunk c over E <= kDemandTableE experts, through the table: zero
// where a token did not pick the expert (a token's picks are distinct
// experts), so each expert's sum is a loop over the chunk's tokens in
// ascending order, and adding the zeros changes no bit of it.  Writes the sum
// to part[c * E + e] when part is non-null, else adds it to hist[e] (and
// stores it as float in delta[e] when delta is non-null).  Uses the whole
// workgroup; begins with a barrier-free write of the table and ends after the
// last read of it (the caller puts a barrier before reusing the memory).
__device__ inline void demand_chunk_table(const int32_t* __restrict__ te,
                                          const float* __restrict__ ts, int T, int k, int E,
                                          int c, float (*table)[kDemandTableE],
                                          double* __restrict__ part, double* __restrict__ hist,
                                          float* __restrict__ delta) {
  const int t0 = c * kDemandChunk;
  const int nt = min(kDemandChunk, T - t0);
  const int n = nt * k;
  for (int i = threadIdx.x; i < kDemandChunk * kDemandTableE; i += blockDim.x)
    (&table[0][0])[i] = 0.f;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int e = te[(size_t)t0 * k + i];
    if (e >= 0 && e < E) table[i / k][e] = ts[(size_t)t0 * k + i];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    double acc = 0.0;
    for (int t = 0; t < nt; ++t) acc += (double)table[t][e];
    if (part) {
      part[(size_t)c * E + e] = acc;
    } else {
      hist[e] += acc;
      if (delta) delta[e] = (float)acc;
    }
  }
}

// hist[e] += the chunk partials part[c][e] added in ascending chunk order;
// delta[e] (when non-null) gets that sum as float.  The loads of a group of 16
// chunks are issued before their additions.  Threads stride over the experts.
__device__ inline void demand_finalize_sums(const double* __restrict__ part, int nchunk, int E,
                                            double* __restrict__ hist,
                                            float* __restrict__ delta) {
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    double acc = 0.0;
    int c = 0;
    for (; c + 16 <= nchunk; c += 16) {
      double v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = part[(size_t)(c + i) * E + e];
#pragma unroll
      for (int i = 0; i < 16; ++i) acc += v[i];
    }
    for (; c < nchunk; ++c) acc += part[(size_t)c * E + e];
    hist[e] += acc;
    if (delta) delta[e] = (float)acc;
  }
}

}  // namespace moe
