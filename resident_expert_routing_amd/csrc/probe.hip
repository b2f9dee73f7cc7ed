// Test-only probes: the block-scaled MXFP4 matrix instructions the expert
// kernels use (one wave, one MFMA on raw per-lane operands, results as the
// lanes hold them), and two microbenchmarks of the achievable read and MXFP4
// matrix rates.
#include "common.hpp"

namespace moe {
typedef int pv8i __attribute__((ext_vector_type(8)));
typedef float pv4f __attribute__((ext_vector_type(4)));
typedef float pv16f __attribute__((ext_vector_type(16)));

template <int SHAPE>
__global__ __launch_bounds__(64) void mxfp4_probe(const uint8_t* a, const uint8_t* as,
                                                  const uint8_t* b, const uint8_t* bs, float* d) {
  const int l = threadIdx.x;
  const uint4 av = reinterpret_cast<const uint4*>(a)[l];
  const uint4 bv = reinterpret_cast<const uint4*>(b)[l];
  const pv8i A = {(int)av.x, (int)av.y, (int)av.z, (int)av.w, 0, 0, 0, 0};
  const pv8i B = {(int)bv.x, (int)bv.y, (int)bv.z, (int)bv.w, 0, 0, 0, 0};
  float4* o = reinterpret_cast<float4*>(d) + 4 * l;
  if (SHAPE == 0) {
    pv4f c = {0.f, 0.f, 0.f, 0.f};
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 4, 4, 0, (int)as[l], 0,
                                                         (int)bs[l]);
    o[0] = make_float4(c[0], c[1], c[2], c[3]);
  } else {
    pv16f c;
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = 0.f;
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, 4, 4, 0, (int)as[l], 0,
                                                        (int)bs[l]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = make_float4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
  }
}
// Achievable read rate: each thread reads 16-byte units i, i + G, i + 2G,
// i + 3G (G = threads in the grid) per round, all four in flight together.
__global__ __launch_bounds__(256) void stream_read(const uint4* __restrict__ src, size_t n16,
                                                   uint32_t* __restrict__ sink) {
  const size_t G = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + 3 * G < n16; i += 4 * G) {
    const uint4 a = src[i], b = src[i + G], c = src[i + 2 * G], d = src[i + 3 * G];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n16; i += G) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// Achievable block-scaled matrix rate: 8 independent 32x32x64 accumulator
// chains per wave; A in E2M1, B in E2M1 or (FP6) E2M3; the operands come from
// the lane index, so nothing folds away.
template <bool FP6>
__global__ __launch_bounds__(256) void mfma_loop(int iters, float* __restrict__ sink) {
  const int l = threadIdx.x;
  const pv8i A = {l, l + 1, l + 2, l + 3, 0, 0, 0, 0};
  const pv8i B = {3 * l, l ^ 5, l + 7, l ^ 9, FP6 ? l + 11 : 0, FP6 ? l ^ 13 : 0, 0, 0};
  constexpr int kBfmt = FP6 ? 2 : 4;  // blgp: E2M3 or E2M1
  pv16f c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) c[j][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c[j], 4, kBfmt, 0, 100 + j, 0,
                                                             120);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[j][i];
  sink[(size_t)blockIdx.x * 256 + l] = s;
}
}  // namespace moe

extern "C" MOE_EXPORT int moe_test_stream_read(const void* src, size_t bytes, uint32_t* sink,
                                               int grid, hipStream_t stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || grid < 1 || grid > 65536)
    return MOE_EINVAL;
  if (!moe::aligned(src, 16)) return MOE_EINVAL;
  moe::stream_read<<<grid, 256, 0, stream>>>(static_cast<const uint4*>(src), bytes / 16, sink);
  return moe::hip_status();
}

extern "C" MOE_EXPORT int moe_test_mfma_loop(int iters, int act_format, float* sink, int grid,
                                             hipStream_t stream) {
  if (!sink || iters < 1 || iters > (1 << 20) || grid < 1 || grid > 65536) return MOE_EINVAL;
  if (act_format != MOE_ACT_MXFP4 && act_format != MOE_ACT_MXFP6) return MOE_EINVAL;
  if (act_format == MOE_ACT_MXFP6)
    moe::mfma_loop<true><<<grid, 256, 0, stream>>>(iters, sink);
  else
    moe::mfma_loop<false><<<grid, 256, 0, stream>>>(iters, sink);
  return moe::hip_status();
}

extern "C" MOE_EXPORT int moe_test_mxfp4_probe(int shape, const uint8_t* a, const uint8_t* a_scale,
                                               const uint8_t* b, const uint8_t* b_scale, float* d,
                                               hipStream_t stream) {
  if (shape != 0 && shape != 1) return MOE_EINVAL;
  if (!a || !a_scale || !b || !b_scale || !d) return MOE_EINVAL;
  if (!moe::aligned(a, 16) || !moe::aligned(b, 16) || !moe::aligned(d, 16)) return MOE_EINVAL;
  if (shape == 0)
    moe::mxfp4_probe<0><<<1, 64, 0, stream>>>(a, a_scale, b, b_scale, d);
  else
    moe::mxfp4_probe<1><<<1, 64, 0, stream>>>(a, a_scale, b, b_scale, d);
  return moe::hip_status();
}
