// Test-only probe of the block-scaled MXFP4 matrix instructions the expert
// kernels use: one wave, one MFMA on raw per-lane operands, results as the
// lanes hold them.
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
}  // namespace moe

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
