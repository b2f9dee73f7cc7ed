// Shared device helpers and host-side checks for libmoe_arena (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_arena.h"

#define MOE_EXPORT __attribute__((visibility("default")))

namespace moe {

constexpr int kWave = 64;
constexpr int kRouterChunk = 32;    // h-chunk of the float64 router sum
constexpr int kSplitRouterMaxT = 64;  // at or below: chunk partials in parallel
constexpr int kDemandChunk = 64;    // tokens per demand partial

// ---------------------------------------------------------------------------
// host helpers
// ---------------------------------------------------------------------------
inline size_t up_to(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline size_t mxfp4_row_bytes(int K) {
  return up_to((size_t)K / 2 + (size_t)K / 32, 16);
}

struct SlotLayout {
  size_t off[6];
  size_t total;
};

inline SlotLayout slot_layout(int H, int I) {
  SlotLayout L;
  const size_t h = (size_t)H, i = (size_t)I;
  const size_t sz[6] = {i * h / 2, i * h / 32, i * h / 2, i * h / 32, h * i / 2, h * i / 32};
  size_t o = 0;
  for (int j = 0; j < 6; ++j) {
    L.off[j] = o;
    o = up_to(o + sz[j], 256);
  }
  L.total = o;
  return L;
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline int hip_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

// Records stage event i when the caller passed an array with a non-null entry
// there; false only if the record itself fails.
inline bool record_stage(hipEvent_t* ev, int i, hipStream_t stream) {
  if (!ev || !ev[i]) return true;
  return hipEventRecord(ev[i], stream) == hipSuccess;
}

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Exponent e of the MX block scale X = 2^e for a block with max |v| = amax > 0:
// floor(log2 amax) - 2, clamped to [-127, 127] (the E8M0 range).
__device__ __forceinline__ int mx_block_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int ex = (int)((u >> 23) & 0xFFu);
  int fl;
  if (ex == 0) {
    const uint32_t m = u & 0x7FFFFFu;  // subnormal: value = m * 2^-149
    fl = (31 - __clz((int)m)) - 149;
  } else {
    fl = ex - 127;
  }
  int e = fl - 2;
  e = e < -127 ? -127 : e;
  e = e > 127 ? 127 : e;
  return e;
}

// E2M1 code of v / 2^e: nearest of {0,.5,1,1.5,2,3,4,6} with ties to the even
// mantissa, magnitudes above 6 saturating; sign bit copied from v.
__device__ __forceinline__ uint32_t e2m1_code(float v, int e) {
  const float a = fabsf(__builtin_amdgcn_ldexpf(v, -e));  // exact power-of-two scaling
  uint32_t m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
               (a >= 3.5f) + (a > 5.0f);
  return m | ((__float_as_uint(v) >> 31) << 3);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
  return v;
}

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmax(v, __shfl_xor(v, d, kWave));
  return v;
}

// Butterfly sum: every lane ends with the same value (a+b == b+a per step).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int d = 1; d <= 32; d <<= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace moe
