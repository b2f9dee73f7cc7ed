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

// MXFP6 (E2M3) activation rows: 24 code bytes per 32-element block, then the
// scale bytes; padded to 16.
inline size_t mxfp6_row_bytes(int K) {
  return up_to((size_t)K / 32 * 24 + (size_t)K / 32, 16);
}

// Byte offset of the scale bytes in an activation row of K elements.
__host__ __device__ inline size_t act_scale_offset(int K, int fmt) {
  return fmt == MOE_ACT_MXFP6 ? (size_t)K / 32 * 24 : (size_t)K / 2;
}

inline size_t act_row_bytes(int K, int fmt) {
  return fmt == MOE_ACT_MXFP6 ? mxfp6_row_bytes(K) : mxfp4_row_bytes(K);
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

// E2M3 code of v / 2^e (OCP MX FP6 E2M3: sign | 2 exponent bits, bias 1 |
// 3 mantissa bits): nearest value with ties to the even mantissa, magnitudes
// above 7.5 saturating; sign bit copied from v.  Within a binade the grid is
// uniform with 8 steps, so the mantissa is the binade offset times 8 rounded
// half to even (exact: a power-of-two scaling and a subtraction in the same
// binade); a round-up to 8 is the next binade's first value.
__device__ __forceinline__ uint32_t e2m3_code(float v, int e) {
  const float a = fabsf(__builtin_amdgcn_ldexpf(v, -e));
  uint32_t mag;
  if (a < 1.0f) {
    mag = (uint32_t)__builtin_rintf(a * 8.0f);                 // subnormal: m / 8 (8 -> 1.0)
  } else {
    const int E = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // 0..2 (a < 8)
    const float m = (__builtin_amdgcn_ldexpf(a, -E) - 1.0f) * 8.0f;
    mag = (uint32_t)(E + 1) * 8u + (uint32_t)__builtin_rintf(m);
  }
  mag = mag > 31u ? 31u : mag;
  return mag | ((__float_as_uint(v) >> 31) << 5);
}

// ---------------------------------------------------------------------------
// Wave reductions through DPP; the result is read from lane 63, so it is a
// uniform value.  Steps: within quads (lane i with i^1, then i^2), half rows
// (i with 7-i), rows (i with 15-i), then lane 15 of each row into rows 1 and
// 3 and lane 31 into rows 2 and 3, after which lane 63 holds the whole wave.
// ---------------------------------------------------------------------------
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppHalfMirror = 0x141,
              kDppMirror = 0x140, kDppBcast15 = 0x142, kDppBcast31 = 0x143;

// Lane values of v moved by one DPP step; rows outside ROW_MASK get `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v, double old) {
  const uint64_t u = (uint64_t)__double_as_longlong(v), o = (uint64_t)__double_as_longlong(old);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)o, (int)(uint32_t)u,
                                                            CTRL, ROW_MASK, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(
      (int)(uint32_t)(o >> 32), (int)(uint32_t)(u >> 32), CTRL, ROW_MASK, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ double lane63_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ double wave_max(double v) {
  v = fmax(v, dpp_f64<kDppQuadXor1, 0xF>(v, v));
  v = fmax(v, dpp_f64<kDppQuadXor2, 0xF>(v, v));
  v = fmax(v, dpp_f64<kDppHalfMirror, 0xF>(v, v));
  v = fmax(v, dpp_f64<kDppMirror, 0xF>(v, v));
  v = fmax(v, dpp_f64<kDppBcast15, 0xA>(v, v));
  v = fmax(v, dpp_f64<kDppBcast31, 0xC>(v, v));
  return lane63_f64(v);
}

// Sum in the fixed order of the steps above (rows outside a step's mask add 0).
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<kDppQuadXor1, 0xF>(v, 0.0);
  v += dpp_f64<kDppQuadXor2, 0xF>(v, 0.0);
  v += dpp_f64<kDppHalfMirror, 0xF>(v, 0.0);
  v += dpp_f64<kDppMirror, 0xF>(v, 0.0);
  v += dpp_f64<kDppBcast15, 0xA>(v, 0.0);
  v += dpp_f64<kDppBcast31, 0xC>(v, 0.0);
  return lane63_f64(v);
}

// Two independent 32-bit maxima (lanes whose DPP source does not exist read
// 0, the identity, so every step can write all rows and fold into v_max_u32).
__device__ __forceinline__ void wave_umax32x2(uint32_t& a, uint32_t& b) {
#define MOE_UMAX_STEP(CTRL)                                                         \
  a = max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)a, CTRL, 0xF, 0xF, true)); \
  b = max(b, (uint32_t)__builtin_amdgcn_mov_dpp((int)b, CTRL, 0xF, 0xF, true));
  MOE_UMAX_STEP(kDppQuadXor1)
  MOE_UMAX_STEP(kDppQuadXor2)
  MOE_UMAX_STEP(kDppHalfMirror)
  MOE_UMAX_STEP(kDppMirror)
  MOE_UMAX_STEP(kDppBcast15)
  MOE_UMAX_STEP(kDppBcast31)
#undef MOE_UMAX_STEP
  a = (uint32_t)__builtin_amdgcn_readlane((int)a, 63);
  b = (uint32_t)__builtin_amdgcn_readlane((int)b, 63);
}

__device__ __forceinline__ uint32_t wave_umax32(uint32_t a) {
  uint32_t b = 0;
  wave_umax32x2(a, b);
  return a;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Direct loads to LDS at lds_base + size * lane (lds_base is wave-uniform and
// goes to M0).  Inline assembly, so that the compiler does not add a wait for
// every outstanding load before each LDS read: the pipeline waits for them
// explicitly, with the count of loads that may still be in flight.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is written here on purpose
__device__ __forceinline__ void dma16(const uint8_t* g, uint8_t* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u8*)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0), "v"(g)
               : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace moe
