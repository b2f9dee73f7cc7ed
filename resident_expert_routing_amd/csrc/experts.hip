// moe_experts_forward: grouped SwiGLU expert FFNs on MXFP4 arena slots and the
// weighted combine (gfx950, block-scaled MXFP4 MFMA).
//
// TideLM README, "How adaptive expert loading works": experts run from arena
// slots (resident set or hot ring).  colibri cluster page: each expert names its
// rows by index (COLIEX01 v2 paragraph), and a row's expert results are added in
// one fixed order (the fixed-summation-order paragraph) -- here ascending
// expert id, which is the order of a token's picks.
//
// Two kernel families, each with one fixed contraction order (so a token's
// result does not depend on the other tokens of its batch within a family):
//
// * Small batches (decode): the weights stream from HBM straight into
//   registers with v_mfma_scale_f32_16x16x128_f8f6f4.  K is walked in
//   512-wide super-chunks (16 MX blocks) in ascending order; MFMA step i
//   (0..3) covers blocks 4i..4i+3, lane group g (lanes 16g..16g+15)
//   supplying block 4i+g, so one load instruction reads 64 contiguous bytes
//   of each of 16 rows.  A lane reads the super-chunk's 16 scale bytes as one
//   16-byte word and shifts its own byte (4i+g) into place for step i; the
//   weight rows' scales are first copied to LDS by the workgroup.
//
// * Larger batches: operands are staged in LDS and the MFMA is
//   v_mfma_scale_f32_32x32x64_f8f6f4 (on gfx950 the 16x16x128 form runs at
//   half the E2M1 rate).  Lane l supplies row (or column) l%32 and one MX
//   block of 32 elements with its E8M0 scale; the 32x32 fp32 result sits in
//   lane l, register v at row 8(v/4) + 4(l/32) + v%4, column l%32.  K is
//   walked in chunks of 128 (4 MX blocks) in ascending order; step s (0, 1)
//   of chunk c takes block 4c + 2s (lanes 0-31) and 4c + 2s + 1 (lanes
//   32-63).
//
// The families agree to float32 rounding of their sums, not bit for bit.
#include <hip/hip_ext.h>

#include <mutex>
#include <type_traits>

#include "common.hpp"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
constexpr int kInlineWorklistMaxS = 1024;

// silu(g) * u, the SwiGLU product of one element.
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// ===========================================================================
// 16x16x128 helpers (small-batch kernels)
// ===========================================================================
__device__ __forceinline__ v4f mfma_fp4(const uint4& a, const uint4& b, v4f c, uint32_t sa,
                                        uint32_t sb) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  // cbsz = blgp = 4: both operands E2M1; the scale is byte 0 of each scale word.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, (int)sa, 0,
                                                          (int)sb);
}

// One super-chunk of an MXFP4 row as this lane supplies it: codes of blocks
// 4i+g (i = 0..3) and, in byte 0 of s[i], their scales.
template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

struct RowSC {
  uint4 q[4];
  uint32_t s[4];
};

// Four MFMA steps of one super-chunk for one 16-row tile.
__device__ __forceinline__ v4f mfma_superchunk(const RowSC& a, const RowSC& b, v4f c) {
#pragma unroll
  for (int i = 0; i < 4; ++i) c = mfma_fp4(a.q[i], b.q[i], c, a.s[i], b.s[i]);
  return c;
}

__device__ __forceinline__ void zero_sc(RowSC& r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.q[i] = make_uint4(0u, 0u, 0u, 0u);
    r.s[i] = 127u;
  }
}

// This lane's code blocks 16sc+g, +4, +8, +12 of a row with a multiple of 16
// blocks (super-chunk sc).
__device__ __forceinline__ void load_codes_full(const uint8_t* codes, int sc, int g, RowSC& r) {
  const uint4* q = reinterpret_cast<const uint4*>(codes + (size_t)sc * 256) + g;
  r.q[0] = q[0];
  r.q[1] = q[4];
  r.q[2] = q[8];
  r.q[3] = q[12];
}

// This lane's scale bytes of those blocks, from the 16 scale bytes of the
// super-chunk.
__device__ __forceinline__ void split_scales(const uint4 sv, int g, RowSC& r) {
  const int sh = 8 * g;
  r.s[0] = sv.x >> sh;
  r.s[1] = sv.y >> sh;
  r.s[2] = sv.z >> sh;
  r.s[3] = sv.w >> sh;
}

// The scale bytes of the same blocks (16-byte aligned scales).
__device__ __forceinline__ void load_scales_full(const uint8_t* scales, int sc, int g, RowSC& r) {
  split_scales(*reinterpret_cast<const uint4*>(scales + sc * 16), g, r);
}

// Load this lane's share of super-chunk sc of an MXFP4 row.  FULL: the row has
// a multiple of 16 blocks and 16-byte aligned scales.  Blocks at or past nblk
// read as zero codes.
template <bool FULL>
__device__ __forceinline__ void load_row_sc(const uint8_t* codes, const uint8_t* scales, int sc,
                                            int g, int nblk, RowSC& r) {
  const int b0 = sc * 16;
  if (FULL) {
    load_codes_full(codes, sc, g, r);
    load_scales_full(scales, sc, g, r);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bi = b0 + 4 * i + g;
      if (bi < nblk) {
        r.q[i] = reinterpret_cast<const uint4*>(codes + (size_t)bi * 16)[0];
        r.s[i] = scales[bi];
      } else {
        r.q[i] = make_uint4(0u, 0u, 0u, 0u);
        r.s[i] = 127u;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Weight codes.  A slot's code sections are stored in tiles of 16 rows x 64
// bytes (128 elements): tile (row block b = row / 16, K-chunk c) starts at
// b * 16 * (K/2) + c * 1024, its rows one after another, each w_c bytes wide
// (64, or what is left of the row for a last partial chunk).  So every 16-byte
// unit a load instruction of the kernels reads for 16 rows lies in one 1 KB
// run of memory.  `blk` is the start of a 16-row block.
// ---------------------------------------------------------------------------
constexpr int kTileBytes = 1024;  // one tile: 16 rows x 64 code bytes

__device__ __forceinline__ const uint8_t* wcode_unit(const uint8_t* blk, size_t crow, int r,
                                                     int bi) {
  const int c = bi >> 2;
  const int w = min(64, (int)crow - 64 * c);
  return blk + (size_t)c * kTileBytes + r * w + (bi & 3) * 16;
}

// This lane's code units of super-chunk sc (K % 512 == 0): chunks 4sc + i,
// unit g, row r of the block.
__device__ __forceinline__ void load_wcodes_full(const uint8_t* blk, int sc, int r, int g,
                                                 RowSC& w) {
  const uint8_t* q = blk + (size_t)sc * 4 * kTileBytes + r * 64 + g * 16;
  w.q[0] = *reinterpret_cast<const uint4*>(q);
  w.q[1] = *reinterpret_cast<const uint4*>(q + kTileBytes);
  w.q[2] = *reinterpret_cast<const uint4*>(q + 2 * kTileBytes);
  w.q[3] = *reinterpret_cast<const uint4*>(q + 3 * kTileBytes);
}

// Super-chunk sc of weight row r of the block at blk (codes) with its scale
// row at `scales`; FULL as load_row_sc.  Blocks at or past nblk read as zero.
template <bool FULL>
__device__ __forceinline__ void load_wrow_sc(const uint8_t* blk, size_t crow, int r,
                                             const uint8_t* scales, int sc, int g, int nblk,
                                             RowSC& w) {
  if (FULL) {
    load_wcodes_full(blk, sc, r, g, w);
    load_scales_full(scales, sc, g, w);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bi = sc * 16 + 4 * i + g;
      if (bi < nblk) {
        w.q[i] = *reinterpret_cast<const uint4*>(wcode_unit(blk, crow, r, bi));
        w.s[i] = scales[bi];
      } else {
        w.q[i] = make_uint4(0u, 0u, 0u, 0u);
        w.s[i] = 127u;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// MXFP6 (E2M3) activation operands of the small-batch kernels: a block of 32
// elements is 24 bytes, element i at bits [6i, 6i+6) -- the six-register
// operand of the block-scaled instruction with the E2M3 format (lane -> row and
// K group as for E2M1, pinned by a probe on the hardware).
// ---------------------------------------------------------------------------
struct RowSC6 {
  uint32_t q[4][6];
  uint32_t s[4];
};

__device__ __forceinline__ v4f mfma_fp4x6(const uint4& a, const uint32_t (&b)[6], v4f c,
                                          uint32_t sa, uint32_t sb) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], (int)b[4], (int)b[5], 0, 0};
  // cbsz = 4: A (weights) E2M1; blgp = 2: B (activations) E2M3
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 2, 0, (int)sa, 0,
                                                          (int)sb);
}

__device__ __forceinline__ v4f mfma_superchunk(const RowSC& a, const RowSC6& b, v4f c) {
#pragma unroll
  for (int i = 0; i < 4; ++i) c = mfma_fp4x6(a.q[i], b.q[i], c, a.s[i], b.s[i]);
  return c;
}

__device__ __forceinline__ void zero_sc(RowSC6& r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 6; ++j) r.q[i][j] = 0u;
    r.s[i] = 127u;
  }
}

// This lane's code blocks 16sc+g, +4, +8, +12 of an MXFP6 row (24 bytes each,
// 8-byte aligned).
__device__ __forceinline__ void load_codes6(const uint8_t* codes, int sc, int g, RowSC6& r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint2* q = reinterpret_cast<const uint2*>(codes + (size_t)(16 * sc + 4 * i + g) * 24);
    const uint2 a = q[0], b = q[1], c = q[2];
    r.q[i][0] = a.x;
    r.q[i][1] = a.y;
    r.q[i][2] = b.x;
    r.q[i][3] = b.y;
    r.q[i][4] = c.x;
    r.q[i][5] = c.y;
  }
}

__device__ __forceinline__ void split_scales(const uint4 sv, int g, RowSC6& r) {
  const int sh = 8 * g;
  r.s[0] = sv.x >> sh;
  r.s[1] = sv.y >> sh;
  r.s[2] = sv.z >> sh;
  r.s[3] = sv.w >> sh;
}

// Super-chunk sc of an MXFP6 row whose length is a multiple of 512 (scales
// 16-byte aligned at `scales`).
__device__ __forceinline__ void load_row_sc6(const uint8_t* codes, const uint8_t* scales, int sc,
                                             int g, RowSC6& r) {
  load_codes6(codes, sc, g, r);
  split_scales(*reinterpret_cast<const uint4*>(scales + sc * 16), g, r);
}

// SwiGLU of one column of a wave's 32 rows of I and its MXFP4 encoding
// (16x16x128 result layout).  Lane (c = lane&15, g) holds rows n0+4g+v (tile
// 0) and n0+16+4g+v (tile 1) of gate (ag*) and up (au*) for column c; the 32
// rows are one MX block of h.  hr: the column's hq row, or null when the
// column is absent (every lane still takes part in the shuffles).
__device__ __forceinline__ void swiglu_quant_store16(const v4f& ag0, const v4f& ag1,
                                                     const v4f& au0, const v4f& au1, int g,
                                                     uint8_t* hr, int n0, int I) {
  float h[8];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    h[v] = silu_mul(ag0[v], au0[v]);
    h[4 + v] = silu_mul(ag1[v], au1[v]);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(h[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
  uint32_t codes[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  uint32_t scale = 0u;
  if (amax > 0.f) {
    const int e = mx_block_exp(amax);
    scale = (uint32_t)(e + 127);
#pragma unroll
    for (int i = 0; i < 8; ++i) codes[i] = e2m1_code(h[i], e);
  }
  if (hr) {
    const uint16_t w0 =
        (uint16_t)(codes[0] | (codes[1] << 4) | (codes[2] << 8) | (codes[3] << 12));
    const uint16_t w1 =
        (uint16_t)(codes[4] | (codes[5] << 4) | (codes[6] << 8) | (codes[7] << 12));
    *reinterpret_cast<uint16_t*>(hr + n0 / 2 + 2 * g) = w0;
    *reinterpret_cast<uint16_t*>(hr + n0 / 2 + 8 + 2 * g) = w1;
    if (g == 0) hr[I / 2 + n0 / 32] = (uint8_t)scale;
  }
}

// The same SwiGLU column encoded as an MXFP6 row: rows n0+4g.. are elements
// 4g..4g+3 of the block (bytes 3g..3g+2 of its 24), rows n0+16+4g.. bytes
// 12+3g..; the scale byte at 3I/4 + n0/32.
__device__ __forceinline__ void swiglu_quant_store16_fp6(const v4f& ag0, const v4f& ag1,
                                                         const v4f& au0, const v4f& au1, int g,
                                                         uint8_t* hr, int n0, int I) {
  float h[8];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    h[v] = silu_mul(ag0[v], au0[v]);
    h[4 + v] = silu_mul(ag1[v], au1[v]);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(h[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
  uint32_t codes[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  uint32_t scale = 0u;
  if (amax > 0.f) {
    const int e = mx_block_exp(amax);
    scale = (uint32_t)(e + 127);
#pragma unroll
    for (int i = 0; i < 8; ++i) codes[i] = e2m3_code(h[i], e);
  }
  if (hr) {
    const uint32_t w0 = codes[0] | (codes[1] << 6) | (codes[2] << 12) | (codes[3] << 18);
    const uint32_t w1 = codes[4] | (codes[5] << 6) | (codes[6] << 12) | (codes[7] << 18);
    uint8_t* b = hr + (size_t)(n0 / 32) * 24 + 3 * g;
    b[0] = (uint8_t)w0;
    b[1] = (uint8_t)(w0 >> 8);
    b[2] = (uint8_t)(w0 >> 16);
    b[12] = (uint8_t)w1;
    b[13] = (uint8_t)(w1 >> 8);
    b[14] = (uint8_t)(w1 >> 16);
    if (g == 0) hr[(size_t)I / 32 * 24 + n0 / 32] = (uint8_t)scale;
  }
}

// ===========================================================================
// 32x32x64 helpers (pipelined kernels)
// ===========================================================================
__device__ __forceinline__ v16f mfma32(const uint4& a, const uint4& b, v16f c, uint32_t sa,
                                       uint32_t sb) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  // cbsz = blgp = 4: both operands E2M1; the scale is byte 0 of each scale word.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, 0, (int)sa, 0,
                                                         (int)sb);
}

__device__ __forceinline__ v16f zero16() {
  v16f z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// ---------------------------------------------------------------------------
// SwiGLU of one column of a wave's 32 rows of I and its MXFP4 encoding
// (32x32x64 result layout).  Lane (column l%32, half hh = l/32) holds gate (G) and up (U) rows
// n0 + 8(v/4) + 4hh + v%4; the 32 rows are one MX block of h.  hr: the
// column's hq row, or null when the column is absent (every lane still takes
// part in the shuffle).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void swiglu_quant_store32(const v16f& G, const v16f& U, int hh,
                                                   uint8_t* hr, int n0, int I) {
  float h[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) h[v] = silu_mul(G[v], U[v]);
  float amax = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) amax = fmaxf(amax, fabsf(h[v]));
  amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
  uint32_t code[16];
  uint32_t scale = 0u;
#pragma unroll
  for (int v = 0; v < 16; ++v) code[v] = 0u;
  if (amax > 0.f) {
    const int e = mx_block_exp(amax);
    scale = (uint32_t)(e + 127);
#pragma unroll
    for (int v = 0; v < 16; ++v) code[v] = e2m1_code(h[v], e);
  }
  if (hr) {
    // rows 8q+4hh .. 8q+4hh+3 are bytes 4q+2hh, 4q+2hh+1 of the block's codes
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint16_t*>(hr + n0 / 2 + 4 * q + 2 * hh) =
          (uint16_t)(code[4 * q] | (code[4 * q + 1] << 4) | (code[4 * q + 2] << 8) |
                     (code[4 * q + 3] << 12));
    if (hh == 0) hr[I / 2 + n0 / 32] = (uint8_t)scale;
  }
}

// y rows n0 + 8q + 4hh .. +3 of one column, rounded to bf16 (a bf16 row of H).
__device__ __forceinline__ void store_y_bf16(uint16_t* yr, int n0, int hh, const v16f& acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<uint2*>(yr + n0 + 8 * q + 4 * hh) =
        make_uint2(f32_to_bf16(acc[4 * q]) | (f32_to_bf16(acc[4 * q + 1]) << 16),
                   f32_to_bf16(acc[4 * q + 2]) | (f32_to_bf16(acc[4 * q + 3]) << 16));
}

// A used slot and its rows [p0, p1) of the bucketed order; s = -1 if none.
struct SlotRange {
  int s, p0, p1;
};

__device__ __forceinline__ bool slot_used(int a, int b, int A) { return b > a && a >= 0 && b <= A; }

// The u-th slot (ascending) that holds assignments, found by one wave from
// slot_offsets (S <= kInlineWorklistMaxS).  Each lane reads its contiguous
// range of offsets in one batch; a wave prefix of the per-lane counts names the
// lane that holds slot u, which hands the slot and its two offsets to the
// others.
__device__ SlotRange wave_nth_used_slot(int u, const int32_t* __restrict__ offsets, int S, int A) {
  constexpr int kPer = kInlineWorklistMaxS / kWave;
  const int lane = threadIdx.x & 63;
  const int per = (S + kWave - 1) / kWave;
  const int lo = min(S, lane * per), hi = min(S, lo + per);
  int ofs[kPer + 1];
#pragma unroll
  for (int i = 0; i <= kPer; ++i)  // i <= per: uniform, so only the loads needed are issued
    ofs[i] = i <= per ? offsets[min(lo + i, S)] : 0;  // in bounds: S + 1 entries
  int local = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    local += (lo + i < hi && slot_used(ofs[i], ofs[i + 1], A)) ? 1 : 0;
  int incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  int run = incl - local;
  int fs = -1, fa = 0, fb = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (lo + i < hi && slot_used(ofs[i], ofs[i + 1], A)) {
      if (run == u) {
        fs = lo + i;
        fa = ofs[i];
        fb = ofs[i + 1];
      }
      ++run;
    }
  }
  const unsigned long long m = __ballot(fs >= 0);
  if (m == 0ull) return SlotRange{-1, 0, 0};
  const int L = __ffsll(m) - 1;
  // uniform across the wave: keep it in scalar registers
  return SlotRange{__builtin_amdgcn_readlane(fs, L), __builtin_amdgcn_readlane(fa, L),
                   __builtin_amdgcn_readlane(fb, L)};
}

// Slot of work item u.  Small slot counts: the u-th used slot, found in place.
// Larger ones (sel_slot given): work item u is position u of the bucketed
// order, and it does the work of its slot when it is the slot's first
// position (perm, sel_slot and slot_offsets come from one moe_route call);
// every other position's item is empty.  Three dependent loads, where a scan
// of thousands of offsets would not fit, and no list to build beforehand.
__device__ __forceinline__ SlotRange work_slot(int u, const int32_t* __restrict__ sel_slot,
                                               const int32_t* __restrict__ perm,
                                               const int32_t* __restrict__ offsets, int S,
                                               int A) {
  if (!sel_slot) return wave_nth_used_slot(u, offsets, S, A);
  if (u >= A) return SlotRange{-1, 0, 0};
  const int a = __builtin_amdgcn_readfirstlane(perm[u]);
  if (a < 0 || a >= A) return SlotRange{-1, 0, 0};
  const int s = __builtin_amdgcn_readfirstlane(sel_slot[a]);
  if (s < 0 || s >= S) return SlotRange{-1, 0, 0};
  const int p0 = __builtin_amdgcn_readfirstlane(offsets[s]);
  const int p1 = __builtin_amdgcn_readfirstlane(offsets[s + 1]);
  if (p0 != u || !slot_used(p0, p1, A)) return SlotRange{-1, 0, 0};
  return SlotRange{s, p0, p1};
}


// ===========================================================================
// Small-batch kernels
// ===========================================================================
// Weight scales of the rows a wave streams are staged in LDS once.  A
// row's scale bytes share one or two cache lines that the K loop would
// otherwise touch once per super-chunk; between touches the workgroup streams
// enough code bytes for the line to leave L2, so it would be fetched again
// from memory every time.  LDS row stride 16*((K/512) | 1) bytes: an odd
// number of 16-byte units, so the 16 rows of one fragment read fall on 16
// distinct 4-bank groups.
constexpr int kStagedRows = 64;             // rows staged per workgroup (one wave)
constexpr int kStagedLdsMax = 32 * 1024;    // LDS budget of the staged scales

__host__ __device__ constexpr int staged_scale_stride(int K) { return 16 * ((K / 512) | 1); }

// Full-row kernels (K a multiple of 512) with staged scales: the workgroup's
// scale rows fit the LDS budget.
static bool staged_ok(int K) {
  return K % 512 == 0 && (size_t)kStagedRows * staged_scale_stride(K) <= (size_t)kStagedLdsMax;
}

// Rows [0, nrows) of NM contiguous scale blocks src[m] (rbytes per row, a
// multiple of 16 and at most 1024) into LDS: row r of block m at
// lds + (m * mrows + r) * stride.  By one wave; each lane issues 4 loads per
// block before it writes any of them to LDS, so a batch costs one memory round
// trip, not one per load.
template <int NM>
__device__ __forceinline__ void stage_scale_rows(const uint8_t* const (&src)[NM], int nrows,
                                                 int rbytes, int stride, int mrows,
                                                 uint8_t* lds) {
  constexpr int kJ = 4;  // rows per thread and block in one batch
  const int per_row = rbytes / 16;
  const int rstep = kWave / per_row;  // rows the wave covers per pass
  const int lane = threadIdx.x & 63;
  const int r0 = lane / per_row, c = lane - r0 * per_row;
  if (r0 >= rstep) return;
  // Rows past the end repeat the last row (same bytes to the same place): no
  // branch, so the compiler keeps every load of a batch ahead of the stores.
  for (int j0 = r0; j0 < nrows; j0 += kJ * rstep) {
    uint4 v[NM][kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int row = min(j0 + j * rstep, nrows - 1);
#pragma unroll
      for (int m = 0; m < NM; ++m)
        v[m][j] = *reinterpret_cast<const uint4*>(src[m] + (size_t)row * rbytes + c * 16);
    }
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int row = min(j0 + j * rstep, nrows - 1);
#pragma unroll
      for (int m = 0; m < NM; ++m)
        *reinterpret_cast<uint4*>(lds + (m * mrows + row) * stride + c * 16) = v[m][j];
    }
  }
}

// Gate/up + SwiGLU + MXFP4(h).  Workgroup = one wave = 32 rows of I of one
// slot (two 16-row tiles of gate and of up).  Columns are the slot's
// assignment rows p, 16 per MFMA tile.  Output: hq row p (an MXFP4 row of I
// elements).  One-wave workgroups let the dispatcher spread the bytes evenly
// over the CUs: each CU streams at a rate of its own, so the CU with the most
// work sets the kernel's time.
// ---------------------------------------------------------------------------
struct GateUpArgs {
  const uint8_t* xq;
  size_t xrow;
  const uint8_t* arena;
  size_t stride;
  size_t off_gc, off_gs, off_uc, off_us;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* sel_slot;  // large slot counts: item u = bucketed position u (else null)
  int32_t* slots;       // out: (slot, p0, p1) of work item u at 3u (slot -1: none), for down
  uint8_t* hq;
  size_t hrow;
  const uint8_t* shared;  // the shared expert's slot bytes, or null
  int T, H, I, k, A, S;
  int maxU;               // work item maxU is the shared expert's (rows A .. A+T, token p - A)
};

// FP6: activations and h in MXFP6 (FULL only).
template <bool FULL, bool FP6>
__global__ __launch_bounds__(kWave, 3) void gateup_kernel(GateUpArgs p) {
  static_assert(FULL || !FP6, "MXFP6 activations need whole super-chunks");
  using XRow = typename std::conditional<FP6, RowSC6, RowSC>::type;
  const int nbps = p.I / 32;
  const int u = blockIdx.x / nbps, nb = blockIdx.x - u * nbps;
  // the shared expert's item: slot id S (never a routed slot), rows A .. A+T
  const bool sh = p.shared && u == p.maxU;
  const SlotRange sr = sh ? SlotRange{p.S, p.A, p.A + p.T}
                          : work_slot(u, p.sel_slot, p.perm, p.offsets, p.S, p.A);
  if (nb == 0 && threadIdx.x == 0) {  // the down kernel takes its work items from here
    p.slots[3 * u] = sr.s;
    p.slots[3 * u + 1] = sr.p0;
    p.slots[3 * u + 2] = sr.p1;
  }
  if (sr.s < 0) return;
  const int s = sr.s, p0 = sr.p0, p1 = sr.p1;
  const int lane = threadIdx.x;
  const int n0 = nb * 32;
  const int r = lane & 15, g = lane >> 4;
  const int H = p.H;
  const int nblk = H / 32;
  const int nsc = (nblk + 15) / 16;
  const uint8_t* base = sh ? p.shared : p.arena + (size_t)s * p.stride;
  const size_t crow = (size_t)H / 2, srow = (size_t)H / 32;
  // 16-row code blocks of the two tiles (rows n0.., n0 + 16..)
  const uint8_t* gc0 = base + p.off_gc + (size_t)n0 * crow;
  const uint8_t* gc1 = gc0 + 16 * crow;
  const uint8_t* uc0 = base + p.off_uc + (size_t)n0 * crow;
  const uint8_t* uc1 = uc0 + 16 * crow;
  const uint8_t* gs0;
  const uint8_t* us0;
  int sstep;  // bytes from a tile-0 scale row to its tile-1 row
  int pa = -1;  // FULL: this lane's perm entry of the first column block, loaded early
  if (FULL) {
    // Issued before the staging waits, so they are in flight together.
    if (!sh && p0 + r < p1) pa = p.perm[p0 + r];
    // gate scales of the wave's 32 rows at LDS row 0.., up scales at row 32..
    extern __shared__ __align__(16) uint8_t wscale[];
    const int sstr = staged_scale_stride(H);
    const uint8_t* const src[2] = {base + p.off_gs + (size_t)n0 * srow,
                                   base + p.off_us + (size_t)n0 * srow};
    stage_scale_rows<2>(src, 32, (int)srow, sstr, 32, wscale);
    __syncthreads();
    gs0 = wscale + r * sstr;
    us0 = gs0 + 32 * sstr;
    sstep = 16 * sstr;
  } else {
    gs0 = base + p.off_gs + (size_t)(n0 + r) * srow;
    us0 = base + p.off_us + (size_t)(n0 + r) * srow;
    sstep = 16 * (int)srow;
  }
  const uint8_t* gs1 = gs0 + sstep;
  const uint8_t* us1 = us0 + sstep;

  // One block of 16 columns (assignment rows cb..) against the wave's 32 rows
  // of gate and of up.  The first block of a FULL kernel takes its perm
  // entries from the early loads.
  auto column_block = [&](int cb, auto first) {
    constexpr bool kFirst = decltype(first)::value;
    // this lane's column (assignment row) for the B operand
    const int pc = cb + r;
    int t = -1;
    if (pc < p1) {
      if (sh) {
        t = pc - p.A;  // the shared expert takes every token, in order
      } else {
        const int a = kFirst ? pa : p.perm[pc];
        if (a >= 0 && a < p.A) t = a / p.k;
      }
    }
    const uint8_t* xc = t >= 0 ? p.xq + (size_t)t * p.xrow : nullptr;
    v4f ag0 = {0.f, 0.f, 0.f, 0.f}, ag1 = ag0, au0 = ag0, au1 = ag0;
    for (int sc = 0; sc < nsc; ++sc) {
      RowSC wg0, wg1, wu0, wu1;
      XRow x;
      load_wrow_sc<FULL>(gc0, crow, r, gs0, sc, g, nblk, wg0);
      load_wrow_sc<FULL>(gc1, crow, r, gs1, sc, g, nblk, wg1);
      load_wrow_sc<FULL>(uc0, crow, r, us0, sc, g, nblk, wu0);
      load_wrow_sc<FULL>(uc1, crow, r, us1, sc, g, nblk, wu1);
      if (!xc)
        zero_sc(x);
      else if constexpr (FP6)
        load_row_sc6(xc, xc + act_scale_offset(H, MOE_ACT_MXFP6), sc, g, x);
      else
        load_row_sc<FULL>(xc, xc + H / 2, sc, g, nblk, x);
      ag0 = mfma_superchunk(wg0, x, ag0);
      ag1 = mfma_superchunk(wg1, x, ag1);
      au0 = mfma_superchunk(wu0, x, au0);
      au1 = mfma_superchunk(wu1, x, au1);
    }
    const int pcol = cb + (lane & 15);
    uint8_t* hr = pcol < p1 ? p.hq + (size_t)pcol * p.hrow : nullptr;
    if constexpr (FP6)
      swiglu_quant_store16_fp6(ag0, ag1, au0, au1, g, hr, n0, p.I);
    else
      swiglu_quant_store16(ag0, ag1, au0, au1, g, hr, n0, p.I);
  };
  int cb = p0;
  if constexpr (FULL) {
    column_block(cb, BoolTag<true>{});
    cb += 16;
  }
  for (; cb < p1; cb += 16) column_block(cb, BoolTag<false>{});
}

// ---------------------------------------------------------------------------
// Down projection.  Workgroup = one wave = 64 rows of H of one slot (four
// 16-row tiles).  B operand: hq rows of the slot.  Output y[a] (fp32 row of
// H), a = perm[p].
// ---------------------------------------------------------------------------
struct DownArgs {
  const uint8_t* hq;
  size_t hrow;
  const uint8_t* arena;
  size_t stride;
  size_t off_dc, off_ds;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* slots;  // (slot, p0, p1) of work item u at 3u, written by the gate/up kernel
  float* y;
  const uint8_t* shared;  // the shared expert's slot bytes (slot id S), or null
  int H, I, A, S;
};

// FP6: h rows in MXFP6 (FULL only).
template <bool FULL, bool FP6>
__global__ __launch_bounds__(kWave, 3) void down_kernel(DownArgs p) {
  static_assert(FULL || !FP6, "MXFP6 activations need whole super-chunks");
  using XRow = typename std::conditional<FP6, RowSC6, RowSC>::type;
  const int nbps = (p.H + 63) / 64;
  const int u = blockIdx.x / nbps, nb = blockIdx.x - u * nbps;
  // one round trip: the gate/up kernel of this call found the slot
  const SlotRange sr = {__builtin_amdgcn_readfirstlane(p.slots[3 * u]),
                        __builtin_amdgcn_readfirstlane(p.slots[3 * u + 1]),
                        __builtin_amdgcn_readfirstlane(p.slots[3 * u + 2])};
  if (sr.s < 0) return;
  const int s = sr.s, p0 = sr.p0, p1 = sr.p1;
  const bool sh = s == p.S;  // the shared expert: y row = its hq row (A + token)
  const int lane = threadIdx.x;
  const int n0 = nb * 64;
  const int r = lane & 15, g = lane >> 4;
  const int I = p.I;
  const int nblk = I / 32;
  const int nsc = (nblk + 15) / 16;
  const uint8_t* base = sh ? p.shared : p.arena + (size_t)s * p.stride;
  const size_t crow = (size_t)I / 2, srow = (size_t)I / 32;
  extern __shared__ __align__(16) uint8_t wscale[];  // FULL: the wave's scale rows
  const int sstr = staged_scale_stride(I);
  const uint8_t* dc[4];
  const uint8_t* ds[4];
  bool tv[4];
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) {
    tv[tl] = n0 + 16 * tl < p.H;  // whole tile valid (H % 16 == 0)
    const int row0 = tv[tl] ? n0 + 16 * tl : n0;  // an idle tile: a block in range
    dc[tl] = base + p.off_dc + (size_t)row0 * crow;  // the tile's 16-row code block
    ds[tl] = FULL ? wscale + (row0 + r - n0) * sstr
                  : base + p.off_ds + (size_t)(row0 + r) * srow;
  }
  RowSC pre[4];  // FULL: super-chunk 0 codes of the first column block, loaded early
  XRow prex;     // FULL: and of its activation rows (codes; scale bytes in prexs)
  uint4 prexs;
  if (FULL) {
    // Issued before the staging waits, so they are in flight together.
#pragma unroll
    for (int tl = 0; tl < 4; ++tl)
      if (tv[tl]) load_wcodes_full(dc[tl], 0, r, g, pre[tl]);
    if (p0 + r < p1) {
      const uint8_t* hc = p.hq + (size_t)(p0 + r) * p.hrow;
      if constexpr (FP6)
        load_codes6(hc, 0, g, prex);
      else
        load_codes_full(hc, 0, g, prex);
      prexs = *reinterpret_cast<const uint4*>(hc + act_scale_offset(I, FP6 ? MOE_ACT_MXFP6
                                                                             : MOE_ACT_MXFP4));
    } else {
      zero_sc(prex);
      prexs = make_uint4(0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu);  // scale 1
    }
    const uint8_t* const src[1] = {base + p.off_ds + (size_t)n0 * srow};
    stage_scale_rows<1>(src, min(64, p.H - n0), (int)srow, sstr, 64, wscale);
    __syncthreads();
  }
  // One block of 16 columns (assignment rows cb..) against the wave's 64 rows;
  // the first block of a FULL kernel takes super-chunk 0 from the early
  // loads (a separate copy of the loop, so those registers are free in the
  // others).
  auto column_block = [&](int cb, auto first) {
    constexpr bool kFirst = decltype(first)::value;
    const int pc = cb + r;
    const uint8_t* hc = pc < p1 ? p.hq + (size_t)pc * p.hrow : nullptr;
    v4f acc[4];
#pragma unroll
    for (int tl = 0; tl < 4; ++tl) acc[tl] = (v4f){0.f, 0.f, 0.f, 0.f};
    int sc0 = 0;
    if constexpr (kFirst) {
      // super-chunk 0 from the early loads
      split_scales(prexs, g, prex);
#pragma unroll
      for (int tl = 0; tl < 4; ++tl) {
        if (tv[tl]) {
          load_scales_full(ds[tl], 0, g, pre[tl]);
          acc[tl] = mfma_superchunk(pre[tl], prex, acc[tl]);
        }
      }
      sc0 = 1;
    }
    for (int sc = sc0; sc < nsc; ++sc) {
      XRow x;
      if (!hc)
        zero_sc(x);
      else if constexpr (FP6)
        load_row_sc6(hc, hc + act_scale_offset(I, MOE_ACT_MXFP6), sc, g, x);
      else
        load_row_sc<FULL>(hc, hc + I / 2, sc, g, nblk, x);
#pragma unroll
      for (int tl = 0; tl < 4; ++tl) {
        if (tv[tl]) {
          RowSC w;
          load_wrow_sc<FULL>(dc[tl], crow, r, ds[tl], sc, g, nblk, w);
          acc[tl] = mfma_superchunk(w, x, acc[tl]);
        }
      }
    }
    const int c = lane & 15;
    const int pcol = cb + c;
    if (pcol < p1) {
      const int a = sh ? pcol : p.perm[pcol];
      if (a >= 0 && (sh || a < p.A)) {
        float* yr = p.y + (size_t)a * p.H;
#pragma unroll
        for (int tl = 0; tl < 4; ++tl) {
          if (tv[tl]) {
            *reinterpret_cast<float4*>(yr + n0 + 16 * tl + 4 * g) =
                make_float4(acc[tl][0], acc[tl][1], acc[tl][2], acc[tl][3]);
          }
        }
      }
    }
  };
  int cb = p0;
  if constexpr (FULL) {
    column_block(cb, BoolTag<true>{});
    cb += 16;
  }
  for (; cb < p1; cb += 16) column_block(cb, BoolTag<false>{});
}

// ---------------------------------------------------------------------------
// Down projection and combine in one launch, for decode-size batches with
// MXFP4 rows (at most kRcMaxRows rows of y, T <= kRcMaxT).  Workgroup = 16
// rows of H (one 16-row block of every slot's down codes) against every work
// item: its sixteen waves take the items in turn, each wave issuing the loads
// of two super-chunks (one when they are partial) before their MFMAs (the same instruction sequence per
// element as down_kernel, so y is the same), and write y for their
// assignments to LDS.  After a barrier, thread (t, row) adds the token's picks in ascending
// pick order with the same fused multiply-adds as combine_kernel, then the
// shared expert's row, and rounds once to bf16: the output is the one the
// two-kernel path gives, without y in memory and without the combine launch.
// With 256 workgroups at H = 4096 every CU streams the same bytes.  Measured
// at decode: 119.3 against 120.7 us per layer step; eight waves with four
// super-chunks in flight each were no faster than the two kernels, and with
// MXFP6 rows (three times the activation load instructions) the single launch
// was slower, so those keep down_kernel and combine_kernel.
// ---------------------------------------------------------------------------
constexpr int kRcMaxRows = 320;  // y rows held in LDS (A, plus T with a shared expert)
constexpr int kRcMaxT = 32;      // tokens: 16 combine threads each
constexpr int kRcWaves = 16;

struct RowsCombineArgs {
  DownArgs d;
  const float* sel_weight;
  const int32_t* sel_slot;
  uint16_t* out;
  int T, k, nwork;
};

template <bool FULL>
__global__ __launch_bounds__(kRcWaves * kWave, 1) void down_rows_combine(RowsCombineArgs q) {
  __shared__ float ybuf[kRcMaxRows * 16];
  const DownArgs& p = q.d;
  const int nb = blockIdx.x;  // rows 16 nb .. 16 nb + 15 of H
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int I = p.I;
  const int nblk = I / 32;
  const int nsc = (nblk + 15) / 16;
  const size_t crow = (size_t)I / 2, srow = (size_t)I / 32;
  for (int u = wave; u < q.nwork; u += kRcWaves) {
    const int s = __builtin_amdgcn_readfirstlane(p.slots[3 * u]);
    if (s < 0) continue;
    const int p0 = __builtin_amdgcn_readfirstlane(p.slots[3 * u + 1]);
    const int p1 = __builtin_amdgcn_readfirstlane(p.slots[3 * u + 2]);
    const bool sh = s == p.S;  // the shared expert: y row = its hq row (A + token)
    const uint8_t* base = sh ? p.shared : p.arena + (size_t)s * p.stride;
    const uint8_t* blk = base + p.off_dc + (size_t)(16 * nb) * crow;
    const uint8_t* srw = base + p.off_ds + (size_t)(16 * nb + r) * srow;
    for (int cb = p0; cb < p1; cb += 16) {
      const int pc = cb + r;
      const uint8_t* hc = pc < p1 ? p.hq + (size_t)pc * p.hrow : nullptr;
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      constexpr int kB = FULL ? 2 : 1;  // super-chunks whose loads are issued together
      for (int sc0 = 0; sc0 < nsc; sc0 += kB) {
        RowSC w[kB];
        RowSC x[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) {
          const int sc = sc0 + j;
          if (sc < nsc) {
            load_wrow_sc<FULL>(blk, crow, r, srw, sc, g, nblk, w[j]);
            if (!hc)
              zero_sc(x[j]);
            else
              load_row_sc<FULL>(hc, hc + I / 2, sc, g, nblk, x[j]);
          }
        }
#pragma unroll
        for (int j = 0; j < kB; ++j)
          if (sc0 + j < nsc) acc = mfma_superchunk(w[j], x[j], acc);
      }
      const int pcol = cb + (lane & 15);
      if (pcol < p1) {
        const int a = sh ? pcol : p.perm[pcol];
        if (a >= 0 && (sh || a < p.A)) {
#pragma unroll
          for (int v = 0; v < 4; ++v) ybuf[a * 16 + 4 * g + v] = acc[v];
        }
      }
    }
  }
  __syncthreads();
  const int T = q.T, k = q.k;
  if (tid < T * 16) {
    const int t = tid >> 4, row = tid & 15;
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const int sl = q.sel_slot[(size_t)t * k + j];
      if (sl >= 0 && sl < p.S) acc = fmaf(q.sel_weight[(size_t)t * k + j], ybuf[(t * k + j) * 16 + row], acc);
    }
    if (p.shared) acc += ybuf[(p.A + t) * 16 + row];
    q.out[(size_t)t * p.H + 16 * nb + row] = (uint16_t)f32_to_bf16(acc);
  }
}

// ---------------------------------------------------------------------------
// Combine: out[t] = sum_j (ascending) w[t,j] * y[t*k+j] in float32, rounded
// once to bf16.  y rows are float32 (small-batch kernels) or bf16 (pipelined).
// ---------------------------------------------------------------------------
// The kEl elements of a y row from element i on, as float32.
template <typename YT>
struct YRow;
template <>
struct YRow<float> {  // small-batch kernels: float32 rows, 4 elements (16 bytes) per thread
  static constexpr int kEl = 4;
  __device__ static void load(const float* y, size_t i, float (&o)[kEl]) {
    const float4 v = *reinterpret_cast<const float4*>(y + i);
    o[0] = v.x;
    o[1] = v.y;
    o[2] = v.z;
    o[3] = v.w;
  }
};
template <>
struct YRow<uint16_t> {  // pipelined kernels: bf16 rows, 8 elements (16 bytes) per thread
  static constexpr int kEl = 8;
  __device__ static void load(const uint16_t* y, size_t i, float (&o)[kEl]) {
    const uint4 v = *reinterpret_cast<const uint4*>(y + i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[2 * q] = bf16_to_f32(w[q] & 0xFFFFu);
      o[2 * q + 1] = bf16_to_f32(w[q] >> 16);
    }
  }
};

// One thread per YRow<YT>::kEl consecutive elements of a token's output row.
// ysh: the shared expert's rows (row t for token t), added unweighted after
// the routed picks, or null.
template <typename YT>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ y,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ sel_slot, int T,
                                                      int H, int k, int S,
                                                      const YT* __restrict__ ysh,
                                                      uint16_t* __restrict__ out) {
  constexpr int kB = 8;  // picks whose rows are loaded together
  constexpr int kEl = YRow<YT>::kEl;
  const int t = blockIdx.x;
  const int h = (blockIdx.y * 256 + threadIdx.x) * kEl;
  if (h >= H) return;  // H % 32 == 0: a thread's elements are all in the row or all past it
  float acc[kEl];
#pragma unroll
  for (int e = 0; e < kEl; ++e) acc[e] = 0.f;
  for (int j0 = 0; j0 < k; j0 += kB) {
    // Every row load of the batch is issued before the first sum: the rows of
    // picks that are skipped (no slot) are read too (they lie in y, whose A
    // rows are all allocated) but never added.  With S == 0, y may be null and
    // nothing is read.
    bool ok[kB];
    float wj[kB];
    float v[kB][kEl];
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      const int j = min(j0 + i, k - 1);
      const int sl = sel_slot[(size_t)t * k + j];
      ok[i] = j0 + i < k && sl >= 0 && sl < S;
      wj[i] = w[(size_t)t * k + j];
    }
    if (S > 0) {
#pragma unroll
      for (int i = 0; i < kB; ++i)
        YRow<YT>::load(y, ((size_t)t * k + min(j0 + i, k - 1)) * H + h, v[i]);
    }
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      if (ok[i]) {
#pragma unroll
        for (int e = 0; e < kEl; ++e) acc[e] = fmaf(wj[i], v[i][e], acc[e]);
      }
    }
  }
  if (ysh) {
    float v[kEl];
    YRow<YT>::load(ysh, (size_t)t * H + h, v);
#pragma unroll
    for (int e = 0; e < kEl; ++e) acc[e] += v[e];
  }
  uint16_t* o = out + (size_t)t * H + h;  // 8-byte aligned: four elements per store
#pragma unroll
  for (int e = 0; e < kEl; e += 4)
    *reinterpret_cast<uint2*>(o + e) =
        make_uint2(f32_to_bf16(acc[e]) | (f32_to_bf16(acc[e + 1]) << 16),
                   f32_to_bf16(acc[e + 2]) | (f32_to_bf16(acc[e + 3]) << 16));
}

// ===========================================================================
// Pipelined path for larger batches (rows of 512-multiple length).  A work
// item is one M-tile of up to kTileM consecutive assignment rows of one slot;
// the grid is work items x N-tiles.  Every operand reaches LDS through direct
// global-to-LDS loads (lane i of a load lands at the LDS base + size * i).
// Code bytes are issued two K chunks ahead of use into a ring of three
// stages; a stage holds one chunk (K = 128: 64 code bytes per row) of the
// N-tile's 256 weight rows (four groups of 64) and of the M-tile's 128
// activation rows.  The E8M0 scales of four stages (16 bytes per row) are
// loaded together, one row per lane, into a group buffer beside the ring: a
// load that touches one cache line per lane then carries 16 bytes instead of
// 4 (with 4-byte loads every stage, the scale loads were half of the cache
// lines requested and cost a fifth of the kernel's time).  Ring and group
// buffer take 78 KB, so two workgroups share a CU.  With MXFP4 rows a
// workgroup is eight waves, each multiplying one weight group by half of the
// M-tile's columns (128 accumulator registers fewer than four waves with all
// columns each), so the kernels fit 128 VGPRs and every SIMD keeps four waves:
// a wave stalls handing its loads to the memory pipeline for about half of
// each stage, and four waves hide more of that than two (gate/up 3 % faster at
// the prefill and the long chunk than four-wave workgroups).  The 16-byte
// block b of a 64-byte stage row r sits at position b ^ ((r >> 2) & 3): a
// fragment read (32 rows, two blocks) spreads over all 16 four-bank groups,
// four lanes each.
// ===========================================================================
constexpr int kTileM = 128;                    // assignment rows per work item
constexpr int kKc = 128;                       // K elements per stage
constexpr int kRowC = kKc / 2;                 // code bytes per row per stage (64)
constexpr int kRowS = kKc / 32;                // scale bytes per row per stage (4)
constexpr int kStageA = 4 * 64 * kRowC;        // weight code rows of the four weight groups
constexpr int kStageB = kTileM * kRowC;        // activation code rows
constexpr int kStage = kStageA + kStageB;      // 24,576 bytes
constexpr int kRing = 3;
constexpr int kAhead = kRing - 1;              // stages issued ahead of the one in use
constexpr int kGroup = 4;                      // stages whose scales are loaded together
constexpr int kGroupRow = kGroup * kRowS;      // scale bytes per row per group (16)
constexpr int kGroupSA = 4 * 64 * kGroupRow;   // weight rows' scales (4,096 bytes)
constexpr int kGroupSB = kTileM * kGroupRow;   // activation rows' scales: 32 rows per wave
constexpr int kPipeLds = kRing * kStage + kGroupSA + kGroupSB;  // 79,872 bytes
static_assert(2 * kPipeLds <= 160 * 1024, "two workgroups per CU");
constexpr int kZeroPage = 256;                 // zeroed workspace bytes absent rows load from
constexpr int kPipeWaves = 8;                  // waves per workgroup (MXFP4 rows)
constexpr int kScalePart = 48 * kGroupRow;     // a wave's part of the group buffer (768 bytes)
static_assert(kPipeWaves * kScalePart == kGroupSA + kGroupSB, "group buffer parts");
// Loads issued by each wave per stage (MXFP4 rows): 2 weight-code and 1
// activation-code load; per group of stages, 1 scale load.
constexpr int kLoadsPerStage = 3;

// Work list of M-tiles of tm rows: items[0] = count, then per item (slot,
// first row of the tile within the slot, index of the slot's first item, the
// slot's item count), slots ascending; with a shared expert (Tsh = T rows),
// its tiles follow as slot S.  Also clears the zero page, and writes the
// first item and the item count of slot defer_slot (0 and 0 when it holds no
// assignment) to defer_info[0..1] when defer_slot >= 0.
__global__ __launch_bounds__(1024) void build_tiles(const int32_t* __restrict__ offsets, int S,
                                                    int A, int tm, int32_t* __restrict__ items,
                                                    uint32_t* __restrict__ zero_page,
                                                    int defer_slot,
                                                    int32_t* __restrict__ defer_info, int Tsh) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid < kZeroPage / 4) zero_page[tid] = 0u;
  const int per = (S + 1023) / 1024;
  const int lo = min(S, tid * per), hi = min(S, lo + per);
  int local = 0;
  for (int s = lo; s < hi; ++s) {
    const int a = offsets[s], b = offsets[s + 1];
    if (b > a && a >= 0 && b <= A) local += (b - a + tm - 1) / tm;
  }
  int incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int run = incl - local;
  for (int i = 0; i < wv; ++i) run += wsum[i];
  for (int s = lo; s < hi; ++s) {
    const int a = offsets[s], b = offsets[s + 1];
    const bool used = b > a && a >= 0 && b <= A;
    if (s == defer_slot) {  // its one owner thread
      defer_info[0] = used ? run : 0;
      defer_info[1] = used ? (b - a + tm - 1) / tm : 0;
    }
    if (used) {
      const int first = run, cnt = (b - a + tm - 1) / tm;
      for (int m = 0; m < cnt; ++m) {
        int32_t* it = items + 1 + 4 * run;
        it[0] = s;
        it[1] = m * tm;
        it[2] = first;
        it[3] = cnt;
        ++run;
      }
    }
  }
  if (tid == 0) {
    int total = 0;
    for (int i = 0; i < 16; ++i) total += wsum[i];
    const int nsh = (Tsh + tm - 1) / tm;  // the shared expert's tiles, last
    for (int m = 0; m < nsh; ++m) {
      int32_t* it = items + 1 + 4 * (total + m);
      it[0] = S;
      it[1] = m * tm;
      it[2] = total;
      it[3] = nsh;
    }
    items[0] = total + nsh;
  }
}

// Work index of this workgroup for n work indices.  Workgroups are dispatched
// round-robin over the 8 XCDs; this mapping gives XCD x the contiguous range
// [x R, x R + R) of R = ceil(n / 8) indices, so all eight share the work the
// batch actually has (the grid is sized for an upper bound of it).  Returns
// -1 for a workgroup with no index.  gridDim.x is a multiple of 8 and at
// least n rounded up to one.
__device__ __forceinline__ int xcd_work_index(int n) {
  const int R = (n + 7) / 8;
  const int j = (int)(blockIdx.x >> 3);
  if (j >= R) return -1;
  const int w = (int)(blockIdx.x & 7u) * R + j;
  return w < n ? w : -1;
}

// The (M-tile, N-tile) of work index w.  A slot's items x nN tiles are
// consecutive work indices, ordered in groups of up to 8 M-tiles: within a
// group the M-tile runs fastest, so the workgroups in flight on one XCD share
// a few weight N-tiles and a few activation M-tiles in its L2.  Returns false
// past the end of the list.
struct TileRef {
  int slot, p0, rows, nt;
};

// Slot S is the shared expert: rows A + m*tm.. of the A + Tsh rows.
__device__ __forceinline__ bool tile_of(int w, int nN, int tm, const int32_t* __restrict__ items,
                                        const int32_t* __restrict__ offsets, int S, int A,
                                        int Tsh, TileRef& t) {
  if (w < 0) return false;
  const int item = w / nN;
  if (item >= items[0]) return false;
  const int32_t* it = items + 1 + 4 * item;
  const int first = it[2], cnt = it[3];
  const int local = w - first * nN;
  const int mg = local / (8 * nN);
  const int gm = min(8, cnt - 8 * mg);
  const int lg = local - mg * 8 * nN;
  const int m = 8 * mg + lg % gm;
  t.slot = it[0];
  t.nt = lg / gm;
  if (t.slot == S) {
    t.p0 = A + m * tm;
    t.rows = min(tm, A + Tsh - t.p0);
  } else {
    t.p0 = offsets[t.slot] + m * tm;
    t.rows = min(tm, offsets[t.slot + 1] - t.p0);
  }
  return true;
}


// Per-wave sources of the direct loads.  Eight waves; wave w loads, per stage,
// the 16-row weight-code blocks 2 (w % 2) and 2 (w % 2) + 1 of weight group
// w / 2 (a group is 64 rows: tile 0 rows 0-31, tile 1 rows 32-63) and the 16
// activation rows 16 w ..; per group of stages one scale load (lanes 0-31:
// weight row 32 (w % 2) + lane of group w / 2; lanes 32-47: activation row
// 16 w + lane - 32; lanes 48-63 load nothing).
struct PipeSrc {
  const uint8_t* a[2];  // weight-code blocks, block already swizzled per lane
  int adst[2];          // their offsets in a stage
  const uint8_t* b;     // activation codes (zero page for an absent row)
  int bstep;            // code bytes per stage (64; 0 for an absent row)
  const uint8_t* s;     // this lane's scale row
  int sstep;            // scale bytes per group (16; 0 for an absent row)
};

struct TileSrc {
  const uint8_t* codes;
  const uint8_t* scales;
  int row0;  // first of the tile's 32 rows
};

__device__ __forceinline__ void pipe_issue(uint8_t* smem, const PipeSrc& src, int q, int wave) {
  uint8_t* st = smem + (q % kRing) * kStage;
#pragma unroll
  for (int j = 0; j < 2; ++j)  // stage q of a 16-row block: its tile q, 1 KB
    dma16(src.a[j] + (size_t)q * kTileBytes, st + src.adst[j]);
  dma16(src.b + (size_t)q * src.bstep, st + kStageA + wave * 1024);
}

// The scale bytes of group g (stages 4g .. 4g+3): 16 bytes per row, in the
// wave's 768-byte part of the group buffer (lane i at 16 i).
__device__ __forceinline__ void pipe_issue_scales(uint8_t* smem, const PipeSrc& src, int g,
                                                  int wave) {
  uint8_t* sg = smem + kRing * kStage;
  if ((threadIdx.x & 63) < 48)  // a partial-lane load
    dma16(src.s + (size_t)g * src.sstep, sg + wave * kScalePart);
}

// Waits until this wave's loads of stage q have landed, with those of its
// scale group (issued before stage q + 1's loads), then a workgroup barrier
// makes every wave's share visible and frees the stage read in the previous
// iteration for reuse.  Issue order: group 0, stages 0 and 1, then in
// iteration q stage q + 2, preceded by group g + 1 when q = 4g + 3; so after
// stage q's loads only stage q + 1's three may still be in flight.
__device__ __forceinline__ void pipe_wait(int q, int Q) {
  static_assert(kLoadsPerStage == 3 && kAhead == 2 && kGroup == 4, "wait counts below");
  if (q + 1 < Q)
    asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// The K loop over Q = K / 128 stages.  Wave w multiplies weight group w % 4
// (two 32-row tiles) by column half w / 4 (two 32-column tiles of the
// M-tile): two MFMA steps of 2 x 2 32x32x64 instructions per stage.
__device__ __forceinline__ void pipe_mainloop(uint8_t* smem, const PipeSrc& src, int Q, int wave,
                                              int lane, v16f (&acc)[2][2]) {
  const int r = lane & 31, hh = lane >> 5;
  const int g = wave & 3, ch = wave >> 2;
  const int swz = (r >> 2) & 3;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[t][c] = zero16();
  pipe_issue_scales(smem, src, 0, wave);
#pragma unroll
  for (int q = 0; q < kAhead; ++q)
    if (q < Q) pipe_issue(smem, src, q, wave);
  for (int q = 0; q < Q; ++q) {
    pipe_wait(q, Q);
    // scale words of stage q: weight tile t row r was loaded by wave 2g + t at
    // lane r; activation row C by wave C / 16 at lane 32 + C % 16
    const uint8_t* sg = smem + kRing * kStage + (q % kGroup) * kRowS;
    uint32_t aw[2], bw[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
      aw[t] = *reinterpret_cast<const uint32_t*>(sg + (2 * g + t) * kScalePart + r * kGroupRow);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int C = 32 * (2 * ch + c) + r;
      bw[c] = *reinterpret_cast<const uint32_t*>(sg + (C >> 4) * kScalePart +
                                                 (32 + (C & 15)) * kGroupRow);
    }
    if (q % kGroup == kGroup - 1 && q + 1 < Q) {
      // every wave holds its last scale words of the group: reload the buffer
      // (stage q's compute hides the load; stage q + 1 waits for it)
      __syncthreads();
      pipe_issue_scales(smem, src, (q + 1) / kGroup, wave);
    }
    if (q + kAhead < Q) pipe_issue(smem, src, q + kAhead, wave);
    const uint8_t* st = smem + (q % kRing) * kStage;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int pb = ((2 * s + hh) ^ swz) * 16;
      uint4 fa[2], fb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        fa[t] = *reinterpret_cast<const uint4*>(st + g * (64 * kRowC) + (32 * t + r) * kRowC + pb);
#pragma unroll
      for (int c = 0; c < 2; ++c)
        fb[c] = *reinterpret_cast<const uint4*>(st + kStageA + (32 * (2 * ch + c) + r) * kRowC +
                                                pb);
      const int sh = 8 * (2 * s + hh);
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t][c] = mfma32(fa[t], fb[c], acc[t][c], aw[t] >> sh, bw[c] >> sh);
    }
  }
}

// Weight-side sources of wave `wave`: tile(wg, t) names the codes, scales and
// first row of tile t of weight group wg.
template <typename TileFn>
__device__ __forceinline__ void pipe_weight_sources(PipeSrc& src, TileFn tile, size_t crow,
                                                    size_t srow, int wave, int lane) {
  const int wg = wave >> 1;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int j = 2 * (wave & 1) + jj;  // block j of the group: tile j / 2, rows 16 (j % 2)..
    const TileSrc ts = tile(wg, j >> 1);
    const int wr = 16 * j + (lane >> 2);  // the lane's row within the group
    const int b = (lane & 3) ^ ((wr >> 2) & 3);
    src.a[jj] = ts.codes + (size_t)(ts.row0 + 16 * (j & 1)) * crow + (lane >> 2) * kRowC + b * 16;
    src.adst[jj] = wg * (64 * kRowC) + j * 1024;
  }
  const TileSrc ts = tile(wg, wave & 1);
  src.s = ts.scales + (size_t)(ts.row0 + (lane & 31)) * srow;  // used by lanes 0-31
  src.sstep = kGroupRow;
}

// Activation-side sources: tile row `row` reads from rowptr(row) (codes at +0,
// scales at +scale_off) or, when absent, from the zero page.
template <typename RowPtr>
__device__ __forceinline__ void pipe_act_sources(PipeSrc& src, RowPtr rowptr, size_t scale_off,
                                                 const uint8_t* zero, int wave, int lane) {
  const int row = 16 * wave + (lane >> 2);
  const int b = (lane & 3) ^ ((row >> 2) & 3);
  const uint8_t* rp = rowptr(row);
  src.b = (rp ? rp : zero) + b * 16;
  src.bstep = rp ? kRowC : 0;
  if (lane >= 32) {  // lanes 32-47 load activation scale rows (48-63 load nothing)
    const uint8_t* sp = rowptr(16 * wave + (lane & 15));
    src.s = sp ? sp + scale_off : zero;
    src.sstep = sp ? kGroupRow : 0;
  }
}

// This lane's scale words of stage q (4 scale bytes of its rows: weight tile
// t row r, column tile cb row r), from the group buffer.
struct StageScales {
  uint32_t aw[2], bw[4];
};

// Weight-side sources: wave row wr (0..63) of the stage is row wrow[wr / 32] +
// wr % 32 of the section at wcodes[wr / 32] / wscales[wr / 32].
template <typename Src>
__device__ __forceinline__ void pipe_weight_src(Src& src, const uint8_t* const (&wcodes)[2],
                                                const uint8_t* const (&wscales)[2],
                                                const int (&wrow)[2], size_t crow, size_t srow,
                                                int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // load j: the 16-row block wrow[t] + (16j % 32).. (a tile row lane/4,
    // unit (lane % 4) ^ swizzle); stage q reads the block's tile q
    const int wr = 16 * j + (lane >> 2), t = wr >> 5;
    const int b = (lane & 3) ^ ((wr >> 2) & 3);
    src.a[j] = wcodes[t] + (size_t)(wrow[t] + ((16 * j) & 31)) * crow + (lane >> 2) * kRowC +
               b * 16;
  }
  const int t = lane >> 5, rr = lane & 31;
  const uint8_t* sbase = t ? wscales[1] : wscales[0];
  src.as = sbase + (size_t)((t ? wrow[1] : wrow[0]) + rr) * srow;
}

struct PipeArgs {
  const uint8_t* act;  // gate/up: xq rows by token; down: hq rows by position p
  size_t arow;
  const uint8_t* arena;
  size_t stride;
  size_t off_c0, off_s0, off_c1, off_s1;  // gate/up: gate, up sections; down: down (c0, s0)
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* items;
  const uint8_t* zero;
  uint8_t* hq;  // gate/up output
  size_t hrow;
  uint16_t* y;  // down output, bf16 rows
  int H, I, k, A, nN;
  int skip_slot;        // gate/up: tiles of this slot are left out (-1: none)
  const int32_t* only;  // gate/up: null, or (first item, item count) of the one slot to run
  const uint8_t* shared;  // the shared expert's slot bytes (its tiles are slot S), or null
  int S, T;
};

// Gate/up: N-tile = 128 rows of I; weight group g: rows n0 = 32g.. of gate
// (tile 0) and of up (tile 1); K = H.
__global__ __launch_bounds__(kPipeWaves * kWave, 2) void gateup_pipe(PipeArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kPipeLds];
  TileRef tr;
  int w;
  if (p.only) {  // one slot's tiles: work indices first * nN .. (first + count) * nN
    const int n = p.only[1] * p.nN;
    w = (int)blockIdx.x < n ? p.only[0] * p.nN + (int)blockIdx.x : -1;
  } else {
    w = xcd_work_index(p.items[0] * p.nN);
  }
  // no barrier yet: a workgroup without a tile (or with the left-out slot's) leaves whole
  if (!tile_of(w, p.nN, kTileM, p.items, p.offsets, p.S, p.A, p.shared ? p.T : 0, tr) ||
      tr.slot == p.skip_slot)
    return;
  const int s = tr.slot, p0 = tr.p0, rows = tr.rows;
  const bool sh = s == p.S;  // the shared expert: row p is token p - A
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r = lane & 31, hh = lane >> 5;
  const int g = wave & 3, ch = wave >> 2;
  const int H = p.H;
  const int nt0 = tr.nt * 128;
  const uint8_t* base = sh ? p.shared : p.arena + (size_t)s * p.stride;
  PipeSrc src;
  pipe_weight_sources(
      src,
      [&](int wg, int t) {
        return TileSrc{base + (t ? p.off_c1 : p.off_c0), base + (t ? p.off_s1 : p.off_s0),
                       nt0 + 32 * wg};
      },
      (size_t)H / 2, (size_t)H / 32, wave, lane);
  pipe_act_sources(
      src,
      [&](int row) -> const uint8_t* {
        if (row >= rows) return nullptr;
        if (sh) return p.act + (size_t)(p0 + row - p.A) * p.arow;
        const int a = p.perm[p0 + row];
        return (a >= 0 && a < p.A) ? p.act + (size_t)(a / p.k) * p.arow : nullptr;
      },
      (size_t)H / 2, p.zero, wave, lane);
  v16f acc[2][2];
  pipe_mainloop(smem, src, H / kKc, wave, lane, acc);
  const int n0 = nt0 + 32 * g;  // I % 128 == 0 on this path: every group is in range
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int cb = 2 * ch + c;
    if (32 * cb < rows) {
      const int lr = 32 * cb + r;
      swiglu_quant_store32(acc[0][c], acc[1][c], hh,
                           lr < rows ? p.hq + (size_t)(p0 + lr) * p.hrow : nullptr, n0, p.I);
    }
  }
}

// Down: N-tile = 256 rows of H; weight group g: rows n0 = 64g.. (two 32-row
// tiles); K = I; the B rows are the slot's hq rows p0.. (contiguous).
__global__ __launch_bounds__(kPipeWaves * kWave, 2) void down_pipe(PipeArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kPipeLds];
  TileRef tr;
  if (!tile_of(xcd_work_index(p.items[0] * p.nN), p.nN, kTileM, p.items, p.offsets, p.S, p.A,
               p.shared ? p.T : 0, tr))
    return;
  const int s = tr.slot, p0 = tr.p0, rows = tr.rows;
  const bool sh = s == p.S;  // the shared expert: y row = its hq row (A + token)
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r = lane & 31, hh = lane >> 5;
  const int g = wave & 3, ch = wave >> 2;
  const int I = p.I;
  const int nt0 = tr.nt * 256;
  const uint8_t* base = sh ? p.shared : p.arena + (size_t)s * p.stride;
  PipeSrc src;
  pipe_weight_sources(
      src,
      [&](int wg, int t) {
        const int row = nt0 + 64 * wg + 32 * t;  // tiles past H load row 0, never stored
        return TileSrc{base + p.off_c0, base + p.off_s0, row < p.H ? row : 0};
      },
      (size_t)I / 2, (size_t)I / 32, wave, lane);
  pipe_act_sources(
      src,
      [&](int row) -> const uint8_t* {
        return row < rows ? p.act + (size_t)(p0 + row) * p.arow : nullptr;
      },
      (size_t)I / 2, p.zero, wave, lane);
  v16f acc[2][2];
  pipe_mainloop(smem, src, I / kKc, wave, lane, acc);
  const int n0 = nt0 + 64 * g;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int lr = 32 * (2 * ch + c) + r;
    if (lr < rows) {
      const int a = sh ? p0 + lr : p.perm[p0 + lr];
      if (a >= 0 && (sh || a < p.A)) {
        uint16_t* yr = p.y + (size_t)a * p.H;
#pragma unroll
        for (int t = 0; t < 2; ++t)
          if (n0 + 32 * t < p.H) store_y_bf16(yr, n0 + 32 * t, hh, acc[t][c]);
      }
    }
  }
}


// ===========================================================================
// Pipelined kernels with MXFP6 activation rows (act_format MOE_ACT_MXFP6):
// the MXFP4 kernels' tiles -- each wave two 32-row weight tiles (gate/up:
// rows n0.. of gate and of up, 128 rows of I per workgroup; down: 64 rows of
// H, 256 per workgroup) against the 128 columns -- with E2M3 B operands.  A B
// row takes 96 bytes per 128-element stage instead of 64, so a stage is 16 KB
// of weight codes and 12 KB of activation codes, and the ring holds two
// stages, one issued ahead: 62 KB with the scale-group buffer, two workgroups
// per CU.  (With two workgroups per CU a ring of two stages ran the MXFP4
// kernels as fast as a ring of three; these tiles read each activation row
// for half as many N-tiles as one 32-row tile per wave did.)  The instruction
// is the same 32x32x64 block-scaled one with E2M1 A and E2M3 B operands
// (measured at the E2M1 x E2M1 rate).
// ===========================================================================
constexpr int kRowB6 = kKc / 32 * 24;            // activation code bytes per row per stage (96)
constexpr int kRing6 = 2;
constexpr int kStageB6 = kTileM * kRowB6;        // activation code rows (12 KB)
constexpr int kStage6 = kStageA + kStageB6;      // 28 KB
constexpr int kPipeLds6 = kRing6 * kStage6 + kGroupSA + kGroupSB;  // 63,488 bytes
static_assert(2 * kPipeLds6 <= 160 * 1024, "two workgroups per CU");
static_assert(kZeroPage >= kRowB6, "an absent activation row reads a stage from the zero page");

struct PipeSrc6 {
  const uint8_t* a[4];   // weight codes, as PipeSrc
  const uint8_t* as;     // weight scales, as PipeSrc
  const uint8_t* b[3];   // activation codes, load j: 16-byte unit 64j + lane of the wave's rows
  int bstep[3];          // code bytes per stage (96; 0 for an absent row on the zero page)
  const uint8_t* bs;     // activation scales (lanes 0-31): tile row 32 wave + lane
  int bsstep;            // scale bytes per group (16; 0 for an absent row)
};

__device__ __forceinline__ void pipe6_issue(uint8_t* smem, const PipeSrc6& src, int q, int wave) {
  uint8_t* st = smem + (q % kRing6) * kStage6;
#pragma unroll
  for (int j = 0; j < 4; ++j)  // stage q of a 16-row block: its tile q, 1 KB
    dma16(src.a[j] + (size_t)q * kTileBytes, st + wave * (64 * kRowC) + j * 1024);
#pragma unroll
  for (int j = 0; j < 3; ++j)
    dma16(src.b[j] + (size_t)q * src.bstep[j], st + kStageA + wave * (32 * kRowB6) + j * 1024);
}

// The scale bytes of group g: the wave's 64 weight rows at lanes 0-63, its
// 32 activation rows at lanes 0-31 (the layout of pipe_issue_scales).
__device__ __forceinline__ void pipe6_issue_scales(uint8_t* smem, const PipeSrc6& src, int g,
                                                   int wave) {
  uint8_t* sg = smem + kRing6 * kStage6;
  dma16(src.as + (size_t)g * kGroupRow, sg + wave * (64 * kGroupRow));
  if ((threadIdx.x & 63) < 32)
    dma16(src.bs + (size_t)g * src.bsstep, sg + kGroupSA + wave * (32 * kGroupRow));
}

// A ring of two stages: every load issued so far (stage q's, and its scale
// group's) has landed; then the barrier makes them visible and frees the
// stage read in the previous iteration.
__device__ __forceinline__ void pipe6_wait() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

__device__ __forceinline__ v16f mfma32x6(const uint4& a, const uint32_t (&b)[6], v16f c,
                                         uint32_t sa, uint32_t sb) {
  const v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  const v8i bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], (int)b[4], (int)b[5], 0, 0};
  // cbsz = 4: A (weights) E2M1; blgp = 2: B (activations) E2M3
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 2, 0, (int)sa, 0,
                                                         (int)sb);
}

struct StepFrags6 {
  uint4 a[2];
  uint32_t b[4][6];
};

// Fragments of MFMA step s: the wave's weight tiles t at row r (16 bytes of
// block 2s+hh, swizzled as in the MXFP4 kernels) and, per column tile, the
// 24 bytes of block 2s+hh of activation row 32cb+r, read as the two 16-byte
// units that hold them (an odd block starts 8 bytes into its first unit).
__device__ __forceinline__ void read_step6(const uint8_t* st, int s, int wave, int r, int hh,
                                           int swz, StepFrags6& f) {
  const int pb = ((2 * s + hh) ^ swz) * 16;
#pragma unroll
  for (int t = 0; t < 2; ++t)
    f.a[t] = *reinterpret_cast<const uint4*>(st + wave * (64 * kRowC) + (32 * t + r) * kRowC + pb);
  const int blk = 2 * s + hh;
  const int u0 = 16 * ((3 * blk) >> 1);
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const uint8_t* rp = st + kStageA + (32 * cb + r) * kRowB6 + u0;
    const uint4 x0 = *reinterpret_cast<const uint4*>(rp);
    const uint4 x1 = *reinterpret_cast<const uint4*>(rp + 16);
    f.b[cb][0] = hh ? x0.z : x0.x;
    f.b[cb][1] = hh ? x0.w : x0.y;
    f.b[cb][2] = hh ? x1.x : x0.z;
    f.b[cb][3] = hh ? x1.y : x0.w;
    f.b[cb][4] = hh ? x1.z : x1.x;
    f.b[cb][5] = hh ? x1.w : x1.y;
  }
}

// This lane's scale words of stage q, from the group buffer (as
// read_stage_scales).
__device__ __forceinline__ void read_stage_scales6(const uint8_t* smem, int q, int wave, int r,
                                                   StageScales& sc) {
  const uint8_t* sg = smem + kRing6 * kStage6 + (q % kGroup) * kRowS;
#pragma unroll
  for (int t = 0; t < 2; ++t)
    sc.aw[t] = *reinterpret_cast<const uint32_t*>(sg + (wave * 64 + 32 * t + r) * kGroupRow);
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
    sc.bw[cb] = *reinterpret_cast<const uint32_t*>(sg + kGroupSA + (32 * cb + r) * kGroupRow);
}

__device__ __forceinline__ void pipe6_compute(const uint8_t* smem, int q, int wave, int r, int hh,
                                              const StageScales& sc, v16f (&acc)[2][4]) {
  const uint8_t* st = smem + (q % kRing6) * kStage6;
  const int swz = (r >> 2) & 3;
  StepFrags6 f[2];
  read_step6(st, 0, wave, r, hh, swz, f[0]);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (s + 1 < 2) read_step6(st, s + 1, wave, r, hh, swz, f[1]);
    __builtin_amdgcn_sched_barrier(0);
    const StepFrags6& cur = f[s];
    const int sh = 8 * (2 * s + hh);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
        acc[t][cb] = mfma32x6(cur.a[t], cur.b[cb], acc[t][cb], sc.aw[t] >> sh, sc.bw[cb] >> sh);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The K loop over Q = K / 128 stages: stage q + 1 is issued into the other
// ring stage once the barrier of iteration q has freed it.
__device__ __forceinline__ void pipe6_mainloop(uint8_t* smem, const PipeSrc6& src, int Q, int wave,
                                               int lane, v16f (&acc)[2][4]) {
  const int r = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[t][cb] = zero16();
  pipe6_issue_scales(smem, src, 0, wave);
  pipe6_issue(smem, src, 0, wave);
  for (int q = 0; q < Q; ++q) {
    pipe6_wait();
    StageScales sc;
    read_stage_scales6(smem, q, wave, r, sc);
    if (q % kGroup == kGroup - 1 && q + 1 < Q) {
      // every wave holds its last scale words of the group: reload the buffer
      __syncthreads();
      pipe6_issue_scales(smem, src, (q + 1) / kGroup, wave);
    }
    if (q + 1 < Q) pipe6_issue(smem, src, q + 1, wave);
    pipe6_compute(smem, q, wave, r, hh, sc, acc);
  }
}

// Activation-side sources: the wave's tile rows 32 wave .. +31, 96 code bytes
// a stage each, as 192 16-byte units (unit c: row c / 6, bytes 16 (c % 6)..);
// rowptr(row) gives the row (codes at +0, scales at +scale_off) or null for
// an absent row, which reads the zero page.
template <typename RowPtr>
__device__ __forceinline__ void pipe6_act_src(PipeSrc6& src, RowPtr rowptr, size_t scale_off,
                                              const uint8_t* zero, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int c = 64 * j + lane;
    const int row = 32 * wave + c / 6, u = c % 6;
    const uint8_t* rp = rowptr(row);
    src.b[j] = (rp ? rp : zero) + u * 16;
    src.bstep[j] = rp ? kRowB6 : 0;
  }
  const int row = 32 * wave + (lane & 31);
  const uint8_t* rp = rowptr(row);
  src.bs = rp ? rp + scale_off : zero;
  src.bsstep = rp ? kGroupRow : 0;
}

// h = silu(gate) * up for one column of a 32-row weight tile pair, as
// swiglu_quant_store32, encoded as MXFP6 (E2M3): the lane's rows
// 8q + 4hh .. +3 are block elements whose 24 bits sit at byte 6q + 3hh of the
// block's 24 code bytes.
__device__ __forceinline__ void swiglu_quant_store32_fp6(const v16f& G, const v16f& U, int hh,
                                                         uint8_t* hr, int n0, int I) {
  float h[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) h[v] = silu_mul(G[v], U[v]);
  float amax = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) amax = fmaxf(amax, fabsf(h[v]));
  amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
  uint32_t code[16];
  uint32_t scale = 0u;
#pragma unroll
  for (int v = 0; v < 16; ++v) code[v] = 0u;
  if (amax > 0.f) {
    const int e = mx_block_exp(amax);
    scale = (uint32_t)(e + 127);
#pragma unroll
    for (int v = 0; v < 16; ++v) code[v] = e2m3_code(h[v], e);
  }
  if (hr) {
    uint8_t* hb = hr + (size_t)(n0 / 32) * 24 + 3 * hh;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w24 = code[4 * q] | (code[4 * q + 1] << 6) | (code[4 * q + 2] << 12) |
                           (code[4 * q + 3] << 18);
      hb[6 * q] = (uint8_t)w24;
      hb[6 * q + 1] = (uint8_t)(w24 >> 8);
      hb[6 * q + 2] = (uint8_t)(w24 >> 16);
    }
    if (hh == 0) hr[(size_t)I / 32 * 24 + n0 / 32] = (uint8_t)scale;
  }
}

// Gate/up with MXFP6 rows: tiles as gateup_pipe (N-tile = 128 rows of I).
__global__ __launch_bounds__(256, 2) void gateup_pipe6(PipeArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kPipeLds6];
  TileRef tr;
  int w;
  if (p.only) {
    const int n = p.only[1] * p.nN;
    w = (int)blockIdx.x < n ? p.only[0] * p.nN + (int)blockIdx.x : -1;
  } else {
    w = xcd_work_index(p.items[0] * p.nN);
  }
  if (!tile_of(w, p.nN, kTileM, p.items, p.offsets, p.S, p.A, p.shared ? p.T : 0, tr) ||
      tr.slot == p.skip_slot)
    return;
  const int s = tr.slot, p0 = tr.p0, rows = tr.rows;
  const bool sh = s == p.S;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 31, hh = lane >> 5;
  const int H = p.H;
  const int n0 = tr.nt * 128 + wave * 32;
  const bool active = n0 < p.I;
  const int nb = active ? n0 : 0;  // an idle wave still loads (row 0) and meets every barrier
  const uint8_t* base = sh ? p.shared : p.arena + (size_t)s * p.stride;
  const uint8_t* const wc[2] = {base + p.off_c0, base + p.off_c1};
  const uint8_t* const wsc[2] = {base + p.off_s0, base + p.off_s1};
  const int wrow[2] = {nb, nb};
  PipeSrc6 src;
  pipe_weight_src(src, wc, wsc, wrow, (size_t)H / 2, (size_t)H / 32, lane);
  pipe6_act_src(
      src,
      [&](int row) -> const uint8_t* {
        if (row >= rows) return nullptr;
        if (sh) return p.act + (size_t)(p0 + row - p.A) * p.arow;
        const int a = p.perm[p0 + row];
        return (a >= 0 && a < p.A) ? p.act + (size_t)(a / p.k) * p.arow : nullptr;
      },
      (size_t)H / 32 * 24, p.zero, wave, lane);
  v16f acc[2][4];
  pipe6_mainloop(smem, src, H / kKc, wave, lane, acc);
  if (!active) return;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    if (32 * cb < rows) {
      const int lr = 32 * cb + r;
      swiglu_quant_store32_fp6(acc[0][cb], acc[1][cb], hh,
                               lr < rows ? p.hq + (size_t)(p0 + lr) * p.hrow : nullptr, n0, p.I);
    }
  }
}

// Down with MXFP6 hq rows: tiles as down_pipe (N-tile = 256 rows of H).
__global__ __launch_bounds__(256, 2) void down_pipe6(PipeArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kPipeLds6];
  TileRef tr;
  if (!tile_of(xcd_work_index(p.items[0] * p.nN), p.nN, kTileM, p.items, p.offsets, p.S, p.A,
               p.shared ? p.T : 0, tr))
    return;
  const int s = tr.slot, p0 = tr.p0, rows = tr.rows;
  const bool sh = s == p.S;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 31, hh = lane >> 5;
  const int I = p.I;
  const int n0 = tr.nt * 256 + wave * 64;
  const uint8_t* base = sh ? p.shared : p.arena + (size_t)s * p.stride;
  const uint8_t* const wc[2] = {base + p.off_c0, base + p.off_c0};
  const uint8_t* const wsc[2] = {base + p.off_s0, base + p.off_s0};
  bool tv[2];
  int wrow[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    tv[t] = n0 + 32 * t < p.H;  // tiles past H load row 0 and are never stored
    wrow[t] = tv[t] ? n0 + 32 * t : 0;
  }
  PipeSrc6 src;
  pipe_weight_src(src, wc, wsc, wrow, (size_t)I / 2, (size_t)I / 32, lane);
  pipe6_act_src(
      src,
      [&](int row) -> const uint8_t* {
        return row < rows ? p.act + (size_t)(p0 + row) * p.arow : nullptr;
      },
      (size_t)I / 32 * 24, p.zero, wave, lane);
  v16f acc[2][4];
  pipe6_mainloop(smem, src, I / kKc, wave, lane, acc);
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int lr = 32 * cb + r;
    if (lr < rows) {
      const int a = sh ? p0 + lr : p.perm[p0 + lr];
      if (a >= 0 && (sh || a < p.A)) {
        uint16_t* yr = p.y + (size_t)a * p.H;
#pragma unroll
        for (int t = 0; t < 2; ++t)
          if (tv[t]) store_y_bf16(yr, n0 + 32 * t, hh, acc[t][cb]);
      }
    }
  }
}

}  // namespace moe

using namespace moe;

struct ExpertsWs {
  size_t items_off, zero_off, hq_off, y_off, total;
};

// Kernel family of a batch: batches of at least kPipeMinA assignments (T*k)
// with H and I multiples of 512 (whole scale groups of 16 bytes per row)
// take the pipelined kernels, every other batch the small-batch kernels.  Measured crossover on the 4096/2048 model with 166
// slots: the small-batch kernels win up to 1024 assignments, the pipelined
// ones from 2048.
constexpr int kPipeMinA = 2048;

enum Family { kFamSmall, kFamPipe };

// MXFP6 activation rows take the same crossover, with their own pipelined
// kernels (gateup_pipe6 / down_pipe6).
static Family family_of(int T, int k, int H, int I, int fmt) {
  (void)fmt;
  if ((size_t)T * k >= (size_t)kPipeMinA && H % 512 == 0 && I % 512 == 0) return kFamPipe;
  return kFamSmall;
}

// N-tiles of the pipelined kernels: gate/up rows of I and down rows of H per
// workgroup (the same for both activation formats).
static int pipe_ntile_gateup(int fmt) { (void)fmt; return 128; }
static int pipe_ntile_down(int fmt) { (void)fmt; return 256; }

// Upper bound on the M-tiles of tm rows of a batch: one partial tile per used
// slot plus the full ones.
static size_t max_tiles(size_t A, int S, int tm) {
  return (A < (size_t)S ? A : (size_t)S) + (A + tm - 1) / tm;
}

// M-tiles of the shared expert's T rows (0 without one).
static size_t shared_tiles(int T, bool shared) {
  return shared ? (size_t)(T + kTileM - 1) / kTileM : 0;
}

static ExpertsWs experts_ws(int T, int H, int k, int I, int S, bool shared, int fmt) {
  ExpertsWs w;
  const size_t A = (size_t)T * k;
  const size_t rows = A + (shared ? (size_t)T : 0);  // hq and y: routed rows, then shared ones
  const Family fam = family_of(T, k, H, I, fmt);
  const bool tiled = fam != kFamSmall;
  w.items_off = 0;
  // pipelined: the M-tile list, then the deferred slot's (first item, item
  // count); small batches: (slot, p0, p1) per work item
  const size_t ntile = max_tiles(A, S, kTileM) + shared_tiles(T, shared);
  const size_t nwork = (S > kInlineWorklistMaxS ? A : (A < (size_t)S ? A : (size_t)S)) +
                       (shared ? 1 : 0);
  const size_t items = tiled ? (1 + 4 * ntile + 2) * sizeof(int32_t)
                             : 3 * nwork * sizeof(int32_t);
  w.zero_off = up_to(w.items_off + items, 256);
  w.hq_off = w.zero_off + (tiled ? kZeroPage : 0);
  w.y_off = up_to(w.hq_off + rows * act_row_bytes(I, fmt), 256);
  w.total = up_to(w.y_off + rows * (size_t)H * sizeof(float), 256);
  return w;
}

size_t moe_experts_ws_bytes_internal(int T, int H, int k, int I, int S, bool shared, int fmt) {
  if (T <= 0) return 0;
  return experts_ws(T, H, k, I, S, shared, fmt).total;
}

// Shape checks shared by both entry points (no HIP call).
static int experts_check_shape(const moe_experts_args* a) {
  if (!a) return MOE_EINVAL;
  const int T = a->T, H = a->H, I = a->I, k = a->k, S = a->S;
  if (T < 0 || H <= 0 || I <= 0 || k <= 0 || S < 0) return MOE_EINVAL;
  if (H % 32 != 0 || I % 32 != 0 || k > MOE_MAX_K || S > MOE_MAX_S) return MOE_EUNSUPPORTED;
  if ((size_t)T * k > (size_t)INT32_MAX) return MOE_EINVAL;
  if (a->act_format != MOE_ACT_MXFP4 && a->act_format != MOE_ACT_MXFP6) return MOE_EINVAL;
  // MXFP6 rows run on the whole-super-chunk kernels only
  if (a->act_format == MOE_ACT_MXFP6 && (!staged_ok(H) || !staged_ok(I)))
    return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// Every argument check of a call that runs with workspace (ws, ws_bytes); no
// HIP call.  MOE_OK means experts_launch may run it.
static int experts_validate(const moe_experts_args* a, const void* ws, size_t ws_bytes) {
  const int r = experts_check_shape(a);
  if (r != MOE_OK) return r;
  const int T = a->T, H = a->H, I = a->I, k = a->k, S = a->S;
  if (T == 0) return MOE_OK;
  if (!a->xq || !a->slot_offsets || !a->perm || !a->sel_slot || !a->sel_weight || !a->out)
    return MOE_EINVAL;
  if (S > 0 && !a->arena) return MOE_EINVAL;  // with no slot, the arena is never read
  const SlotLayout L = slot_layout(H, I);
  if (a->slot_stride < L.total || a->slot_stride % 256 != 0) return MOE_EINVAL;
  if (!aligned(a->xq, 16) || !aligned(a->arena, 256) || !aligned(a->out, 8)) return MOE_EINVAL;
  const bool shared = a->shared_expert != nullptr;
  if (!aligned(a->shared_expert, 256)) return MOE_EINVAL;
  const int fmt = a->act_format;
  const ExpertsWs W = experts_ws(T, H, k, I, S, shared, fmt);
  if (ws_bytes < W.total) return MOE_EWORKSPACE;
  if (!ws || !aligned(ws, 256)) return MOE_EINVAL;
  const int defer = a->defer_slot;
  if (defer < -1 || defer >= S || (defer >= 0 && !a->defer_event)) return MOE_EINVAL;
  if (family_of(T, k, H, I, fmt) != kFamSmall) {
    const size_t ntile = max_tiles((size_t)T * k, S, kTileM) + shared_tiles(T, shared);
    const int n1 = pipe_ntile_gateup(fmt), n2 = pipe_ntile_down(fmt);
    if (up_to(ntile * (size_t)((I + n1 - 1) / n1), 8) > 0x7FFFFFFFu ||
        up_to(ntile * (size_t)((H + n2 - 1) / n2), 8) > 0x7FFFFFFFu)
      return MOE_EUNSUPPORTED;
  }
  return MOE_OK;
}

// Enqueues the work of a validated call with workspace ws.
static int experts_launch(const moe_experts_args* a, void* ws_ptr, hipStream_t stream) {
  const int T = a->T, H = a->H, I = a->I, k = a->k, S = a->S;
  if (T == 0) return MOE_OK;
  const SlotLayout L = slot_layout(H, I);
  const bool shared = a->shared_expert != nullptr;
  const int fmt = a->act_format;
  const ExpertsWs W = experts_ws(T, H, k, I, S, shared, fmt);
  const int defer = a->defer_slot;
  const int A = T * k;
  const Family fam = family_of(T, k, H, I, fmt);
  const size_t ntile = max_tiles((size_t)A, S, kTileM) + shared_tiles(T, shared);
  // N-tiles: gate/up 128 rows of I, down 256 rows of H (MXFP6 rows: 64 and 128)
  const bool fp6 = fmt == MOE_ACT_MXFP6;
  const int nN1 = (I + pipe_ntile_gateup(fmt) - 1) / pipe_ntile_gateup(fmt);
  const int nN2 = (H + pipe_ntile_down(fmt) - 1) / pipe_ntile_down(fmt);
  const size_t g1 = up_to(ntile * (size_t)nN1, 8);
  const size_t g2 = up_to(ntile * (size_t)nN2, 8);
  if (S == 0 && !shared) {
    // nothing routable: every pick is padding, the output is zero
    dim3 grid(T, (H + 256 * YRow<float>::kEl - 1) / (256 * YRow<float>::kEl));
    combine_kernel<float><<<grid, 256, 0, stream>>>(nullptr, a->sel_weight, a->sel_slot, T, H,
                                                    k, S, nullptr, a->out);
    return hip_status();
  }
  uint8_t* ws = static_cast<uint8_t*>(ws_ptr);
  uint8_t* hq = ws + W.hq_off;
  float* y = reinterpret_cast<float*>(ws + W.y_off);
  hipEvent_t* ev = a->stage_events;

  if (fam == kFamPipe) {
    int32_t* items = reinterpret_cast<int32_t*>(ws + W.items_off);
    int32_t* defer_info = items + 1 + 4 * ntile;
    uint8_t* zero = ws + W.zero_off;
    if (!record_stage(ev, 0, stream)) return MOE_EHIP;
    build_tiles<<<1, 1024, 0, stream>>>(a->slot_offsets, S, A, kTileM, items,
                                        reinterpret_cast<uint32_t*>(zero), defer, defer_info,
                                        shared ? T : 0);
    PipeArgs t;
    t.act = a->xq;
    t.arow = act_row_bytes(H, fmt);
    t.arena = a->arena;
    t.stride = a->slot_stride;
    t.off_c0 = L.off[0];
    t.off_s0 = L.off[1];
    t.off_c1 = L.off[2];
    t.off_s1 = L.off[3];
    t.offsets = a->slot_offsets;
    t.perm = a->perm;
    t.items = items;
    t.zero = zero;
    t.hq = hq;
    t.hrow = act_row_bytes(I, fmt);
    t.y = reinterpret_cast<uint16_t*>(y);
    t.H = H;
    t.I = I;
    t.k = k;
    t.A = A;
    t.nN = nN1;
    t.skip_slot = defer;
    t.only = nullptr;
    t.shared = a->shared_expert;
    t.S = S;
    t.T = T;
    hipExtLaunchKernelGGL(fp6 ? gateup_pipe6 : gateup_pipe, dim3((unsigned)g1),
                          dim3(fp6 ? 256 : kPipeWaves * kWave), 0, stream, ev ? ev[1] : nullptr,
                          ev ? ev[2] : nullptr, 0, t);
    if (defer >= 0) {
      // the deferred slot's tiles, once its bytes are in place: at most one
      // assignment per token, so at most ceil(T / 128) M-tiles
      if (hipStreamWaitEvent(stream, a->defer_event, 0) != hipSuccess) return MOE_EHIP;
      t.skip_slot = -1;
      t.only = defer_info;
      const size_t g3 = (size_t)((T + kTileM - 1) / kTileM) * (size_t)nN1;
      if (fp6)
        gateup_pipe6<<<(unsigned)g3, 256, 0, stream>>>(t);
      else
        gateup_pipe<<<(unsigned)g3, kPipeWaves * kWave, 0, stream>>>(t);
      t.only = nullptr;
    }
    t.act = hq;
    t.arow = t.hrow;
    t.off_c0 = L.off[4];
    t.off_s0 = L.off[5];
    t.nN = nN2;
    if (fp6)
      down_pipe6<<<(unsigned)g2, 256, 0, stream>>>(t);
    else
      down_pipe<<<(unsigned)g2, kPipeWaves * kWave, 0, stream>>>(t);
    if (!record_stage(ev, 3, stream)) return MOE_EHIP;
  } else {
    // work items: the used slots, found in place, for small slot counts; the
    // bucketed positions (an item per slot's first position) for larger ones
    const bool by_position = S > kInlineWorklistMaxS;
    const int maxU = by_position ? A : (S < A ? S : A);
    // small batches run every slot in one pass: the deferred slot's bytes
    // must be in place before it
    if (defer >= 0 && hipStreamWaitEvent(stream, a->defer_event, 0) != hipSuccess)
      return MOE_EHIP;
    if (!record_stage(ev, 0, stream)) return MOE_EHIP;
    GateUpArgs g;
    g.xq = a->xq;
    g.xrow = act_row_bytes(H, fmt);
    g.arena = a->arena;
    g.stride = a->slot_stride;
    g.off_gc = L.off[0];
    g.off_gs = L.off[1];
    g.off_uc = L.off[2];
    g.off_us = L.off[3];
    g.offsets = a->slot_offsets;
    g.perm = a->perm;
    g.sel_slot = by_position ? a->sel_slot : nullptr;
    int32_t* slots = reinterpret_cast<int32_t*>(ws + W.items_off);
    g.slots = slots;
    g.hq = hq;
    g.hrow = act_row_bytes(I, fmt);
    g.T = T;
    g.H = H;
    g.I = I;
    g.k = k;
    g.A = A;
    g.S = S;
    g.shared = a->shared_expert;
    g.maxU = maxU;
    const int nwork = maxU + (shared ? 1 : 0);  // the shared expert's item last
    const int gblocks = nwork * (I / 32);
    hipEvent_t gu0 = ev ? ev[1] : nullptr, gu1 = ev ? ev[2] : nullptr;
    const size_t glds = 2 * 32 * staged_scale_stride(H);
    if (fmt == MOE_ACT_MXFP6)  // validated: staged_ok(H) and staged_ok(I)
      hipExtLaunchKernelGGL(gateup_kernel<true, true>, dim3(gblocks), dim3(kWave), glds, stream,
                            gu0, gu1, 0, g);
    else if (staged_ok(H))
      hipExtLaunchKernelGGL(gateup_kernel<true, false>, dim3(gblocks), dim3(kWave), glds, stream,
                            gu0, gu1, 0, g);
    else
      hipExtLaunchKernelGGL(gateup_kernel<false, false>, dim3(gblocks), dim3(kWave), 0, stream,
                            gu0, gu1, 0, g);
    DownArgs d;
    d.hq = hq;
    d.hrow = g.hrow;
    d.arena = a->arena;
    d.stride = a->slot_stride;
    d.off_dc = L.off[4];
    d.off_ds = L.off[5];
    d.offsets = a->slot_offsets;
    d.perm = a->perm;
    d.slots = slots;
    d.y = y;
    d.H = H;
    d.I = I;
    d.A = A;
    d.S = S;
    d.shared = a->shared_expert;
    const int yrows = A + (shared ? T : 0);
    if (fmt == MOE_ACT_MXFP4 && yrows <= kRcMaxRows && T <= kRcMaxT) {
      // decode-size batches: down and combine in one launch (same output)
      RowsCombineArgs q;
      q.d = d;
      q.sel_weight = a->sel_weight;
      q.sel_slot = a->sel_slot;
      q.out = a->out;
      q.T = T;
      q.k = k;
      q.nwork = nwork;
      const unsigned rblocks = (unsigned)(H / 16);
      if (I % 512 == 0)
        down_rows_combine<true><<<rblocks, kRcWaves * kWave, 0, stream>>>(q);
      else
        down_rows_combine<false><<<rblocks, kRcWaves * kWave, 0, stream>>>(q);
      if (!record_stage(ev, 3, stream) || !record_stage(ev, 4, stream)) return MOE_EHIP;
      return hip_status();
    }
    const int dblocks = nwork * ((H + 63) / 64);
    const size_t dlds = 64 * staged_scale_stride(I);
    if (fmt == MOE_ACT_MXFP6)
      down_kernel<true, true><<<dblocks, kWave, dlds, stream>>>(d);
    else if (staged_ok(I))
      down_kernel<true, false><<<dblocks, kWave, dlds, stream>>>(d);
    else
      down_kernel<false, false><<<dblocks, kWave, 0, stream>>>(d);
    if (!record_stage(ev, 3, stream)) return MOE_EHIP;
  }
  // a workgroup covers 256 threads x YRow<YT>::kEl elements of a token's row; the
  // shared expert's rows follow the A routed ones
  if (fam != kFamSmall) {
    const int per = 256 * YRow<uint16_t>::kEl;
    const uint16_t* yb = reinterpret_cast<const uint16_t*>(y);
    combine_kernel<uint16_t><<<dim3(T, (H + per - 1) / per), 256, 0, stream>>>(
        yb, a->sel_weight, a->sel_slot, T, H, k, S, shared ? yb + (size_t)A * H : nullptr,
        a->out);
  } else {
    const int per = 256 * YRow<float>::kEl;
    combine_kernel<float><<<dim3(T, (H + per - 1) / per), 256, 0, stream>>>(
        y, a->sel_weight, a->sel_slot, T, H, k, S, shared ? y + (size_t)A * H : nullptr, a->out);
  }
  if (!record_stage(ev, 4, stream)) return MOE_EHIP;
  return hip_status();
}

extern "C" MOE_EXPORT int moe_experts_forward(const moe_experts_args* a, hipStream_t stream) {
  const int r = a ? experts_validate(a, a->ws, a->ws_bytes) : MOE_EINVAL;
  if (r != MOE_OK) return r;
  return experts_launch(a, a->ws, stream);
}

// ---------------------------------------------------------------------------
// moe_experts_forward_noalloc: the same call with the workspace taken from a
// device array of the library's own (kNoAllocScratch bytes, one copy per GPU,
// held until the process ends).  Its device address is looked up once per
// device, with that device current, and kept; host code never passes the
// array's name itself to a kernel (on the host it is only a stand-in).
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratch = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kNoAllocScratch];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];  // per device: the array's device address

// The scratch array's address on the current device (looked up on the first
// call there); null if the lookup fails.
static void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

extern "C" MOE_EXPORT int moe_experts_forward_noalloc(const moe_experts_args* a,
                                                      hipStream_t stream) {
  int r = experts_check_shape(a);
  if (r != MOE_OK) return r;
  if (a->ws || a->ws_bytes) return MOE_EINVAL;  // the workspace is the library's own
  if (a->T == 0) return MOE_OK;
  const size_t need =
      experts_ws(a->T, a->H, a->k, a->I, a->S, a->shared_expert != nullptr, a->act_format).total;
  if (need > kNoAllocScratch) return MOE_ESCRATCH;
  // every other check, against a stand-in for the scratch (256-aligned, not read)
  r = experts_validate(a, reinterpret_cast<const void*>(uintptr_t{256}), kNoAllocScratch);
  if (r != MOE_OK) return r;
  void* ws = scratch_on_current_device();
  if (!ws) return MOE_EHIP;
  return experts_launch(a, ws, stream);
}
