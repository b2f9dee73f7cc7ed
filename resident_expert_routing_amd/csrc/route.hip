// moe_route: router logits, demand picks, masked top-k, renormalisation,
// token-to-slot bucketing and MXFP4 activation rows (gfx950).
//
// TideLM README, "How adaptive expert loading works", items 1-2: the router
// scores every expert; demand is recorded over the unrestricted top-k; the
// router then picks only resident (or hot-ring) experts, a miss replaced by the
// next-best resident expert; the chosen weights are renormalised.  Rows are
// then named by index per slot (colibri cluster page, COLIEX01 v2 paragraph).
#include <algorithm>

#include "common.hpp"
#include "demand_sums.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Router logits in float64 (every bf16 x fp32 product is exact).  Two regimes,
// each with one fixed summation order, so within a regime a token's z does
// not depend on the rest of its batch: router_small_f64 (chunk chains, then
// runs of chunk sums) and router_full_f64 (the float64 matrix instruction).
// ---------------------------------------------------------------------------

// Activation rows, one element per thread: each aligned group of 32 threads
// encodes one block (amax by shuffles within the group).  MXFP4: even lanes
// write a byte of two codes; MXFP6: every fourth lane writes the 3 bytes of
// four codes.  Lane 0 writes the scale.  gid and gstride are multiples of 32
// and T*H is a multiple of 32, so a group is always whole.
__device__ void quantize_x_elements(const uint16_t* __restrict__ x, int T, int H,
                                    uint8_t* __restrict__ xq, size_t xq_row, size_t gid,
                                    size_t gstride, int fmt) {
  const size_t n = (size_t)T * H;
  const size_t sc_off = act_scale_offset(H, fmt);
  for (size_t q = gid; q < n; q += gstride) {
    const int t = (int)(q / H), h = (int)(q % H);
    const float v = bf16_to_f32(x[q]);
    float a = fabsf(v);
#pragma unroll
    for (int d = 16; d >= 1; d >>= 1) a = fmaxf(a, __shfl_xor(a, d, 32));
    const int li = (int)(q & 31);
    uint8_t* row = xq + (size_t)t * xq_row;
    uint32_t scale = 0u;
    if (fmt == MOE_ACT_MXFP6) {
      uint32_t code = 0u;
      if (a > 0.f) {
        const int e = mx_block_exp(a);
        code = e2m3_code(v, e);
        scale = (uint32_t)(e + 127);
      }
      const uint32_t c1 = __shfl_down(code, 1, 32), c2 = __shfl_down(code, 2, 32),
                     c3 = __shfl_down(code, 3, 32);
      if ((li & 3) == 0) {
        const uint32_t w = code | (c1 << 6) | (c2 << 12) | (c3 << 18);  // elements li..li+3
        uint8_t* dst = row + (size_t)(h / 32) * 24 + (li / 4) * 3;
        dst[0] = (uint8_t)w;
        dst[1] = (uint8_t)(w >> 8);
        dst[2] = (uint8_t)(w >> 16);
      }
    } else {
      uint32_t code = 0u;
      if (a > 0.f) {
        const int e = mx_block_exp(a);
        code = e2m1_code(v, e);
        scale = (uint32_t)(e + 127);
      }
      const uint32_t odd = __shfl_down(code, 1, 32);
      if ((li & 1) == 0) row[h / 2] = (uint8_t)(code | (odd << 4));
    }
    if (li == 0) row[sc_off + h / 32] = (uint8_t)scale;
  }
}

// Small T (decode batches): a workgroup owns one expert and up to RS_T tokens;
// thread c owns chunk c for all of them (the router chunk is loaded once, RS_T
// independent fma chains) -- or, with at most 128 chunks (SPLIT), threads c and
// c + 128 own chunk c for half of the tokens each, so every thread works and
// holds half the x registers; the chunk sums meet in LDS.  They are added in runs
// of RS_RUN consecutive chunks (ascending, from 0), and the run sums in
// ascending order (from 0).  Workgroups from `nrb` on encode the activation
// rows instead (one element per thread), alongside the dot products.
// Workgroup 0 also zeroes `counter` (nullable) for the selection kernel that
// follows.
typedef double v4d __attribute__((ext_vector_type(4)));
constexpr int RS_T = 8;
constexpr int RS_MAX_CHUNKS = 256;
constexpr int RS_RUN = 16;
// z[tok[i], e] for the nt (<= RS_T) tokens tok[0..nt) and one expert, by the
// whole workgroup (thread c owns chunk c).
template <bool SPLIT>
__device__ __forceinline__ void small_dot_block(const uint16_t* __restrict__ x,
                                                const float* __restrict__ w, int H, int E,
                                                double* __restrict__ z, int e, const int* tok,
                                                int nt) {
  __shared__ double part[RS_T][RS_MAX_CHUNKS + 1];
  __shared__ double runs[RS_T][RS_MAX_CHUNKS / RS_RUN];
  const int nchunk = H / kRouterChunk;  // H % 32 == 0 (SPLIT: at most 128 chunks)
  // SPLIT: thread (c, half) takes chunk c for tokens 4 half .. 4 half + 3
  constexpr int kTok = SPLIT ? RS_T / 2 : RS_T;
  const int c = SPLIT ? (int)(threadIdx.x & 127) : (int)threadIdx.x;
  const int ibeg = SPLIT ? (int)(threadIdx.x >> 7) * kTok : 0;
  if (c < nchunk) {
    const int h0 = c * kRouterChunk;
    const float4* w4 = reinterpret_cast<const float4*>(w + (size_t)e * H + h0);
    float4 wv[kRouterChunk / 4];
#pragma unroll
    for (int q = 0; q < kRouterChunk / 4; ++q) wv[q] = w4[q];
    // every token's x chunk is loaded before the first chain starts (tokens
    // past the batch load its last one and are never stored): loads inside
    // `if (i < nt)` were issued one token at a time, a round trip each
    uint4 xv_all[kTok][kRouterChunk / 8];
#pragma unroll
    for (int ii = 0; ii < kTok; ++ii) {
      const int i = ibeg + ii;
      const uint4* x4 = reinterpret_cast<const uint4*>(x + (size_t)tok[min(i, nt - 1)] * H + h0);
#pragma unroll
      for (int q = 0; q < kRouterChunk / 8; ++q) xv_all[ii][q] = x4[q];
    }
#pragma unroll
    for (int ii = 0; ii < kTok; ++ii) {
      const int i = ibeg + ii;
      {
        const uint4 (&xv)[kRouterChunk / 8] = xv_all[ii];
        double s = 0.0;
#pragma unroll
        for (int q = 0; q < kRouterChunk / 8; ++q) {
          const uint32_t xw[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
          const float4 wa = wv[2 * q], wb = wv[2 * q + 1];
          const float ww[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const uint32_t bits = (r & 1) ? (xw[r >> 1] >> 16) : (xw[r >> 1] & 0xFFFFu);
            s = fma((double)bf16_to_f32(bits), (double)ww[r], s);
          }
        }
        if (i < nt) part[i][c] = s;
      }
    }
  }
  __syncthreads();
  // thread (token i, run q) adds the chunk sums of run q
  const int nrun = (nchunk + RS_RUN - 1) / RS_RUN;
  const int tc = threadIdx.x;
  {
    const int i = tc / nrun, q = tc % nrun;
    if (i < nt) {
      double acc = 0.0;
      const int c1 = min(nchunk, (q + 1) * RS_RUN);
      for (int cc = q * RS_RUN; cc < c1; ++cc) acc += part[i][cc];
      runs[i][q] = acc;
    }
  }
  __syncthreads();
  if (tc < nt) {
    double acc = 0.0;
    for (int q = 0; q < nrun; ++q) acc += runs[tc][q];
    z[(size_t)tok[tc] * E + e] = acc;
  }
}

template <bool SPLIT>
__global__ __launch_bounds__(256) void router_small_f64(const uint16_t* __restrict__ x,
                                                        const float* __restrict__ w, int T, int H,
                                                        int E, double* __restrict__ z,
                                                        uint8_t* __restrict__ xq, size_t xq_row,
                                                        int fmt, int nrb,
                                                        uint32_t* __restrict__ counter) {
  if (counter && blockIdx.x == 0 && threadIdx.x == 0) *counter = 0u;
  if ((int)blockIdx.x >= nrb) {
    quantize_x_elements(x, T, H, xq, xq_row, (size_t)(blockIdx.x - nrb) * 256 + threadIdx.x,
                        (size_t)(gridDim.x - nrb) * 256, fmt);
    return;
  }
  const int ntg = (T + RS_T - 1) / RS_T;
  const int e = blockIdx.x / ntg, t0 = (blockIdx.x % ntg) * RS_T;
  const int nt = min(RS_T, T - t0);
  int tok[RS_T];
#pragma unroll
  for (int i = 0; i < RS_T; ++i) tok[i] = t0 + i;
  small_dot_block<SPLIT>(x, w, H, E, z, e, tok, nt);
}

// Float64 logits where a flagged token's picks can still change.  With every
// stored z~ within `bound` of its exact value, an expert whose z~ (bias
// included) is below the k-th stored value minus twice the bound has at least
// k experts certainly above it, so it is out of the top-k; only the experts at
// or above that line (in the order over all experts, and over the routable
// ones) can be picked.  Those get the float64 logit, every other entry keeps
// its z~, and the token is selected again: the picks are the float64 logits'.
// One workgroup per listed token (a fixed grid walks the list).  The token's
// candidates are decided first, from the bounded logits, into an LDS mask per
// 64 experts; a barrier then separates those reads from the rewrites of z, and
// the four waves take the candidates in turn.  Lane l sums h in
// [l H/64, (l+1) H/64) as a fused multiply-add chain, then the wave adds the
// lanes' sums in the fixed DPP order.
__global__ __launch_bounds__(256) void router_f64_candidates(
    const uint16_t* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    const int32_t* __restrict__ expert_slot, int H, int E, int S, double* __restrict__ z,
    const int32_t* __restrict__ tlist, const double* __restrict__ cert) {
  constexpr int kPass = 64;  // elements per lane whose loads are issued together
  __shared__ uint64_t cmask[MOE_MAX_E / 64];
  const int n = tlist[0];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per = H / 64;  // H % 512 == 0, H <= 8192: at most two passes
  const int nb = (E + 63) / 64;
  for (int i = blockIdx.x; i < n; i += gridDim.x) {  // uniform
    const int t = tlist[1 + i];
    const double ku = cert[3 * (size_t)t], km = cert[3 * (size_t)t + 1];
    const double line = 2.0 * cert[3 * (size_t)t + 2];
    for (int b = wave; b < nb; b += 4) {
      const int e = 64 * b + lane;
      bool cand = false;
      if (e < E) {
        const double v = z[(size_t)t * E + e] + (bias ? (double)bias[e] : 0.0);
        const int sl = expert_slot[e];
        cand = v >= ku - line || (sl >= 0 && sl < S && v >= km - line);
      }
      const uint64_t m = __ballot(cand);
      if (lane == 0) cmask[b] = m;
    }
    __syncthreads();  // every candidate decided before any z of the token is rewritten
    const uint16_t* xr = x + (size_t)t * H + (size_t)lane * per;
    int j = 0;  // candidate rank over all blocks; wave j % 4 takes it
    for (int b = 0; b < nb; ++b) {
      uint64_t m = cmask[b];
      for (; m; ++j) {  // uniform
        const int c = 64 * b + __builtin_ctzll(m);
        m &= m - 1;
        if ((j & 3) != wave) continue;
        const float* wr = w + (size_t)c * H + (size_t)lane * per;
        double acc = 0.0;  // h ascending over the lane's range (per = H/64, a multiple of 8)
        for (int h0 = 0; h0 < per; h0 += kPass) {
          // every load of the pass before its first product: one memory round
          // trip per pass instead of one per 8 elements
          uint4 xv[kPass / 8];
          float4 wv[kPass / 4];
#pragma unroll
          for (int q = 0; q < kPass / 8; ++q) {
            if (h0 + 8 * q < per) {
              xv[q] = *reinterpret_cast<const uint4*>(xr + h0 + 8 * q);
              wv[2 * q] = *reinterpret_cast<const float4*>(wr + h0 + 8 * q);
              wv[2 * q + 1] = *reinterpret_cast<const float4*>(wr + h0 + 8 * q + 4);
            }
          }
#pragma unroll
          for (int q = 0; q < kPass / 8; ++q) {
            if (h0 + 8 * q < per) {
              const uint32_t xw[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
              const float ww[8] = {wv[2 * q].x,     wv[2 * q].y,     wv[2 * q].z,
                                   wv[2 * q].w,     wv[2 * q + 1].x, wv[2 * q + 1].y,
                                   wv[2 * q + 1].z, wv[2 * q + 1].w};
#pragma unroll
              for (int jj = 0; jj < 8; ++jj) {
                const uint32_t bits = (jj & 1) ? (xw[jj >> 1] >> 16) : (xw[jj >> 1] & 0xFFFFu);
                acc = fma((double)bf16_to_f32(bits), (double)ww[jj], acc);
              }
            }
          }
        }
        const double sum = wave_sum(acc);
        if (lane == 0) z[(size_t)t * E + c] = sum;
      }
    }
    __syncthreads();  // cmask is rewritten for the next token only after every wave read it
  }
}

// Router for larger T on the float64 matrix cores (v_mfma_f64_16x16x4f64):
// bf16 x fp32 products are exact in float64 and every sum is float64; each
// z[t,e] is the chain, over h in steps of 4 ascending, of the instruction's
// float64 sum of its four products added to the running value (one fixed,
// batch-independent order).  A workgroup owns 16 tokens x 64 experts; wave w
// owns the 16x16 tile of experts 16w..16w+15.  16-token workgroups put two
// waves on every SIMD at 2048 tokens (the float64 instruction's issue rate
// rose from 32 to 45 TFLOP/s with a second wave in a probe; a second
// accumulator chain in the same wave added little).  K tiles of 32 are staged
// in LDS as float32 (exact for bf16 and fp32), k-major (the weight rows with a
// 16-float pad) so a fragment read hits 64 distinct banks, and double-buffered
// through registers.
constexpr int RM_T = 16, RM_E = 64, RM_K = 32;
constexpr int RM_XS = RM_T, RM_WS = RM_E + 16;

// tlist (nullable): the tokens to compute, tlist[0] = n then n token ids
// ascending; tile row i is then token tlist[1 + t0 + i] (workgroups past n
// leave at once).  Without it, tile row i is token t0 + i.
__global__ __launch_bounds__(256) void router_full_f64(const uint16_t* __restrict__ x,
                                                       const float* __restrict__ w, int T, int H,
                                                       int E, double* __restrict__ z,
                                                       const int32_t* __restrict__ tlist) {
  __shared__ float xs[2][RM_K][RM_XS];
  __shared__ float ws[2][RM_K][RM_WS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = blockIdx.y * RM_T, e0 = blockIdx.x * RM_E;
  const int nt = tlist ? tlist[0] : T;  // rows of this call
  if (t0 >= nt) return;                  // uniform: before any barrier
  // token of tile row i (i < RM_T), or -1
  auto token_of = [&](int i) -> int {
    if (t0 + i >= nt) return -1;
    return tlist ? tlist[1 + t0 + i] : t0 + i;
  };
  // staging roles: x -- token tid/8, h 4(tid%8)..+3 (threads 0-127); w -- expert
  // tid/4, h 8(tid%4)..+7
  const int xt = (tid >> 3) & (RM_T - 1), xq = tid & 7;
  const int we = tid >> 2, wq = tid & 3;
  const bool xrole = tid < RM_T * 8;
  const int xtok = token_of(xt);
  const bool xin = xrole && xtok >= 0, win = e0 + we < E;
  const uint16_t* xrow = x + (size_t)(xin ? xtok : 0) * H + 4 * xq;
  const float* wrow = w + (size_t)(win ? e0 + we : 0) * H + 8 * wq;
  uint2 xv = xin ? *reinterpret_cast<const uint2*>(xrow) : make_uint2(0u, 0u);
  float4 w0 = win ? *reinterpret_cast<const float4*>(wrow) : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 w1 = win ? *reinterpret_cast<const float4*>(wrow + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
  auto stage = [&](int b) {
    if (xrole) {
      xs[b][4 * xq + 0][xt] = bf16_to_f32(xv.x & 0xFFFFu);
      xs[b][4 * xq + 1][xt] = bf16_to_f32(xv.x >> 16);
      xs[b][4 * xq + 2][xt] = bf16_to_f32(xv.y & 0xFFFFu);
      xs[b][4 * xq + 3][xt] = bf16_to_f32(xv.y >> 16);
    }
    ws[b][8 * wq + 0][we] = w0.x;
    ws[b][8 * wq + 1][we] = w0.y;
    ws[b][8 * wq + 2][we] = w0.z;
    ws[b][8 * wq + 3][we] = w0.w;
    ws[b][8 * wq + 4][we] = w1.x;
    ws[b][8 * wq + 5][we] = w1.y;
    ws[b][8 * wq + 6][we] = w1.z;
    ws[b][8 * wq + 7][we] = w1.w;
  };
  stage(0);
  __syncthreads();
  v4d acc0 = {0.0, 0.0, 0.0, 0.0};
  const int r = lane & 15, kq = lane >> 4;
  const int ntile = H / RM_K;
  for (int c = 0; c < ntile; ++c) {
    const int b = c & 1;
    if (c + 1 < ntile) {
      const int h0 = (c + 1) * RM_K;
      xv = xin ? *reinterpret_cast<const uint2*>(xrow + h0) : make_uint2(0u, 0u);
      w0 = win ? *reinterpret_cast<const float4*>(wrow + h0) : make_float4(0.f, 0.f, 0.f, 0.f);
      w1 = win ? *reinterpret_cast<const float4*>(wrow + h0 + 4)
               : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int ks = 0; ks < RM_K / 4; ++ks) {
      const int k = 4 * ks + kq;
      const double a0 = (double)xs[b][k][r];
      const double bw = (double)ws[b][k][16 * wave + r];
      acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, bw, acc0, 0, 0, 0);
    }
    if (c + 1 < ntile) stage(b ^ 1);
    __syncthreads();
  }
  // lane l holds rows (tokens) l/16 + 4v, column (expert) l%16 of the tile
  // (the float64 instruction's result layout, confirmed on the hardware)
  const int e = e0 + 16 * wave + r;
  if (e >= E) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int ta = token_of(kq + 4 * v);
    if (ta >= 0) z[(size_t)ta * E + e] = acc0[v];
  }
}

// ---------------------------------------------------------------------------
// Larger batches, first pass: the logits on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16).  Every fp32 router weight splits exactly into
// three bf16 parts, w = w1 + w2 + w3 (w1 = w cut to 8 significant bits, w2 =
// the rest cut the same way, w3 = what remains, at most 8 bits: split_w_bf16x3,
// once per call), so every product x*w_i is exact in fp32.  Per 64-wide slice
// of h, the products of each part go to an fp32 accumulator of their own (a
// chain of 4 instructions each); at the end of the slice the three are added,
// w1's first, to a float64 sum.  Bound on the result's error (the selection
// uses it to decide which tokens need float64 logits): if one instruction's
// result (accumulator plus 16 exact products) is off by at most c*u times
// (|accumulator| + sum of |products|), c = 34 and u = 2^-24 (sixteen rounded
// additions, each allowed twice the rounding of round-to-nearest), a chain of
// 4 instructions is off by at most 4*c*u times the sum of |products| of its
// part; with |w2| + |w3| < 2^-7 (1 + 2^-7) |w| that is c*u*4 (1 + 2^-7 (1 +
// 2^-7)) <= 4.04 c u times sum_h |x_h w_h| per slice, and over the slices
// (float64 additions adding ~1e-16 relative) |z~ - z| <= 4.04 c u ||x_t||
// ||w_e|| (Cauchy-Schwarz).  Workgroup: MT tokens x 64 experts, one wave per
// 32 x 32 tile, h staged in LDS 64 at a time.  Every z[t,e] is a fixed chain of
// its own operands: batch-independent.
// ---------------------------------------------------------------------------
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
constexpr int RB_E = 64, RB_K = 64;

__device__ __forceinline__ uint32_t bf16_hi(float v) { return __float_as_uint(v) >> 16; }

// w [E][H] fp32 -> planes [3][E][H] bf16 with w = w1 + w2 + w3 exactly, and
// wnorm2[e] = ||w_e||^2 (float64 sums of exact squares; one workgroup per row).
// Also zeroes *count (the flagged-token count of the selection that follows).
__global__ __launch_bounds__(256) void split_w_bf16x3(const float* __restrict__ w, int E, int H,
                                                      uint16_t* __restrict__ planes,
                                                      double* __restrict__ wnorm2,
                                                      int32_t* __restrict__ count) {
  __shared__ double part[4];
  const int e = blockIdx.x, tid = threadIdx.x;
  if (e == 0 && tid == 0) *count = 0;
  const float* row = w + (size_t)e * H;
  const size_t plane = (size_t)E * H;
  double nrm = 0.0;
  for (int h = 4 * tid; h < H; h += 1024) {  // H % 64 == 0: whole float4s
    const float4 v4 = *reinterpret_cast<const float4*>(row + h);
    const float f[4] = {v4.x, v4.y, v4.z, v4.w};
    uint32_t p[3][2] = {{0u, 0u}, {0u, 0u}, {0u, 0u}};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v = f[j];
      nrm += (double)v * (double)v;
      const uint32_t h1 = bf16_hi(v);
      const float r1 = v - __uint_as_float(h1 << 16);   // exact
      const uint32_t h2 = bf16_hi(r1);
      const float r2 = r1 - __uint_as_float(h2 << 16);  // exact, at most 8 bits
      const uint32_t h3 = bf16_hi(r2);
      p[0][j >> 1] |= h1 << (16 * (j & 1));
      p[1][j >> 1] |= h2 << (16 * (j & 1));
      p[2][j >> 1] |= h3 << (16 * (j & 1));
    }
#pragma unroll
    for (int q = 0; q < 3; ++q)
      *reinterpret_cast<uint2*>(planes + q * plane + (size_t)e * H + h) = make_uint2(p[q][0], p[q][1]);
  }
  nrm = wave_sum(nrm);
  if ((tid & 63) == 0) part[tid >> 6] = nrm;
  __syncthreads();
  if (tid == 0) wnorm2[e] = ((part[0] + part[1]) + part[2]) + part[3];
}

// Workgroup: 128 tokens x 64 experts, 8 waves (4 x 2 tiles of 32 x 32), h in
// [z*H/KS, (z+1)*H/KS) for blockIdx.z = z: the float64 sum of those slices
// goes to zpart[z][t][e] (the selection adds the KS parts in order of z).
// Operands reach LDS by direct global-to-LDS loads into a ring of three
// 40 KB stages (64 h of the 128 x rows and of the three planes' 64 rows), two
// stages issued ahead; each load moves 8 rows x 128 bytes.  The 16-byte block
// b of a 128-byte LDS row r sits at b ^ ((r >> 1) & 7), so a fragment read
// (32 rows, one block each) is free of bank conflicts.  Rows past T or E read
// row 0 of the batch: their results are never stored.
constexpr int RB_MT = 128, RB_THREADS = 512;
constexpr int RB_ROW = 2 * RB_K;                          // bytes per LDS row per stage
constexpr int RB_XB = RB_MT * RB_ROW;                     // x rows of a stage (16 KB)
constexpr int RB_WB = 3 * RB_E * RB_ROW;                  // the planes' rows (24 KB)
constexpr int RB_STAGE = RB_XB + RB_WB;
constexpr int RB_RING = 3;
constexpr int RB_XL = RB_XB / 1024 / (RB_THREADS / 64);  // x loads per wave per stage (2)
constexpr int RB_WL = RB_WB / 1024 / (RB_THREADS / 64);  // plane loads per wave per stage (3)
static_assert(RB_XL == 2 && RB_WL == 3, "vmcnt below counts 5 loads per stage");

__device__ __forceinline__ int rb_swz(int row) { return (row >> 1) & 7; }

__global__ __launch_bounds__(RB_THREADS) void router_bf16x3(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ planes,
                                                           int T, int H, int E, int KS,
                                                           double* __restrict__ zpart) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[RB_RING * RB_STAGE];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int t0 = blockIdx.y * RB_MT, e0 = blockIdx.x * RB_E;
  const int hk = H / KS;  // a multiple of RB_K
  const int hbeg = blockIdx.z * hk;
  const size_t plane = (size_t)E * H;
  // load j of the wave: x rows 8 (RB_XL w + j) + lane/8, or plane unit
  // u = RB_WL w + j: plane u / 8, rows 8 (u % 8) + lane/8; lane i lands at
  // position i % 8 of its row, so it reads block (i % 8) ^ swz(row)
  const uint8_t* xsrc[RB_XL];
#pragma unroll
  for (int j = 0; j < RB_XL; ++j) {
    const int row = 8 * (RB_XL * wave + j) + (lane >> 3);
    const int b = (lane & 7) ^ rb_swz(row);
    xsrc[j] = reinterpret_cast<const uint8_t*>(x + (size_t)(t0 + row < T ? t0 + row : 0) * H +
                                               hbeg + 8 * b);
  }
  const uint8_t* wsrc[RB_WL];
#pragma unroll
  for (int j = 0; j < RB_WL; ++j) {
    const int u = RB_WL * wave + j, q = u >> 3, row = 8 * (u & 7) + (lane >> 3);
    const int b = (lane & 7) ^ rb_swz(row);
    wsrc[j] = reinterpret_cast<const uint8_t*>(planes + q * plane +
                                               (size_t)(e0 + row < E ? e0 + row : 0) * H + hbeg +
                                               8 * b);
  }
  const int nchunk = hk / RB_K;
  auto issue = [&](int c) {
    uint8_t* st = smem + (c % RB_RING) * RB_STAGE;
#pragma unroll
    for (int j = 0; j < RB_XL; ++j)
      dma16(xsrc[j] + (size_t)c * RB_ROW, st + (RB_XL * wave + j) * 1024);
#pragma unroll
    for (int j = 0; j < RB_WL; ++j)
      dma16(wsrc[j] + (size_t)c * RB_ROW, st + RB_XB + (RB_WL * wave + j) * 1024);
  };
  const int wr = wave >> 1, wcl = wave & 1;  // the wave's 32 x 32 tile
  const int r = lane & 31, hh = lane >> 5;
  const int swz = rb_swz(r);  // = swz(32 wr + r) = swz(32 wcl + r)
  v16f acc[3];
  double zs[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    acc[0][v] = 0.f;
    acc[1][v] = 0.f;
    acc[2][v] = 0.f;
    zs[v] = 0.0;
  }
  issue(0);
  if (nchunk > 1) issue(1);
  for (int c = 0; c < nchunk; ++c) {
    // after chunk c's loads only chunk c + 1's five may still be in flight
    if (c + 1 < nchunk)
      asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every wave's share landed; chunk c - 1's slot is free
    if (c + 2 < nchunk) issue(c + 2);
    const uint8_t* st = smem + (c % RB_RING) * RB_STAGE;
    const uint8_t* xa = st + (32 * wr + r) * RB_ROW;
    const uint8_t* wb = st + RB_XB + (32 * wcl + r) * RB_ROW;
#pragma unroll
    for (int s = 0; s < RB_K / 16; ++s) {
      const int pos = ((2 * s + hh) ^ swz) * 16;
      const v8bf a = *reinterpret_cast<const v8bf*>(xa + pos);
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const v8bf bq = *reinterpret_cast<const v8bf*>(wb + q * (RB_E * RB_ROW) + pos);
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq, acc[q], 0, 0, 0);
      }
    }
    // end of a 64-wide slice: w1's sum, then w2's, then w3's, into float64
#pragma unroll
    for (int v = 0; v < 16; ++v) {
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        zs[v] += (double)acc[q][v];
        acc[q][v] = 0.f;
      }
    }
  }
  // lane l, register v: token row 8(v/4) + 4(l/32) + v%4, expert column l%32
  const int e = e0 + 32 * wcl + r;
  if (e >= E) return;
  double* zp = zpart + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int t = t0 + 32 * wr + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (t < T) zp[(size_t)t * E + e] = zs[v];
  }
}

// Error constant of router_bf16x3: |z~ - z| <= kRouteBound * ||x_t|| * max ||w_e||
// (34 * 2^-24 * 4.04, raised by 1 % for the roundings of the norms and of
// the float64 additions).
constexpr double kRouteBound = 34.0 * 5.9604644775390625e-8 * 4.04 * 1.01;

// ---------------------------------------------------------------------------
// Per-token selection: one wave per token, expert e = lane + 64*i.
// ---------------------------------------------------------------------------
// NPER: experts per lane held in registers (4 for E <= 256, 16 for E <= 1024).

// Order-preserving map of a finite double to an unsigned key (larger z,
// larger key; every key of a finite value is nonzero).
__device__ __forceinline__ uint64_t order_key(double z) {
  const uint64_t u = (uint64_t)__double_as_longlong(z);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Top-k selection: the min(want, #allowed) allowed experts with the largest
// key, ties to the lower expert id (bit i of a lane's masks = expert
// lane+64i).  Each lane first sorts its allowed experts (key descending, ties
// to the lower i); a round then takes the wave maximum of the upper key words
// of the lanes' list heads, and the lane holding the winner drops its head.
// Only when several heads share that maximum are the lower words compared,
// and only when full keys tie does the lowest id decide (a lane's equal keys
// are already in id order, so the lowest id is always a head).
// The unrestricted and the masked selection share the rounds, so their two
// reductions overlap.
template <int NPER>
struct LaneList {
  uint32_t hi[NPER], lo[NPER];
  int idx[NPER];
  bool ok[NPER];
  int n;  // allowed experts of this lane not yet taken; entry 0 is the head
};

// Compare-exchange of entries A < B, placing first the one that goes first
// (FIRST_FIRST) or last: an allowed entry before a disallowed one, then the
// larger key, then the lower i.
template <int A, int B, bool FIRST_FIRST, int NPER>
__device__ __forceinline__ void lane_ce(LaneList<NPER>& L) {
  const uint64_t ka = ((uint64_t)L.hi[A] << 32) | L.lo[A];
  const uint64_t kb = ((uint64_t)L.hi[B] << 32) | L.lo[B];
  const bool a_first =
      (L.ok[A] != L.ok[B]) ? L.ok[A] : (ka != kb ? ka > kb : L.idx[A] < L.idx[B]);
  const bool sw = FIRST_FIRST ? !a_first : a_first;
  const uint32_t ha = L.hi[A], la = L.lo[A];
  const int ia = L.idx[A];
  const bool oa = L.ok[A];
  L.hi[A] = sw ? L.hi[B] : ha;
  L.lo[A] = sw ? L.lo[B] : la;
  L.idx[A] = sw ? L.idx[B] : ia;
  L.ok[A] = sw ? L.ok[B] : oa;
  L.hi[B] = sw ? ha : L.hi[B];
  L.lo[B] = sw ? la : L.lo[B];
  L.idx[B] = sw ? ia : L.idx[B];
  L.ok[B] = sw ? oa : L.ok[B];
}

// Bitonic sorting network over the NPER entries, generated at compile time
// so that every index is a constant (the lists stay in registers).
template <int NPER, int KK, int JJ, int A>
struct BitonicPass {
  __device__ static __forceinline__ void run(LaneList<NPER>& L) {
    if constexpr ((A ^ JJ) > A) lane_ce<A, (A ^ JJ), (A & KK) == 0, NPER>(L);
    if constexpr (A + 1 < NPER) BitonicPass<NPER, KK, JJ, A + 1>::run(L);
  }
};

template <int NPER, int KK, int JJ>
struct BitonicMerge {
  __device__ static __forceinline__ void run(LaneList<NPER>& L) {
    BitonicPass<NPER, KK, JJ, 0>::run(L);
    if constexpr (JJ > 1) BitonicMerge<NPER, KK, JJ / 2>::run(L);
  }
};

template <int NPER, int KK>
struct BitonicSort {
  __device__ static __forceinline__ void run(LaneList<NPER>& L) {
    BitonicMerge<NPER, KK, KK / 2>::run(L);
    if constexpr (KK < NPER) BitonicSort<NPER, KK * 2>::run(L);
  }
};

template <int NPER>
__device__ __forceinline__ void build_list(const uint64_t* key, uint32_t allowed,
                                           LaneList<NPER>& L) {
  L.n = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    L.ok[i] = (allowed >> i) & 1u;
    L.hi[i] = (uint32_t)(key[i] >> 32);
    L.lo[i] = (uint32_t)key[i];
    L.idx[i] = i;
    L.n += L.ok[i] ? 1 : 0;
  }
  BitonicSort<NPER, 2>::run(L);
}

template <int NPER>
__device__ __forceinline__ uint32_t head_hi(const LaneList<NPER>& L) {
  return L.n > 0 ? L.hi[0] : 0u;
}

// The winner among the heads whose upper word is `best` leaves its list (the
// lists shift down; all indices are static, so they stay in registers).
template <int NPER>
__device__ __forceinline__ void take_head(LaneList<NPER>& L, uint32_t best, uint32_t& sel) {
  const int lane = threadIdx.x & 63;
  bool hit = L.n > 0 && L.hi[0] == best;
  uint64_t b = __ballot(hit);
  int winner;
  if (__popcll(b) == 1) {
    winner = __builtin_ctzll(b);
  } else {  // uniform; ties in the upper word are rare
    // (the reductions run in every lane: never under a short-circuit)
    const uint32_t l = hit ? L.lo[0] : 0u;
    const uint32_t lb = wave_umax32(l);
    hit = hit && l == lb;
    b = __ballot(hit);
    if (__popcll(b) == 1) {
      winner = __builtin_ctzll(b);
    } else {  // equal keys: the lowest expert id (the maximum of ~id)
      const uint32_t ne = hit ? ~(uint32_t)(lane + 64 * L.idx[0]) : 0u;
      const uint32_t nmax = wave_umax32(ne);
      winner = (int)(~nmax & 63u);
    }
  }
  const bool won = lane == winner;
  sel |= won ? 1u << L.idx[0] : 0u;
#pragma unroll
  for (int i = 0; i + 1 < NPER; ++i) {
    L.hi[i] = won ? L.hi[i + 1] : L.hi[i];
    L.lo[i] = won ? L.lo[i + 1] : L.lo[i];
    L.idx[i] = won ? L.idx[i + 1] : L.idx[i];
  }
  L.n -= won ? 1 : 0;
}

template <int NPER>
__device__ __forceinline__ int count_allowed(uint32_t allowed) {
  int total = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) total += __popcll(__ballot((allowed >> i) & 1u));
  return total;
}

// do_u / do_m (uniform): which of the two selections to make.
template <int NPER>
__device__ void wave_select_pair(const uint64_t* key, uint32_t allow_u, uint32_t allow_m, int want,
                                 bool do_u, bool do_m, uint32_t& sel_u, uint32_t& sel_m,
                                 int& got_m) {
  LaneList<NPER> U, M;
  U.n = 0;
  M.n = 0;
  if (do_u) build_list<NPER>(key, allow_u, U);
  if (do_m) build_list<NPER>(key, allow_m, M);
  const int nu = do_u ? min(want, count_allowed<NPER>(allow_u)) : 0;
  const int nm = do_m ? min(want, count_allowed<NPER>(allow_m)) : 0;
  sel_u = 0u;
  sel_m = 0u;
  const int rounds = max(nu, nm);
  for (int j = 0; j < rounds; ++j) {
    uint32_t bu = head_hi<NPER>(U), bm = head_hi<NPER>(M);
    wave_umax32x2(bu, bm);
    if (j < nu) take_head<NPER>(U, bu, sel_u);
    if (j < nm) take_head<NPER>(M, bm, sel_m);
  }
  got_m = nm;
}

// Position of each selected expert in ascending-id order.
template <int NPER>
__device__ __forceinline__ void selected_positions(uint32_t sel, int nper, int* pos) {
  const uint64_t lt = lanemask_lt();
  int base = 0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    if (i < nper) {
      const uint64_t m = __ballot((sel >> i) & 1u);
      pos[i] = base + __popcll(m & lt);
      base += __popcll(m);
    }
  }
}

struct SelectArgs {
  double* z;  // [T][E] logits without bias
  const float* bias;
  const int32_t* expert_slot;
  const uint16_t* x;
  int T, H, E, k, S;
  int32_t* topk_expert;
  float* topk_score;
  int32_t* sel_expert;
  float* sel_weight;
  int32_t* sel_slot;
  uint8_t* xq;
  size_t xq_row;
  int quantize_x;   // encode the activation row here (else the router kernel did)
  int act_format;   // MOE_ACT_MXFP4 or MOE_ACT_MXFP6
  double* hist;     // nullable: demand accumulated by the one-workgroup kernel
  float* delta;
  // Logits from router_bf16x3 (nullable otherwise): token t is appended to
  // the list flags[1 ..] (count in flags[0], zeroed beforehand) when its k-th
  // and (k+1)-th logits, in either order (all experts; routable experts), lie
  // within twice the bound of each other, so its picks need float64 logits;
  // wnorm2: ||w_e||^2 per expert.
  int32_t* flags;
  double* cert;           // per token: k-th value (all experts), k-th (routable), bound
  const double* wnorm2;
  // nullable: select only the tokens tlist[1 .. tlist[0]] (the second pass)
  const int32_t* tlist;
  // nullable: router_bf16x3's KS partial sums [KS][T][E]; the selection adds
  // them in order (z = ((p0 + p1) + p2) + ...) and stores the sum in z
  const double* zpart;
  int KS;
};

// Routed picks of token t (bit i of msel: expert lane+64i), in ascending id,
// with weights renormalised over them; positions past `got` are padding.
template <int NPER>
__device__ __forceinline__ void select_write_routed(const SelectArgs& p, int t, uint32_t msel,
                                                    int got, const double* ex, double denom,
                                                    const int* slot_of) {
  const int lane = threadIdx.x & 63;
  const int k = p.k, nper = (p.E + 63) / 64;
  int pos[NPER];
  selected_positions<NPER>(msel, nper, pos);
  double psel = 0.0;
#pragma unroll
  for (int i = 0; i < NPER; ++i)
    if (i < nper && ((msel >> i) & 1u)) psel += ex[i] / denom;
  const double wsum = wave_sum(psel);
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    if (i < nper && ((msel >> i) & 1u)) {
      const size_t o = (size_t)t * k + pos[i];
      p.sel_expert[o] = lane + 64 * i;
      p.sel_weight[o] = (float)((ex[i] / denom) / wsum);
      p.sel_slot[o] = slot_of[i];
    }
  }
  for (int j = got + lane; j < k; j += 64) {
    const size_t o = (size_t)t * k + j;
    p.sel_expert[o] = -1;
    p.sel_weight[o] = 0.f;
    p.sel_slot[o] = -1;
  }
}

// Activation row of token t (when p.quantize_x): lane per 32-block, MXFP4 or
// MXFP6 (FP6; the kernels are instantiated per format, so each keeps the
// registers of its own encoder).  Returns ||x_t||^2 (float64 sums of exact squares,
// wave-uniform), or -1 when the row was not read.
template <bool FP6>
__device__ __forceinline__ double quantize_row(const SelectArgs& p, int t) {
  if (!p.quantize_x) return -1.0;
  const int lane = threadIdx.x & 63;
  const int H = p.H;
  const int nblk = H / 32;
  constexpr bool fp6 = FP6;
  const size_t sc_off = act_scale_offset(H, FP6 ? MOE_ACT_MXFP6 : MOE_ACT_MXFP4);
  const uint16_t* xr = p.x + (size_t)t * H;
  uint8_t* qr = p.xq + (size_t)t * p.xq_row;
  double sq = 0.0;
  for (int b = lane; b < nblk; b += 64) {
    const uint4* src = reinterpret_cast<const uint4*>(xr + b * 32);
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 u = src[q];
      const uint32_t wds[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[q * 8 + r * 2 + 0] = bf16_to_f32(wds[r] & 0xFFFFu);
        v[q * 8 + r * 2 + 1] = bf16_to_f32(wds[r] >> 16);
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      amax = fmaxf(amax, fabsf(v[i]));
      sq += (double)v[i] * (double)v[i];
    }
    uint32_t scale = 0u;
    if constexpr (fp6) {
      uint32_t words[6] = {0u, 0u, 0u, 0u, 0u, 0u};  // element i at bits [6i, 6i+6)
      if (amax > 0.f) {
        const int e = mx_block_exp(amax);
        scale = (uint32_t)(e + 127);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const uint32_t c = e2m3_code(v[i], e);
          words[(6 * i) >> 5] |= c << ((6 * i) & 31);
          if (((6 * i) & 31) > 26) words[((6 * i) >> 5) + 1] |= c >> (32 - ((6 * i) & 31));
        }
      }
      uint2* dst = reinterpret_cast<uint2*>(qr + (size_t)b * 24);  // 8-byte aligned
      dst[0] = make_uint2(words[0], words[1]);
      dst[1] = make_uint2(words[2], words[3]);
      dst[2] = make_uint2(words[4], words[5]);
    } else {
      uint32_t words[4] = {0u, 0u, 0u, 0u};
      if (amax > 0.f) {
        const int e = mx_block_exp(amax);
        scale = (uint32_t)(e + 127);
#pragma unroll
        for (int i = 0; i < 32; ++i) words[i >> 3] |= e2m1_code(v[i], e) << (4 * (i & 7));
      }
      *reinterpret_cast<uint4*>(qr + (size_t)b * 16) =
          make_uint4(words[0], words[1], words[2], words[3]);
    }
    qr[sc_off + b] = (uint8_t)scale;
  }
  return wave_sum(sq);
}

// Certification of token t's picks made on router_bf16x3's logits: the k-th
// and (k+1)-th values in both orders (z here includes the bias) must differ
// by more than twice the logits' error bound kRouteBound * ||x_t|| * max
// ||w_e||; otherwise the token is flagged for the exact float64 logits.
// ||x_t||^2 is summed in float64 from exact float32 squares.
template <int NPER>
__device__ void certify_token(const SelectArgs& p, int t, const double* z, uint32_t valid,
                              uint32_t routable, uint32_t usel, uint32_t msel, double xn2) {
  const int lane = threadIdx.x & 63;
  const int nper = (p.E + 63) / 64;
  double ku = INFINITY, nu = -INFINITY, km = INFINITY, nm = -INFINITY, wmax = 0.0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    if (i >= nper || !((valid >> i) & 1u)) continue;
    const double v = z[i];
    if ((usel >> i) & 1u) ku = fmin(ku, v); else nu = fmax(nu, v);
    if ((routable >> i) & 1u) {
      if ((msel >> i) & 1u) km = fmin(km, v); else nm = fmax(nm, v);
    }
    wmax = fmax(wmax, p.wnorm2[lane + 64 * i]);
  }
  ku = -wave_max(-ku);
  nu = wave_max(nu);
  km = -wave_max(-km);
  nm = wave_max(nm);
  wmax = wave_max(wmax);
  double xn = xn2;
  if (xn < 0.0) {  // the row was not read for the activation encoding
    const uint16_t* xr = p.x + (size_t)t * p.H;
    xn = 0.0;
    for (int h = 8 * lane; h < p.H; h += 512) {
      const uint4 u = *reinterpret_cast<const uint4*>(xr + h);
      const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double a = (double)bf16_to_f32(wd[q] & 0xFFFFu);
        const double b = (double)bf16_to_f32(wd[q] >> 16);
        xn += a * a + b * b;
      }
    }
    xn = wave_sum(xn);
  }
  const double bound = kRouteBound * sqrt(xn) * sqrt(wmax);
  // no (k+1)-th value (every candidate picked): nothing to certify in that order
  const bool close_u = nu != -INFINITY && !(ku - nu > 2.0 * bound);
  const bool close_m = nm != -INFINITY && !(km - nm > 2.0 * bound);
  if (lane == 0) {
    if (close_u || close_m) {
      // the list's order does not matter: every listed token is handled on its own
      const int slot = (int)atomicAdd(reinterpret_cast<unsigned*>(p.flags), 1u);
      p.flags[1 + slot] = t;
    }
    p.cert[3 * (size_t)t] = ku;
    p.cert[3 * (size_t)t + 1] = km;   // +inf when nothing is routable
    p.cert[3 * (size_t)t + 2] = bound;
  }
}

// What one wave does for its token: the demand picks (unrestricted top-k
// and scores), the routed picks (masked top-k, renormalised weights, slots),
// or both.  Each selection is a serial chain of rounds, so two waves that
// split them finish sooner than one wave doing both.
constexpr int kSelDemand = 1, kSelRouted = 2, kSelBoth = 3;

// One wave, token t.  Activation rows are encoded too when p.quantize_x.
template <int NPER, bool FP6>
__device__ void select_token(const SelectArgs& p, int t, int role) {
  const int lane = threadIdx.x & 63;
  const int E = p.E, k = p.k;
  const int nper = (E + 63) / 64;

  // ---- logits plus bias ----
  // every load is issued before the first use (lanes past E load expert
  // E - 1 and drop it): loads under the per-expert branch went one round trip
  // at a time
  double zl[NPER];
  float bl[NPER];
  int sl[NPER];
  // without a bias the loads read the (E-entry) slot table and are dropped:
  // a load under `if (bias)` made the compiler wait for it before the next
  const bool has_bias = p.bias != nullptr;
  const float* bsrc = has_bias ? p.bias : reinterpret_cast<const float*>(p.expert_slot);
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = min(lane + 64 * i, E - 1);
    zl[i] = p.zpart ? p.zpart[(size_t)t * E + e] : p.z[(size_t)t * E + e];
    bl[i] = bsrc[e];
    sl[i] = p.expert_slot[e];
  }
  if (p.zpart) {  // the K parts of router_bf16x3, added in order and kept in z
    const size_t part = (size_t)p.T * E;
    for (int q = 1; q < p.KS; ++q) {
#pragma unroll
      for (int i = 0; i < NPER; ++i)
        zl[i] += p.zpart[q * part + (size_t)t * E + min(lane + 64 * i, E - 1)];
    }
#pragma unroll
    for (int i = 0; i < NPER; ++i)
      if (lane + 64 * i < E) p.z[(size_t)t * E + lane + 64 * i] = zl[i];
  }
#pragma unroll
  for (int i = 0; i < NPER; ++i) bl[i] = has_bias ? bl[i] : 0.f;
  double z[NPER];
  uint32_t valid = 0, routable = 0;
  int slot_of[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    z[i] = -INFINITY;
    slot_of[i] = -1;
    const int e = lane + 64 * i;
    if (i < nper && e < E) {
      z[i] = zl[i] + (double)bl[i];
      valid |= 1u << i;
      const int s = sl[i];
      if (s >= 0 && s < p.S) {
        routable |= 1u << i;
        slot_of[i] = s;
      }
    }
  }

  // ---- softmax over all experts (float64) ----
  double m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NPER; ++i)
    if (i < nper) m = fmax(m, z[i]);
  m = wave_max(m);
  double ex[NPER];
  double lsum = 0.0;
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    ex[i] = 0.0;
    if (i < nper && ((valid >> i) & 1u)) {
      ex[i] = exp(z[i] - m);
      lsum += ex[i];
    }
  }
  const double denom = wave_sum(lsum);

  // ---- selections: demand picks (all experts), routed picks (routable) ----
  uint64_t key[NPER];
#pragma unroll
  for (int i = 0; i < NPER; ++i) key[i] = order_key(z[i] + 0.0);  // -0 and +0 tie
  const bool do_u = role & kSelDemand, do_m = role & kSelRouted;
  uint32_t usel = 0, msel = 0;
  int got = 0;
  wave_select_pair<NPER>(key, valid, routable, k, do_u, do_m, usel, msel, got);
  int pos[NPER];
  if (do_u) {
    selected_positions<NPER>(usel, nper, pos);
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
      if (i < nper && ((usel >> i) & 1u)) {
        const size_t o = (size_t)t * k + pos[i];
        p.topk_expert[o] = lane + 64 * i;
        p.topk_score[o] = (float)(ex[i] / denom);
      }
    }
  }
  if (do_m) select_write_routed<NPER>(p, t, msel, got, ex, denom, slot_of);
  double xn2 = -1.0;
  if (role & kSelRouted) xn2 = quantize_row<FP6>(p, t);
  if (p.flags && role == kSelBoth) certify_token<NPER>(p, t, z, valid, routable, usel, msel, xn2);
}

template <int NPER, bool FP6>
__global__ __launch_bounds__(256) void route_select(SelectArgs p) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (!p.tlist) {
    if (i < p.T) select_token<NPER, FP6>(p, i, kSelBoth);  // wave-uniform
    return;
  }
  const int n = p.tlist[0];  // a fixed grid walks the list
  for (int j = i; j < n; j += gridDim.x * 4)
    select_token<NPER, FP6>(p, p.tlist[1 + j], kSelBoth);
}

// ---------------------------------------------------------------------------
// Bucketing.  Counts per slot, exclusive offsets, and a stable scatter
// (ascending assignment index within a slot).
// ---------------------------------------------------------------------------

// Batches of up to kFusedMaxT tokens (E <= 256, small-T router): selection,
// demand and bucketing in one launch.  Workgroup b selects tokens 2b and
// 2b+1, two waves each (one per SIMD): one for the demand picks, one for the
// routed picks.  Each workgroup then counts itself done on a
// counter that the router kernel of the same call set to zero; the last one
// reads every token's picks back and does the demand update and the
// bucketing alone.  Both bucket picks with 64-bit token masks -- demand picks
// by expert, routed picks by slot (a token picks an expert, and a slot, at
// most once) -- so a pick's rank in its bucket is the number of earlier
// tokens in the mask.  Expert e's demand: its bucket of scores added in
// ascending token order -- the float64 additions of moe_demand_accumulate.
constexpr int kFusedMaxT = 64;
constexpr int kFusedWgTokens = 2;
constexpr int kFusedMaxA = kFusedMaxT * MOE_MAX_K;

// One DPP step of an inclusive wave scan: adds the value of the lane that
// CTRL names (0 where it names none, or in rows outside ROW_MASK).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int scan_add(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive scans of two values over the wave: shifts 1, 2, 4, 8 within rows
// of 16 lanes (row_shr), then row 15 into rows 1 and 3 and lane 31 into rows
// 2 and 3 (row_bcast), steps of the two scans interleaved.
__device__ __forceinline__ void wave_inclusive_scan2(int& a, int& b) {
  a = scan_add<0x111, 0xF>(a);  // row_shr:1
  b = scan_add<0x111, 0xF>(b);
  a = scan_add<0x112, 0xF>(a);  // row_shr:2
  b = scan_add<0x112, 0xF>(b);
  a = scan_add<0x114, 0xF>(a);  // row_shr:4
  b = scan_add<0x114, 0xF>(b);
  a = scan_add<0x118, 0xF>(a);  // row_shr:8
  b = scan_add<0x118, 0xF>(b);
  a = scan_add<0x142, 0xA>(a);  // row_bcast:15
  b = scan_add<0x142, 0xA>(b);
  a = scan_add<0x143, 0xC>(a);  // row_bcast:31
  b = scan_add<0x143, 0xC>(b);
}

// Exclusive scans of two values (one of each per thread) over the
// workgroup's 256 threads; `part` holds 8 ints of LDS.  Returns the thread's
// offsets in a and b and the totals in ta and tb.  Ends with a barrier.
__device__ __forceinline__ void wg256_exclusive_scan2(int& a, int& b, int* part, int& ta,
                                                      int& tb) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int ia = a, ib = b;
  wave_inclusive_scan2(ia, ib);
  if (lane == 63) {
    part[wv] = ia;
    part[4 + wv] = ib;
  }
  __syncthreads();
  int ra = ia - a, rb = ib - b;
  for (int i = 0; i < wv; ++i) {
    ra += part[i];
    rb += part[4 + i];
  }
  ta = part[0] + part[1] + part[2] + part[3];
  tb = part[4] + part[5] + part[6] + part[7];
  __syncthreads();
  a = ra;
  b = rb;
}

__global__ __launch_bounds__(256) void route_fused(SelectArgs p, uint32_t* __restrict__ counter,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ perm) {
  __shared__ unsigned long long smask[MOE_MAX_S];  // tokens routed to slot s
  __shared__ unsigned long long emask[256];        // tokens with a demand pick of expert e
  __shared__ int off[MOE_MAX_S];                   // first perm position of slot s
  __shared__ int eoff[256];                        // first bucket position of expert e
  __shared__ int te[kFusedMaxA];
  __shared__ float ts[kFusedMaxA];
  __shared__ int sl[kFusedMaxA];
  __shared__ float elist[kFusedMaxA];  // demand scores bucketed by expert
  __shared__ int part[8];
  __shared__ int last;
  const int tid = threadIdx.x;
  const int T = p.T, k = p.k, E = p.E, S = p.S, A = T * k;
  double h_old = 0.0;
  if (p.hist && tid < E) h_old = p.hist[tid];  // used only by the last workgroup
  // waves 2j and 2j+1: demand and routed picks of token kFusedWgTokens*b + j
  const int t = blockIdx.x * kFusedWgTokens + (tid >> 7);
  // the small router encodes x (quantize_x is 0 here): the MXFP4 instance serves both formats
  if (t < T) select_token<4, false>(p, t, (tid >> 6) & 1 ? kSelRouted : kSelDemand);
  __threadfence();  // this workgroup's picks, visible device-wide before it counts itself
  __syncthreads();
  if (tid == 0) last = atomicAdd(counter, 1u) == gridDim.x - 1;
  __syncthreads();
  if (!last) return;
  __threadfence();  // every other workgroup's picks

  for (int a = tid; a < A; a += 256) {
    te[a] = p.topk_expert[a];
    ts[a] = p.topk_score[a];
    sl[a] = p.sel_slot[a];
  }
  for (int s = tid; s < S; s += 256) smask[s] = 0ull;
  emask[tid] = 0ull;
  __syncthreads();
  for (int a = tid; a < A; a += 256) {
    const unsigned long long bit = 1ull << (a / k);
    const int e = te[a], s = sl[a];
    if (e >= 0 && e < E) atomicOr(&emask[e], bit);
    if (s >= 0 && s < S) atomicOr(&smask[s], bit);
  }
  __syncthreads();

  // ---- bucket offsets: experts one per thread, slots a range per thread ----
  const int ecount = tid < E ? __popcll(emask[tid]) : 0;
  const int per = (S + 255) / 256;
  const int lo = min(S, tid * per), hi = min(S, lo + per);
  int local = 0;
  for (int s = lo; s < hi; ++s) local += __popcll(smask[s]);
  int eo = ecount, run = local, etot, total;
  wg256_exclusive_scan2(eo, run, part, etot, total);
  eoff[tid] = eo;
  for (int s = lo; s < hi; ++s) {
    off[s] = run;
    offsets[s] = run;
    run += __popcll(smask[s]);
  }
  if (tid == 0) offsets[S] = total;
  __syncthreads();

  // ---- place: demand scores by expert, assignments by slot ----
  for (int a = tid; a < A; a += 256) {
    const unsigned long long before = (1ull << (a / k)) - 1ull;
    const int e = te[a], s = sl[a];
    if (e >= 0 && e < E) elist[eoff[e] + __popcll(emask[e] & before)] = ts[a];
    if (s >= 0 && s < S) perm[off[s] + __popcll(smask[s] & before)] = a;
  }
  for (int a = total + tid; a < A; a += 256) perm[a] = -1;
  __syncthreads();

  // ---- demand ----
  if (p.hist && tid < E) {
    double acc = 0.0;
    const int b0 = eoff[tid];
    for (int q = 0; q < ecount; ++q) acc += (double)elist[b0 + q];
    p.hist[tid] = h_old + acc;
    if (p.delta) p.delta[tid] = (float)acc;
  }
}

// Bucketing for larger batches, stable by (slot, assignment).  The k picks of
// a token lie in distinct slots (distinct routable experts have distinct
// slots), so within a slot the assignments of a chunk of 64 tokens are
// ordered by token, and a token's rank among them is the number of the
// chunk's earlier tokens whose bit is set in the slot's 64-bit token mask.
constexpr int kBucketChunk = 64;

// Token mask of every slot for chunk blockIdx.x, in LDS (S 64-bit words).
__device__ void chunk_token_masks(const int32_t* __restrict__ sel_slot, int T, int k, int S,
                                  unsigned long long* bits) {
  const int c = blockIdx.x, t0 = c * kBucketChunk;
  const int n = min(kBucketChunk, T - t0) * k;
  for (int s = threadIdx.x; s < S; s += blockDim.x) bits[s] = 0ull;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int s = sel_slot[(size_t)t0 * k + i];
    if (s >= 0 && s < S) atomicOr(&bits[s], 1ull << (i / k));
  }
  __syncthreads();
}

// counts[s * nchunk + c] = tokens of chunk c with a pick in slot s.
__global__ __launch_bounds__(256) void bucket_hist(const int32_t* __restrict__ sel_slot, int T,
                                                   int k, int S, int nchunk,
                                                   int32_t* __restrict__ counts) {
  extern __shared__ unsigned long long bits[];
  chunk_token_masks(sel_slot, T, k, S, bits);
  for (int s = threadIdx.x; s < S; s += blockDim.x)
    counts[(size_t)s * nchunk + blockIdx.x] = __popcll(bits[s]);
}

// bucket_hist with, first, the demand partial of the same chunk of tokens
// (E <= kDemandTableE): part[c][e] as moe_demand_accumulate's chunk sums.  The
// dynamic LDS (max(kDemandTableBytes, S * 8) bytes) holds the score table,
// then the token masks.
__global__ __launch_bounds__(256) void bucket_hist_demand(const int32_t* __restrict__ sel_slot,
                                                          int T, int k, int S, int nchunk,
                                                          int32_t* __restrict__ counts,
                                                          const int32_t* __restrict__ te,
                                                          const float* __restrict__ ts, int E,
                                                          double* __restrict__ part) {
  extern __shared__ unsigned long long bits[];
  demand_chunk_table(te, ts, T, k, E, blockIdx.x, reinterpret_cast<float(*)[kDemandTableE]>(bits),
                     part, nullptr, nullptr);
  __syncthreads();  // the table's last reads before the masks overwrite it
  chunk_token_masks(sel_slot, T, k, S, bits);
  for (int s = threadIdx.x; s < S; s += blockDim.x)
    counts[(size_t)s * nchunk + blockIdx.x] = __popcll(bits[s]);
}

// One workgroup: offsets = exclusive scan of the slot totals (S+1 entries),
// and counts[s][c] replaced by the first perm position of chunk c's
// assignments in slot s.  perm entries past the total are set to -1.  When
// the S x nchunk counts fit kScanLdsInts, they are first copied to LDS with
// every load of a thread's batch issued before its stores (one round trip
// per batch of 8), and a wave handles one slot at a time from LDS (lanes over
// chunks).  Otherwise, with few chunks a thread walks whole slots in global
// memory; with many, a wave handles one slot at a time.  One pass of 1024
// threads scans the totals.
constexpr int kScanWaveMinChunks = 16;
constexpr int kScanLdsInts = 24 * 1024;  // counts staged in LDS (dynamic, 96 KB at most)

__global__ __launch_bounds__(1024) void bucket_scan(int32_t* __restrict__ counts, int S,
                                                    int nchunk, int A,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ perm) {
  __shared__ int tot[MOE_MAX_S];
  __shared__ int wsum[16];
  extern __shared__ int cl[];  // staged counts, when they fit
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ncount = S * nchunk;
  const bool staged = ncount > 0 && ncount <= kScanLdsInts;
  const bool by_wave = staged || nchunk >= kScanWaveMinChunks;
  if (staged) {
    for (int i0 = 0; i0 < ncount; i0 += 8 * 1024) {
      int v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = counts[min(i0 + j * 1024 + tid, ncount - 1)];
#pragma unroll
      for (int j = 0; j < 8; ++j) cl[min(i0 + j * 1024 + tid, ncount - 1)] = v[j];  // same value
    }
    __syncthreads();
  }
  // count c of slot s, from LDS when staged
  auto cnt = [&](int s, int c) { return staged ? cl[s * nchunk + c] : counts[(size_t)s * nchunk + c]; };
  if (by_wave) {
    for (int s = wv; s < S; s += 16) {
      int v = 0;
      for (int c = lane; c < nchunk; c += 64) v += cnt(s, c);
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
      if (lane == 0) tot[s] = v;
    }
  } else {
    for (int s = tid; s < S; s += 1024) {
      const int32_t* cs = counts + (size_t)s * nchunk;
      int v = 0;
      for (int c = 0; c < nchunk; ++c) v += cs[c];
      tot[s] = v;
    }
  }
  __syncthreads();
  const int per = (S + 1023) / 1024;
  const int lo = min(S, tid * per), hi = min(S, lo + per);
  int local = 0;
  for (int s = lo; s < hi; ++s) local += tot[s];
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
    const int n = tot[s];
    tot[s] = run;  // exclusive offset of slot s
    offsets[s] = run;
    run += n;
  }
  int total = 0;
  for (int i = 0; i < 16; ++i) total += wsum[i];
  if (tid == 0) offsets[S] = total;
  __syncthreads();
  if (by_wave) {
    for (int s = wv; s < S; s += 16) {
      int32_t* cs = counts + (size_t)s * nchunk;
      int carry = tot[s];
      for (int c0 = 0; c0 < nchunk; c0 += 64) {
        const int c = c0 + lane;
        const int v = c < nchunk ? cnt(s, c) : 0;
        int inc = v;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int o = __shfl_up(inc, d, kWave);
          if (lane >= d) inc += o;
        }
        if (c < nchunk) cs[c] = carry + inc - v;
        carry += __shfl(inc, 63, kWave);
      }
    }
  } else {
    for (int s = tid; s < S; s += 1024) {
      int32_t* cs = counts + (size_t)s * nchunk;
      int b = tot[s];
      for (int c = 0; c < nchunk; ++c) {
        const int n = cs[c];
        cs[c] = b;
        b += n;
      }
    }
  }
  for (int a = total + tid; a < A; a += 1024) perm[a] = -1;
}

// perm[base[s][c] + rank] = a for every assignment a of chunk c in slot s.
__global__ __launch_bounds__(256) void bucket_place(const int32_t* __restrict__ sel_slot, int T,
                                                    int k, int S, int nchunk,
                                                    const int32_t* __restrict__ base,
                                                    int32_t* __restrict__ perm) {
  extern __shared__ unsigned long long bits[];
  chunk_token_masks(sel_slot, T, k, S, bits);
  const int c = blockIdx.x, t0 = c * kBucketChunk;
  const int n = min(kBucketChunk, T - t0) * k;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int s = sel_slot[(size_t)t0 * k + i];
    if (s >= 0 && s < S) {
      const int tl = i / k;
      const int rank = __popcll(bits[s] & ((1ull << tl) - 1ull));
      perm[base[(size_t)s * nchunk + c] + rank] = t0 * k + i;
    }
  }
}

// Placement with the scan folded in, for count tables of at most
// kFusedScanMaxInts entries and S <= kFusedScanMaxS: every workgroup reads
// the whole S x nchunk table (slot totals, and per slot the counts of the
// chunks before its own), scans the totals, and places its chunk's
// assignments at offsets[s] + (earlier chunks of s) + rank.  Workgroup 0
// writes offsets; perm positions past the total are set to -1, spread over
// the workgroups.  Same perm and offsets as bucket_scan then bucket_place.
// With dpart non-null the grid has one more workgroup, which finishes the
// demand from the chunk partials that bucket_hist_demand wrote.
constexpr int kFusedScanMaxS = 2048;
constexpr int kFusedScanMaxInts = 32 * 1024;

__global__ __launch_bounds__(256) void bucket_place_scan(const int32_t* __restrict__ sel_slot,
                                                         int T, int k, int S, int nchunk, int A,
                                                         const int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ perm,
                                                         const double* __restrict__ dpart, int E,
                                                         double* __restrict__ hist,
                                                         float* __restrict__ delta) {
  if (blockIdx.x == nchunk) {
    // the extra workgroup (launched when dpart is non-null): the demand's
    // chunk partials added into hist
    demand_finalize_sums(dpart, nchunk, E, hist, delta);
    return;
  }
  extern __shared__ unsigned long long bits[];  // S token masks, then tot[S], pre[S]
  int* tot = reinterpret_cast<int*>(bits + S);
  int* pre = tot + S;
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = blockIdx.x;
  for (int s = tid; s < S; s += 256) {
    const int32_t* cs = counts + (size_t)s * nchunk;
    int ts = 0, ps = 0;
#pragma unroll 8
    for (int q = 0; q < nchunk; ++q) {
      const int v = cs[q];
      ts += v;
      ps += q < c ? v : 0;
    }
    tot[s] = ts;
    pre[s] = ps;
  }
  chunk_token_masks(sel_slot, T, k, S, bits);  // begins and ends with a barrier
  // exclusive scan of the totals: thread tid owns slots [lo, hi)
  const int per = (S + 255) / 256;
  const int lo = min(S, tid * per), hi = min(S, lo + per);
  int local = 0;
  for (int s = lo; s < hi; ++s) local += tot[s];
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
  const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  for (int s = lo; s < hi; ++s) {
    const int n = tot[s];
    tot[s] = run;  // exclusive offset of slot s
    if (c == 0) offsets[s] = run;
    run += n;
  }
  if (c == 0 && tid == 0) offsets[S] = total;
  __syncthreads();
  const int t0 = c * kBucketChunk;
  const int n = min(kBucketChunk, T - t0) * k;
  for (int i = tid; i < n; i += 256) {
    const int s = sel_slot[(size_t)t0 * k + i];
    if (s >= 0 && s < S) {
      const int tl = i / k;
      const int rank = __popcll(bits[s] & ((1ull << tl) - 1ull));
      perm[tot[s] + pre[s] + rank] = t0 * k + i;
    }
  }
  for (int a = total + c * 256 + tid; a < A; a += nchunk * 256) perm[a] = -1;
}

__global__ void fill_i32(int32_t* p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace moe

using namespace moe;

size_t moe_demand_ws_bytes_internal(int T, int E);
int moe_demand_launch_internal(const int32_t* te, const float* ts, int T, int k, int E,
                               double* hist, float* delta, void* ws, hipStream_t stream);

// Workspace: float64 logits [T][E], then the demand partials of the batch.
static size_t route_z_bytes(int T, int E) { return up_to((size_t)T * E * sizeof(double), 256); }

// Per-(slot, chunk) bucket counts of the larger-batch bucketing.
static size_t route_bucket_bytes(int T, int S) {
  const size_t nchunk = (size_t)(T + kBucketChunk - 1) / kBucketChunk;
  return up_to(nchunk * (size_t)(S > 0 ? S : 1) * sizeof(int32_t), 256);
}

// The certified path (router_bf16x3): ||w_e||^2 [E] float64, flags [T] int32
// and the flagged-token list [1 + T] int32.
// K parts of router_bf16x3 (1, 2, 4 or 8, each a whole number of 64-wide
// slices): one workgroup runs per CU (its LDS ring takes 135 KB), so the
// split that keeps the most of the 256 CUs busy over the launch's rounds,
// the fewest parts among equals.
static int route_ksplit(int T, int H, int E) {
  const long tiles = (long)((T + 127) / 128) * ((E + 63) / 64);
  int best = 1;
  double best_use = 0.0;
  for (int ks = 1; ks <= 8 && (H / ks) % 64 == 0 && H % ks == 0; ks *= 2) {
    const long wgs = tiles * ks;
    const double use = (double)wgs / (256.0 * (double)((wgs + 255) / 256));
    if (use > best_use + 1e-9) {
      best = ks;
      best_use = use;
    }
  }
  return best;
}

// H a multiple of 512: whole 64-wide slices, and whole 16-byte x loads for each
// lane's H/64 elements in router_f64_candidates.
static bool route_approx(int T, int H) {
  return T > kSplitRouterMaxT && H % 512 == 0 && H / kRouterChunk <= RS_MAX_CHUNKS;
}
static size_t route_cert_bytes(int T, int H, int E) {
  return up_to((size_t)E * sizeof(double), 256) +
         up_to((size_t)(T + 1) * sizeof(int32_t), 256) +   // flagged tokens: count, ids
         up_to((size_t)3 * E * H * sizeof(uint16_t), 256) +  // the bf16 planes of w
         up_to((size_t)3 * T * sizeof(double), 256) +         // per token: k-th values, bound
         up_to((size_t)route_ksplit(T, H, E) * T * E * sizeof(double), 256);  // K parts of z
}

static size_t route_ws_bytes(int T, int H, int E, int S) {
  if (T <= 0) return 0;
  return route_z_bytes(T, E) + moe_demand_ws_bytes_internal(T, E) + route_bucket_bytes(T, S) +
         (route_approx(T, H) ? route_cert_bytes(T, H, E) : 0);
}

size_t moe_route_ws_bytes_internal(int T, int H, int E, int S) {
  return route_ws_bytes(T, H, E, S);
}

extern "C" MOE_EXPORT int moe_route(const moe_route_args* a, hipStream_t stream) {
  if (!a) return MOE_EINVAL;
  const int T = a->T, H = a->H, E = a->E, k = a->k, S = a->S;
  if (T < 0 || H <= 0 || E <= 0 || k <= 0 || S < 0) return MOE_EINVAL;
  if (H % 32 != 0 || k > MOE_MAX_K || k > E || E > MOE_MAX_E || S > MOE_MAX_S)
    return MOE_EUNSUPPORTED;
  if ((size_t)T * k > (size_t)INT32_MAX || (size_t)T * H > ((size_t)1 << 40)) return MOE_EINVAL;
  if (!a->slot_offsets) return MOE_EINVAL;
  if (a->hist_row && !aligned(a->hist_row, 8)) return MOE_EINVAL;
  if (a->act_format != MOE_ACT_MXFP4 && a->act_format != MOE_ACT_MXFP6) return MOE_EINVAL;
  if (T > 0) {
    if (!a->x || !a->w_router || !a->expert_slot || !a->topk_expert || !a->topk_score ||
        !a->sel_expert || !a->sel_weight || !a->sel_slot || !a->perm || !a->xq)
      return MOE_EINVAL;
    if (!aligned(a->x, 16) || !aligned(a->w_router, 16) || !aligned(a->xq, 16)) return MOE_EINVAL;
    const size_t need = route_ws_bytes(T, H, E, S);
    if (a->ws_bytes < need) return MOE_EWORKSPACE;
    if (need > 0 && (!a->ws || !aligned(a->ws, 256))) return MOE_EINVAL;
  }

  if (T == 0) {
    fill_i32<<<(S + 1 + 255) / 256, 256, 0, stream>>>(a->slot_offsets, S + 1, 0);
    if (a->hist_row && a->delta)
      fill_i32<<<(E + 255) / 256, 256, 0, stream>>>((int32_t*)a->delta, E, 0);
    return hip_status();
  }
  hipEvent_t* ev = a->stage_events;
  double* z = static_cast<double*>(a->ws);
  void* dws = static_cast<uint8_t*>(a->ws) + route_z_bytes(T, E);
  const int nchunk = H / kRouterChunk;
  const int fmt = a->act_format;
  const size_t xq_row = act_row_bytes(H, fmt);
  const bool small_router = T <= kSplitRouterMaxT && nchunk <= RS_MAX_CHUNKS;
  // the fused kernel's completion counter: the first word of the bucket-count
  // area, which that path does not use otherwise
  const bool fused = small_router && T <= kFusedMaxT && E <= 256;
  uint32_t* counter = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(a->ws) +
                                                  route_z_bytes(T, E) +
                                                  moe_demand_ws_bytes_internal(T, E));
  const bool approx = !small_router && route_approx(T, H);
  uint8_t* cert = static_cast<uint8_t*>(a->ws) + route_z_bytes(T, E) +
                  moe_demand_ws_bytes_internal(T, E) + route_bucket_bytes(T, S);
  double* wnorm2 = reinterpret_cast<double*>(cert);
  int32_t* flags = reinterpret_cast<int32_t*>(cert + up_to((size_t)E * sizeof(double), 256));
  uint16_t* planes = reinterpret_cast<uint16_t*>(
      reinterpret_cast<uint8_t*>(flags) + up_to((size_t)(T + 1) * sizeof(int32_t), 256));
  double* cert_info = reinterpret_cast<double*>(
      reinterpret_cast<uint8_t*>(planes) + up_to((size_t)3 * E * H * sizeof(uint16_t), 256));
  double* zpart = reinterpret_cast<double*>(reinterpret_cast<uint8_t*>(cert_info) +
                                            up_to((size_t)3 * T * sizeof(double), 256));
  const int ks = route_ksplit(T, H, E);
  if (!record_stage(ev,0, stream)) return MOE_EHIP;
  if (a->reuse_logits) {
    // z and xq stay from the previous call; only the fused kernel's counter,
    // which the router would zero, and the flagged-token count need clearing
    if (fused) fill_i32<<<1, 256, 0, stream>>>(reinterpret_cast<int32_t*>(counter), 1, 0);
    if (approx) fill_i32<<<1, 256, 0, stream>>>(flags, 1, 0);
  } else if (small_router) {
    const int nrb = E * ((T + RS_T - 1) / RS_T);
    const size_t nx = ((size_t)T * H + 255) / 256;
    const int nxb = (int)(nx < 1024 ? nx : 1024);
    if (nchunk <= 128)
      router_small_f64<true><<<nrb + nxb, 256, 0, stream>>>(a->x, a->w_router, T, H, E, z, a->xq,
                                                            xq_row, fmt, nrb,
                                                            fused ? counter : nullptr);
    else
      router_small_f64<false><<<nrb + nxb, 256, 0, stream>>>(a->x, a->w_router, T, H, E, z,
                                                             a->xq, xq_row, fmt, nrb,
                                                             fused ? counter : nullptr);
  } else if (approx) {
    split_w_bf16x3<<<E, 256, 0, stream>>>(a->w_router, E, H, planes, wnorm2, flags);
    router_bf16x3<<<dim3((E + RB_E - 1) / RB_E, (T + RB_MT - 1) / RB_MT, ks), RB_THREADS, 0,
                    stream>>>(a->x, planes, T, H, E, ks, zpart);
  } else {
    dim3 grid((E + RM_E - 1) / RM_E, (T + RM_T - 1) / RM_T);
    router_full_f64<<<grid, 256, 0, stream>>>(a->x, a->w_router, T, H, E, z, nullptr);
  }
  if (!record_stage(ev,1, stream)) return MOE_EHIP;
  SelectArgs p;
  p.z = z;
  p.bias = a->bias;
  p.expert_slot = a->expert_slot;
  p.x = a->x;
  p.T = T;
  p.H = H;
  p.E = E;
  p.k = k;
  p.S = S;
  p.topk_expert = a->topk_expert;
  p.topk_score = a->topk_score;
  p.sel_expert = a->sel_expert;
  p.sel_weight = a->sel_weight;
  p.sel_slot = a->sel_slot;
  p.xq = a->xq;
  p.xq_row = xq_row;
  p.quantize_x = (small_router || a->reuse_logits) ? 0 : 1;
  p.act_format = fmt;
  p.hist = nullptr;
  p.delta = nullptr;
  p.flags = approx ? flags : nullptr;
  p.cert = cert_info;
  p.zpart = (approx && !a->reuse_logits) ? zpart : nullptr;
  p.KS = ks;
  p.wnorm2 = wnorm2;
  p.tlist = nullptr;
  const int A = T * k;
  if (fused) {
    // selection, demand and bucketing in one kernel; the remaining stage
    // events are recorded back to back
    p.hist = a->hist_row;
    p.delta = a->delta;
    route_fused<<<(T + kFusedWgTokens - 1) / kFusedWgTokens, 256, 0, stream>>>(
        p, counter, a->slot_offsets, a->perm);
    for (int i = 2; i <= 4; ++i)
      if (!record_stage(ev,i, stream)) return MOE_EHIP;
    return hip_status();
  }
  const bool fp6 = fmt == MOE_ACT_MXFP6;
  auto launch_select = [&](unsigned nwg) {
    if (E <= 256) {
      if (fp6) route_select<4, true><<<nwg, 256, 0, stream>>>(p);
      else route_select<4, false><<<nwg, 256, 0, stream>>>(p);
    } else {
      if (fp6) route_select<16, true><<<nwg, 256, 0, stream>>>(p);
      else route_select<16, false><<<nwg, 256, 0, stream>>>(p);
    }
  };
  launch_select((unsigned)((T + 3) / 4));
  if (approx) {
    // the flagged tokens: exact float64 logits, then their picks again (the
    // grids are sized for every token; workgroups past the list leave at once)
    router_f64_candidates<<<T < 2048 ? T : 2048, 256, 0, stream>>>(
        a->x, a->w_router, a->bias, a->expert_slot, H, E, S, z, flags, cert_info);
    p.flags = nullptr;
    p.zpart = nullptr;   // z now holds the sums, with the float64 candidates
    p.tlist = flags;
    p.quantize_x = 0;
    const int nwg = (T + 3) / 4 < 512 ? (T + 3) / 4 : 512;
    launch_select((unsigned)nwg);
  }
  const int nbc = (T + kBucketChunk - 1) / kBucketChunk;
  const bool fused_scan =
      S > 0 && S <= kFusedScanMaxS && (size_t)S * nbc <= (size_t)kFusedScanMaxInts;
  // the demand's chunk sums ride on the bucket counting, its final sums on
  // the placement (same chunks of 64 tokens; same float64 sums and order)
  const bool demand_in_buckets = a->hist_row && fused_scan && E <= kDemandTableE &&
                                 T > kDemandChunk && kDemandChunk == kBucketChunk;
  if (a->hist_row && !demand_in_buckets) {
    const int st = moe_demand_launch_internal(a->topk_expert, a->topk_score, T, k, E, a->hist_row,
                                              a->delta, dws, stream);
    if (st != MOE_OK) return st;
  }
  if (!record_stage(ev,2, stream)) return MOE_EHIP;
  int32_t* counts = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(a->ws) + route_z_bytes(T, E) +
                                               moe_demand_ws_bytes_internal(T, E));
  const size_t mask_lds = (size_t)(S > 0 ? S : 1) * sizeof(unsigned long long);
  double* dpart = demand_in_buckets ? static_cast<double*>(dws) : nullptr;
  if (demand_in_buckets)
    bucket_hist_demand<<<nbc, 256, std::max(mask_lds, kDemandTableBytes), stream>>>(
        a->sel_slot, T, k, S, nbc, counts, a->topk_expert, a->topk_score, E, dpart);
  else if (S > 0)
    bucket_hist<<<nbc, 256, mask_lds, stream>>>(a->sel_slot, T, k, S, nbc, counts);
  if (fused_scan) {
    // small count tables: every placement workgroup scans them itself
    if (!record_stage(ev,3, stream)) return MOE_EHIP;
    bucket_place_scan<<<nbc + (dpart ? 1 : 0), 256, (size_t)S * 16, stream>>>(
        a->sel_slot, T, k, S, nbc, A, counts, a->slot_offsets, a->perm, dpart, E, a->hist_row,
        a->delta);
  } else {
    const size_t scan_lds =
        (size_t)S * nbc <= (size_t)kScanLdsInts ? (size_t)S * nbc * sizeof(int32_t) : 0;
    bucket_scan<<<1, 1024, scan_lds, stream>>>(counts, S, nbc, A, a->slot_offsets, a->perm);
    if (!record_stage(ev,3, stream)) return MOE_EHIP;
    if (S > 0)
      bucket_place<<<nbc, 256, mask_lds, stream>>>(a->sel_slot, T, k, S, nbc, counts, a->perm);
  }
  if (!record_stage(ev,4, stream)) return MOE_EHIP;
  return hip_status();
}
