// moe_route: router logits, demand picks, masked top-k, renormalisation,
// token-to-slot bucketing and MXFP4 activation rows (gfx950).
//
// TideLM README, "How adaptive expert loading works", items 1-2: the router
// scores every expert; demand is recorded over the unrestricted top-k; the
// router then picks only resident (or hot-ring) experts, a miss replaced by the
// next-best resident expert; the chosen weights are renormalised.  Rows are
// then named by index per slot (colibri cluster page, COLIEX01 v2 paragraph).
#include "common.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Router logits in float64.  Definition shared by both kernels below:
//   S_c = fma chain over h in chunk c (128 wide), ascending, starting from 0
//   z   = S_0 + S_1 + ... (ascending c, starting from 0); bias added later.
// Both kernels compute bit-identical values for a (t, e) whatever T is.
// ---------------------------------------------------------------------------

// One thread per (t, e, c): chunk partials, for small T (decode batches).
__global__ __launch_bounds__(256) void router_chunks_f64(const uint16_t* __restrict__ x,
                                                         const float* __restrict__ w, int T, int H,
                                                         int E, double* __restrict__ zpart) {
  const int e = blockIdx.x * 64 + (threadIdx.x & 63);
  const int t = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int c = blockIdx.z;
  if (e >= E || t >= T) return;
  const int h0 = c * kRouterChunk;
  const int hn = min(kRouterChunk, H - h0);  // multiple of 32
  const float4* wr = reinterpret_cast<const float4*>(w + (size_t)e * H + h0);
  const uint2* xr = reinterpret_cast<const uint2*>(x + (size_t)t * H + h0);
  double s = 0.0;
  for (int q = 0; q < hn / 4; ++q) {
    const float4 wv = wr[q];
    const uint2 xv = xr[q];
    s = fma((double)bf16_to_f32(xv.x & 0xFFFFu), (double)wv.x, s);
    s = fma((double)bf16_to_f32(xv.x >> 16), (double)wv.y, s);
    s = fma((double)bf16_to_f32(xv.y & 0xFFFFu), (double)wv.z, s);
    s = fma((double)bf16_to_f32(xv.y >> 16), (double)wv.w, s);
  }
  zpart[((size_t)c * T + t) * E + e] = s;
}

// Tiled full-K router for larger T: a workgroup owns 64 experts x 16 tokens; the
// 128-wide chunk of W and x is staged in LDS; each thread keeps 4 tokens x 1
// expert, with a per-chunk fma chain added into the running sum.
constexpr int RT_E = 64, RT_T = 16, RT_TPT = 4;
__global__ __launch_bounds__(256) void router_full_f64(const uint16_t* __restrict__ x,
                                                       const float* __restrict__ w, int T, int H,
                                                       int E, double* __restrict__ z) {
  __shared__ float ws[RT_E][kRouterChunk + 1];
  __shared__ double xs[kRouterChunk][RT_T];
  const int tid = threadIdx.x;
  const int el = tid & 63, tg = tid >> 6;
  const int e0 = blockIdx.x * RT_E, t0 = blockIdx.y * RT_T;
  double acc[RT_TPT], part[RT_TPT];
#pragma unroll
  for (int i = 0; i < RT_TPT; ++i) acc[i] = 0.0;
  const int nchunk = (H + kRouterChunk - 1) / kRouterChunk;
  for (int c = 0; c < nchunk; ++c) {
    const int h0 = c * kRouterChunk;
    const int hn = min(kRouterChunk, H - h0);
    // W tile: 64 rows x hn floats
    for (int i = tid; i < RT_E * (kRouterChunk / 4); i += 256) {
      const int r = i / (kRouterChunk / 4), q = i % (kRouterChunk / 4);
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e0 + r < E && q * 4 < hn)
        v = *reinterpret_cast<const float4*>(w + (size_t)(e0 + r) * H + h0 + q * 4);
      ws[r][q * 4 + 0] = v.x;
      ws[r][q * 4 + 1] = v.y;
      ws[r][q * 4 + 2] = v.z;
      ws[r][q * 4 + 3] = v.w;
    }
    // x tile: 16 tokens x hn bf16, stored [h][t] as float64
    for (int i = tid; i < RT_T * (kRouterChunk / 4); i += 256) {
      const int r = i / (kRouterChunk / 4), q = i % (kRouterChunk / 4);
      uint2 v = make_uint2(0u, 0u);
      if (t0 + r < T && q * 4 < hn)
        v = *reinterpret_cast<const uint2*>(x + (size_t)(t0 + r) * H + h0 + q * 4);
      xs[q * 4 + 0][r] = (double)bf16_to_f32(v.x & 0xFFFFu);
      xs[q * 4 + 1][r] = (double)bf16_to_f32(v.x >> 16);
      xs[q * 4 + 2][r] = (double)bf16_to_f32(v.y & 0xFFFFu);
      xs[q * 4 + 3][r] = (double)bf16_to_f32(v.y >> 16);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < RT_TPT; ++i) part[i] = 0.0;
    for (int h = 0; h < hn; ++h) {
      const double wv = (double)ws[el][h];
#pragma unroll
      for (int i = 0; i < RT_TPT; ++i) part[i] = fma(xs[h][tg * RT_TPT + i], wv, part[i]);
    }
#pragma unroll
    for (int i = 0; i < RT_TPT; ++i) acc[i] += part[i];
    __syncthreads();
  }
  const int e = e0 + el;
  if (e >= E) return;
#pragma unroll
  for (int i = 0; i < RT_TPT; ++i) {
    const int t = t0 + tg * RT_TPT + i;
    if (t < T) z[(size_t)t * E + e] = acc[i];
  }
}

// ---------------------------------------------------------------------------
// Per-token selection: one wave per token, expert e = lane + 64*i.
// ---------------------------------------------------------------------------
constexpr int kMaxPerLane = MOE_MAX_E / 64;

// Adds to `sel` (bit i = expert lane+64i) the best `want` experts among
// `allowed & ~sel` by key (higher z, then lower id).  Returns how many were found.
__device__ int wave_select(const double* z, uint32_t allowed, int nper, int want,
                           uint32_t& sel) {
  const int lane = threadIdx.x & 63;
  int got = 0;
  for (int r = 0; r < want; ++r) {
    double bz = -INFINITY;
    int be = 0x7FFFFFFF;
    const uint32_t cand = allowed & ~sel;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      if (i < nper && ((cand >> i) & 1u)) {
        const int e = lane + 64 * i;
        if (z[i] > bz || (z[i] == bz && e < be)) {
          bz = z[i];
          be = e;
        }
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      const double oz = __shfl_xor(bz, d, kWave);
      const int oe = __shfl_xor(be, d, kWave);
      if (oz > bz || (oz == bz && oe < be)) {
        bz = oz;
        be = oe;
      }
    }
    if (be == 0x7FFFFFFF) break;  // wave-uniform: no candidate left
    if ((be & 63) == lane) sel |= 1u << (be >> 6);
    ++got;
  }
  return got;
}

// Position of each selected expert in ascending-id order.
__device__ __forceinline__ void selected_positions(uint32_t sel, int nper, int* pos) {
  const uint64_t lt = lanemask_lt();
  int base = 0;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    if (i < nper) {
      const uint64_t m = __ballot((sel >> i) & 1u);
      pos[i] = base + __popcll(m & lt);
      base += __popcll(m);
    }
  }
}

__global__ __launch_bounds__(256) void route_select(
    const double* __restrict__ zsrc, int nsplit, const float* __restrict__ bias,
    const int32_t* __restrict__ expert_slot, const uint16_t* __restrict__ x, int T, int H, int E,
    int k, int S, int32_t* __restrict__ topk_expert, float* __restrict__ topk_score,
    int32_t* __restrict__ sel_expert, float* __restrict__ sel_weight,
    int32_t* __restrict__ sel_slot, uint8_t* __restrict__ xq, size_t xq_row) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform
  const int nper = (E + 63) / 64;

  // ---- logits: ascending chunk sums, then bias ----
  double z[kMaxPerLane];
  uint32_t valid = 0, routable = 0;
  int slot_of[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    z[i] = -INFINITY;
    slot_of[i] = -1;
    const int e = lane + 64 * i;
    if (i < nper && e < E) {
      double s = 0.0;
      if (nsplit > 0) {
        for (int c = 0; c < nsplit; ++c) s += zsrc[((size_t)c * T + t) * E + e];
      } else {
        s = zsrc[(size_t)t * E + e];
      }
      z[i] = s + (bias ? (double)bias[e] : 0.0);
      valid |= 1u << i;
      const int sl = expert_slot[e];
      if (sl >= 0 && sl < S) {
        routable |= 1u << i;
        slot_of[i] = sl;
      }
    }
  }

  // ---- softmax over all experts (float64) ----
  double m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i)
    if (i < nper) m = fmax(m, z[i]);
  m = wave_max(m);
  double ex[kMaxPerLane];
  double lsum = 0.0;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    ex[i] = 0.0;
    if (i < nper && ((valid >> i) & 1u)) {
      ex[i] = exp(z[i] - m);
      lsum += ex[i];
    }
  }
  const double denom = wave_sum(lsum);

  // ---- unrestricted top-k (demand picks) ----
  uint32_t usel = 0;
  wave_select(z, valid, nper, k, usel);
  int pos[kMaxPerLane];
  selected_positions(usel, nper, pos);
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    if (i < nper && ((usel >> i) & 1u)) {
      const size_t o = (size_t)t * k + pos[i];
      topk_expert[o] = lane + 64 * i;
      topk_score[o] = (float)(ex[i] / denom);
    }
  }

  // ---- masked top-k over routable experts, renormalised ----
  uint32_t msel = 0;
  const int got = wave_select(z, routable, nper, k, msel);
  selected_positions(msel, nper, pos);
  double psel = 0.0;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i)
    if (i < nper && ((msel >> i) & 1u)) psel += ex[i] / denom;
  const double wsum = wave_sum(psel);
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    if (i < nper && ((msel >> i) & 1u)) {
      const size_t o = (size_t)t * k + pos[i];
      sel_expert[o] = lane + 64 * i;
      sel_weight[o] = (float)((ex[i] / denom) / wsum);
      sel_slot[o] = slot_of[i];
    }
  }
  for (int j = got + lane; j < k; j += 64) {
    const size_t o = (size_t)t * k + j;
    sel_expert[o] = -1;
    sel_weight[o] = 0.f;
    sel_slot[o] = -1;
  }

  // ---- MXFP4 activation row: lane per 32-block ----
  const int nblk = H / 32;
  const uint16_t* xr = x + (size_t)t * H;
  uint8_t* qr = xq + (size_t)t * xq_row;
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
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    uint32_t words[4] = {0u, 0u, 0u, 0u};
    uint32_t scale = 0u;
    if (amax > 0.f) {
      const int e = mx_block_exp(amax);
      scale = (uint32_t)(e + 127);
#pragma unroll
      for (int i = 0; i < 32; ++i) words[i >> 3] |= e2m1_code(v[i], e) << (4 * (i & 7));
    }
    *reinterpret_cast<uint4*>(qr + (size_t)b * 16) = make_uint4(words[0], words[1], words[2], words[3]);
    qr[H / 2 + b] = (uint8_t)scale;
  }
}

// ---------------------------------------------------------------------------
// Bucketing: counts + exclusive scan in one workgroup, then a stable scatter
// with one workgroup per slot scanning the assignments in ascending order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void bucket_count_scan(const int32_t* __restrict__ sel_slot,
                                                          int A, int S,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ perm) {
  __shared__ int cnt[MOE_MAX_S];
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  for (int s = tid; s < S; s += 1024) cnt[s] = 0;
  __syncthreads();
  for (int a = tid; a < A; a += 1024) {
    const int s = sel_slot[a];
    if (s >= 0 && s < S) atomicAdd(&cnt[s], 1);
  }
  __syncthreads();
  const int per = (S + 1023) / 1024;
  const int lo = min(S, tid * per), hi = min(S, lo + per);
  int local = 0;
  for (int s = lo; s < hi; ++s) local += cnt[s];
  // block exclusive scan of `local`
  const int lane = tid & 63, wv = tid >> 6;
  int incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int wbase = 0;
  for (int i = 0; i < wv; ++i) wbase += wsum[i];
  int run = wbase + incl - local;
  for (int s = lo; s < hi; ++s) {
    offsets[s] = run;
    run += cnt[s];
  }
  int total = 0;
  for (int i = 0; i < 16; ++i) total += wsum[i];
  if (tid == 0) offsets[S] = total;
  for (int a = total + tid; a < A; a += 1024) perm[a] = -1;
}

__global__ __launch_bounds__(256) void bucket_scatter(const int32_t* __restrict__ sel_slot, int A,
                                                      const int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ perm) {
  __shared__ int wcnt[4];
  const int s = blockIdx.x;
  const int base0 = offsets[s];
  const int n = offsets[s + 1] - base0;
  if (n <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int found = 0;
  for (int a0 = 0; a0 < A && found < n; a0 += 256) {
    const int a = a0 + tid;
    const bool hit = a < A && sel_slot[a] == s;
    const uint64_t m = __ballot(hit);
    if (lane == 0) wcnt[wv] = __popcll(m);
    __syncthreads();
    int before = 0;
    for (int i = 0; i < wv; ++i) before += wcnt[i];
    if (hit) perm[base0 + found + before + __popcll(m & lanemask_lt())] = a;
    found += wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    __syncthreads();
  }
}

__global__ void fill_i32(int32_t* p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace moe

using namespace moe;

static size_t route_ws_bytes(int T, int H, int E) {
  if (T <= 0) return 0;
  const size_t nchunk = (size_t)(H + kRouterChunk - 1) / kRouterChunk;
  const size_t zb = T <= kSplitRouterMaxT ? nchunk * T * E * sizeof(double)
                                          : (size_t)T * E * sizeof(double);
  return up_to(zb, 256);
}

size_t moe_route_ws_bytes_internal(int T, int H, int E) { return route_ws_bytes(T, H, E); }

extern "C" MOE_EXPORT int moe_route(const moe_route_args* a, hipStream_t stream) {
  if (!a) return MOE_EINVAL;
  const int T = a->T, H = a->H, E = a->E, k = a->k, S = a->S;
  if (T < 0 || H <= 0 || E <= 0 || k <= 0 || S < 0) return MOE_EINVAL;
  if (H % 32 != 0 || k > MOE_MAX_K || k > E || E > MOE_MAX_E || S > MOE_MAX_S)
    return MOE_EUNSUPPORTED;
  if ((size_t)T * k > (size_t)INT32_MAX || (size_t)T * H > ((size_t)1 << 40)) return MOE_EINVAL;
  if (!a->slot_offsets) return MOE_EINVAL;
  if (T > 0) {
    if (!a->x || !a->w_router || !a->expert_slot || !a->topk_expert || !a->topk_score ||
        !a->sel_expert || !a->sel_weight || !a->sel_slot || !a->perm || !a->xq)
      return MOE_EINVAL;
    if (!aligned(a->x, 16) || !aligned(a->w_router, 16) || !aligned(a->xq, 16)) return MOE_EINVAL;
    const size_t need = route_ws_bytes(T, H, E);
    if (a->ws_bytes < need) return MOE_EWORKSPACE;
    if (need > 0 && (!a->ws || !aligned(a->ws, 256))) return MOE_EINVAL;
  }

  if (T == 0) {
    fill_i32<<<(S + 1 + 255) / 256, 256, 0, stream>>>(a->slot_offsets, S + 1, 0);
    return hip_status();
  }
  hipEvent_t* ev = a->stage_events;
  double* zbuf = static_cast<double*>(a->ws);
  const int nchunk = (H + kRouterChunk - 1) / kRouterChunk;
  int nsplit = 0;
  if (ev && hipEventRecord(ev[0], stream) != hipSuccess) return MOE_EHIP;
  if (T <= kSplitRouterMaxT) {
    dim3 grid((E + 63) / 64, (T + 3) / 4, nchunk);
    router_chunks_f64<<<grid, 256, 0, stream>>>(a->x, a->w_router, T, H, E, zbuf);
    nsplit = nchunk;
  } else {
    dim3 grid((E + RT_E - 1) / RT_E, (T + RT_T - 1) / RT_T);
    router_full_f64<<<grid, 256, 0, stream>>>(a->x, a->w_router, T, H, E, zbuf);
  }
  if (ev && hipEventRecord(ev[1], stream) != hipSuccess) return MOE_EHIP;
  route_select<<<(T + 3) / 4, 256, 0, stream>>>(
      zbuf, nsplit, a->bias, a->expert_slot, a->x, T, H, E, k, S, a->topk_expert, a->topk_score,
      a->sel_expert, a->sel_weight, a->sel_slot, a->xq, mxfp4_row_bytes(H));
  const int A = T * k;
  if (ev && hipEventRecord(ev[2], stream) != hipSuccess) return MOE_EHIP;
  bucket_count_scan<<<1, 1024, 0, stream>>>(a->sel_slot, A, S, a->slot_offsets, a->perm);
  if (ev && hipEventRecord(ev[3], stream) != hipSuccess) return MOE_EHIP;
  if (S > 0) bucket_scatter<<<S, 256, 0, stream>>>(a->sel_slot, A, a->slot_offsets, a->perm);
  if (ev && hipEventRecord(ev[4], stream) != hipSuccess) return MOE_EHIP;
  return hip_status();
}
