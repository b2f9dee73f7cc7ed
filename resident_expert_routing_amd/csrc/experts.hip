// moe_experts_forward: grouped SwiGLU expert FFNs on MXFP4 arena slots and the
// weighted combine (gfx950, block-scaled MXFP4 MFMA).
//
// TideLM README, "How adaptive expert loading works": experts run from arena
// slots (resident set or hot ring).  colibri cluster page: each expert names its
// rows by index (COLIEX01 v2 paragraph), and a row's expert results are added in
// one fixed order (the fixed-summation-order paragraph) -- here ascending
// expert id, which is the order of a token's picks.
//
// Contraction layout shared by every GEMM here (so any token's result is the
// same whatever batch it runs in): K is walked in 512-wide super-chunks
// (16 MX blocks) in ascending order; MFMA step i (0..3) of a super-chunk covers
// blocks 4i..4i+3, lane group g (lanes 16g..16g+15) supplying block 4i+g.  One
// load instruction thus reads 64 contiguous bytes of each of 16 rows.  A lane
// reads the super-chunk's 16 scale bytes as one 16-byte word and shifts its
// own byte (4i+g) into place for step i.
#include "common.hpp"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
constexpr int kInlineWorklistMaxS = 1024;
typedef float v4f __attribute__((ext_vector_type(4)));

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

// Load this lane's share of super-chunk sc of an MXFP4 row.  FULL: the row has
// a multiple of 16 blocks and 16-byte aligned scales.  Blocks at or past nblk
// read as zero codes.
template <bool FULL>
__device__ __forceinline__ void load_row_sc(const uint8_t* codes, const uint8_t* scales, int sc,
                                            int g, int nblk, RowSC& r) {
  const int b0 = sc * 16;
  if (FULL) {
    const uint4* p = reinterpret_cast<const uint4*>(codes + (size_t)b0 * 16) + g;
    r.q[0] = p[0];
    r.q[1] = p[4];
    r.q[2] = p[8];
    r.q[3] = p[12];
    const uint4 sv = *reinterpret_cast<const uint4*>(scales + b0);
    const int sh = 8 * g;
    r.s[0] = sv.x >> sh;
    r.s[1] = sv.y >> sh;
    r.s[2] = sv.z >> sh;
    r.s[3] = sv.w >> sh;
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

// The u-th slot (ascending) that holds assignments, found by the whole
// workgroup from slot_offsets; -1 if fewer slots are used.  Each thread scans a
// contiguous range, then a workgroup prefix of the per-thread counts.
__device__ int wg_nth_used_slot(int u, const int32_t* __restrict__ offsets, int S, int A) {
  __shared__ int wsum[4];
  __shared__ int found;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (tid == 0) found = -1;
  const int per = (S + 255) / 256;
  const int lo = min(S, tid * per), hi = min(S, lo + per);
  int local = 0;
  for (int s = lo; s < hi; ++s) {
    const int a = offsets[s], b = offsets[s + 1];
    local += (b > a && a >= 0 && b <= A) ? 1 : 0;
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
  if (u >= run && u < run + local) {
    for (int s = lo; s < hi; ++s) {
      const int a = offsets[s], b = offsets[s + 1];
      if (b > a && a >= 0 && b <= A) {
        if (run == u) found = s;
        ++run;
      }
    }
  }
  __syncthreads();
  return found;
}

// Slot of work item u: from the prebuilt list when there is one, else found
// in place (small slot counts).
__device__ __forceinline__ int work_slot(int u, const int32_t* used, const int32_t* offsets, int S,
                                         int A) {
  if (used) return u < used[0] ? used[1 + u] : -1;
  return wg_nth_used_slot(u, offsets, S, A);
}

// ---------------------------------------------------------------------------
// Work list: the slots that hold assignments, ascending, from slot_offsets.
// used[0] = count, used[1..] = slot ids.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void build_used(const int32_t* __restrict__ offsets, int S,
                                                   int A, int32_t* __restrict__ used) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = (S + 1023) / 1024;
  const int lo = min(S, tid * per), hi = min(S, lo + per);
  int local = 0;
  for (int s = lo; s < hi; ++s) {
    const int a = offsets[s], b = offsets[s + 1];
    local += (b > a && a >= 0 && b <= A) ? 1 : 0;
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
    if (b > a && a >= 0 && b <= A) used[1 + run++] = s;
  }
  if (tid == 0) {
    int total = 0;
    for (int i = 0; i < 16; ++i) total += wsum[i];
    used[0] = total;
  }
}

// ---------------------------------------------------------------------------
// Gate/up + SwiGLU + MXFP4(h).  Workgroup = 4 waves = 128 rows of I of one
// slot; wave = 32 rows (two 16-row tiles of gate and of up).  Columns are the
// slot's assignment rows p, 16 per MFMA tile.  Output: hq row p (an MXFP4 row
// of I elements).
// ---------------------------------------------------------------------------
struct GateUpArgs {
  const uint8_t* xq;
  size_t xrow;
  const uint8_t* arena;
  size_t stride;
  size_t off_gc, off_gs, off_uc, off_us;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* used;  // prebuilt work list, or null: found in place
  uint8_t* hq;
  size_t hrow;
  int T, H, I, k, A, S;
};

template <bool FULL>
__global__ __launch_bounds__(256) void gateup_kernel(GateUpArgs p) {
  const int nbps = (p.I + 127) / 128;
  const int u = blockIdx.x / nbps, nb = blockIdx.x % nbps;
  const int s = work_slot(u, p.used, p.offsets, p.S, p.A);
  if (s < 0) return;
  const int p0 = p.offsets[s], p1 = p.offsets[s + 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = nb * 128 + wave * 32;
  if (n0 >= p.I) return;
  const int r = lane & 15, g = lane >> 4;
  const int H = p.H;
  const int nblk = H / 32;
  const int nsc = (nblk + 15) / 16;
  const uint8_t* base = p.arena + (size_t)s * p.stride;
  const size_t crow = (size_t)H / 2, srow = (size_t)H / 32;
  const uint8_t* gc0 = base + p.off_gc + (size_t)(n0 + r) * crow;
  const uint8_t* gc1 = gc0 + 16 * crow;
  const uint8_t* gs0 = base + p.off_gs + (size_t)(n0 + r) * srow;
  const uint8_t* gs1 = gs0 + 16 * srow;
  const uint8_t* uc0 = base + p.off_uc + (size_t)(n0 + r) * crow;
  const uint8_t* uc1 = uc0 + 16 * crow;
  const uint8_t* us0 = base + p.off_us + (size_t)(n0 + r) * srow;
  const uint8_t* us1 = us0 + 16 * srow;

  for (int cb = p0; cb < p1; cb += 16) {
    // this lane's column (assignment row) for the B operand
    const int pc = cb + r;
    int t = -1;
    if (pc < p1) {
      const int a = p.perm[pc];
      if (a >= 0 && a < p.A) t = a / p.k;
    }
    const uint8_t* xc = t >= 0 ? p.xq + (size_t)t * p.xrow : nullptr;
    v4f ag0 = {0.f, 0.f, 0.f, 0.f}, ag1 = ag0, au0 = ag0, au1 = ag0;
    for (int sc = 0; sc < nsc; ++sc) {
      RowSC wg0, wg1, wu0, wu1, x;
      load_row_sc<FULL>(gc0, gs0, sc, g, nblk, wg0);
      load_row_sc<FULL>(gc1, gs1, sc, g, nblk, wg1);
      load_row_sc<FULL>(uc0, us0, sc, g, nblk, wu0);
      load_row_sc<FULL>(uc1, us1, sc, g, nblk, wu1);
      if (xc)
        load_row_sc<FULL>(xc, xc + H / 2, sc, g, nblk, x);
      else
        zero_sc(x);
      ag0 = mfma_superchunk(wg0, x, ag0);
      ag1 = mfma_superchunk(wg1, x, ag1);
      au0 = mfma_superchunk(wu0, x, au0);
      au1 = mfma_superchunk(wu1, x, au1);
    }
    // Epilogue.  Lane (c = lane&15, g) holds rows n0+4g+v (tile 0) and
    // n0+16+4g+v (tile 1) of column c.
    const int c = lane & 15;
    const int pcol = cb + c;
    float h[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      h[v] = ag0[v] / (1.0f + expf(-ag0[v])) * au0[v];
      h[4 + v] = ag1[v] / (1.0f + expf(-ag1[v])) * au1[v];
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
    if (pcol < p1) {
      uint8_t* hr = p.hq + (size_t)pcol * p.hrow;
      const uint16_t w0 = (uint16_t)(codes[0] | (codes[1] << 4) | (codes[2] << 8) | (codes[3] << 12));
      const uint16_t w1 = (uint16_t)(codes[4] | (codes[5] << 4) | (codes[6] << 8) | (codes[7] << 12));
      *reinterpret_cast<uint16_t*>(hr + n0 / 2 + 2 * g) = w0;
      *reinterpret_cast<uint16_t*>(hr + n0 / 2 + 8 + 2 * g) = w1;
      if (g == 0) hr[p.I / 2 + n0 / 32] = (uint8_t)scale;
    }
  }
}

// ---------------------------------------------------------------------------
// Down projection.  Workgroup = 4 waves = 256 rows of H of one slot; wave = 64
// rows (four 16-row tiles).  B operand: hq rows of the slot.  Output y[a] (fp32
// row of H), a = perm[p].
// ---------------------------------------------------------------------------
struct DownArgs {
  const uint8_t* hq;
  size_t hrow;
  const uint8_t* arena;
  size_t stride;
  size_t off_dc, off_ds;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* used;  // prebuilt work list, or null: found in place
  float* y;
  int H, I, A, S;
};

template <bool FULL>
__global__ __launch_bounds__(256) void down_kernel(DownArgs p) {
  const int nbps = (p.H + 255) / 256;
  const int u = blockIdx.x / nbps, nb = blockIdx.x % nbps;
  const int s = work_slot(u, p.used, p.offsets, p.S, p.A);
  if (s < 0) return;
  const int p0 = p.offsets[s], p1 = p.offsets[s + 1];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = nb * 256 + wave * 64;
  if (n0 >= p.H) return;
  const int r = lane & 15, g = lane >> 4;
  const int I = p.I;
  const int nblk = I / 32;
  const int nsc = (nblk + 15) / 16;
  const uint8_t* base = p.arena + (size_t)s * p.stride;
  const size_t crow = (size_t)I / 2, srow = (size_t)I / 32;
  const uint8_t* dc[4];
  const uint8_t* ds[4];
  bool tv[4];
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) {
    tv[tl] = n0 + 16 * tl < p.H;  // whole tile valid (H % 16 == 0)
    const int row = tv[tl] ? n0 + 16 * tl + r : n0 + r;
    dc[tl] = base + p.off_dc + (size_t)row * crow;
    ds[tl] = base + p.off_ds + (size_t)row * srow;
  }
  for (int cb = p0; cb < p1; cb += 16) {
    const int pc = cb + r;
    const uint8_t* hc = pc < p1 ? p.hq + (size_t)pc * p.hrow : nullptr;
    v4f acc[4];
#pragma unroll
    for (int tl = 0; tl < 4; ++tl) acc[tl] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int sc = 0; sc < nsc; ++sc) {
      RowSC x;
      if (hc)
        load_row_sc<FULL>(hc, hc + I / 2, sc, g, nblk, x);
      else
        zero_sc(x);
#pragma unroll
      for (int tl = 0; tl < 4; ++tl) {
        if (tv[tl]) {
          RowSC w;
          load_row_sc<FULL>(dc[tl], ds[tl], sc, g, nblk, w);
          acc[tl] = mfma_superchunk(w, x, acc[tl]);
        }
      }
    }
    const int c = lane & 15;
    const int pcol = cb + c;
    if (pcol < p1) {
      const int a = p.perm[pcol];
      if (a >= 0 && a < p.A) {
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
  }
}

// ---------------------------------------------------------------------------
// Combine: out[t] = sum_j (ascending) w[t,j] * y[t*k+j], rounded once to bf16.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ sel_slot, int T,
                                                      int H, int k, int S,
                                                      uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int h = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (h >= H) return;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int j = 0; j < k; ++j) {
    const int sl = sel_slot[(size_t)t * k + j];
    if (sl < 0 || sl >= S) continue;
    const float wj = w[(size_t)t * k + j];
    const float4 v = *reinterpret_cast<const float4*>(y + ((size_t)t * k + j) * H + h);
    a0 = fmaf(wj, v.x, a0);
    a1 = fmaf(wj, v.y, a1);
    a2 = fmaf(wj, v.z, a2);
    a3 = fmaf(wj, v.w, a3);
  }
  const uint32_t lo = f32_to_bf16(a0) | (f32_to_bf16(a1) << 16);
  const uint32_t hi = f32_to_bf16(a2) | (f32_to_bf16(a3) << 16);
  *reinterpret_cast<uint2*>(out + (size_t)t * H + h) = make_uint2(lo, hi);
}

}  // namespace moe

using namespace moe;

struct ExpertsWs {
  size_t used_off, hq_off, y_off, total;
};

static ExpertsWs experts_ws(int T, int H, int k, int I, int S) {
  ExpertsWs w;
  const size_t A = (size_t)T * k;
  w.used_off = 0;
  w.hq_off = up_to((size_t)(S + 2) * sizeof(int32_t), 256);
  w.y_off = up_to(w.hq_off + A * mxfp4_row_bytes(I), 256);
  w.total = up_to(w.y_off + A * (size_t)H * sizeof(float), 256);
  return w;
}

size_t moe_experts_ws_bytes_internal(int T, int H, int k, int I, int S) {
  if (T <= 0) return 0;
  return experts_ws(T, H, k, I, S).total;
}

extern "C" MOE_EXPORT int moe_experts_forward(const moe_experts_args* a, hipStream_t stream) {
  if (!a) return MOE_EINVAL;
  const int T = a->T, H = a->H, I = a->I, k = a->k, S = a->S;
  if (T < 0 || H <= 0 || I <= 0 || k <= 0 || S < 0) return MOE_EINVAL;
  if (H % 32 != 0 || I % 32 != 0 || k > MOE_MAX_K || S > MOE_MAX_S) return MOE_EUNSUPPORTED;
  if ((size_t)T * k > (size_t)INT32_MAX) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!a->xq || !a->slot_offsets || !a->perm || !a->sel_slot || !a->sel_weight || !a->out)
    return MOE_EINVAL;
  if (S > 0 && !a->arena) return MOE_EINVAL;  // with no slot, the arena is never read
  const SlotLayout L = slot_layout(H, I);
  if (a->slot_stride < L.total || a->slot_stride % 256 != 0) return MOE_EINVAL;
  if (!aligned(a->xq, 16) || !aligned(a->arena, 256) || !aligned(a->out, 8)) return MOE_EINVAL;
  const ExpertsWs W = experts_ws(T, H, k, I, S);
  if (a->ws_bytes < W.total) return MOE_EWORKSPACE;
  if (!a->ws || !aligned(a->ws, 256)) return MOE_EINVAL;
  if (S == 0) {
    // nothing routable: every pick is padding, the output is zero
    dim3 grid(T, (H + 1023) / 1024);
    combine_kernel<<<grid, 256, 0, stream>>>(nullptr, a->sel_weight, a->sel_slot, T, H, k, S,
                                             a->out);
    return hip_status();
  }
  uint8_t* ws = static_cast<uint8_t*>(a->ws);
  int32_t* used = reinterpret_cast<int32_t*>(ws + W.used_off);
  uint8_t* hq = ws + W.hq_off;
  float* y = reinterpret_cast<float*>(ws + W.y_off);
  const int A = T * k;
  const int maxU = S < A ? S : A;
  hipEvent_t* ev = a->stage_events;

  // Work list of used slots: built once for large slot counts, else each
  // workgroup finds its slot in place (saves a launch on decode batches).
  const bool prebuilt = S > kInlineWorklistMaxS;
  if (!record_stage(ev,0, stream)) return MOE_EHIP;
  if (prebuilt) build_used<<<1, 1024, 0, stream>>>(a->slot_offsets, S, A, used);
  if (!record_stage(ev,1, stream)) return MOE_EHIP;

  GateUpArgs g;
  g.xq = a->xq;
  g.xrow = mxfp4_row_bytes(H);
  g.arena = a->arena;
  g.stride = a->slot_stride;
  g.off_gc = L.off[0];
  g.off_gs = L.off[1];
  g.off_uc = L.off[2];
  g.off_us = L.off[3];
  g.offsets = a->slot_offsets;
  g.perm = a->perm;
  g.used = prebuilt ? used : nullptr;
  g.hq = hq;
  g.hrow = mxfp4_row_bytes(I);
  g.T = T;
  g.H = H;
  g.I = I;
  g.k = k;
  g.A = A;
  g.S = S;
  const int gblocks = maxU * ((I + 127) / 128);
  if (H % 512 == 0)
    gateup_kernel<true><<<gblocks, 256, 0, stream>>>(g);
  else
    gateup_kernel<false><<<gblocks, 256, 0, stream>>>(g);

  if (!record_stage(ev,2, stream)) return MOE_EHIP;

  DownArgs d;
  d.hq = hq;
  d.hrow = g.hrow;
  d.arena = a->arena;
  d.stride = a->slot_stride;
  d.off_dc = L.off[4];
  d.off_ds = L.off[5];
  d.offsets = a->slot_offsets;
  d.perm = a->perm;
  d.used = prebuilt ? used : nullptr;
  d.y = y;
  d.H = H;
  d.I = I;
  d.A = A;
  d.S = S;
  const int dblocks = maxU * ((H + 255) / 256);
  if (I % 512 == 0)
    down_kernel<true><<<dblocks, 256, 0, stream>>>(d);
  else
    down_kernel<false><<<dblocks, 256, 0, stream>>>(d);
  if (!record_stage(ev,3, stream)) return MOE_EHIP;

  dim3 cgrid(T, (H + 1023) / 1024);
  combine_kernel<<<cgrid, 256, 0, stream>>>(y, a->sel_weight, a->sel_slot, T, H, k, S, a->out);
  if (!record_stage(ev,4, stream)) return MOE_EHIP;
  return hip_status();
}
