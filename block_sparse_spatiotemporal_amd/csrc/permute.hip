// Raster <-> block-order gathers ("Video Sparse Attention" explainer,
// section 3: the tokens of each cube are made contiguous so the fine stage
// runs on whole blocks).  Pure data movement, HBM bound: 16-byte vector
// accesses, each 64-token block row-run read and written contiguously.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "attn_common.h"
#include "fva_internal.h"

namespace {

using fva_attn::vt_slot_key;

constexpr int kThreads = 256;

// Element loads/stores for the rotary path: bf16 (uint16 bit patterns) or
// fp32.  st_val rounds an fp64 value once to the element type.
__device__ __forceinline__ float ld_val(const uint16_t* p) { return __uint_as_float((uint32_t)(*p) << 16); }
__device__ __forceinline__ float ld_val(const float* p) { return *p; }
template <typename T>
__device__ __forceinline__ T st_val(double v);
// Correctly rounded fp64 -> bf16 (nearest, ties to even).  f = (float)v is
// within half an fp32 ulp of v, so the two bf16 values around f, lo (f
// truncated) and hi (one bf16 ulp further from zero), bracket v's nearest
// bf16; the distances are exact in fp64.  Infinity and NaN pass through.
template <>
__device__ __forceinline__ uint16_t st_val<uint16_t>(double v) {
  const uint32_t fb = __float_as_uint((float)v);
  if ((fb & 0x7F800000u) == 0x7F800000u) return (uint16_t)((fb >> 16) | ((fb & 0x7FFFFFu) ? 0x40u : 0u));
  const uint32_t lo = fb & 0xFFFF0000u, hi = lo + 0x10000u;
  const double dlo = fabs(v - (double)__uint_as_float(lo)), dhi = fabs(v - (double)__uint_as_float(hi));
  const uint32_t r = dlo < dhi ? lo : (dhi < dlo ? hi : (((lo >> 16) & 1u) ? hi : lo));
  return (uint16_t)(r >> 16);
}
template <>
__device__ __forceinline__ float st_val<float>(double v) { return (float)v; }
constexpr int kUnroll = 4;  // 16-byte chunks per thread per block of work

// x_perm[b,h,pos,:] = x_raster[b, perm[pos], h, :] (or zero for a pad).
// gridDim.y = B*H; each workgroup moves kThreads*kUnroll 16-byte chunks.
__global__ __launch_bounds__(kThreads) void k_permute_rows(const uint4* __restrict__ src,
                                                           uint4* __restrict__ dst,
                                                           const int32_t* __restrict__ perm,
                                                           int64_t n_tok, int heads, int64_t n_pad,
                                                           int cpr /* chunks per row */) {
  const int bh = blockIdx.y;
  const int b = bh / heads, h = bh - b * heads;
  const int64_t total = n_pad * cpr;
  const int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
  uint4 v[kUnroll];
  int64_t idx[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    idx[u] = base + (int64_t)u * kThreads;
    v[u] = make_uint4(0, 0, 0, 0);
    if (idx[u] < total) {
      const int64_t pos = idx[u] / cpr;
      const int ch = (int)(idx[u] - pos * cpr);
      const int tok = perm[pos];
      if (tok >= 0) v[u] = src[(((int64_t)b * n_tok + tok) * heads + h) * cpr + ch];
    }
  }
  uint4* out = dst + (int64_t)bh * total;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (idx[u] < total) out[idx[u]] = v[u];
}

// x_raster[b, perm[pos], h, :] = x_perm[b,h,pos,:] for valid positions.
__global__ __launch_bounds__(kThreads) void k_unpermute_rows(const uint4* __restrict__ src,
                                                             uint4* __restrict__ dst,
                                                             const int32_t* __restrict__ perm,
                                                             int64_t n_tok, int heads, int64_t n_pad,
                                                             int cpr) {
  const int bh = blockIdx.y;
  const int b = bh / heads, h = bh - b * heads;
  const int64_t total = n_pad * cpr;
  const int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
  const uint4* in = src + (int64_t)bh * total;
  uint4 v[kUnroll];
  int64_t idx[kUnroll];
  int tok[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    idx[u] = base + (int64_t)u * kThreads;
    tok[u] = -1;
    if (idx[u] < total) {
      tok[u] = perm[idx[u] / cpr];
      if (tok[u] >= 0) v[u] = in[idx[u]];
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    if (tok[u] >= 0) {
      const int64_t pos = idx[u] / cpr;
      const int ch = (int)(idx[u] - pos * cpr);
      dst[(((int64_t)b * n_tok + tok[u]) * heads + h) * cpr + ch] = v[u];
    }
  }
}

// One workgroup per (b, h, block).  The block's 64 rows come in as 16-byte
// chunks into an LDS tile (rows padded by one chunk); each 16-byte output
// chunk of the two [D][32] halves (one d, E consecutive key slots) is then
// gathered from the tile and written with one 16-byte store.  T is the
// element type (2 or 4 bytes).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void k_permute_vt(const T* __restrict__ src, T* __restrict__ dst,
                                                         const int32_t* __restrict__ perm,
                                                         int64_t n_tok, int heads, int n_blk) {
  constexpr int E = 16 / sizeof(T);        // elements per 16-byte chunk
  constexpr int CPR = D / E;               // chunks per row
  constexpr int RS = (CPR + 1) * E;        // tile row stride in elements
  constexpr int NCH = 64 * CPR;            // chunks per block, in and out
  constexpr int OPD = 32 / E;              // output chunks per d row of a half
  __shared__ uint4 tile16[64 * (CPR + 1)];
  const T* tile = (const T*)tile16;
  const int blk = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / heads, h = bh - b * heads;
  const uint4* src16 = (const uint4*)src;
#pragma unroll
  for (int e = threadIdx.x; e < NCH; e += kThreads) {
    const int key = e / CPR, c = e - key * CPR;
    const int tok = perm[(int64_t)blk * 64 + key];
    tile16[key * (CPR + 1) + c] =
        tok >= 0 ? src16[(((int64_t)b * n_tok + tok) * heads + h) * CPR + c] : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
  uint4* out = (uint4*)(dst + ((int64_t)bh * n_blk + blk) * 64 * D);
#pragma unroll
  for (int o = threadIdx.x; o < NCH; o += kThreads) {
    const int half = o / (D * OPD);
    const int rem = o - half * (D * OPD);
    const int d = rem / OPD, s0 = (rem - d * OPD) * E;
    union {
      T e[E];
      uint4 v;
    } u;
#pragma unroll
    for (int i = 0; i < E; ++i) u.e[i] = tile[(32 * half + vt_slot_key(s0 + i)) * RS + d];
    out[o] = u.v;
  }
}

// --------------------------------------------------------------- rotary
// Pairs of the t, h and w axes for a head dimension: D/2 split as evenly as
// possible, t first.
__host__ __device__ inline void rope_split(int D, int* pt, int* ph, int* pw) {
  const int n = D / 2, q = n / 3, r = n % 3;
  *pt = q + (r > 0);
  *ph = q + (r > 1);
  *pw = q;
}

// cos/sin table of one call: rows are axis positions (T rows for t, then H
// for h, then W for w), each with D/2 columns of (cos, sin); only the
// columns of the row's own axis are filled.
__global__ __launch_bounds__(256) void k_rope_table(double2* __restrict__ tab, int T, int Hh, int W, int D,
                                                    int t_offset, double base) {
  int pt, ph, pw;
  rope_split(D, &pt, &ph, &pw);
  const int rows = T + Hh + W, np = D / 2;
  for (int e = blockIdx.x * 256 + threadIdx.x; e < rows * np; e += gridDim.x * 256) {
    const int row = e / np, p = e - row * np;
    int axis, pos, first, cnt;
    if (row < T) axis = 0, pos = row + t_offset, first = 0, cnt = pt;
    else if (row < T + Hh) axis = 1, pos = row - T, first = pt, cnt = ph;
    else axis = 2, pos = row - T - Hh, first = pt + ph, cnt = pw;
    (void)axis;
    double2 cs = make_double2(1.0, 0.0);
    if (p >= first && p < first + cnt) {
      const double ang = (double)pos * pow(base, -(double)(p - first) / (double)cnt);
      double sn, c;
      sincos(ang, &sn, &c);
      cs = make_double2(c, sn);
    }
    tab[e] = cs;
  }
}

// Two fp64 values rounded once to bf16 (nearest, ties to even), packed
// first | second << 16.  Rounding to fp32 and then to bf16 (the hardware's
// nearest-even pack) gives the same bits as one rounding unless the fp32
// value lies exactly halfway between two bf16 values (low 16 bits 0x8000):
// any other fp32 value is on the same side of every bf16 midpoint as the
// fp64 value it came from, since those midpoints are fp32 values.  Those
// halfway cases, and non-finite or subnormal fp32 values, set `rare`, and
// the caller rounds that chunk again with st_val.
__device__ __forceinline__ uint32_t bf16x2_once(double a, double b, bool& rare) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const float fa = (float)a, fb = (float)b;
  constexpr int kOdd = 0x297;   // class mask: NaN, infinities, subnormals
  rare |= (__float_as_uint(fa) & 0xFFFFu) == 0x8000u || (__float_as_uint(fb) & 0xFFFFu) == 0x8000u ||
          __builtin_amdgcn_class(fa, kOdd) || __builtin_amdgcn_class(fb, kOdd);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){fa, fb}, bf16x2));
}

// Chunks per thread of the rotary gather: 2 measured 0.37 ms at the Wan-14B
// 480P shape against 0.41 (1), 0.49 (4) and 0.89 ms (8), bit-identical.
constexpr int kRopeUnroll = 2;

// x_perm[b,h,pos,:] = rope(x_raster[b, perm[pos], h, :]) (zero for a pad):
// each thread moves kRopeUnroll 16-byte chunks (E/2 dimension pairs each) with
// 16-byte loads and stores; the rotation is fp64 with the call's (cos, sin)
// table, each output rounded once.  All of a thread's row and table loads
// are issued before any of them is used: a table load issued after the
// first chunk's arithmetic would wait behind every row load in flight.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void k_permute_rope(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                           const int32_t* __restrict__ perm,
                                                           const double2* __restrict__ tab, int64_t n_tok,
                                                           int heads, int64_t n_pad, int Tg, int Hg, int Wg,
                                                           float inv_w, float inv_h) {
  constexpr int E = 16 / sizeof(T);       // elements per chunk
  constexpr int CPR = D / E, NP = D / 2;  // chunks per row, pairs per row
  const int bh = blockIdx.y;
  const int b = bh / heads, h = bh - b * heads;
  const int64_t total = n_pad * CPR;
  int pt, ph, pw;
  rope_split(D, &pt, &ph, &pw);
  (void)pw;
  const int64_t base = (int64_t)blockIdx.x * kThreads * kRopeUnroll + threadIdx.x;
  union Chunk {
    uint4 v;
    T x[E];
    uint32_t w[4];
  };
  int tok[kRopeUnroll];
#pragma unroll
  for (int u = 0; u < kRopeUnroll; ++u) {
    const int64_t e = base + (int64_t)u * kThreads;
    tok[u] = e < total ? perm[e / CPR] : -1;
  }
  Chunk in[kRopeUnroll];
  double2 cs[kRopeUnroll][E / 2];
#pragma unroll
  for (int u = 0; u < kRopeUnroll; ++u) {
    const int c = (int)((base + (int64_t)u * kThreads) % CPR);
    const int tk = max(tok[u], 0);   // pads read token 0's table rows, unused
    // token -> (t, h, w): quotients from an fp32 reciprocal, corrected by
    // one step (tokens < 2^24, so the fp32 product is within one of them)
    int th = (int)((float)tk * inv_w);
    int w = tk - th * Wg;
    if (w < 0) w += Wg, --th;
    else if (w >= Wg) w -= Wg, ++th;
    int t = (int)((float)th * inv_h);
    int hh = th - t * Hg;
    if (hh < 0) hh += Hg, --t;
    else if (hh >= Hg) hh -= Hg, ++t;
    in[u].v = make_uint4(0, 0, 0, 0);
    if (tok[u] >= 0) in[u].v = src[(((int64_t)b * n_tok + tok[u]) * heads + h) * CPR + c];
#pragma unroll
    for (int j = 0; j < E / 2; ++j) {
      const int p = c * (E / 2) + j;
      const int row = p < pt ? t : (p < pt + ph ? Tg + hh : Tg + Hg + w);
      cs[u][j] = tab[row * NP + p];
    }
  }
  uint4* out = dst + (int64_t)bh * total;
#pragma unroll
  for (int u = 0; u < kRopeUnroll; ++u) {
    const int64_t e = base + (int64_t)u * kThreads;
    if (e >= total) continue;
    Chunk o;
    o.v = make_uint4(0, 0, 0, 0);
    if (tok[u] >= 0) {
      double r[E];
#pragma unroll
      for (int j = 0; j < E / 2; ++j) {
        const double x0 = (double)ld_val(&in[u].x[2 * j]), x1 = (double)ld_val(&in[u].x[2 * j + 1]);
        r[2 * j] = x0 * cs[u][j].x - x1 * cs[u][j].y;
        r[2 * j + 1] = x0 * cs[u][j].y + x1 * cs[u][j].x;
      }
      if constexpr (sizeof(T) == 2) {
        bool rare = false;
#pragma unroll
        for (int j = 0; j < E / 2; ++j) o.w[j] = bf16x2_once(r[2 * j], r[2 * j + 1], rare);
        if (rare) {
#pragma unroll
          for (int i = 0; i < E; ++i) o.x[i] = st_val<T>(r[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < E; ++i) o.x[i] = st_val<T>(r[i]);
      }
    }
    out[e] = o.v;
  }
}

// fva_permute (rows) of one block plus its pooled means, so the selection
// need not read the block-order tensor again ("Video Sparse Attention"
// explainer, section 3: one mean per (4,4,4) cube; "DFSAttn" trick 2: one
// per (2,2,2) sub-block for K when the plan has sub-blocks).  One workgroup
// per (block, b*h): the rows move as in k_permute_rows and a copy stays in
// LDS, from which the means are summed in fp64 in the order the separate
// pooling kernels use (row groups g, g+RG, ... per column, then the groups
// in order; sub-block members in table order), so the means are the same
// bits.  Pad rows are zero, so the sums run over all 64 rows.
template <typename T, int D, bool SUB>
__global__ __launch_bounds__(kThreads) void k_permute_pool(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                           const int32_t* __restrict__ perm, int64_t n_tok,
                                                           int heads, int64_t n_pad, int n_blk,
                                                           const int32_t* __restrict__ blk_cnt,
                                                           const uint8_t* __restrict__ sub_pos,
                                                           const int32_t* __restrict__ sub_cnt,
                                                           double* __restrict__ bar) {
  constexpr int CPR = D * (int)sizeof(T) / 16;   // 16-byte chunks per row
  constexpr int NCH = 64 * CPR;                  // chunks per block
  constexpr int PER = NCH / kThreads;
  constexpr int RG = 64 / CPR;                   // row groups of the column sums
  constexpr int RPL = 64 / RG;
  static_assert(NCH % kThreads == 0, "whole chunks per thread");
  __shared__ uint4 tile[NCH];
  __shared__ double part[SUB ? 1 : RG][D];
  __shared__ uint8_t s_pos[SUB ? 64 : 1];   // the block's sub-block member positions
  __shared__ int s_cnt[SUB ? 8 : 1];
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / heads, h = bh - b * heads;
  const int t = threadIdx.x;
  if (SUB) {
    if (t < 64) s_pos[t] = sub_pos[(int64_t)blk * 64 + t];
    if (t < 8) s_cnt[t] = sub_cnt[blk * 8 + t];
  }
  uint4* out = dst + ((int64_t)bh * n_pad + (int64_t)blk * 64) * CPR;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int c = t + kThreads * u;
    const int row = c / CPR, ch = c - row * CPR;
    const int tok = perm[blk * 64 + row];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (tok >= 0) v = src[(((int64_t)b * n_tok + tok) * heads + h) * CPR + ch];
    out[c] = v;
    tile[c] = v;
  }
  __syncthreads();
  const T* x = (const T*)tile;   // x[row * D + d]
  if (!SUB) {
    for (int e = t; e < RG * D; e += kThreads) {
      const int g = e / D, d = e - g * D;
      double acc = 0.0;
#pragma unroll 8
      for (int i = 0; i < RPL; ++i) acc += (double)ld_val(x + (g + RG * i) * D + d);
      part[g][d] = acc;
    }
    __syncthreads();
    if (t < D) {
      double sum = 0.0;
#pragma unroll
      for (int g = 0; g < RG; ++g) sum += part[g][t];
      bar[((int64_t)bh * n_blk + blk) * D + t] = sum / (double)blk_cnt[blk];
    }
  } else {
    double* o = bar + ((int64_t)bh * n_blk + blk) * 8 * D;
    for (int e = t; e < 8 * D; e += kThreads) {
      const int sb = e / D, d = e - sb * D;
      const uint8_t* pos = s_pos + sb * 8;
      double acc = 0.0;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += (double)ld_val(x + (int)pos[i] * D + d);
      const int cnt = s_cnt[sb];
      o[e] = cnt ? acc / (double)cnt : 0.0;
    }
  }
}

int check_common(fva_plan_t plan, const void* a, const void* b) {
  if (!plan) return fva_fail(FVA_EINVAL, "plan is NULL");
  if (!a || !b) return fva_fail(FVA_EINVAL, "tensor pointer is NULL");
  return FVA_OK;
}

}  // namespace

extern "C" int fva_permute(fva_plan_t plan, const void* x_raster, void* x_perm, int32_t layout,
                           hipStream_t stream) {
  int rc = check_common(plan, x_raster, x_perm);
  if (rc) return rc;
  if (layout != FVA_LAYOUT_ROWS && layout != FVA_LAYOUT_VT)
    return fva_fail(FVA_EINVAL, "unknown layout %d", layout);
  const fva_plan_desc& d = plan->desc;
  const fva_plan_info& in = plan->info;
  const int bh = d.batch * d.heads;
  if (layout == FVA_LAYOUT_ROWS) {
    const int cpr = d.head_dim * plan->esize / 16;
    const int64_t total = in.n_pad * cpr;
    dim3 grid((unsigned)((total + kThreads * kUnroll - 1) / (kThreads * kUnroll)), bh);
    hipLaunchKernelGGL(k_permute_rows, grid, dim3(kThreads), 0, stream, (const uint4*)x_raster,
                       (uint4*)x_perm, plan->perm, in.n_tokens, d.heads, in.n_pad, cpr);
  } else {
    dim3 grid(in.n_blk, bh);
    if (d.dtype == FVA_DTYPE_BF16) {
      if (d.head_dim == 128)
        hipLaunchKernelGGL((k_permute_vt<uint16_t, 128>), grid, dim3(kThreads), 0, stream,
                           (const uint16_t*)x_raster, (uint16_t*)x_perm, plan->perm, in.n_tokens, d.heads, in.n_blk);
      else
        hipLaunchKernelGGL((k_permute_vt<uint16_t, 64>), grid, dim3(kThreads), 0, stream,
                           (const uint16_t*)x_raster, (uint16_t*)x_perm, plan->perm, in.n_tokens, d.heads, in.n_blk);
    } else {
      if (d.head_dim == 128)
        hipLaunchKernelGGL((k_permute_vt<float, 128>), grid, dim3(kThreads), 0, stream,
                           (const float*)x_raster, (float*)x_perm, plan->perm, in.n_tokens, d.heads, in.n_blk);
      else
        hipLaunchKernelGGL((k_permute_vt<float, 64>), grid, dim3(kThreads), 0, stream,
                           (const float*)x_raster, (float*)x_perm, plan->perm, in.n_tokens, d.heads, in.n_blk);
    }
  }
  return fva_after_launch(stream, "fva_permute");
}

extern "C" int fva_permute_pool(fva_plan_t plan, const void* x_raster, void* x_perm, int32_t which,
                                hipStream_t stream) {
  int rc = check_common(plan, x_raster, x_perm);
  if (rc) return rc;
  if (which != FVA_POOL_Q && which != FVA_POOL_K) return fva_fail(FVA_EINVAL, "unknown pooled tensor %d", which);
  const fva_plan_desc& d = plan->desc;
  const fva_plan_info& in = plan->info;
  const bool sub = which == FVA_POOL_K && in.n_sub != 0;
  double* bar = which == FVA_POOL_Q ? plan->qbar : plan->kbar;
  dim3 grid(in.n_blk, d.batch * d.heads);
#define FVA_PP(T, DD, S)                                                                                        \
  hipLaunchKernelGGL((k_permute_pool<T, DD, S>), grid, dim3(kThreads), 0, stream, (const uint4*)x_raster,        \
                     (uint4*)x_perm, plan->perm, in.n_tokens, d.heads, in.n_pad, (int)in.n_blk, plan->blk_cnt,  \
                     plan->sub_pos, plan->sub_cnt, bar)
  if (d.dtype == FVA_DTYPE_BF16) {
    if (d.head_dim == 128) { if (sub) FVA_PP(uint16_t, 128, true); else FVA_PP(uint16_t, 128, false); }
    else { if (sub) FVA_PP(uint16_t, 64, true); else FVA_PP(uint16_t, 64, false); }
  } else {
    if (d.head_dim == 128) { if (sub) FVA_PP(float, 128, true); else FVA_PP(float, 128, false); }
    else { if (sub) FVA_PP(float, 64, true); else FVA_PP(float, 64, false); }
  }
#undef FVA_PP
  plan->pooled |= 1 << which;
  return fva_after_launch(stream, "fva_permute_pool");
}

extern "C" int fva_unpermute(fva_plan_t plan, const void* x_perm, void* x_raster, hipStream_t stream) {
  int rc = check_common(plan, x_perm, x_raster);
  if (rc) return rc;
  const fva_plan_desc& d = plan->desc;
  const fva_plan_info& in = plan->info;
  const int cpr = d.head_dim * plan->esize / 16;
  const int64_t total = in.n_pad * cpr;
  dim3 grid((unsigned)((total + kThreads * kUnroll - 1) / (kThreads * kUnroll)), d.batch * d.heads);
  hipLaunchKernelGGL(k_unpermute_rows, grid, dim3(kThreads), 0, stream, (const uint4*)x_perm,
                     (uint4*)x_raster, plan->perm, in.n_tokens, d.heads, in.n_pad, cpr);
  return fva_after_launch(stream, "fva_unpermute");
}

extern "C" int fva_permute_rope(fva_plan_t plan, const void* x_raster, void* x_perm, int32_t t_offset, double base,
                                hipStream_t stream) {
  int rc = check_common(plan, x_raster, x_perm);
  if (rc) return rc;
  if (t_offset < 0) return fva_fail(FVA_EINVAL, "t_offset %d must be >= 0", t_offset);
  if (!(base > 1.0)) return fva_fail(FVA_EINVAL, "base %g must be > 1", base);
  const fva_plan_desc& d = plan->desc;
  const fva_plan_info& in = plan->info;
  const int T = d.grid[0], Hg = d.grid[1], Wg = d.grid[2], D = d.head_dim;
  const int entries = (T + Hg + Wg) * (D / 2);
  hipLaunchKernelGGL(k_rope_table, dim3((entries + 255) / 256), dim3(256), 0, stream, plan->rope_tab, T, Hg, Wg, D,
                     t_offset, base);
  const int64_t total = in.n_pad * (D * plan->esize / 16);
  dim3 grid((unsigned)((total + kThreads * kRopeUnroll - 1) / (kThreads * kRopeUnroll)), d.batch * d.heads);
  const float inv_w = 1.0f / (float)Wg, inv_h = 1.0f / (float)Hg;
#define FVA_ROPE(TY, DD)                                                                                   \
  hipLaunchKernelGGL((k_permute_rope<TY, DD>), grid, dim3(kThreads), 0, stream, (const uint4*)x_raster,   \
                     (uint4*)x_perm, plan->perm, plan->rope_tab, in.n_tokens, d.heads, in.n_pad, T, Hg, Wg, \
                     inv_w, inv_h)
  if (d.dtype == FVA_DTYPE_BF16) {
    if (D == 128) FVA_ROPE(uint16_t, 128);
    else FVA_ROPE(uint16_t, 64);
  } else {
    if (D == 128) FVA_ROPE(float, 128);
    else FVA_ROPE(float, 64);
  }
#undef FVA_ROPE
  return fva_after_launch(stream, "fva_permute_rope");
}
