// Raster <-> block-order gathers ("Video Sparse Attention" explainer,
// section 3: the tokens of each cube are made contiguous so the fine stage
// runs on whole blocks).  Pure data movement, HBM bound: 16-byte vector
// accesses, each 64-token block row-run read and written contiguously.
#include <hip/hip_runtime.h>

#include "fva_internal.h"

namespace {

constexpr int kThreads = 256;
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

// Key slot order inside one 32-key half of the VT layout: slot s holds key
// 16*c + 8*(j/4) + 4*g + j%4 with c = s/16, g = (s%16)/8, j = s%8.  This is
// the key order in which a 32x32x16 bf16 matrix-core instruction's B-operand
// lanes receive P^T when P^T comes straight from the S^T accumulators, so the
// matching A operand (V^T) is one contiguous 16-byte load per lane.
__device__ __forceinline__ int vt_slot_key(int s) {
  const int c = s >> 4, g = (s >> 3) & 1, j = s & 7;
  return 16 * c + 8 * (j >> 2) + 4 * g + (j & 3);
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
