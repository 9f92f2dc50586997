// Fine stage: block-sparse attention over the selected key blocks only
// ("Video Sparse Attention" explainer, section 3), with online softmax, and
// the one-GPU share of run-time load balancing ("FVAttn" review, section 02):
// rows of very different cost are sorted longest-first into a device work
// list and pulled by a persistent grid, so no compute unit idles while
// another still holds a long row.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "fva_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct AttnArgs {
  const uint16_t* q;        // [B*H, n_pad, D] rows
  const uint16_t* k;        // [B*H, n_pad, D] rows
  const uint16_t* vt;       // [B*H, n_blk, 2, D, 32] VT layout
  const float* qf;          // fp32 variants of the same
  const float* kf;
  const float* vtf;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const uint64_t* blk_mask;
  void* o;
  const int32_t* worklist;
  int32_t* cursor;
  uint64_t* wg_times;
  int64_t n_pad;
  int n_items;
  int n_blk;
  int persistent;
  float scale;              // 1/sqrt(D)
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Next row for this workgroup: from the atomic cursor (persistent) or the
// workgroup index (plain).  Returns -1 when the work list is exhausted.
__device__ __forceinline__ int next_item(const AttnArgs& a, int* s_item, bool first) {
  if (!a.persistent) return first ? (int)blockIdx.x : -1;
  __syncthreads();
  if (threadIdx.x == 0) *s_item = atomicAdd(a.cursor, 1);
  __syncthreads();
  const int it = *s_item;
  return it < a.n_items ? it : -1;
}

// ------------------------------------------------------------------ bf16
// Workgroup = 2 waves = one 64-query block; wave w owns queries 32w..32w+31.
// Per 32-key half of a selected block:
//   S^T (32 keys x 32 queries) = K_half . Q^T     (D/16 MFMA 32x32x16 bf16)
//   online softmax in fp32 on the accumulators (each lane owns one query)
//   O^T (D x 32 queries) += V^T_half . P^T        (D/32 x 2 MFMA)
// P^T feeds the second product straight from the accumulators (the VT key
// slot order makes that consistent).  K and V^T halves are staged through
// LDS with an XOR swizzle so the 16-byte operand reads are conflict free.
template <int D>
__global__ __launch_bounds__(128, 2) void k_attn_bf16(AttnArgs a) {
  constexpr int KS = D / 16;   // k-steps of S^T
  constexpr int DT = D / 32;   // d tiles of O^T
  constexpr int KCH = D / 8;   // 16-byte chunks per K row
  __shared__ uint4 k_lds[32 * KCH];
  __shared__ uint4 v_lds[D * 4];
  __shared__ int s_item;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const uint64_t t0 = wall_clock64();
  const float sl2 = a.scale * 1.44269504088896340736f;   // scores in log2 units
  for (int item = next_item(a, &s_item, true); item >= 0; item = next_item(a, &s_item, false)) {
    const int r = a.worklist[item];
    const int bh = r / a.n_blk;
    const int I = r - bh * a.n_blk;
    const int64_t head = (int64_t)bh * a.n_pad;
    bf16x8 qreg[KS];
    {
      const uint4* qrow = (const uint4*)(a.q + (head + (int64_t)I * 64 + 32 * w + l32) * D);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qreg[ks] = as_bf16x8(qrow[2 * ks + h]);
    }
    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f;
    const int e0 = a.row_ptr[r], e1 = a.row_ptr[r + 1];
    for (int e = e0; e < e1; ++e) {
      const int J = a.col_idx[e];
      if ((unsigned)J >= (unsigned)a.n_blk) continue;   // ids outside the plan are skipped
      const uint64_t mJ = a.blk_mask[J];
      const uint16_t* kblk = a.k + (head + (int64_t)J * 64) * D;
      const uint16_t* vblk = a.vt + (head + (int64_t)J * 64) * D;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t mh = (uint32_t)(mJ >> (32 * u));
        if (mh == 0) continue;   // half holds only pad keys (uniform over the workgroup)
        __syncthreads();
        for (int c = tid; c < 32 * KCH; c += 128) {
          const int row = c / KCH, ch = c % KCH;
          k_lds[row * KCH + (ch ^ (row & 7))] = *(const uint4*)(kblk + (32 * u + row) * D + ch * 8);
        }
        for (int c = tid; c < D * 4; c += 128) {
          const int d = c >> 2, ch = c & 3;
          v_lds[d * 4 + (ch ^ ((d >> 1) & 3))] = *(const uint4*)(vblk + u * 32 * D + d * 32 + ch * 8);
        }
        __syncthreads();
        f32x16 s = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k_lds[l32 * KCH + ((2 * ks + h) ^ (l32 & 7))]),
                                                      qreg[ks], s, 0, 0, 0);
        // s[i]: key 8*(i/4) + 4*h + i%4 of this half, query l32
        float t[16];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 8 * (i >> 2) + 4 * h + (i & 3);
          t[i] = (mh >> key & 1) ? s[i] * sl2 : -INFINITY;
          mx = fmaxf(mx, t[i]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
        m_run = m_new;
        f32x8 p0, p1;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p0[i] = exp2f(t[i] - m_new);
          p1[i] = exp2f(t[8 + i] - m_new);
          l_run += p0[i] + p1[i];
        }
        const bf16x8 pb0 = __builtin_convertvector(p0, bf16x8);
        const bf16x8 pb1 = __builtin_convertvector(p1, bf16x8);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int d = 32 * dt + l32;
          const int sw = (d >> 1) & 3;
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(v_lds[d * 4 + ((0 + h) ^ sw)]), pb0, o[dt], 0, 0, 0);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(v_lds[d * 4 + ((2 + h) ^ sw)]), pb1, o[dt], 0, 0, 0);
        }
      }
    }
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const bool qvalid = a.blk_mask[I] >> (32 * w + l32) & 1;
    uint16_t* orow = (uint16_t*)a.o + (head + (int64_t)I * 64 + 32 * w + l32) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float4 v = make_float4(o[dt][4 * g4] * inv, o[dt][4 * g4 + 1] * inv, o[dt][4 * g4 + 2] * inv,
                               o[dt][4 * g4 + 3] * inv);
        if (!qvalid) v = make_float4(0.f, 0.f, 0.f, 0.f);
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 b = __builtin_convertvector((f32x4{v.x, v.y, v.z, v.w}), bf16x4);
        *(uint2*)(orow + 32 * dt + 8 * g4 + 4 * h) = __builtin_bit_cast(uint2, b);
      }
    }
  }
  if (a.wg_times && tid == 0) {
    a.wg_times[2 * blockIdx.x] = t0;
    a.wg_times[2 * blockIdx.x + 1] = wall_clock64();
  }
}

// ------------------------------------------------------------------ fp32
// Reference-precision path (fp32 throughout).  Workgroup = 256 threads = one
// 64-query block, 4 threads per query each owning D/4 dimensions; keys are
// staged 32 at a time.
template <int D>
__global__ __launch_bounds__(256) void k_attn_f32(AttnArgs a) {
  constexpr int DP = D / 4;
  __shared__ float k_lds[32][D + 1];
  __shared__ float v_lds[32][D + 1];
  __shared__ int s_item;
  const int tid = threadIdx.x;
  const int qi = tid >> 2, part = tid & 3;
  const uint64_t t0 = wall_clock64();
  for (int item = next_item(a, &s_item, true); item >= 0; item = next_item(a, &s_item, false)) {
    const int r = a.worklist[item];
    const int bh = r / a.n_blk;
    const int I = r - bh * a.n_blk;
    const int64_t head = (int64_t)bh * a.n_pad;
    float q[DP], o[DP];
    const float* qrow = a.qf + (head + (int64_t)I * 64 + qi) * D + part * DP;
#pragma unroll
    for (int d = 0; d < DP; ++d) {
      q[d] = qrow[d];
      o[d] = 0.0f;
    }
    float m_run = -INFINITY, l_run = 0.0f;
    const int e0 = a.row_ptr[r], e1 = a.row_ptr[r + 1];
    for (int e = e0; e < e1; ++e) {
      const int J = a.col_idx[e];
      if ((unsigned)J >= (unsigned)a.n_blk) continue;   // ids outside the plan are skipped
      const uint64_t mJ = a.blk_mask[J];
      for (int u = 0; u < 2; ++u) {
        const uint32_t mh = (uint32_t)(mJ >> (32 * u));
        if (mh == 0) continue;   // uniform: the half holds only pad keys
        const float* kblk = a.kf + (head + (int64_t)J * 64 + 32 * u) * D;
        const float* vblk = a.vtf + (head + (int64_t)J * 64) * D + u * 32 * D;
        __syncthreads();
        for (int c = tid; c < 32 * D; c += 256) {
          const int key = c / D, d = c - key * D;
          k_lds[key][d] = kblk[c];
          // VT element (d, slot) of this half -> V[key][d]
          const int dv = c >> 5, sl = c & 31;
          const int cc = sl >> 4, g = (sl >> 3) & 1, j = sl & 7;
          v_lds[16 * cc + 8 * (j >> 2) + 4 * g + (j & 3)][dv] = vblk[c];
        }
        __syncthreads();
        float sc[32];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          float acc = 0.0f;
#pragma unroll
          for (int d = 0; d < DP; ++d) acc = fmaf(q[d], k_lds[j][part * DP + d], acc);
          acc += __shfl_xor(acc, 1);
          acc += __shfl_xor(acc, 2);
          sc[j] = (mh >> j & 1) ? acc * a.scale : -INFINITY;
          mx = fmaxf(mx, sc[j]);
        }
        const float m_new = fmaxf(m_run, mx);
        const float alpha = expf(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < DP; ++d) o[d] *= alpha;
        m_run = m_new;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const float pj = expf(sc[j] - m_new);
          l_run += pj;
#pragma unroll
          for (int d = 0; d < DP; ++d) o[d] = fmaf(pj, v_lds[j][part * DP + d], o[d]);
        }
      }
    }
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    const bool qvalid = a.blk_mask[I] >> qi & 1;
    float* orow = (float*)a.o + (head + (int64_t)I * 64 + qi) * D + part * DP;
#pragma unroll
    for (int d = 0; d < DP; ++d) orow[d] = qvalid ? o[d] * inv : 0.0f;
  }
  if (a.wg_times && tid == 0) {
    a.wg_times[2 * blockIdx.x] = t0;
    a.wg_times[2 * blockIdx.x + 1] = wall_clock64();
  }
}

// ------------------------------------------------------------------ schedule
// Counting sort of rows by cost (kept blocks), longest first, into the work
// list; resets the work-queue cursor.  One workgroup.
__global__ __launch_bounds__(1024) void k_sched(const int32_t* __restrict__ row_ptr, int64_t n_rows, int n_blk,
                                                int32_t* __restrict__ worklist, int32_t* __restrict__ cursor) {
  __shared__ int hist[FVA_MAX_NBLK + 1];
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int nb = n_blk + 1;
  for (int i = tid; i < nb; i += 1024) hist[i] = 0;
  __syncthreads();
  for (int64_t r = tid; r < n_rows; r += 1024) {
    const int c = min(max(row_ptr[r + 1] - row_ptr[r], 0), n_blk);
    atomicAdd(&hist[n_blk - c], 1);   // bin 0 = most expensive
  }
  __syncthreads();
  const int per = (nb + 1023) / 1024;
  const int b0 = min(tid * per, nb), b1 = min(b0 + per, nb);
  int s = 0;
  for (int i = b0; i < b1; ++i) s += hist[i];
  part[tid] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (int i = b0; i < b1; ++i) {
    const int c = hist[i];
    hist[i] = run;
    run += c;
  }
  __syncthreads();
  for (int64_t r = tid; r < n_rows; r += 1024) {
    const int c = min(max(row_ptr[r + 1] - row_ptr[r], 0), n_blk);
    const int pos = atomicAdd(&hist[n_blk - c], 1);
    worklist[pos] = (int32_t)r;
  }
  if (tid == 0) *cursor = 0;
}

template <typename K>
int occupancy(K kernel, int threads) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, 0) != hipSuccess || nb < 1) nb = 1;
  return nb;
}

}  // namespace

extern "C" int fva_attention(fva_plan_t plan, const void* q_perm, const void* k_perm, const void* vt_perm,
                             const int32_t* row_ptr, const int32_t* col_idx, void* o_perm, int32_t sched_mode,
                             uint64_t* wg_times, hipStream_t stream) {
  if (!plan) return fva_fail(FVA_EINVAL, "plan is NULL");
  if (!q_perm || !k_perm || !vt_perm || !o_perm) return fva_fail(FVA_EINVAL, "tensor pointer is NULL");
  if (!row_ptr || !col_idx) return fva_fail(FVA_EINVAL, "row_ptr / col_idx is NULL");
  if (sched_mode != FVA_SCHED_PERSISTENT && sched_mode != FVA_SCHED_PLAIN)
    return fva_fail(FVA_EINVAL, "unknown sched_mode %d", sched_mode);
  const fva_plan_desc& d = plan->desc;
  const fva_plan_info& in = plan->info;
  hipLaunchKernelGGL(k_sched, dim3(1), dim3(1024), 0, stream, row_ptr, in.n_rows, in.n_blk, plan->worklist,
                     plan->counters);
  AttnArgs a{};
  a.q = (const uint16_t*)q_perm;
  a.k = (const uint16_t*)k_perm;
  a.vt = (const uint16_t*)vt_perm;
  a.qf = (const float*)q_perm;
  a.kf = (const float*)k_perm;
  a.vtf = (const float*)vt_perm;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.blk_mask = plan->blk_mask;
  a.o = o_perm;
  a.worklist = plan->worklist;
  a.cursor = plan->counters;
  a.wg_times = wg_times;
  a.n_pad = in.n_pad;
  a.n_items = (int)in.n_rows;
  a.n_blk = in.n_blk;
  a.persistent = sched_mode == FVA_SCHED_PERSISTENT;
  a.scale = 1.0f / sqrtf((float)d.head_dim);

#define FVA_LAUNCH(KERNEL, THREADS)                                                              \
  do {                                                                                           \
    int grid = (int)in.n_rows;                                                                   \
    if (a.persistent)                                                                            \
      grid = (int)std::min<int64_t>(std::min<int64_t>(in.n_rows, in.max_wg),                     \
                                    (int64_t)plan->num_cu * occupancy(KERNEL, THREADS));         \
    hipLaunchKernelGGL(KERNEL, dim3(grid), dim3(THREADS), 0, stream, a);                        \
  } while (0)
  if (d.dtype == FVA_DTYPE_BF16) {
    if (d.head_dim == 128) FVA_LAUNCH(k_attn_bf16<128>, 128);
    else FVA_LAUNCH(k_attn_bf16<64>, 128);
  } else {
    if (d.head_dim == 128) FVA_LAUNCH(k_attn_f32<128>, 256);
    else FVA_LAUNCH(k_attn_f32<64>, 256);
  }
#undef FVA_LAUNCH
  return fva_after_launch(stream, "fva_attention");
}
