// Coarse stage and routing:
//   pool   - "Video Sparse Attention" explainer, dialogue and section 3
//            (pooled (4,4,4) tiles), "DFSAttn" explainer trick 2 (sub-blocks)
//   score  - pooled q_bar . k_bar / sqrt(D) in fp64, softmax over key blocks
//   select - "FVAttn" review, sections 00 and 02: adaptive Top-p with a
//            Top-k safety floor, emitted as CSR block lists
//   slack  - "FVAttn" section 02 slack-aware augmentation, one-GPU reading:
//            light heads are filled up to the median head's block count
#include <hip/hip_runtime.h>

#include <cmath>

#include "fva_internal.h"

namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ helpers
__device__ __forceinline__ float ld_elem(const uint16_t* p) {
  return __uint_as_float((uint32_t)(*p) << 16);
}
__device__ __forceinline__ float ld_elem(const float* p) { return *p; }

// Selection view of a score: NaN and s <= 0 -> +0, s > 1 -> 1; returns bits.
__device__ __forceinline__ uint32_t clamp_bits(float s) {
  if (!(s > 0.0f)) return 0u;
  if (s >= 1.0f) return 0x3F800000u;
  return __float_as_uint(s);
}

// floor(s * 2^47) for the fp32 value with bits b in [0, 1], exactly.
__device__ __forceinline__ uint64_t fix_mass(uint32_t b) {
  if (b == 0) return 0;
  const uint32_t e = b >> 23;
  const uint64_t mant = (b & 0x7FFFFFu) | (e ? 0x800000u : 0u);
  const int sh = (int)(e ? e : 1) - 103;
  if (sh >= 0) return mant << sh;
  return sh > -64 ? (mant >> (-sh)) : 0;
}

__device__ __forceinline__ uint64_t p_threshold(float p) {
  // ceil(p * 2^47): exact, p is an fp32 value in (0, 1).
  return (uint64_t)ceil((double)p * 140737488355328.0);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// Inclusive wave prefix sum with DPP moves (no LDS traffic): row_shr 1, 2,
// 4, 8 scan each row of 16 lanes, then row_bcast 15 and 31 carry the row
// totals into the rows above.  Lanes a DPP move cannot source read 0.
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x, int ctrl_id) {
  switch (ctrl_id) {
    case 0: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);   // row_shr:1
    case 1: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);   // row_shr:2
    case 2: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);   // row_shr:4
    case 3: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);   // row_shr:8
    case 4: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);   // row_bcast:15
    default: return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  }
}
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v, int lane) {
  (void)lane;
#pragma unroll
  for (int c = 0; c < 6; ++c) {
    if constexpr (sizeof(T) == 8) {
      const uint64_t u = (uint64_t)v;
      const uint64_t t = ((uint64_t)dpp_u32((uint32_t)(u >> 32), c) << 32) | dpp_u32((uint32_t)u, c);
      v = (T)(u + t);
    } else {
      v = (T)((uint32_t)v + dpp_u32((uint32_t)v, c));
    }
  }
  return v;
}
// The value of lane `src` (wave-uniform) of x.
template <typename T>
__device__ __forceinline__ T lane_value(T x, int src) {
  if constexpr (sizeof(T) == 8) {
    const uint64_t u = (uint64_t)x;
    return (T)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(u >> 32), src) << 32) |
               (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, src));
  } else {
    return (T)__builtin_amdgcn_readlane((int)x, src);
  }
}

// The values of lanes l and l^16 (X = 16) or l and l^32 (X = 32) of an fp64
// x, in some order, without an LDS round trip: v_permlane16/32_swap of each
// 32-bit half with itself.  Max and sum of the pair are then exact and
// symmetric, the same bits as combining x with __shfl_xor(x, X).
template <int X>
__device__ __forceinline__ void lane_pair(double x, double& a, double& b) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  uint32_t l0, l1, h0, h1;
  if constexpr (X == 16) {
    const auto rl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto rh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    l0 = rl[0], l1 = rl[1], h0 = rh[0], h1 = rh[1];
  } else {
    const auto rl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto rh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    l0 = rl[0], l1 = rl[1], h0 = rh[0], h1 = rh[1];
  }
  a = __builtin_bit_cast(double, ((uint64_t)h0 << 32) | l0);
  b = __builtin_bit_cast(double, ((uint64_t)h1 << 32) | l1);
}
template <int X>
__device__ __forceinline__ double pair_max(double x) {
  double a, b;
  lane_pair<X>(x, a, b);
  return fmax(a, b);
}
template <int X>
__device__ __forceinline__ double pair_sum(double x) {
  double a, b;
  lane_pair<X>(x, a, b);
  return a + b;
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------------ pool
// Mean of the 64 rows of one block (pads are zero rows, so the sum over all
// rows is the sum over valid rows), divided by the valid count, in fp64.
// One wave per (block, b*h, tensor), four blocks per workgroup; lanes own
// 16-byte column chunks of interleaved rows.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_pool(const T* __restrict__ q, const T* __restrict__ k,
                                              double* __restrict__ qbar, double* __restrict__ kbar,
                                              const int32_t* __restrict__ blk_cnt, int n_blk, int64_t n_pad) {
  constexpr int EPC = 16 / sizeof(T);   // elements per 16-byte chunk
  constexpr int CPR = D / EPC;          // chunks per row
  constexpr int RG = 64 / CPR;          // row groups
  __shared__ double part_all[4][RG][D];
  const int wv = threadIdx.x >> 6;
  const int blk = blockIdx.x * 4 + wv, bh = blockIdx.y;
  if (blk >= n_blk) return;             // whole wave; only wave-level syncs below
  double (*part)[D] = part_all[wv];
  const T* src = (blockIdx.z == 0 ? q : k) + ((int64_t)bh * n_pad + (int64_t)blk * 64) * D;
  double* dst = (blockIdx.z == 0 ? qbar : kbar) + ((int64_t)bh * n_blk + blk) * D;
  const int lane = threadIdx.x & 63;
  const int ch = lane % CPR, g = lane / CPR;
  double acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
  // 16-byte loads, eight rows in flight per lane before they are summed
  constexpr int RPL = 64 / RG;          // rows per lane
  constexpr int BATCH = RPL < 8 ? RPL : 8;
  const uint4* src16 = (const uint4*)src;
#pragma unroll
  for (int r0 = 0; r0 < RPL; r0 += BATCH) {
    uint4 v[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) v[i] = src16[(g + (r0 + i) * RG) * CPR + ch];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const T* e16 = (const T*)&v[i];
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] += (double)ld_elem(e16 + e);
    }
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) part[g][ch * EPC + e] = acc[e];
  wave_sync_lds();
  const double cnt = (double)blk_cnt[blk];
  for (int d = lane; d < D; d += 64) {
    double s = 0.0;
#pragma unroll
    for (int gg = 0; gg < RG; ++gg) s += part[gg][d];
    dst[d] = s / cnt;
  }
}

// Sub-block means of K ("DFSAttn" trick 2), fp64: kbar[(bh, blk, s), :] =
// mean of the valid rows of sub-block s; an empty sub-block gets zeros (its
// logit is masked by the score kernel through sub_cnt).
template <typename T, int D>
__global__ __launch_bounds__(64) void k_pool_sub(const T* __restrict__ k, double* __restrict__ kbar,
                                                 const uint8_t* __restrict__ sub_pos,
                                                 const int32_t* __restrict__ sub_cnt, int n_blk,
                                                 int64_t n_pad) {
  const int blk = blockIdx.x, bh = blockIdx.y;
  const T* src = k + ((int64_t)bh * n_pad + (int64_t)blk * 64) * D;
  double* dst = kbar + ((int64_t)bh * n_blk + blk) * 8 * D;
  for (int e = threadIdx.x; e < 8 * D; e += 64) {
    const int s = e / D, d = e - s * D;
    const uint8_t* pos = sub_pos + ((int64_t)blk * 8 + s) * 8;
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += (double)ld_elem(src + (int64_t)pos[i] * D + d);
    const int c = sub_cnt[blk * 8 + s];
    dst[e] = c ? acc / (double)c : 0.0;
  }
}

// exp(x) for x <= 0, in fp64 with a 64-entry table: x = k ln2/64 + r,
// |r| <= ln2/128, with ln2/64 split in a 32-bit head (k * head exact for
// |k| < 2^20) and a tail; exp(r) by its degree-5 Taylor polynomial
// (remainder below 4e-17); exp(x) = 2^(k >> 6) * tab[k & 63] * exp(r) with
// tab[j] = 2^(j/64), the power of two added to the exponent field as an
// integer.  Arguments below -700 (and -inf) are taken as -700, so the result
// stays a normal number: exp(-700) ~ 1e-304 in place of a smaller value or
// 0, which changes no sum of at least 1 and no score rounded to fp32.  About
// 12 fp64 instructions against about 20 for the library exp, within 5e-16
// relative (tests/test_host_fp64_math.py restates it on the host).
__device__ __forceinline__ double exp_neg(double x, const double* tab) {
  const double xc = fmax(x, -700.0);
  const double k = __builtin_rint(xc * 92.33248261689366);          // 64 / ln 2
  double r = fma(-k, 0.010830424695086549, xc);                     // head of ln 2 / 64
  r = fma(-k, 1.162596423439437e-12, r);                            // tail of ln 2 / 64
  double p = fma(r, 1.0 / 120.0, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  const int ki = (int)k;
  const double v = tab[ki & 63] * p;   // in [0.99, 2.02]: normal
  return __longlong_as_double(__double_as_longlong(v) + ((long long)(ki >> 6) << 52));
}

// tab[j] = 2^(j/64) for exp_neg; filled by the first 64 threads (callers
// synchronise before use).
__device__ __forceinline__ void exp_neg_table(double* tab) {
  if (threadIdx.x < 64) tab[threadIdx.x] = exp2((double)threadIdx.x / 64.0);
}

// log(x) for finite x >= 1 in fp64 with a 128-entry table: x = 2^k m with m
// in [1, 2) taken from the bits; c = m cut to 7 fractional bits, so m - c is
// exact and r = (m - c) / c lies in [0, 2^-7); log x = k ln 2 + log c +
// log1p(r), with 1/c and log c from the table (tab[2j], tab[2j+1] for
// c = 1 + j/128), log1p(r) by its degree-7 Taylor polynomial (remainder below
// 2e-18) and ln 2 split in a head exact in k * head and a tail.  About 13
// fp64 instructions against about 75 for the library log; within 4e-16 of
// log x on [1, 8], exactly 0 at x = 1 (tests/test_host_fp64_math.py restates
// it on the host).
__device__ __forceinline__ double log_ge1(double x, const double* tab) {
  const uint64_t xb = (uint64_t)__double_as_longlong(x);
  const uint32_t hx = (uint32_t)(xb >> 32);
  const int k = (int)(hx >> 20) - 1023;
  const uint32_t hm = (hx & 0x000FFFFFu) | 0x3FF00000u;
  const double m = __longlong_as_double((long long)(((uint64_t)hm << 32) | (uint32_t)xb));
  const double c = __longlong_as_double((long long)((uint64_t)(hm & 0xFFFFE000u) << 32));
  const int j = (int)(hx >> 13) & 127;
  const double2 t = *(const double2*)(tab + 2 * j);
  const double r = (m - c) * t.x;
  double q = fma(1.0 / 7.0, r, -1.0 / 6.0);
  q = fma(q, r, 1.0 / 5.0);
  q = fma(q, r, -0.25);
  q = fma(q, r, 1.0 / 3.0);
  q = fma(q, r, -0.5);
  q = fma(q, r, 1.0);
  const double kd = (double)k;
  return fma(kd, 0.6931471803691238, fma(kd, 1.9082149292705877e-10, t.y + q * r));
}

// tab for log_ge1: tab[2j] = 1 / (1 + j/128), tab[2j+1] = log(1 + j/128);
// filled by the first 128 threads (callers synchronise before use).
__device__ __forceinline__ void log_ge1_table(double* tab) {
  if (threadIdx.x < 128) {
    const double c = 1.0 + (double)threadIdx.x / 128.0;
    tab[2 * threadIdx.x] = 1.0 / c;
    tab[2 * threadIdx.x + 1] = log1p((double)threadIdx.x / 128.0);
  }
}

// ------------------------------------------------------------------ score
// Block logits Y[bh, i, j] = q_bar_i . k_bar_j / sqrt(D) in fp64 (with
// sub-blocks: the log-sum-exp over the non-empty sub-blocks of j, which makes
// exp(Y) the sum of the sub-block terms), plus the row max of Y.
// fp64 matrix cores (v_mfma_f64_16x16x4_f64).  Workgroup = 4 waves, each
// wave one 16-query tile; every wave sweeps the 16-key tiles of its
// workgroup's key range (gridDim.z ranges split the tiles evenly, so the grid
// fills whole rounds of the compute units), computing Z^T = Kbar . Qbar^T so
// that lane l owns query l%16 and keys l/16 + 4*i.  Each range writes its
// own row max (rowmax[range][row]); the selection takes their maximum.
// fp64 keeps the logits exact to ~1e-15, so the fp32 scores the selection
// reads carry only their final rounding.
template <bool SUB, int D>
__global__ __launch_bounds__(256, 3) void k_score(const double* __restrict__ qbar, const double* __restrict__ kbar,
                                               const int32_t* __restrict__ sub_cnt, double* __restrict__ y,
                                               double* __restrict__ rowmax, int n_blk, double scale) {
  constexpr int QD = D / 4;   // d values per lane group (k-steps of 4)
  const int bh = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int q0 = blockIdx.x * 64 + w * 16;   // a wave past the last query still helps load keys
  const int qi = q0 + l16;
  const bool qvalid = qi < n_blk;
  const int nkeys = SUB ? n_blk * 8 : n_blk;
  const int ntiles = (nkeys + 15) / 16;
  // this workgroup's key tiles [t0, t1) and logit columns [c0, c1)
  const int t0 = (int)((int64_t)ntiles * blockIdx.z / gridDim.z);
  const int t1 = (int)((int64_t)ntiles * (blockIdx.z + 1) / gridDim.z);
  const int c0 = SUB ? 2 * t0 : 16 * t0, c1 = min(SUB ? 2 * t1 : 16 * t1, n_blk);
  double qv[QD];
  {
    const double2* src = (const double2*)(qbar + ((int64_t)bh * n_blk + min(qi, n_blk - 1)) * D + QD * g);
#pragma unroll
    for (int c = 0; c < QD / 2; ++c) {
      const double2 t = src[c];
      qv[2 * c] = t.x, qv[2 * c + 1] = t.y;
    }
  }
  // Key tiles (16 keys x D) are shared by the workgroup's four waves through
  // a double-buffered LDS tile: each thread prefetches its share of tile
  // kt+1 into registers while tile kt is multiplied, then stores it.
  constexpr int KS = D + 2;                        // padded LDS row (doubles)
  constexpr int KV = 16 * D / 2 / 256;             // double2 per thread per tile
  __shared__ double ks_lds[2][16][KS];
  const double* kh = kbar + (int64_t)bh * nkeys * D;
  // The tile in flight is a value returned by kfetch and consumed by kstore
  // in the same iteration, fetched unconditionally (the last iteration
  // re-reads the last tile into the idle buffer), so it stays in registers:
  // an array kept across the loop with conditional writes ended up in
  // scratch memory, and every prefetch then waited for its loads at once.
  struct KTile { double2 v[KV]; };
  // The last tile may run up to 15 rows past the head's keys: those rows are
  // read (the workspace keeps slack rows behind the pooled keys) and their
  // logits masked, so the loads need no per-lane clamp, only a wave-uniform
  // tile base plus a fixed lane offset.
  auto kfetch = [&](int kt) -> KTile {
    KTile t;
    const double* tb = kh + (int64_t)min(kt, ntiles - 1) * 16 * D;
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int e = threadIdx.x + 256 * v;         // double2 index within the tile
      const int r = e / (D / 2), d2 = e - r * (D / 2);
      t.v[v] = *(const double2*)(tb + r * D + 2 * d2);
    }
    return t;
  };
  auto kstore = [&](int buf, const KTile& t) {
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int e = threadIdx.x + 256 * v;
      const int r = e / (D / 2), d2 = e - r * (D / 2);
      *(double2*)&ks_lds[buf][r][2 * d2] = t.v[v];
    }
  };
  // non-empty sub-blocks of every block, one byte per block (bit s: sub-block s)
  __shared__ uint8_t sub_ok[SUB ? FVA_MAX_NBLK : 1];
  if (SUB)
    for (int j = threadIdx.x; j < n_blk; j += 256) {
      uint32_t mbits = 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) mbits |= (sub_cnt[j * 8 + t] > 0 ? 1u : 0u) << t;
      sub_ok[j] = (uint8_t)mbits;
    }
  __shared__ double exp_tab[64];
  exp_neg_table(exp_tab);
  __shared__ __attribute__((aligned(16))) double log_tab[SUB ? 256 : 2];
  if (SUB) log_ge1_table(log_tab);
  kstore(t0 & 1, kfetch(t0));
  __syncthreads();
  // Logits go out through a per-wave LDS tile of 16 query rows x YC block
  // columns, written back as YC * 8-byte row pieces, 64 / YC rows per store.
  // The tile is kept that small so three workgroups fit the LDS of a
  // compute unit.
  constexpr int YC = SUB ? 16 : 32;
  constexpr int TPF = SUB ? YC / 2 : YC / 16;   // key tiles per flush
  __shared__ double yt[4][16][YC + 1];
  double* yw = y + ((int64_t)bh * n_blk + q0) * n_blk;
  auto flush = [&](int kt) {
    wave_sync_lds();
    const int j = (kt / TPF) * YC + lane % YC;   // only this range's columns of the group
#pragma unroll
    for (int q2 = 0; q2 < 16; q2 += 64 / YC) {
      const int q = q2 + lane / YC;
      if (q0 + q < n_blk && j >= c0 && j < c1) yw[(int64_t)q * n_blk + j] = yt[w][q][lane % YC];
    }
    wave_sync_lds();
  };
  double m_run = -INFINITY;
  double c_held = -INFINITY, e_held = 0.0;   // block max and sum of a held even tile (sub-blocks)
  // The products of tile kt run on the matrix cores while the same wave does
  // the fp64 log-sum-exp of tile kt-1 (independent work, so the two overlap
  // inside the wave): the loop carries the previous tile's accumulator.
  // With sub-blocks the tile's rows are read permuted, row r of the product
  // taking sub-key 4 (r % 4) + r / 4: lane group g then holds sub-keys
  // 4g..4g+3, half of one block, so a block's log-sum-exp needs one exchange
  // between lane groups g and g ^ 1 instead of two rounds over all four.
  const int arow = SUB ? 4 * (l16 & 3) + (l16 >> 2) : l16;
  auto products = [&](int kt) __attribute__((always_inline)) -> f64x4 {
    const double2* ks = (const double2*)&ks_lds[kt & 1][arow][QD * g];
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int c = 0; c < QD / 2; ++c) {
      const double2 a = ks[c];
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a.x, qv[2 * c], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a.y, qv[2 * c + 1], acc, 0, 0, 0);
    }
    return acc;
  };
  // acc[i]: key kt*16 + g + 4*i, query l16 (fp64 16x16x4 accumulator layout).
  // Only the row max is kept here: the selection kernel takes every
  // exponential of the row anyway and sums them there, so the score kernel's
  // fp64 vector work (which does not overlap its fp64 products) stays small.
  auto lse = [&](int kt, const f64x4& acc) __attribute__((always_inline)) {
    if (!SUB) {
      double yv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = kt * 16 + g + 4 * i;
        yv[i] = j < n_blk ? acc[i] * scale : -INFINITY;
        m_run = fmax(m_run, yv[i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) yt[w][l16][(kt % TPF) * 16 + g + 4 * i] = yv[i];
    } else {
      // acc[i] is sub-key 4g + i of the tile: sub-block 4 (g % 2) + i of
      // block kt*2 + g/2.  Log-sum-exp over the block's 8 sub-blocks (4 per
      // lane, lane groups g and g ^ 1): the max first, then one exponential
      // per sub-block.  Lane groups g and g ^ 1 then hold the same block
      // max c and sum e, so a tile's log would be taken twice: an even tile
      // keeps (c, e) instead, and the next (odd) tile takes one log for
      // both, the even lane groups for the held tile's blocks and the odd
      // ones for its own.  A tile with no partner in the range (first and
      // odd, or last and even) takes its own log.
      const int blk = kt * 2 + (g >> 1);
      const uint32_t ok = blk < n_blk ? (uint32_t)sub_ok[blk] >> (4 * (g & 1)) : 0u;
      double v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (ok >> i & 1) ? acc[i] * scale : -INFINITY;
      double c = fmax(fmax(v[0], v[1]), fmax(v[2], v[3]));
      c = pair_max<16>(c);
      const double e4 = (exp_neg(v[0] - c, exp_tab) + exp_neg(v[1] - c, exp_tab)) +
                        (exp_neg(v[2] - c, exp_tab) + exp_neg(v[3] - c, exp_tab));
      double e = c > -INFINITY ? e4 : 0.0;
      e = pair_sum<16>(e);
      const bool even = (kt & 1) == 0;
      if (even && kt + 1 < t1) {   // hold for the next tile's log
        c_held = c;
        e_held = e;
        return;
      }
      const bool pair = !even && kt > t0;   // an even tile is held
      const bool mine = !pair || (g & 1);    // this lane's log is for its own tile
      const double cc = mine ? c : c_held, ee = mine ? e : e_held;
      // e >= 1 (the max term is 1) whenever the block has a sub-block
      const double lg = cc + log_ge1(cc > -INFINITY ? ee : 1.0, log_tab);
      const double yo = (pair || (g & 1) == 0) && cc > -INFINITY ? lg : -INFINITY;
      m_run = fmax(m_run, yo);
      if (!pair) {
        if ((g & 1) == 0) yt[w][l16][(kt % TPF) * 2 + (g >> 1)] = yo;
      } else {   // even lane groups: the held tile kt - 1; odd ones: tile kt
        yt[w][l16][(((g & 1) ? kt : kt - 1) % TPF) * 2 + (g >> 1)] = yo;
      }
    }
  };
  f64x4 acc_prev = products(t0);
  {
    const KTile nxt = kfetch(t0 + 1);
    kstore((t0 + 1) & 1, nxt);
    __syncthreads();
  }
  for (int kt = t0 + 1; kt < t1; ++kt) {
    const KTile nxt = kfetch(kt + 1);
    const f64x4 acc = products(kt);
    lse(kt - 1, acc_prev);
    if ((kt - 1) % TPF == TPF - 1) flush(kt - 1);
    kstore((kt + 1) & 1, nxt);
    __syncthreads();
    acc_prev = acc;
  }
  lse(t1 - 1, acc_prev);
  flush(t1 - 1);
  // the row max over the four lane groups that share query l16
  m_run = pair_max<32>(pair_max<16>(m_run));
  if (g == 0 && qvalid) rowmax[(int64_t)blockIdx.z * gridDim.y * n_blk + (int64_t)bh * n_blk + qi] = m_run;
}

// ------------------------------------------------------------------ select
// One wave per row (b, h, I).  Scores are either computed from the fp64
// block logits (S = exp(y - max) / sum in fp64, rounded once to fp32) or
// read from scores_in.  The kept set
// is the shortest prefix in (score desc, id asc) order whose fixed-point
// mass reaches p, extended to the floor min(k_min, n).  It is found by an
// MSD radix select over the 48-bit key (score bits << 16 | (0xFFFF - J)),
// starting below its always-zero sign bit so the first digit is the score's
// exponent: each level builds a 256-bin histogram of mass and count in LDS
// (prefix sums across the wave by DPP row shifts and broadcasts), keeps the
// bin where the mass target or the count target is crossed, and as soon as
// that bin holds <= 64 keys they are sorted across the wave (bitonic) and the
// exact cut is read off a prefix sum.  Output: a bitmask of kept ids per row
// and the kept count.
// Ten mask words (up to 640 blocks, the 480P shapes) fit four waves per SIMD
// in 128 VGPRs (2 of them spilled); the selection then took
// 0.87 instead of 0.90 ms at the Wan-14B 480P shape, lists unchanged.  Wider
// rows keep the compiler's choice: forcing four waves spills 23 and more.
template <int NI>
__global__ __launch_bounds__(256, NI == 10 ? 4 : 1) void k_select(const double* __restrict__ z, const double* __restrict__ rowmax,
                                                int nsplit,
                                                const float* __restrict__ scores_in, float* __restrict__ s_out,
                                                SelectArgs pa, int p_count, int k_min, int n_blk,
                                                int64_t n_rows, int32_t* __restrict__ rowcnt,
                                                uint64_t* __restrict__ rowmask, int nw) {
  // two copies of each wave's histograms (even and odd lanes), which halves
  // the same-bin atomics of one instruction: at the first level the digit
  // is the score's exponent, shared by many lanes
  __shared__ unsigned long long hmass[4][2][256];
  __shared__ unsigned int hcnt[4][2][256];
  __shared__ unsigned long long lkey[4][64];
  __shared__ double exp_tab[64];
  exp_neg_table(exp_tab);
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wv;
  if (r >= n_rows) return;
  const int n = n_blk;
  const int bh = (int)(r / n);
  const float p = pa.p[p_count == 1 ? 0 : bh];

  uint32_t bits[NI];
  {
    const float* sr = scores_in ? scores_in + r * n : nullptr;
    float* so = s_out ? s_out + r * n : nullptr;
    if (sr) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int j = lane + 64 * i;
        bits[i] = 0;
        if (j < n) {
          const float s = sr[j];
          if (so) so[j] = s;
          bits[i] = clamp_bits(s);
        }
      }
    } else {
      // S_j = exp(y_j - max) / sum_j' exp(y_j' - max): the exponentials in
      // fp64 against the row max, their sum per lane in slot order and then
      // across the wave by a butterfly (commutative pairwise adds, so every
      // lane holds the same sum), each score rounded once to fp32
      double m = rowmax[r];
      for (int sp = 1; sp < nsplit; ++sp) m = fmax(m, rowmax[sp * n_rows + r]);
      const double* zr = z + r * n;
      double e[NI];
      double sl = 0.0;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int j = lane + 64 * i;
        e[i] = j < n ? exp_neg(zr[j] - m, exp_tab) : 0.0;
        sl += e[i];
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) sl += __shfl_xor(sl, o);
      const double inv = 1.0 / sl;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int j = lane + 64 * i;
        bits[i] = 0;
        if (j < n) {
          const float s = (float)(e[i] * inv);
          if (so) so[j] = s;
          bits[i] = clamp_bits(s);
        }
      }
    }
  }
  auto key_of = [&](int i) -> uint64_t {
    return ((uint64_t)bits[i] << 16) | (uint64_t)(0xFFFF - (lane + 64 * i));
  };

  uint64_t thr = 0;   // keep ids whose key >= thr
  int kept = n;
  const int kf = min(k_min, n);
  if (p < 1.0f) {
    uint64_t needP = p_threshold(p);
    int needF = kf;
    bool useP = true, useF = kf > 0;
    int kAbove = 0;
    uint64_t active = 0;   // bit i: element i of this lane still a candidate
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (lane + 64 * i < n) active |= 1ull << i;
    bool all = false;
    for (int level = 0; level < 6; ++level) {
      // key bit 47 (the score's sign) is 0 for every clamped score, so the
      // levels take bits 46..39, 38..31, ..., 14..7, then 7..0 (bit 7 is
      // already fixed by the prefix there): the first digit is the whole
      // exponent, which splits a row over more bins than sign + 7 bits
      const int shift = level < 5 ? 39 - 8 * level : 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        hmass[wv][0][lane * 4 + t] = 0;
        hmass[wv][1][lane * 4 + t] = 0;
        hcnt[wv][0][lane * 4 + t] = 0;
        hcnt[wv][1][lane * 4 + t] = 0;
      }
      wave_sync_lds();
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (active >> i & 1) {
          const int dg = 255 - (int)((key_of(i) >> shift) & 0xFF);
          atomicAdd(&hmass[wv][lane & 1][dg], (unsigned long long)fix_mass(bits[i]));
          atomicAdd(&hcnt[wv][lane & 1][dg], 1u);
        }
      }
      wave_sync_lds();
      uint64_t bm[4];
      uint32_t bc[4];
      uint64_t lm = 0;
      uint32_t lc = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bm[t] = hmass[wv][0][lane * 4 + t] + hmass[wv][1][lane * 4 + t];
        bc[t] = hcnt[wv][0][lane * 4 + t] + hcnt[wv][1][lane * 4 + t];
        lm += bm[t];
        lc += bc[t];
      }
      const uint64_t mi = wave_incl_scan<uint64_t>(lm, lane);
      const uint32_t ci = wave_incl_scan<uint32_t>(lc, lane);
      const uint64_t mtot = lane_value(mi, 63);
      if (level == 0 && useP && mtot < needP) {   // total mass never reaches p: keep all
        all = true;
        break;
      }
      // crossing bins for each live criterion (bin index, -1 when unused)
      int bP = -1, bF = -1;
      {
        uint64_t me = mi - lm;
        uint32_t ce = ci - lc;
        int myP = -1, myF = -1;
        if (useP && me < needP && mi >= needP) {
          uint64_t a = me;
          for (int t = 0; t < 4; ++t) {
            a += bm[t];
            if (a >= needP) { myP = lane * 4 + t; break; }
          }
        }
        if (useF && (int)ce < needF && (int)ci >= needF) {
          uint32_t a = ce;
          for (int t = 0; t < 4; ++t) {
            a += bc[t];
            if ((int)a >= needF) { myF = lane * 4 + t; break; }
          }
        }
        const uint64_t vp = __ballot(myP >= 0), vf = __ballot(myF >= 0);
        if (vp) bP = lane_value(myP, __ffsll((unsigned long long)vp) - 1);
        if (vf) bF = lane_value(myF, __ffsll((unsigned long long)vf) - 1);
      }
      const int bs = max(bP, bF);
      if (bP < bs) useP = false;
      if (bF < bs) useF = false;
      // mass / count strictly above bin bs: the lanes before the one owning
      // bs (its exclusive prefix) plus that lane's bins before bs
      uint64_t ma;
      uint32_t ca;
      {
        uint64_t pm = mi - lm;
        uint32_t pc = ci - lc;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (lane * 4 + t < bs) {
            pm += bm[t];
            pc += bc[t];
          }
        }
        ma = bs > 0 ? lane_value(pm, bs >> 2) : 0;
        ca = bs > 0 ? lane_value(pc, bs >> 2) : 0;
      }
      if (useP) needP -= ma;
      if (useF) needF -= (int)ca;
      kAbove += (int)ca;
      const uint32_t cstar = hcnt[wv][0][bs] + hcnt[wv][1][bs];
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if ((active >> i & 1) && 255 - (int)((key_of(i) >> shift) & 0xFF) != bs) active &= ~(1ull << i);
      if (cstar <= 64) break;
    }
    if (!all) {
      // gather the <= 64 candidates, sort descending across the wave
      int base = 0;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const bool a = active >> i & 1;
        const uint64_t b = __ballot(a);
        if (a) lkey[wv][base + __popcll(b & ((1ull << lane) - 1))] = key_of(i);
        base += __popcll(b);
      }
      wave_sync_lds();
      uint64_t kk = lane < base ? lkey[wv][lane] : 0ull;
      // a bitonic network over the smallest power of two holding the
      // candidates (lanes past it never meet lanes below it): most rows
      // end with a handful of candidates, e.g. 8 or fewer in three rows of
      // four at the Wan-14B 480P shape, and need 6 of the 21 stages
      const int span = base <= 2 ? 2 : 1 << (32 - __builtin_clz((unsigned)(base - 1)));
      for (int kb = 2; kb <= span; kb <<= 1) {
        for (int jb = kb >> 1; jb > 0; jb >>= 1) {
          const uint64_t o = __shfl_xor(kk, jb);
          const bool up = (lane & kb) == 0, lower = (lane & jb) == 0;
          kk = (up == lower) ? (kk > o ? kk : o) : (kk < o ? kk : o);
        }
      }
      const uint64_t qm = lane < base ? fix_mass((uint32_t)(kk >> 16)) : 0;
      const uint64_t qi = wave_incl_scan<uint64_t>(qm, lane);
      int tP = 0;
      if (useP) {
        const uint64_t hit = __ballot(lane < base && qi >= needP);
        tP = hit ? __ffsll((unsigned long long)hit) : base;   // 1-based position
      }
      const int tF = useF ? needF : 0;
      const int t = max(max(tP, tF), 1);
      thr = lane_value(kk, t - 1);
      kept = kAbove + t;
    }
  }
  // emit the bitmask of kept ids
  uint64_t* mrow = rowmask + r * nw;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (i < nw) {
      const bool sel = (lane + 64 * i < n) && key_of(i) >= thr;
      const uint64_t b = __ballot(sel);
      if (lane == 0) mrow[i] = b;
    }
  }
  if (lane == 0) rowcnt[r] = kept;
}

// ------------------------------------------------------------------ slack
// Lower median of the per-(b,h) kept counts and the deficit of every head.
__global__ __launch_bounds__(1024) void k_slack_target(const int32_t* __restrict__ rowcnt, int n_blk, int n_bh,
                                                       int32_t* __restrict__ headcnt,
                                                       int32_t* __restrict__ deficit) {
  __shared__ int hn[FVA_MAX_PHEAD];
  __shared__ int target;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int bh = wv; bh < n_bh; bh += 16) {
    int s = 0;
    for (int i = lane; i < n_blk; i += 64) s += rowcnt[(int64_t)bh * n_blk + i];
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    if (lane == 0) hn[bh] = s;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n_bh; i += 1024) {
    int rank = 0;
    for (int j = 0; j < n_bh; ++j) rank += (hn[j] < hn[i]) || (hn[j] == hn[i] && j < i);
    if (rank == (n_bh - 1) / 2) target = hn[i];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n_bh; i += 1024) {
    headcnt[i] = hn[i];
    deficit[i] = max(0, target - hn[i]);
  }
}

// Per deficient head: the key (score bits << 32 | ~(I*n + J)) of the d-th best
// unselected pair, by an MSD radix select over all n^2 pairs, 8 bits a level.
// Each level is two launches: k_slack_hist spreads a head's pairs over many
// workgroups (LDS histogram of the level's digit among the pairs that match
// the prefix so far, merged into the head's global histogram), then
// k_slack_pick keeps the digit where the count of larger keys crosses the
// remaining need, extends the prefix and clears the histogram.  When the kept
// digit's whole bin is needed the head is resolved (need 0): the prefix with
// zero lower digits already admits exactly that bin, so later levels skip the
// head.  With distinct fp32 scores that happens once the score's four digits
// are known, so the four index digits are only walked for ties.
constexpr int kSlackChunk = 2048;   // pairs per histogram workgroup

__global__ __launch_bounds__(256) void k_slack_hist(const float* __restrict__ S,
                                                    const uint64_t* __restrict__ rowmask, int nw, int n_blk,
                                                    const int32_t* __restrict__ deficit,
                                                    const int32_t* __restrict__ need,
                                                    const uint64_t* __restrict__ prefix, int level,
                                                    uint32_t* __restrict__ hist) {
  __shared__ unsigned int h[256];
  const int bh = blockIdx.y, tid = threadIdx.x;
  if (deficit[bh] <= 0 || (level > 0 && need[bh] == 0)) return;   // no deficit, or resolved
  const int shift = 56 - 8 * level;
  const uint64_t pre = level == 0 ? 0 : prefix[bh];
  h[tid] = 0;
  __syncthreads();
  const uint32_t n = (uint32_t)n_blk, nn = n * n;   // n^2 < 2^31: the block lists are int32
  const float* Sh = S + (int64_t)bh * nn;
  const uint64_t* mh = rowmask + (int64_t)bh * n * nw;
  const uint32_t e0 = blockIdx.x * (uint32_t)kSlackChunk, e1 = min(e0 + (uint32_t)kSlackChunk, nn);
  for (uint32_t e = e0 + tid; e < e1; e += 256) {
    const uint32_t I = e / n, J = e - I * n;
    if (mh[I * nw + (J >> 6)] >> (J & 63) & 1) continue;
    const uint64_t key = ((uint64_t)clamp_bits(Sh[e]) << 32) | (uint64_t)(0xFFFFFFFFu - e);
    if (level > 0 && (key >> (shift + 8)) != (pre >> (shift + 8))) continue;
    atomicAdd(&h[(key >> shift) & 0xFF], 1u);
  }
  __syncthreads();
  const unsigned v = h[tid];
  if (v) atomicAdd(&hist[bh * 256 + tid], v);
}

// Thread t holds digit 255 - t: an inclusive scan gives the count of keys
// whose digit is at least its own, and exactly one thread holds the crossing.
__global__ __launch_bounds__(256) void k_slack_pick(uint32_t* __restrict__ hist, const int32_t* __restrict__ deficit,
                                                    int32_t* __restrict__ need, uint64_t* __restrict__ prefix,
                                                    int level) {
  __shared__ int wtot[4];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nd = level == 0 ? deficit[bh] : need[bh];   // every thread reads it before one rewrites it
  if (deficit[bh] <= 0 || nd <= 0) return;
  const int shift = 56 - 8 * level;
  const uint64_t pre = level == 0 ? 0 : prefix[bh];
  uint32_t* hh = hist + bh * 256 + 255 - tid;
  const int c = (int)*hh;
  *hh = 0;
  const int incl = wave_incl_scan<int>(c, lane);
  if (lane == 63) wtot[wv] = incl;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) before += k < wv ? wtot[k] : 0;
  const int hi = before + incl, lo = hi - c;
  if (lo < nd && nd <= hi) {
    prefix[bh] = pre | ((uint64_t)(255 - tid) << shift);
    need[bh] = nd == hi ? 0 : nd - lo;
  }
}

// Add the pairs at or above a deficient head's threshold to its rows.
__global__ __launch_bounds__(256) void k_slack_apply(const float* __restrict__ S, uint64_t* __restrict__ rowmask,
                                                     int32_t* __restrict__ rowcnt, int nw, int n_blk,
                                                     int64_t n_rows, const int32_t* __restrict__ deficit,
                                                     const uint64_t* __restrict__ slack_thr) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wv;
  if (r >= n_rows) return;
  const int bh = (int)(r / n_blk);
  if (deficit[bh] <= 0) return;
  const uint64_t thr = slack_thr[bh];
  const int I = (int)(r - (int64_t)bh * n_blk);
  const float* Sr = S + r * n_blk;
  int added = 0;
  for (int i = 0; i < nw; ++i) {
    const int J = lane + 64 * i;
    const uint64_t old = rowmask[r * nw + i];
    bool add = false;
    if (J < n_blk && !(old >> lane & 1)) {
      const uint32_t e = (uint32_t)I * (uint32_t)n_blk + (uint32_t)J;
      const uint64_t key = ((uint64_t)clamp_bits(Sr[J]) << 32) | (uint64_t)(0xFFFFFFFFu - e);
      add = key >= thr;
    }
    const uint64_t b = __ballot(add);
    if (lane == 0 && b) rowmask[r * nw + i] = old | b;
    added += __popcll(b);
  }
  if (lane == 0) rowcnt[r] += added;
}

// ------------------------------------------------------------------ CSR
// Row pointers in two levels: k_scan_rows writes each head's exclusive scan
// of its rows' kept counts (head-local) and the head's total; k_scan_heads
// turns the totals into head offsets, head_nnz and row_ptr[n_rows]; k_emit
// adds the head offset, writes the final row_ptr[r] and the column ids.
__global__ __launch_bounds__(1024) void k_scan_rows(const int32_t* __restrict__ cnt, int n_blk,
                                                    int32_t* __restrict__ row_ptr, int32_t* __restrict__ headcnt) {
  __shared__ int wsum[16];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int32_t* c = cnt + (int64_t)bh * n_blk;
  int32_t* out = row_ptr + (int64_t)bh * n_blk;
  int carry = 0;
  for (int base = 0; base < n_blk; base += 1024) {
    const int i = base + tid;
    const int v = i < n_blk ? c[i] : 0;
    const int incl = wave_incl_scan<int>(v, lane);
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      before += k < wv ? wsum[k] : 0;
      total += wsum[k];
    }
    if (i < n_blk) out[i] = carry + before + incl - v;
    carry += total;
    __syncthreads();
  }
  if (tid == 0) headcnt[bh] = carry;
}

__global__ __launch_bounds__(1024) void k_scan_heads(const int32_t* __restrict__ headcnt, int n_bh,
                                                     int32_t* __restrict__ headoff, int32_t* __restrict__ head_nnz,
                                                     int32_t* __restrict__ row_ptr, int64_t n_rows) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int carry = 0;
  for (int base = 0; base < n_bh; base += 1024) {
    const int i = base + tid;
    const int v = i < n_bh ? headcnt[i] : 0;
    const int incl = wave_incl_scan<int>(v, lane);
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      before += k < wv ? wsum[k] : 0;
      total += wsum[k];
    }
    if (i < n_bh) {
      headoff[i] = carry + before + incl - v;
      if (head_nnz) head_nnz[i] = v;
    }
    carry += total;
    __syncthreads();
  }
  if (tid == 0) row_ptr[n_rows] = carry;
}

// Kept-id bitmask -> ascending column indices at row_ptr[r] (after adding
// the head offset to the head-local pointer).
__global__ __launch_bounds__(256) void k_emit(const uint64_t* __restrict__ rowmask, int32_t* __restrict__ row_ptr,
                                              const int32_t* __restrict__ headoff, int32_t* __restrict__ col_idx,
                                              int nw, int n_blk, int64_t n_rows) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wv;
  if (r >= n_rows) return;
  int base = row_ptr[r] + headoff[r / n_blk];
  if (lane == 0) row_ptr[r] = base;
  const uint64_t below = (1ull << lane) - 1;
  for (int i = 0; i < nw; ++i) {
    const uint64_t m = rowmask[r * nw + i];
    if (m >> lane & 1) col_idx[base + __popcll(m & below)] = 64 * i + lane;
    base += __popcll(m);
  }
}

template <typename T, int D>
void launch_pool(fva_plan_t plan, const void* q, const void* k, hipStream_t s) {
  const fva_plan_info& in = plan->info;
  const int bh = plan->desc.batch * plan->desc.heads;
  const bool sub = in.n_sub != 0;
  dim3 grid((in.n_blk + 3) / 4, bh, sub ? 1 : 2);
  hipLaunchKernelGGL((k_pool<T, D>), grid, dim3(256), 0, s, (const T*)q, (const T*)k, plan->qbar, plan->kbar,
                     plan->blk_cnt, in.n_blk, in.n_pad);
  if (sub)
    hipLaunchKernelGGL((k_pool_sub<T, D>), dim3(in.n_blk, bh), dim3(64), 0, s, (const T*)k, plan->kbar,
                       plan->sub_pos, plan->sub_cnt, in.n_blk, in.n_pad);
}

// Key ranges of the score grid.  Every workgroup does the same work (64
// queries x its key tiles), so the launch takes ceil(wg * n / slots) rounds
// of the resident workgroups; each range adds a fixed cost of about two
// tiles (the query load, the tables, the prefetch start).  n minimises
// rounds x (tiles / n + 2): at the 720P Hilbert shape 920 workgroups on
// 512 slots take 2 rounds unsplit and 9 (of 8.98) with five ranges.
int score_split(int wg, int ntiles, int slots) {
  int best = 1;
  double best_cost = 1e300;
  for (int n = 1; n <= FVA_MAX_SCORE_SPLIT && n <= ntiles; ++n) {
    const int64_t rounds = ((int64_t)wg * n + slots - 1) / slots;
    const double cost = (double)rounds * ((double)ntiles / n + 2.0);
    if (cost < best_cost * 0.99) best = n, best_cost = cost;
  }
  return best;
}

template <typename K>
int resident_blocks(K kernel) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, 256, 0) != hipSuccess || nb < 1) nb = 1;
  return nb;
}

template <int D>
void launch_score(fva_plan_t plan, hipStream_t s) {
  const fva_plan_info& in = plan->info;
  const int bh = plan->desc.batch * plan->desc.heads;
  const int wg = (in.n_blk + 63) / 64 * bh;
  const int ntiles = ((in.n_sub ? 8 : 1) * in.n_blk + 15) / 16;
  const double scale = 1.0 / sqrt((double)D);
  if (in.n_sub) {
    static const int per_cu = resident_blocks(k_score<true, D>);
    plan->score_split = score_split(wg, ntiles, plan->num_cu * per_cu);
    dim3 grid((in.n_blk + 63) / 64, bh, plan->score_split);
    hipLaunchKernelGGL((k_score<true, D>), grid, dim3(256), 0, s, plan->qbar, plan->kbar, plan->sub_cnt,
                       plan->ybuf, plan->rowmax, in.n_blk, scale);
  } else {
    static const int per_cu = resident_blocks(k_score<false, D>);
    plan->score_split = score_split(wg, ntiles, plan->num_cu * per_cu);
    dim3 grid((in.n_blk + 63) / 64, bh, plan->score_split);
    hipLaunchKernelGGL((k_score<false, D>), grid, dim3(256), 0, s, plan->qbar, plan->kbar, plan->sub_cnt,
                       plan->ybuf, plan->rowmax, in.n_blk, scale);
  }
}

// fva_select's body.  pooled: the means come from fva_permute_pool calls
// (already in qbar / kbar), so q_perm / k_perm are not read.
int select_impl(fva_plan_t plan, const void* q_perm, const void* k_perm, bool pooled, const float* p,
                int32_t p_count, int32_t k_min, int32_t slack_mode, const float* scores_in, float* scores_out,
                int32_t* row_ptr, int32_t* col_idx, int32_t* head_nnz, hipStream_t stream) {
  if (!plan) return fva_fail(FVA_EINVAL, "plan is NULL");
  const fva_plan_desc& d = plan->desc;
  const fva_plan_info& in = plan->info;
  const int n_bh = d.batch * d.heads;
  if (!p) return fva_fail(FVA_EINVAL, "p is NULL");
  if (p_count != 1 && p_count != n_bh)
    return fva_fail(FVA_EINVAL, "p_count %d must be 1 or B*H = %d", p_count, n_bh);
  if (p_count > FVA_MAX_PHEAD)
    return fva_fail(FVA_EUNSUPPORTED, "per-head p supports at most %d heads", FVA_MAX_PHEAD);
  SelectArgs pa;
  for (int i = 0; i < p_count; ++i) {
    if (!(p[i] > 0.0f)) return fva_fail(FVA_EINVAL, "p[%d] = %g must be > 0", i, (double)p[i]);
    pa.p[i] = p[i];
  }
  if (k_min < 0) return fva_fail(FVA_EINVAL, "k_min %d must be >= 0", k_min);
  if (slack_mode != FVA_SLACK_NONE && slack_mode != FVA_SLACK_MEDIAN)
    return fva_fail(FVA_EINVAL, "unknown slack mode %d", slack_mode);
  if (slack_mode == FVA_SLACK_MEDIAN && n_bh > FVA_MAX_PHEAD)
    return fva_fail(FVA_EUNSUPPORTED, "slack fill supports at most %d heads", FVA_MAX_PHEAD);
  if (!row_ptr || !col_idx) return fva_fail(FVA_EINVAL, "row_ptr / col_idx is NULL");
  if (!scores_in && !pooled && (!q_perm || !k_perm)) return fva_fail(FVA_EINVAL, "q_perm / k_perm is NULL");
  if (pooled && (plan->pooled & 3) != 3)
    return fva_fail(FVA_EINVAL, "fva_permute_pool has not produced the pooled means of both Q and K");

  if (!scores_in && !pooled) {
    plan->pooled = 0;   // qbar / kbar now hold the means of q_perm / k_perm
    if (d.dtype == FVA_DTYPE_BF16) {
      if (d.head_dim == 128) launch_pool<uint16_t, 128>(plan, q_perm, k_perm, stream);
      else launch_pool<uint16_t, 64>(plan, q_perm, k_perm, stream);
    } else {
      if (d.head_dim == 128) launch_pool<float, 128>(plan, q_perm, k_perm, stream);
      else launch_pool<float, 64>(plan, q_perm, k_perm, stream);
    }
  }
  if (!scores_in) {
    if (d.head_dim == 128) launch_score<128>(plan, stream);
    else launch_score<64>(plan, stream);
  }
  // fp32 scores are kept in the workspace only when the slack fill reads them
  float* s_out = scores_out ? scores_out
                            : (scores_in || slack_mode != FVA_SLACK_MEDIAN ? nullptr : plan->sbuf);
  const float* s_read = scores_in ? scores_in : s_out;
  const unsigned sel_grid = (unsigned)((in.n_rows + 3) / 4);
  const int ni = (in.n_blk + 63) / 64;
#define FVA_SELECT(NI)                                                                                  \
  hipLaunchKernelGGL((k_select<NI>), dim3(sel_grid), dim3(256), 0, stream, plan->ybuf, plan->rowmax,   \
                     plan->score_split,                                                                 \
                     scores_in, s_out, pa, p_count, k_min, in.n_blk, in.n_rows, plan->rowcnt,           \
                     plan->rowmask, plan->nw)
  if (ni <= 4) FVA_SELECT(4);
  else if (ni <= 8) FVA_SELECT(8);
  else if (ni <= 10) FVA_SELECT(10);
  else if (ni <= 12) FVA_SELECT(12);
  else if (ni <= 16) FVA_SELECT(16);
  else if (ni <= 24) FVA_SELECT(24);
  else if (ni <= 32) FVA_SELECT(32);
  else FVA_SELECT(64);
#undef FVA_SELECT
  if (slack_mode == FVA_SLACK_MEDIAN) {
    hipLaunchKernelGGL(k_slack_target, dim3(1), dim3(1024), 0, stream, plan->rowcnt, in.n_blk, n_bh,
                       plan->headcnt, plan->deficit);
    const unsigned chunks = (unsigned)(((int64_t)in.n_blk * in.n_blk + kSlackChunk - 1) / kSlackChunk);
    for (int level = 0; level < 8; ++level) {
      hipLaunchKernelGGL(k_slack_hist, dim3(chunks, n_bh), dim3(256), 0, stream, s_read, plan->rowmask, plan->nw,
                         in.n_blk, plan->deficit, plan->slack_need, plan->slack_thr, level, plan->slack_hist);
      hipLaunchKernelGGL(k_slack_pick, dim3(n_bh), dim3(256), 0, stream, plan->slack_hist, plan->deficit,
                         plan->slack_need, plan->slack_thr, level);
    }
    hipLaunchKernelGGL(k_slack_apply, dim3(sel_grid), dim3(256), 0, stream, s_read, plan->rowmask,
                       plan->rowcnt, plan->nw, in.n_blk, in.n_rows, plan->deficit, plan->slack_thr);
  }
  hipLaunchKernelGGL(k_scan_rows, dim3(n_bh), dim3(1024), 0, stream, plan->rowcnt, in.n_blk, row_ptr,
                     plan->headcnt);
  hipLaunchKernelGGL(k_scan_heads, dim3(1), dim3(1024), 0, stream, plan->headcnt, n_bh, plan->headoff, head_nnz,
                     row_ptr, in.n_rows);
  hipLaunchKernelGGL(k_emit, dim3(sel_grid), dim3(256), 0, stream, plan->rowmask, row_ptr, plan->headoff, col_idx,
                     plan->nw, in.n_blk, in.n_rows);
  return fva_after_launch(stream, pooled ? "fva_select_pooled" : "fva_select");
}

}  // namespace

extern "C" int fva_select(fva_plan_t plan, const void* q_perm, const void* k_perm, const float* p,
                          int32_t p_count, int32_t k_min, int32_t slack_mode, const float* scores_in,
                          float* scores_out, int32_t* row_ptr, int32_t* col_idx, int32_t* head_nnz,
                          hipStream_t stream) {
  return select_impl(plan, q_perm, k_perm, false, p, p_count, k_min, slack_mode, scores_in, scores_out, row_ptr,
                     col_idx, head_nnz, stream);
}

extern "C" int fva_select_pooled(fva_plan_t plan, const float* p, int32_t p_count, int32_t k_min,
                                 int32_t slack_mode, float* scores_out, int32_t* row_ptr, int32_t* col_idx,
                                 int32_t* head_nnz, hipStream_t stream) {
  return select_impl(plan, nullptr, nullptr, true, p, p_count, k_min, slack_mode, nullptr, scores_out, row_ptr,
                     col_idx, head_nnz, stream);
}

// ------------------------------------------------------------------ reuse
namespace {

__global__ __launch_bounds__(256) void k_zero_i64(int64_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

// One wave per row: both rows' id sets become LDS bitmaps, lane l then
// counts word l of their intersection and union; per-head totals by atomics.
__global__ __launch_bounds__(256) void k_mask_overlap(const int32_t* __restrict__ rpa, const int32_t* __restrict__ cia,
                                                      const int32_t* __restrict__ rpb, const int32_t* __restrict__ cib,
                                                      int n_blk, int64_t n_rows, unsigned long long* __restrict__ counts) {
  __shared__ unsigned int bits[4][2][128];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wv;
  if (r >= n_rows) return;   // whole wave; only wave-level syncs below
  for (int t = lane; t < 256; t += 64) bits[wv][t >> 7][t & 127] = 0;
  wave_sync_lds();
  for (int j = rpa[r] + lane; j < rpa[r + 1]; j += 64) {
    const int J = cia[j];
    if ((unsigned)J < (unsigned)n_blk) atomicOr(&bits[wv][0][J >> 5], 1u << (J & 31));
  }
  for (int j = rpb[r] + lane; j < rpb[r + 1]; j += 64) {
    const int J = cib[j];
    if ((unsigned)J < (unsigned)n_blk) atomicOr(&bits[wv][1][J >> 5], 1u << (J & 31));
  }
  wave_sync_lds();
  unsigned long long inter = 0, uni = 0;
  for (int t = lane; t < (n_blk + 31) / 32; t += 64) {
    const unsigned a = bits[wv][0][t], b = bits[wv][1][t];
    inter += __popc(a & b);
    uni += __popc(a | b);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    inter += __shfl_xor(inter, o);
    uni += __shfl_xor(uni, o);
  }
  if (lane == 0) {
    const int64_t bh = r / n_blk;
    atomicAdd(&counts[2 * bh], inter);
    atomicAdd(&counts[2 * bh + 1], uni);
  }
}

// Row r of a selection, as a set, added into its row of counts.
__global__ __launch_bounds__(256) void k_mask_accumulate(const int32_t* __restrict__ rp, const int32_t* __restrict__ ci,
                                                         int n_blk, int64_t n_rows, int32_t* __restrict__ counts) {
  __shared__ unsigned int bits[4][128];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wv;
  if (r >= n_rows) return;   // whole wave; only wave-level syncs below
  for (int t = lane; t < 128; t += 64) bits[wv][t] = 0;
  wave_sync_lds();
  for (int j = rp[r] + lane; j < rp[r + 1]; j += 64) {
    const int J = ci[j];
    if ((unsigned)J < (unsigned)n_blk) atomicOr(&bits[wv][J >> 5], 1u << (J & 31));
  }
  wave_sync_lds();
  int32_t* c = counts + r * n_blk;
  for (int J = lane; J < n_blk; J += 64)
    if (bits[wv][J >> 5] >> (J & 31) & 1) c[J] += 1;
}

// Kept-pair bitmask and count of each row from the counts.
__global__ __launch_bounds__(256) void k_mask_threshold(const int32_t* __restrict__ counts, int32_t min_count,
                                                        int n_blk, int64_t n_rows, int nw,
                                                        uint64_t* __restrict__ rowmask, int32_t* __restrict__ rowcnt) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wv;
  if (r >= n_rows) return;
  const int32_t* c = counts + r * n_blk;
  int kept = 0;
  for (int i = 0; i < nw; ++i) {
    const int J = 64 * i + lane;
    const uint64_t b = __ballot(J < n_blk && c[J] >= min_count);
    if (lane == 0) rowmask[r * nw + i] = b;
    kept += __popcll(b);
  }
  if (lane == 0) rowcnt[r] = kept;
}

}  // namespace

extern "C" int fva_mask_accumulate(fva_plan_t plan, const int32_t* row_ptr, const int32_t* col_idx, int32_t* counts,
                                   hipStream_t stream) {
  if (!plan) return fva_fail(FVA_EINVAL, "plan is NULL");
  if (!row_ptr || !col_idx || !counts) return fva_fail(FVA_EINVAL, "CSR or counts pointer is NULL");
  const fva_plan_info& in = plan->info;
  hipLaunchKernelGGL(k_mask_accumulate, dim3((unsigned)((in.n_rows + 3) / 4)), dim3(256), 0, stream, row_ptr, col_idx,
                     (int)in.n_blk, in.n_rows, counts);
  return fva_after_launch(stream, "fva_mask_accumulate");
}

extern "C" int fva_mask_from_counts(fva_plan_t plan, const int32_t* counts, int32_t min_count, int32_t* row_ptr,
                                    int32_t* col_idx, int32_t* head_nnz, hipStream_t stream) {
  if (!plan) return fva_fail(FVA_EINVAL, "plan is NULL");
  if (!counts || !row_ptr || !col_idx) return fva_fail(FVA_EINVAL, "counts / row_ptr / col_idx is NULL");
  if (min_count < 1) return fva_fail(FVA_EINVAL, "min_count %d must be >= 1", min_count);
  const fva_plan_info& in = plan->info;
  const int n_bh = plan->desc.batch * plan->desc.heads;
  const unsigned g = (unsigned)((in.n_rows + 3) / 4);
  hipLaunchKernelGGL(k_mask_threshold, dim3(g), dim3(256), 0, stream, counts, min_count, (int)in.n_blk, in.n_rows,
                     plan->nw, plan->rowmask, plan->rowcnt);
  hipLaunchKernelGGL(k_scan_rows, dim3(n_bh), dim3(1024), 0, stream, plan->rowcnt, (int)in.n_blk, row_ptr,
                     plan->headcnt);
  hipLaunchKernelGGL(k_scan_heads, dim3(1), dim3(1024), 0, stream, plan->headcnt, n_bh, plan->headoff, head_nnz,
                     row_ptr, in.n_rows);
  hipLaunchKernelGGL(k_emit, dim3(g), dim3(256), 0, stream, plan->rowmask, row_ptr, plan->headoff, col_idx, plan->nw,
                     (int)in.n_blk, in.n_rows);
  return fva_after_launch(stream, "fva_mask_from_counts");
}

extern "C" int fva_mask_overlap(fva_plan_t plan, const int32_t* row_ptr_a, const int32_t* col_idx_a,
                                const int32_t* row_ptr_b, const int32_t* col_idx_b, int64_t* counts,
                                hipStream_t stream) {
  if (!plan) return fva_fail(FVA_EINVAL, "plan is NULL");
  if (!row_ptr_a || !col_idx_a || !row_ptr_b || !col_idx_b || !counts)
    return fva_fail(FVA_EINVAL, "CSR or counts pointer is NULL");
  const fva_plan_info& in = plan->info;
  const int n_bh = plan->desc.batch * plan->desc.heads;
  hipLaunchKernelGGL(k_zero_i64, dim3((2 * n_bh + 255) / 256), dim3(256), 0, stream, counts, 2 * n_bh);
  hipLaunchKernelGGL(k_mask_overlap, dim3((unsigned)((in.n_rows + 3) / 4)), dim3(256), 0, stream, row_ptr_a,
                     col_idx_a, row_ptr_b, col_idx_b, (int)in.n_blk, in.n_rows, (unsigned long long*)counts);
  return fva_after_launch(stream, "fva_mask_overlap");
}

// Per-row 64-bit id masks ([n_rows][nw]) -> CSR with ascending ids, through
// the selection's row-count, two-level scan and emit kernels.
namespace {
__global__ __launch_bounds__(256) void k_bits_rowcnt(const uint64_t* __restrict__ bits, int nw, int64_t n_rows,
                                                     int32_t* __restrict__ cnt) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= n_rows) return;
  int c = 0;
  for (int i = 0; i < nw; ++i) c += __popcll(bits[r * nw + i]);
  cnt[r] = c;
}
}  // namespace

int fva_bits_to_csr(fva_plan_t plan, const uint64_t* bits, int32_t* row_ptr, int32_t* col_idx, hipStream_t stream) {
  const fva_plan_info& in = plan->info;
  const int n_bh = plan->desc.batch * plan->desc.heads;
  hipLaunchKernelGGL(k_bits_rowcnt, dim3((unsigned)((in.n_rows + 255) / 256)), dim3(256), 0, stream, bits, plan->nw,
                     in.n_rows, plan->rowcnt);
  hipLaunchKernelGGL(k_scan_rows, dim3(n_bh), dim3(1024), 0, stream, plan->rowcnt, (int)in.n_blk, row_ptr,
                     plan->headcnt);
  hipLaunchKernelGGL(k_scan_heads, dim3(1), dim3(1024), 0, stream, plan->headcnt, n_bh, plan->headoff,
                     (int32_t*)nullptr, row_ptr, in.n_rows);
  hipLaunchKernelGGL(k_emit, dim3((unsigned)((in.n_rows + 3) / 4)), dim3(256), 0, stream, bits, row_ptr,
                     plan->headoff, col_idx, plan->nw, (int)in.n_blk, in.n_rows);
  return FVA_OK;
}
