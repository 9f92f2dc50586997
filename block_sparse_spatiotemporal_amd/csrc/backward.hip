// Backward pass of the block-sparse attention over the same block lists as
// the forward pass ("Video Sparse Attention" explainer, section 3: the
// sparse kernel serves training as well as inference).  With scaled scores
// s_ij = q_i . k_j / sqrt(D), P = softmax over the selected keys of each
// query, and dO the gradient of the output:
//   dP = dO V^T,  delta_i = sum_d dO_id O_id,  dS = P * (dP - delta)
//   dQ = dS K / sqrt(D),  dK = dS^T Q / sqrt(D),  dV = P^T dO
// Each kernel owns its outputs outright (no atomics, so the gradients are
// bitwise reproducible):
//   k_bwd_dq    groups of query blocks, walking their rows of the selection
//               (like the forward pass); also writes minus delta, where
//               the dK products start their dP accumulators (dS = P * dP);
//   k_bwd_dkv   groups of key blocks, walking the transposed selection (the
//               query blocks that listed them), once for dV and once for dK;
//   k_bwd_dkdv  dK and dV in one kernel (a selectable variant: holding both
//               accumulators costs it half the waves per SIMD).
// P is recomputed from the forward pass's per-query log-sum-exp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "attn_common.h"
#include "fva_internal.h"

namespace {

using namespace fva_attn;

// ------------------------------------------------------------------ lists
// CSR -> one 64-bit-word bitmap per row (a row read as a set; ids outside
// [0, n_blk) dropped).  One wave per row.
__global__ __launch_bounds__(256) void k_csr_bits(const int32_t* __restrict__ row_ptr,
                                                  const int32_t* __restrict__ col_idx, int n_blk, int nw,
                                                  int64_t n_rows, uint64_t* __restrict__ bits) {
  __shared__ unsigned long long wbuf[4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t r = (int64_t)blockIdx.x * 4 + wv;
  wbuf[wv][lane] = 0;
  __syncthreads();
  if (r < n_rows) {
    const int beg = row_ptr[r], end = row_ptr[r + 1];
    for (int j = beg + lane; j < end; j += 64) {
      const int J = col_idx[j];
      if ((unsigned)J < (unsigned)n_blk) atomicOr(&wbuf[wv][J >> 6], 1ull << (J & 63));
    }
  }
  __syncthreads();
  if (r < n_rows && lane < nw) bits[r * nw + lane] = wbuf[wv][lane];
}

// Per-head transpose of the block bitmap, one 64 x 64 bit tile per wave:
// lane i holds word wj of row 64*wi + i; the ballot of bit c over the lanes
// is word wi of row 64*wj + c of the transpose.  grid (ceil(nw*nw / 4), B*H).
__global__ __launch_bounds__(256) void k_bits_transpose(const uint64_t* __restrict__ bits, int n_blk, int nw,
                                                        uint64_t* __restrict__ bits_t) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= nw * nw) return;   // whole waves; no barrier follows
  const int wi = t / nw, wj = t - wi * nw;
  const int64_t head = (int64_t)blockIdx.y * n_blk;
  const int I = 64 * wi + lane;
  const uint64_t x = I < n_blk ? bits[(head + I) * nw + wj] : 0;
  uint64_t out = 0;
#pragma unroll 8
  for (int c = 0; c < 64; ++c) {
    const uint64_t b = __ballot((x >> c) & 1);
    if (lane == c) out = b;
  }
  const int J = 64 * wj + lane;
  if (J < n_blk) bits_t[(head + J) * nw + wi] = out;
}

// ------------------------------------------------------------------ kernels
struct BwdArgs {
  const uint16_t* q;        // [B*H, n_pad, D] rows
  const uint16_t* k;        // rows
  const uint16_t* v;        // rows
  const float* o32;         // forward output before rounding, rows
  const float* lse;         // [B*H, n_pad] log2-sum-exp2 of the scaled scores (forward pass)
  const uint16_t* dout;     // dO rows
  const uint16_t* dot;      // dO in the VT layout
  const uint64_t* bits;     // [n_rows][nw] query block -> key blocks
  const uint64_t* bits_t;   // [n_rows][nw] key block -> query blocks
  const uint64_t* blk_mask;
  const uint64_t* blk_full;
  float* ndelta;            // [B*H, n_pad]: minus delta, the start value of the dK kernel's dP
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int64_t n_pad;
  int n_blk;
  int nw;
  int n_items;              // B*H*ceil(n_blk / G) groups
  int chunk;
  int persistent;           // 1: resident grid popping groups from per-XCD cursors
  int32_t* cursor;          // [16] per-XCD cursors, then per-XCD exhausted flags (zeroed before launch)
  const int32_t* order;     // persistent: groups in schedule order (list position -> group)
  const int2* pairs;        // optional (G = 2): the two blocks of each group, second -1 if none
  float scale;              // 1/sqrt(D)
};

// Next group of G consecutive blocks of one head for this workgroup, or -1
// when none is left.  Plain grid: workgroup b is on XCD b % 8 and takes its
// XCD's (b / 8)-th group.  Persistent grid: one cursor per XCD over the
// XCD's chunks of the group list; an XCD whose share is done steals from the
// others.  Uniform across the workgroup (an LDS broadcast).
__device__ __forceinline__ int bwd_next(const BwdArgs& a, int* s_item, bool first) {
  if (!a.persistent) {
    if (!first) return -1;
    const int64_t it = xcd_item(blockIdx.x % kXcds, blockIdx.x / kXcds, a.chunk);
    return it < a.n_items ? (int)it : -1;
  }
  __syncthreads();   // the previous group's ring reads are done
  if (threadIdx.x == 0) {
    const int x0 = blockIdx.x % kXcds;
    int found = -1;
    for (int t = 0; t < kXcds && found < 0; ++t) {
      const int x = (x0 + t) % kXcds;
      if (__hip_atomic_load(&a.cursor[kXcds + x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) continue;
      const int64_t it = xcd_item(x, atomicAdd(&a.cursor[x], 1), a.chunk);
      if (it < a.n_items) found = a.order[it];
      else __hip_atomic_store(&a.cursor[kXcds + x], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    *s_item = found;
  }
  __syncthreads();
  return *s_item;
}

// Schedule order of one head's groups of G blocks (one workgroup per head):
// decreasing cost, the number of set bits of the group's bitmap rows (ties
// by group id), so each XCD runs a head's long groups first and its short
// ones last.
__global__ __launch_bounds__(1024) void k_bwd_order(const uint64_t* __restrict__ bits, int n_blk, int nw, int G,
                                                    const int2* __restrict__ pairs, int32_t* __restrict__ order) {
  __shared__ int cost[4096];
  const int ngh = (n_blk + G - 1) / G;
  const int bh = blockIdx.x;
  for (int g = threadIdx.x; g < ngh; g += 1024) {
    int c = 0;
    for (int i = 0; i < G; ++i) {
      const int b = pairs ? (i == 0 ? pairs[(int64_t)bh * ngh + g].x : pairs[(int64_t)bh * ngh + g].y)
                          : (g * G + i < n_blk ? g * G + i : -1);
      if (b < 0) continue;
      const uint64_t* row = bits + ((int64_t)bh * n_blk + b) * nw;
      for (int wd = 0; wd < nw; ++wd) c += __popcll(row[wd]);
    }
    cost[g] = c;
  }
  __syncthreads();
  for (int g = threadIdx.x; g < ngh; g += 1024) {
    int rk = 0;
    const int c = cost[g];
    for (int o = 0; o < ngh; ++o) rk += (cost[o] > c) || (cost[o] == c && o < g);
    order[(int64_t)bh * ngh + rk] = bh * ngh + g;
  }
}

__global__ __launch_bounds__(64) void k_zero_i32(int32_t* __restrict__ p, int n) {
  for (int i = threadIdx.x; i < n; i += 64) p[i] = 0;
}

// Wait until at most `ahead` steps of this wave's direct loads (PW each) are
// still in flight.
template <int PW, int NST>
__device__ __forceinline__ void wait_steps(int st, int total) {
  // the loads of step st are this wave's oldest except for those of the
  // min(NST - 2, total - 1 - st) steps issued after it
  static_assert(NST >= 2 && NST <= 4 && (NST - 1) * PW < 64, "vmcnt range");
  if (st + NST - 2 < total) wait_vm<(NST - 2) * PW>();
  else if (NST >= 4 && st + 2 < total) wait_vm<(NST >= 4 ? 2 * PW : 0)>();
  else if (NST >= 3 && st + 1 < total) wait_vm<PW>();
  else wait_vm<0>();
}

// bf16x4 store of 4 consecutive fp32 values (times f), or zeros.
__device__ __forceinline__ void store4(uint16_t* dst, const f32x16& acc, int g4, float f, bool ok) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  f32x4 v = {acc[4 * g4] * f, acc[4 * g4 + 1] * f, acc[4 * g4 + 2] * f, acc[4 * g4 + 3] * f};
  if (!ok) v = f32x4{0.f, 0.f, 0.f, 0.f};
  *(uint2*)dst = __builtin_bit_cast(uint2, __builtin_convertvector(v, bf16x4));
}

// Chunk swizzle of the row tiles of the backward kernels.  Physical 16-byte
// chunk pc of row r holds logical chunk pc ^ kswz_t(r).  For D = 128 the
// swizzle puts r % 4 in the high two bits and (r / 4) % 4 in the low two:
// a plain row read (16 consecutive rows, one chunk each) still touches 16
// different chunks, and a transposed read, whose 16-lane group takes two
// neighbouring chunks of four consecutive rows (and whose other 16-lane group
// in the same pass the next two chunks of those rows), touches 16 different
// chunks over the 32 lanes: every bank once.  With r % 16 (the forward
// kernel's swizzle) the four rows of a group share their chunks, and half the
// LDS cycles of the dQ and dK kernels went to bank conflicts.
template <int D>
__device__ __forceinline__ int kswz_t(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : kswz<D>(row);
}

// Source offsets (bytes within one 32-row half) of a wave's direct loads of
// a row tile (XOR swizzle kswz_t by row) and of a VT tile (vswz by d).
// Load j of wave w (of NW) fills LDS bytes [1024 (NW j + w), +1024) of the half.
template <int D, int LPW, int NW>
__device__ __forceinline__ void tile_offsets(int w, int lane, uint32_t* roff, uint32_t* toff) {
  constexpr int KCH = D / 8;
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int off = (NW * j + w) * 1024 + lane * 16;
    const int row = off / (KCH * 16), pc = (off / 16) % KCH;
    roff[j] = row * (D * 2) + ((pc ^ kswz_t<D>(row)) * 16);
    const int d = off / 64, pv = (off / 16) & 3;
    toff[j] = d * 64 + ((pv ^ vswz(d)) * 16);
  }
}

// Transposed LDS reads (ds_read_b64_tr_b16).  In each group of 16 lanes,
// every lane names 8 bytes (4 bf16) of LDS; lane j of the group receives, as
// its element e (e = 0..3), element j % 4 of what lane 4 e + j / 4 named.  So
// if source lane s names row r0 + s / 4 at columns c0 + 4 (s % 4)..+3 of a
// row-major tile, lane j receives column c0 + j of rows r0..r0+3.
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;

// Lane parts of the transposed-read addresses.  For D = 128 every address
// tr_operand<128> forms is one of eight lane constants (column tile dt and
// the first or second 8-row run of a 16-row step) plus an immediate: with
// r = 16 ks + 8 u + rl the swizzle is 4 (rl % 4) + 2 u + rl / 4, so the
// physical chunk of logical chunk 4 dt + c (c < 4) is
// 4 (dt ^ (rl % 4)) + (c ^ (2 u + rl / 4)).
struct TrBase {
  uint32_t b[4][2];
};
template <int D>
__device__ __forceinline__ TrBase tr_base(uint32_t ring_lds, int lane) {
  TrBase t{};
  if constexpr (D == 128) {
    const int g = lane >> 4, s = lane & 15, gb = g >> 1;
    const int rl = 4 * gb + (s >> 2);                    // row within 8
    const int c = 2 * (g & 1) + ((s & 3) >> 1);          // logical chunk within the column tile
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        t.b[dt][u] = ring_lds + (8 * u + rl) * 256 + 16 * (4 * (dt ^ (rl & 3)) + (c ^ (2 * u + gb))) + (s & 1) * 8;
  } else {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) t.b[dt][0] = t.b[dt][1] = ring_lds;
  }
  return t;
}

// A operand (32 x 16) of a product whose k index runs over the rows of a
// 32-row, D-column tile in LDS (16-byte chunks swizzled by kswz_t, as the row
// tiles of the ring are stored), taken in the key order of the B operand fed
// from an S-shaped accumulator: lane (i, h) element e holds row
// 16 ks + 8 (e / 4) + 4 h + e % 4 at column 32 dt + i.  Two transposed reads,
// one per 4-row run; `tile` is the tile's byte offset inside the ring.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(uint32_t tile, const TrBase& tb, int dt, int ks, int lane) {
  uint32_t o0, o1;
  if constexpr (D == 128) {
    // column 32 dt + 16 (g&1) + 4 (s&3) of rows 16 ks + rl and 16 ks + 8 + rl
    o0 = tb.b[dt][0] + tile + (16 * ks) * 256;
    o1 = tb.b[dt][1] + tile + (16 * ks) * 256;
  } else {
    const int g = lane >> 4, s = lane & 15;
    const int d = 32 * dt + 16 * (g & 1) + 4 * (s & 3);
    const int r0 = 16 * ks + 4 * (g >> 1) + (s >> 2), r1 = r0 + 8;
    o0 = tb.b[0][0] + tile + r0 * (D * 2) + (((d >> 3) ^ kswz_t<D>(r0)) << 4) + ((d & 7) << 1);
    o1 = tb.b[0][0] + tile + r1 * (D * 2) + (((d >> 3) ^ kswz_t<D>(r1)) << 4) + ((d & 7) << 1);
  }
  // whole-vector casts: element-wise extraction from the builtin's bf16x4
  // result is avoided
  const bf16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)o0);
  const bf16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(uintptr_t)o1);
  const uint2 ux = __builtin_bit_cast(uint2, x), uy = __builtin_bit_cast(uint2, y);
  return __builtin_bit_cast(bf16x8, make_uint4(ux.x, ux.y, uy.x, uy.y));
}

// The blocks of group `item` (G consecutive ids from I0, or a pair from the
// pair table), -1 past the head's last block.  Wave-uniform.
template <int G>
__device__ __forceinline__ void group_blocks(const int2* pairs, int item, int I0, int n_blk, int* blk) {
  if (G == 2 && pairs) {
    const uint64_t v = sload((const uint64_t*)pairs, item);   // (x, y) of an int2
    blk[0] = (int)(uint32_t)v;
    blk[G - 1] = (int)(uint32_t)(v >> 32);
  } else {
#pragma unroll
    for (int i = 0; i < G; ++i) blk[i] = I0 + i < n_blk ? I0 + i : -1;
  }
}

// The G bitmaps of a group (rows head_row0 + blk[i] of `bits`; a -1 block
// is empty): this wave's own one (member g) and their union, one 64-bit
// word per lane.
template <int G>
__device__ __forceinline__ void group_bits(const uint64_t* bits, int64_t head_row0, const int* blk, int nw, int lane,
                                           int g, uint32_t* own_lo, uint32_t* own_hi, uint32_t* un_lo,
                                           uint32_t* un_hi) {
  uint64_t own = 0, un = 0;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const uint64_t x = (lane < nw && blk[i] >= 0) ? bits[(head_row0 + blk[i]) * nw + lane] : 0;
    un |= x;
    if (i == g) own = x;
  }
  *own_lo = (uint32_t)own;
  *own_hi = (uint32_t)(own >> 32);
  *un_lo = (uint32_t)un;
  *un_hi = (uint32_t)(un >> 32);
}

// dQ and delta.  Workgroup = G query blocks, 2 waves each; wave w serves
// block w/2, queries 32 (w%2)..+31, one per lane pair (lanes l and l+32
// split D).  Steps walk the union of the G rows of the selection, one
// 32-key half of a block per step, loaded once into the LDS ring for every
// wave pair whose row holds it:
//   S^T  (32 keys x 32 queries) = K_half . Q^T      (Q in registers)
//   dP^T (32 keys x 32 queries) = V_half . dO^T     (dO in registers)
//   dS^T = P^T * (dP^T - delta),  P^T = exp2(S^T * scale * log2 e - lse)
//   dQ^T (D x 32 queries) += K^T_half . dS^T        (dS^T straight from the accumulators)
// K rows and V rows of each half stream through an NST-stage ring of direct
// loads, published by one barrier per step; K^T is read from the K rows by
// transposed LDS reads.
template <int D, int NST, int G>
__global__ __launch_bounds__(128 * G, 2) void k_bwd_dq(BwdArgs a) {
  constexpr int NW = 2 * G;
  constexpr int KS = D / 16, DT = D / 32, KCH = D / 8;
  constexpr int HALF = 32 * D * 2;
  constexpr int STAGE = 2 * HALF;
  constexpr int LPW = HALF / 1024 / NW;  // direct loads per wave per tile
  constexpr int PW = 2 * LPW;            // per wave per step
  static_assert(LPW >= 1 && (HALF / 1024) % NW == 0, "tile loads split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) uint4 ring[NST * STAGE / 16];
  __shared__ int s_item;
  for (int item = bwd_next(a, &s_item, true); item >= 0; item = bwd_next(a, &s_item, false)) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qg = w >> 1, w2 = w & 1;
  const int h = lane >> 5, l32 = lane & 31;
  const int ngh = (a.n_blk + G - 1) / G;
  const int bh = item / ngh, I0 = (item - bh * ngh) * G;
  int blk[G];
  group_blocks<G>(a.pairs, item, I0, a.n_blk, blk);
  const bool has_row = blk[qg] >= 0;
  const int I = has_row ? blk[qg] : blk[0];
  const int64_t head = (int64_t)bh * a.n_pad;
  const int64_t tok = head + (int64_t)I * 64 + 32 * w2 + l32;
  const float sl2 = a.scale * 1.44269504088896340736f;
  const bool qvalid = has_row && (sload(a.blk_mask, I) >> (32 * w2 + l32) & 1);

  uint32_t roff[LPW], toff[LPW];
  tile_offsets<D, LPW, NW>(w, lane, roff, toff);
  uint32_t own_lo, own_hi, un_lo, un_hi;
  group_bits<G>(a.bits, (int64_t)bh * a.n_blk, blk, a.nw, lane, qg, &own_lo, &own_hi, &un_lo, &un_hi);
  const uint64_t fw = lane < a.nw ? a.blk_full[lane] : 0;
  const uint32_t full_lo = (uint32_t)fw, full_hi = (uint32_t)(fw >> 32);

  // Q, dO in registers (lane: d chunk 2ks + h of its query); delta from O.
  bf16x8 qreg[KS], doreg[KS];
  float lse2, delta;
  {
    const uint4* qrow = (const uint4*)(a.q + tok * D);
    const uint4* drow = (const uint4*)(a.dout + tok * D);
    const f32x8* orow = (const f32x8*)(a.o32 + tok * D);
    float dl = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qreg[ks] = as_bf16x8(qrow[2 * ks + h]);
      doreg[ks] = as_bf16x8(drow[2 * ks + h]);
      const f32x8 ov = orow[2 * ks + h];
#pragma unroll
      for (int e = 0; e < 8; ++e) dl = fmaf((float)doreg[ks][e], ov[e], dl);
    }
    const float dsum = xhalf_sum(dl);   // lanes l and l+32 hold the two halves of D
    delta = qvalid ? dsum : 0.0f;
    lse2 = qvalid ? a.lse[tok] : INFINITY;   // pad queries: P = 0
    // settle these loads before the ring's direct loads are counted
    wait_vm<0>();
    if (h == 0 && has_row) a.ndelta[tok] = -delta;
  }

  BitWalk iw, cw;
  const char* kbase = (const char*)(a.k + head * D);
  const char* vbase = (const char*)(a.v + head * D);
  int curJ = 0;
  const int total = union_steps(un_lo, un_hi);   // two halves per union block
  // loads of half u of the walk's next block into ring stage `stage` (a
  // compile-time constant at every call site of the unrolled loop)
  auto issue_next = [&](int stage, int u) __attribute__((always_inline)) {
    if (u == 0) curJ = iw.next_known(un_lo, un_hi);
    const int64_t roff0 = ((int64_t)curJ * 64 + 32 * u) * D * 2;
    const uint32_t dst = lds_addr(ring) + stage * STAGE;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const uint32_t o1 = (NW * j + w) * 1024;
      dma16(kbase + roff0, roff[j], dst + o1);
      dma16(vbase + roff0, roff[j], dst + HALF + o1);
    }
  };

  const TrBase trb = tr_base<D>(lds_addr(ring), lane);
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < total) issue_next(st, st & 1);

  int J = 0;
  // valid-key mask of the current block for this wave (zero when the row
  // does not list it), a scalar word taken once per block
  uint64_t kmask = 0;
  // unrolled by the ring depth: copy kk reads stage kk (offsets fold into
  // the LDS reads' immediates) and loads into stage (kk + NST - 1) % NST
  for (int st0 = 0; st0 < total; st0 += NST) {
#pragma unroll
  for (int kk = 0; kk < NST; ++kk) {
    const int st = st0 + kk;
    if (st >= total) break;
    if ((st & 1) == 0) {
      J = cw.next_known(un_lo, un_hi);
      const bool mine = lane_word(own_lo, own_hi, J >> 6) >> (J & 63) & 1;
      const bool full = lane_word(full_lo, full_hi, J >> 6) >> (J & 63) & 1;
      kmask = !mine ? 0ull : (full ? ~0ull : sload(a.blk_mask, J));
    }
    wait_steps<PW, NST>(st, total);
    barrier_no_fence();
    if (st + NST - 1 < total) issue_next((kk + NST - 1) % NST, (st + NST - 1) & 1);

    const int u = st & 1;
    const uint32_t mh = (uint32_t)(kmask >> (32 * u));
    if (mh == 0) continue;   // not in this row, or a half of pad keys
    const uint4* kst = ring + kk * (STAGE / 16);
    const uint4* vst = kst + HALF / 16;
    f32x16 s = {}, dp = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = l32 * KCH + ((2 * ks + h) ^ kswz_t<D>(l32));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kst[c]), qreg[ks], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vst[c]), doreg[ks], dp, 0, 0, 0);
    }
    // From the exponentials to the end of the step's last products the wave
    // runs at a raised priority, as in the forward kernel: a wave finishing
    // a step issues ahead of a co-resident wave starting one (bit-identical;
    // backward kernels 52.3 -> 51.1 ms at the Wan-14B 480P shape).
    __builtin_amdgcn_s_setprio(2);
    // element i: key 8*(i/4) + 4*h + i%4 of this half, query l32.  Pad keys
    // get s = -inf (P = 0) only in blocks that have any (a uniform branch):
    // a pad key's zero K row would otherwise meet P = 2^-lse, which need not
    // be finite
    if (mh != 0xFFFFFFFFu) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * h + (i & 3);
        if (!(mh >> key & 1)) s[i] = -INFINITY;
      }
    }
    f32x8 d0, d1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[i], sl2, -lse2));
      const float ds = p * (dp[i] - delta);
      if (i < 8) d0[i] = ds;
      else d1[i - 8] = ds;
    }
    const bf16x8 db0 = __builtin_convertvector(d0, bf16x8);
    const bf16x8 db1 = __builtin_convertvector(d1, bf16x8);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(kk * STAGE, trb, dt, 0, lane), db0, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(kk * STAGE, trb, dt, 1, lane), db1, acc[dt], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  }
  }
  if (!has_row) continue;
  // acc[dt][r]: dQ^T[32 dt + 8 (r/4) + 4 h + r%4][query l32]
  uint16_t* out = a.dq + tok * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) store4(out + 32 * dt + 8 * g4 + 4 * h, acc[dt], g4, a.scale, qvalid);
  }
}

// dK and dV.  Workgroup = G key blocks, 2 waves each; wave w owns keys
// 32 (w%2)..+31 of block w/2 (K and V rows in registers).  Steps walk the
// union of the G columns (the query blocks whose rows list the key
// blocks), one 32-query half per step:
//   S  (32 queries x 32 keys) = Q_half . K^T,   dP = dO_half . V^T
//   P = exp2(S * scale * log2 e - lse),  dS = P * (dP - delta)
//   dV^T (D x 32 keys) += dO^T_half . P,   dK^T += Q^T_half . dS
// The ring stage holds Q rows, dO rows and dO^T (VT layout) of the half
// (Q^T is read from the Q rows by transposed LDS reads), and the half's 32
// lse then 32 minus-delta values (each wave brings 256/NW bytes of those).
template <int D, int NST, int G>
__global__ __launch_bounds__(128 * G, G) void k_bwd_dkdv(BwdArgs a) {
  constexpr int NW = 2 * G;
  constexpr int KS = D / 16, DT = D / 32, KCH = D / 8;
  constexpr int HALF = 32 * D * 2;
  constexpr int STAGE = 3 * HALF + 256;
  constexpr int LPW = HALF / 1024 / NW;
  constexpr int PW = 3 * LPW + 1;
  constexpr int LDW = 64 / NW;           // lse/delta floats each wave brings
  static_assert(LPW >= 1 && (HALF / 1024) % NW == 0, "tile loads split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) uint4 ring[NST * STAGE / 16];
  __shared__ int s_item;
  for (int item = bwd_next(a, &s_item, true); item >= 0; item = bwd_next(a, &s_item, false)) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = w >> 1, w2 = w & 1;
  const int h = lane >> 5, l32 = lane & 31;
  const int ngh = (a.n_blk + G - 1) / G;
  const int bh = item / ngh, J0 = (item - bh * ngh) * G;
  int blk[G];
  group_blocks<G>(a.pairs, item, J0, a.n_blk, blk);
  const bool has_blk = blk[kg] >= 0;
  const int J = has_blk ? blk[kg] : blk[0];
  const int64_t head = (int64_t)bh * a.n_pad;
  const int64_t tok = head + (int64_t)J * 64 + 32 * w2 + l32;   // this lane's key token
  const float sl2 = a.scale * 1.44269504088896340736f;
  const uint32_t kmask = has_blk ? (uint32_t)(sload(a.blk_mask, J) >> (32 * w2)) : 0u;
  const bool kvalid = kmask >> l32 & 1;

  uint32_t roff[LPW], toff[LPW];
  tile_offsets<D, LPW, NW>(w, lane, roff, toff);
  uint32_t own_lo, own_hi, un_lo, un_hi;
  group_bits<G>(a.bits_t, (int64_t)bh * a.n_blk, blk, a.nw, lane, kg, &own_lo, &own_hi, &un_lo, &un_hi);

  bf16x8 kreg[KS], vreg[KS];
  {
    const uint4* krow = (const uint4*)(a.k + tok * D);
    const uint4* vrow = (const uint4*)(a.v + tok * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kreg[ks] = as_bf16x8(krow[2 * ks + h]);
      vreg[ks] = as_bf16x8(vrow[2 * ks + h]);
    }
    wait_vm<0>();
  }

  BitWalk iw, cw;
  const char* qbase = (const char*)(a.q + head * D);
  const char* dbase = (const char*)(a.dout + head * D);
  const char* dtbase = (const char*)(a.dot + head * D);
  // floats [LDW w, LDW (w+1)) of the stage's [32 lse | 32 -delta]
  const float* lbase = (LDW * w < 32 ? a.lse + LDW * w : (const float*)a.ndelta + (LDW * w - 32)) + head;
  int issued = 0, curI = 0;
  const int total = union_steps(un_lo, un_hi);   // two halves per union block
  auto issue_next = [&]() __attribute__((always_inline)) {
    if ((issued & 1) == 0) curI = iw.next_known(un_lo, un_hi);
    const int u = issued & 1;
    const int64_t roff0 = ((int64_t)curI * 64 + 32 * u) * D * 2;
    const int64_t toff0 = (int64_t)curI * 64 * D * 2 + u * HALF;
    const uint32_t dst = lds_addr(ring) + (issued % NST) * STAGE;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const uint32_t o1 = (NW * j + w) * 1024;
      dma16u(qbase + roff0, roff[j], dst + o1);
      dma16u(dbase + roff0, roff[j], dst + HALF + o1);
      dma16u(dtbase + toff0, toff[j], dst + 2 * HALF + o1);
    }
    if (lane < LDW / 4) dma16u(lbase + (int64_t)curI * 64 + 32 * u, lane * 16, dst + 3 * HALF + 4 * LDW * w);
    ++issued;
  };

  const TrBase trb = tr_base<D>(lds_addr(ring), lane);
  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dk[dt] = dv[dt] = f32x16{};
#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < total) issue_next();

  int I = 0;
  // valid-query mask of the current block for this wave (zero when the
  // column does not list it), a scalar word taken once per block
  uint64_t qm64 = 0;
  for (int st = 0; st < total; ++st) {
    if ((st & 1) == 0) {
      I = cw.next_known(un_lo, un_hi);
      const bool mine = lane_word(own_lo, own_hi, I >> 6) >> (I & 63) & 1;
      qm64 = mine && kmask != 0 ? sload(a.blk_mask, I) : 0ull;
    }
    wait_steps<PW, NST>(st, total);
    barrier_no_fence();
    if (st + NST - 1 < total) issue_next();

    const int u = st & 1;
    const uint32_t qm = (uint32_t)(qm64 >> (32 * u));
    if (qm == 0) continue;   // not in this column, pad queries, or a wave of pad keys
    const uint4* qst = ring + (st % NST) * (STAGE / 16);
    const uint4* dst_ = qst + HALF / 16;
    const uint4* dtst = qst + 2 * HALF / 16;
    const float* lds_l = (const float*)(qst + 3 * HALF / 16);
    const uint32_t qtile = (uint32_t)((st % NST) * STAGE);   // Q rows: Q^T by transposed reads
    // Two phases keep the live registers low enough for two waves per
    // SIMD: S -> P -> dV, then dP -> dS -> dK (P kept in fp32 between).
    // element r of S, dP: query 8*(r/4) + 4*h + r%4 of this half, key l32
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qst[l32 * KCH + ((2 * ks + h) ^ kswz_t<D>(l32))]),
                                                  kreg[ks], s, 0, 0, 0);
    f32x16 p;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 L = *(const f32x4*)(lds_l + 8 * c + 4 * h);
#pragma unroll
      for (int j = 0; j < 4; ++j) p[4 * c + j] = __builtin_amdgcn_exp2f(fmaf(s[4 * c + j], sl2, -L[j]));
    }
    {
      const bf16x8 pb0 = __builtin_convertvector(p.lo, bf16x8), pb1 = __builtin_convertvector(p.hi, bf16x8);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 32 * dt + l32;
        const int sw = vswz(d);
        dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(dtst[d * 4 + ((0 + h) ^ sw)]), pb0, dv[dt], 0, 0, 0);
        dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(dtst[d * 4 + ((2 + h) ^ sw)]), pb1, dv[dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16 dp;   // starts at minus delta (the stage holds -delta), so dS = P * dP
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 nD = *(const f32x4*)(lds_l + 32 + 8 * c + 4 * h);
#pragma unroll
      for (int j = 0; j < 4; ++j) dp[4 * c + j] = nD[j];
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(dst_[l32 * KCH + ((2 * ks + h) ^ kswz_t<D>(l32))]),
                                                   vreg[ks], dp, 0, 0, 0);
    f32x16 ds;
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = p[r] * dp[r];
    {
      const bf16x8 db0 = __builtin_convertvector(ds.lo, bf16x8), db1 = __builtin_convertvector(ds.hi, bf16x8);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(qtile, trb, dt, 0, lane), db0, dk[dt], 0, 0, 0);
        dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(qtile, trb, dt, 1, lane), db1, dk[dt], 0, 0, 0);
      }
    }
  }
  if (!has_blk) continue;
  // dk[dt][r], dv[dt][r]: [32 dt + 8 (r/4) + 4 h + r%4][key l32]
  uint16_t* ok = a.dk + tok * D;
  uint16_t* ov = a.dv + tok * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      store4(ok + 32 * dt + 8 * g4 + 4 * h, dk[dt], g4, a.scale, kvalid);
      store4(ov + 32 * dt + 8 * g4 + 4 * h, dv[dt], g4, 1.0f, kvalid);
    }
  }
}

// dV or dK alone (DK selects), for two waves per SIMD: the fused kernel
// above needs both accumulators and K, V in registers at once.  Workgroup =
// G key blocks, 2 waves each, wave w owning keys 32 (w%2)..+31 of block
// w/2; steps walk the union of the G columns, one 32-query half per step.
//   dV:  S = Q_half . K^T,  P,  dV^T += dO^T_half . P
//        stage: Q rows, dO^T (VT layout), 32 lse
//   dK:  S = Q_half . K^T,  dP = dO_half . V^T,  P,  dS = P (dP - delta),
//        dK^T += Q^T_half . dS
//        stage: Q rows, dO rows, 32 lse, 32 -delta (Q^T by transposed reads
//        of the Q rows)
template <int D, int NST, int G, bool DK, int OCC>
__global__ __launch_bounds__(128 * G, OCC) void k_bwd_dkv(BwdArgs a) {
  constexpr int NW = 2 * G;
  constexpr int KS = D / 16, DT = D / 32, KCH = D / 8;
  constexpr int HALF = 32 * D * 2;
  constexpr int NT = 2;                   // 32-row tiles per stage
  constexpr int LDB = DK ? 256 : 128;     // lse (and delta) bytes per stage
  constexpr int STAGE = NT * HALF + LDB;
  constexpr int LPW = HALF / 1024 / NW;
  constexpr int PW = NT * LPW + 1;
  constexpr int LDW = LDB / 4 / NW;       // lse / delta floats each wave brings
  static_assert(LPW >= 1 && (HALF / 1024) % NW == 0 && LDW % 4 == 0, "loads split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) uint4 ring[NST * STAGE / 16];
  __shared__ int s_item;
  for (int item = bwd_next(a, &s_item, true); item >= 0; item = bwd_next(a, &s_item, false)) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = w >> 1, w2 = w & 1;
  const int h = lane >> 5, l32 = lane & 31;
  const int ngh = (a.n_blk + G - 1) / G;
  const int bh = item / ngh, J0 = (item - bh * ngh) * G;
  int blk[G];
  group_blocks<G>(a.pairs, item, J0, a.n_blk, blk);
  const bool has_blk = blk[kg] >= 0;
  const int J = has_blk ? blk[kg] : blk[0];
  const int64_t head = (int64_t)bh * a.n_pad;
  const int64_t tok = head + (int64_t)J * 64 + 32 * w2 + l32;   // this lane's key token
  const float sl2 = a.scale * 1.44269504088896340736f;
  const uint32_t kmask = has_blk ? (uint32_t)(sload(a.blk_mask, J) >> (32 * w2)) : 0u;
  const bool kvalid = kmask >> l32 & 1;

  uint32_t roff[LPW], toff[LPW];
  tile_offsets<D, LPW, NW>(w, lane, roff, toff);
  uint32_t own_lo, own_hi, un_lo, un_hi;
  group_bits<G>(a.bits_t, (int64_t)bh * a.n_blk, blk, a.nw, lane, kg, &own_lo, &own_hi, &un_lo, &un_hi);

  bf16x8 kreg[KS], vreg[DK ? KS : 1];
  {
    const uint4* krow = (const uint4*)(a.k + tok * D);
    const uint4* vrow = (const uint4*)(a.v + tok * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kreg[ks] = as_bf16x8(krow[2 * ks + h]);
      if (DK) vreg[DK ? ks : 0] = as_bf16x8(vrow[2 * ks + h]);
    }
    wait_vm<0>();
  }

  BitWalk iw, cw;
  const char* qbase = (const char*)(a.q + head * D);
  const char* dbase = (const char*)(a.dout + head * D);
  const char* dtbase = (const char*)(a.dot + head * D);
  // floats [LDW w, LDW (w+1)) of the stage's [32 lse | 32 -delta]
  const float* lbase = (LDW * w < 32 ? a.lse + LDW * w : (const float*)a.ndelta + (LDW * w - 32)) + head;
  int curI = 0;
  const int total = union_steps(un_lo, un_hi);   // two halves per union block
  // the loads of one step into a ring stage known at compile time (the step
  // loop below is unrolled by the ring depth, so the stage offsets need no
  // readfirstlane): Q rows, then dO rows (dK) or dO^T (dV), then lse (and
  // delta)
  auto issue_at = [&](int stage, int u) __attribute__((always_inline)) {
    if (u == 0) curI = iw.next_known(un_lo, un_hi);
    const int64_t roff0 = ((int64_t)curI * 64 + 32 * u) * D * 2;
    const int64_t toff0 = (int64_t)curI * 64 * D * 2 + u * HALF;
    const uint32_t dst = lds_addr(ring) + stage * STAGE;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const uint32_t o1 = (NW * j + w) * 1024;
      dma16(qbase + roff0, roff[j], dst + o1);
      if (DK) dma16(dbase + roff0, roff[j], dst + HALF + o1);
      else dma16(dtbase + toff0, toff[j], dst + HALF + o1);
    }
    if (lane < LDW / 4) dma16(lbase + (int64_t)curI * 64 + 32 * u, lane * 16, dst + NT * HALF + 4 * LDW * w);
  };

  const TrBase trb = tr_base<D>(lds_addr(ring), lane);
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < total) issue_at(st, st & 1);

  int I = 0;
  // valid-query mask of the current block for this wave (zero when the
  // column does not list it), a scalar word taken once per block
  uint64_t qm64 = 0;
  // unrolled by the ring depth, so copy kk reads stage kk (offsets fold
  // into the LDS reads' immediates) and loads into stage (kk + NST - 1) % NST
  constexpr int UNR = NST;
  for (int st0 = 0; st0 < total; st0 += UNR) {
#pragma unroll
  for (int kk = 0; kk < UNR; ++kk) {
    const int st = st0 + kk;
    if (st >= total) break;
    if ((st & 1) == 0) {
      I = cw.next_known(un_lo, un_hi);
      const bool mine = lane_word(own_lo, own_hi, I >> 6) >> (I & 63) & 1;
      qm64 = mine && kmask != 0 ? sload(a.blk_mask, I) : 0ull;
    }
    wait_steps<PW, NST>(st, total);
    barrier_no_fence();
    if (st + NST - 1 < total) issue_at((kk + NST - 1) % NST, (st + NST - 1) & 1);

    const int u = st & 1;
    const uint32_t qm = (uint32_t)(qm64 >> (32 * u));
    if (qm == 0) continue;   // not in this column, pad queries, or a wave of pad keys
    const uint4* qst = ring + kk * (STAGE / 16);
    const uint4* t1 = qst + HALF / 16;       // dO rows (dK) or dO^T (dV)
    const float* lds_l = (const float*)(qst + NT * HALF / 16);
    // element r: query 8*(r/4) + 4*h + r%4 of this half, key l32.  No
    // per-element mask: a pad query has zero Q, dO and delta rows and lse 0,
    // so its P is exactly 1 and every product it enters (dO^T P for dV,
    // Q^T dS with dS = P (0 - 0) for dK) adds exact zeros; a pad key's column
    // only reaches its own output row, which the store writes as zero.
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    f32x16 s = {}, dp = {};
    if (DK) {   // dP starts at minus delta (the stage holds -delta), so dS = P * dP
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 nD = *(const f32x4*)(lds_l + 32 + 8 * c + 4 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j) dp[4 * c + j] = nD[j];
      }
    }
    // dK: the eight Q operand reads of the S products are issued together
    // ahead of them, held there by a scheduling fence, as in the forward
    // kernel (246 VGPRs; backward kernels 51.0 -> 50.7 ms at the Wan-14B
    // 480P shape, bit-identical).  The dV form, at three waves per SIMD, has
    // no registers to spare for it.
    bf16x8 qf[KS];
    if constexpr (DK) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(qst[l32 * KCH + ((2 * ks + h) ^ kswz_t<D>(l32))]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = l32 * KCH + ((2 * ks + h) ^ kswz_t<D>(l32));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(DK ? qf[ks] : as_bf16x8(qst[c]), kreg[ks], s, 0, 0, 0);
      if (DK) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(t1[c]), vreg[DK ? ks : 0], dp, 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(2);   // raised priority to the end of the step, as in k_bwd_dq
    f32x16 x;   // P (dV) or dS (dK)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 L = *(const f32x4*)(lds_l + 8 * c + 4 * h);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * c + j;
        const float p = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -L[j]));
        x[r] = DK ? p * dp[r] : p;
      }
    }
    const bf16x8 xb0 = __builtin_convertvector(x.lo, bf16x8), xb1 = __builtin_convertvector(x.hi, bf16x8);
    // dK: Q^T by transposed reads of the stage's Q rows; dV: the dO^T tile
    const uint32_t qtile = (uint32_t)(kk * STAGE);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 32 * dt + l32;
      const int sw = vswz(d);
      const bf16x8 a0 = DK ? tr_operand<D>(qtile, trb, dt, 0, lane) : as_bf16x8(t1[d * 4 + ((0 + h) ^ sw)]);
      const bf16x8 a1 = DK ? tr_operand<D>(qtile, trb, dt, 1, lane) : as_bf16x8(t1[d * 4 + ((2 + h) ^ sw)]);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, xb0, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, xb1, acc[dt], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  }
  }
  if (!has_blk) continue;
  // acc[dt][r]: [32 dt + 8 (r/4) + 4 h + r%4][key l32]
  uint16_t* out = (DK ? a.dk : a.dv) + tok * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) store4(out + 32 * dt + 8 * g4 + 4 * h, acc[dt], g4, DK ? a.scale : 1.0f, kvalid);
  }
}

// dK/dV kernels: 0 = dK and dV in separate kernels of two key blocks per
// workgroup (default); 1 or 2 = the fused kernel with that many key blocks
// per workgroup.  FVA_BWD_KGROUP overrides it.
int bwd_kgroup() {
  const char* v = getenv("FVA_BWD_KGROUP");
  const int n = v ? atoi(v) : 0;
  return n == 1 || n == 2 ? n : 0;
}

// Tuning switches of the split dK / dV kernels: FVA_BWD_DV_OCC = 2|3
// (waves per SIMD the dV kernel is compiled for), FVA_BWD_DK_NST = 2|3
// (ring depth of the dK kernel).
int env_pick(const char* name, int a, int b, int dflt) {
  const char* v = getenv(name);
  const int n = v ? atoi(v) : dflt;
  return n == a || n == b ? n : dflt;
}

// Schedule of the backward grids.  Persistent (default): a resident grid
// pops groups from per-XCD cursors, one head's groups per XCD chunk (or an
// equal part of a head when the head count is not a multiple of 8), so a
// head's Q, dO (or K, V) is fetched into one XCD's L2.  Plain
// (FVA_BWD_SCHED=plain): one workgroup per group in chunks of 16 groups per
// XCD (in-order dispatch cannot take head-sized chunks).  FVA_BWD_CHUNK
// overrides the chunk of either.
bool bwd_persistent() {
  const char* v = getenv("FVA_BWD_SCHED");
  return !(v && strcmp(v, "plain") == 0);
}

int bwd_chunk(int dflt) {
  const char* v = getenv("FVA_BWD_CHUNK");
  int n = v ? atoi(v) : dflt;
  if (n < 1 || n > 65536) n = dflt;
  return n;
}

template <typename K>
int bwd_occupancy(K kernel, int threads) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, 0) != hipSuccess || nb < 1) nb = 1;
  return nb;
}

// Launch one backward kernel over the groups of G blocks of every head, with
// its own cursor set (16 counters, zeroed by the caller).
template <typename K>
void bwd_launch(K kernel, int threads, int G, BwdArgs a, fva_plan_t plan, int32_t* cursor, const int32_t* order,
                const int2* pairs, hipStream_t stream) {
  const int n_bh = plan->desc.batch * plan->desc.heads;
  const int ngh = (int)((plan->info.n_blk + G - 1) / G);
  a.n_items = n_bh * ngh;
  a.persistent = bwd_persistent() ? 1 : 0;
  a.cursor = cursor;
  a.order = order;
  a.pairs = G == 2 ? pairs : nullptr;
  // whole heads per XCD chunk, cut into 8 / gcd(heads, 8) parts so every
  // XCD gets the same number of chunks
  int gc = n_bh, bb = kXcds;
  while (bb) { const int t = gc % bb; gc = bb; bb = t; }
  const int parts = kXcds / gc;
  a.chunk = bwd_chunk(a.persistent ? (ngh + parts - 1) / parts : 16);
  int64_t grid;
  if (a.persistent) {
    grid = std::min<int64_t>(a.n_items, (int64_t)plan->num_cu * bwd_occupancy(kernel, threads));
  } else {
    const int64_t deal = (int64_t)kXcds * a.chunk;
    grid = (a.n_items + deal - 1) / deal * deal;
  }
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(threads), 0, stream, a);
}

// Row bitmaps of a CSR and their per-head transpose into the plan's workspace.
void launch_lists(fva_plan_t plan, const int32_t* row_ptr, const int32_t* col_idx, hipStream_t stream) {
  const fva_plan_info& in = plan->info;
  const int n_bh = plan->desc.batch * plan->desc.heads;
  hipLaunchKernelGGL(k_csr_bits, dim3((unsigned)((in.n_rows + 3) / 4)), dim3(256), 0, stream, row_ptr, col_idx,
                     (int)in.n_blk, plan->nw, in.n_rows, plan->rowmask);
  hipLaunchKernelGGL(k_bits_transpose, dim3((unsigned)((plan->nw * plan->nw + 3) / 4), n_bh), dim3(256), 0, stream,
                     plan->rowmask, (int)in.n_blk, plan->nw, plan->bits_t);
}

}  // namespace

void fva_csr_bits(fva_plan_t plan, const int32_t* row_ptr, const int32_t* col_idx, uint64_t* bits,
                  hipStream_t stream) {
  const fva_plan_info& in = plan->info;
  hipLaunchKernelGGL(k_csr_bits, dim3((unsigned)((in.n_rows + 3) / 4)), dim3(256), 0, stream, row_ptr, col_idx,
                     (int)in.n_blk, plan->nw, in.n_rows, bits);
}

extern "C" int fva_mask_transpose(fva_plan_t plan, const int32_t* row_ptr, const int32_t* col_idx,
                                  int32_t* t_row_ptr, int32_t* t_col_idx, hipStream_t stream) {
  if (!plan) return fva_fail(FVA_EINVAL, "plan is NULL");
  if (!row_ptr || !col_idx || !t_row_ptr || !t_col_idx)
    return fva_fail(FVA_EINVAL, "row_ptr / col_idx / t_row_ptr / t_col_idx is NULL");
  launch_lists(plan, row_ptr, col_idx, stream);
  const int rc = fva_bits_to_csr(plan, plan->bits_t, t_row_ptr, t_col_idx, stream);
  if (rc != FVA_OK) return rc;
  return fva_after_launch(stream, "fva_mask_transpose");
}

extern "C" int fva_attention_backward(fva_plan_t plan, const void* q_perm, const void* k_perm, const void* v_perm,
                                      const float* o32, const float* lse, const void* do_perm, const void* do_vt,
                                      const int32_t* row_ptr, const int32_t* col_idx, void* dq_perm, void* dk_perm,
                                      void* dv_perm, hipStream_t stream) {
  if (!plan) return fva_fail(FVA_EINVAL, "plan is NULL");
  if (!q_perm || !k_perm || !v_perm || !o32 || !lse || !do_perm || !do_vt)
    return fva_fail(FVA_EINVAL, "input pointer is NULL");
  if (!row_ptr || !col_idx) return fva_fail(FVA_EINVAL, "row_ptr / col_idx is NULL");
  if (!dq_perm || !dk_perm || !dv_perm) return fva_fail(FVA_EINVAL, "gradient pointer is NULL");
  const fva_plan_desc& d = plan->desc;
  const fva_plan_info& in = plan->info;
  if (d.dtype != FVA_DTYPE_BF16) return fva_fail(FVA_EUNSUPPORTED, "the backward pass is bf16 only");
  launch_lists(plan, row_ptr, col_idx, stream);
  BwdArgs a{};
  a.q = (const uint16_t*)q_perm;
  a.k = (const uint16_t*)k_perm;
  a.v = (const uint16_t*)v_perm;
  a.o32 = o32;
  a.lse = lse;
  a.dout = (const uint16_t*)do_perm;
  a.dot = (const uint16_t*)do_vt;
  a.bits = plan->rowmask;
  a.bits_t = plan->bits_t;
  a.blk_mask = plan->blk_mask;
  a.blk_full = plan->blk_full;
  a.ndelta = plan->bwd_delta;
  a.dq = (uint16_t*)dq_perm;
  a.dk = (uint16_t*)dk_perm;
  a.dv = (uint16_t*)dv_perm;
  a.n_pad = in.n_pad;
  a.n_blk = (int)in.n_blk;
  a.nw = plan->nw;
  a.scale = 1.0f / sqrtf((float)d.head_dim);
  constexpr int GQ = 2;   // query blocks per workgroup of the dQ kernel
  const int kmode = bwd_kgroup();
  const int dv_occ = env_pick("FVA_BWD_DV_OCC", 2, 3, 3);
  const int dk_nst = env_pick("FVA_BWD_DK_NST", 2, 3, 2);
  // cursor sets: dQ, dV (or fused dK/dV), dK
  int32_t* cq = plan->counters + 16;
  int32_t* cv = plan->counters + 32;
  int32_t* ck = plan->counters + 48;
  hipLaunchKernelGGL(k_zero_i32, dim3(1), dim3(64), 0, stream, cq, 48);
  // longest-first order inside each head: query-block groups by row lengths
  // (dQ), key-block groups by column lengths (dK, dV)
  const int n_bh = d.batch * d.heads;
  const int GK = kmode == 1 ? 1 : 2;
  int32_t* oq = plan->worklist;
  int32_t* ok = plan->worklist_t;
  // groups of two by list overlap: query blocks over rows, key blocks over
  // columns (FVA_BWD_PAIR=0: consecutive ids)
  const bool paired = env_pick("FVA_BWD_PAIR", 0, 1, 1) == 1;
  const int2* pq = paired ? plan->pairs : nullptr;
  const int2* pk = paired && GK == 2 ? plan->pairs_t : nullptr;
  if (paired) {
    fva_pair_blocks(plan, plan->rowmask, plan->pairs, stream);
    if (GK == 2) fva_pair_blocks(plan, plan->bits_t, plan->pairs_t, stream);
  }
  if (bwd_persistent()) {
    hipLaunchKernelGGL(k_bwd_order, dim3(n_bh), dim3(1024), 0, stream, plan->rowmask, (int)in.n_blk, plan->nw, GQ, pq,
                       oq);
    hipLaunchKernelGGL(k_bwd_order, dim3(n_bh), dim3(1024), 0, stream, plan->bits_t, (int)in.n_blk, plan->nw, GK, pk,
                       ok);
  }
  if (d.head_dim == 128) {
    bwd_launch(k_bwd_dq<128, 4, GQ>, 128 * GQ, GQ, a, plan, cq, oq, pq, stream);
    if (kmode == 0) {
      if (dv_occ == 3) bwd_launch(k_bwd_dkv<128, 3, 2, false, 3>, 256, 2, a, plan, cv, ok, pk, stream);
      else bwd_launch(k_bwd_dkv<128, 3, 2, false, 2>, 256, 2, a, plan, cv, ok, pk, stream);
      if (dk_nst == 3) bwd_launch(k_bwd_dkv<128, 3, 2, true, 2>, 256, 2, a, plan, ck, ok, pk, stream);
      else bwd_launch(k_bwd_dkv<128, 2, 2, true, 2>, 256, 2, a, plan, ck, ok, pk, stream);
    } else if (kmode == 2) {
      bwd_launch(k_bwd_dkdv<128, 2, 2>, 256, 2, a, plan, cv, ok, pk, stream);
    } else {
      bwd_launch(k_bwd_dkdv<128, 2, 1>, 128, 1, a, plan, cv, ok, pk, stream);
    }
  } else {
    bwd_launch(k_bwd_dq<64, 4, GQ>, 128 * GQ, GQ, a, plan, cq, oq, pq, stream);
    if (kmode == 0) {
      if (dv_occ == 3) bwd_launch(k_bwd_dkv<64, 3, 2, false, 3>, 256, 2, a, plan, cv, ok, pk, stream);
      else bwd_launch(k_bwd_dkv<64, 3, 2, false, 2>, 256, 2, a, plan, cv, ok, pk, stream);
      if (dk_nst == 3) bwd_launch(k_bwd_dkv<64, 3, 2, true, 2>, 256, 2, a, plan, ck, ok, pk, stream);
      else bwd_launch(k_bwd_dkv<64, 2, 2, true, 2>, 256, 2, a, plan, ck, ok, pk, stream);
    } else if (kmode == 2) {
      bwd_launch(k_bwd_dkdv<64, 2, 2>, 256, 2, a, plan, cv, ok, pk, stream);
    } else {
      bwd_launch(k_bwd_dkdv<64, 2, 1>, 128, 1, a, plan, cv, ok, pk, stream);
    }
  }
  return fva_after_launch(stream, "fva_attention_backward");
}
