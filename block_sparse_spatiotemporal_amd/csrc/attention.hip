// Fine stage: block-sparse attention over the selected key blocks only
// ("Video Sparse Attention" explainer, section 3), with online softmax, and
// the one-GPU share of run-time load balancing ("FVAttn" review, section 02):
// rows of very different cost are sorted longest-first into a device work
// list and pulled by a persistent grid, so no compute unit idles while
// another still holds a long row.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <mutex>

#include "attn_common.h"
#include "fva_internal.h"

namespace {

using namespace fva_attn;

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
  const uint64_t* blk_full; // [64] bitmap of blocks with every position valid
  void* o;
  const int32_t* worklist;
  const int2* pairs;        // optional (G = 2): the two query blocks of each group
  int32_t* cursor;
  uint64_t* wg_times;
  float* lse;               // optional [B*H, n_pad]: log2 sum exp2 of the scaled scores
  float* o32;               // optional [B*H, n_pad, D]: the output before rounding to bf16
  const int32_t* perm;      // optional: write O in raster order [B, N, H, D] (position -> token)
  int64_t n_tok;            // raster tokens per batch entry (with perm)
  int heads;                // H (with perm)
  int64_t n_pad;
  int n_items;
  int n_blk;
  int persistent;
  int chunk;                // work-list chunk dealt to one XCD at a time
  float scale;              // 1/sqrt(D)
};


// Next row for this workgroup, or -1 when the work list is exhausted.
// Plain: workgroup b is on XCD b % 8 and takes its XCD's (b / 8)-th row.
// Persistent: one cursor per XCD; an XCD whose share is done steals from
// the others, so every workgroup leaves only when all rows are taken.
__device__ __forceinline__ int next_item(const AttnArgs& a, int* s_item, bool first) {
  if (!a.persistent) {
    if (!first) return -1;
    const int64_t it = xcd_item(blockIdx.x % kXcds, blockIdx.x / kXcds, a.chunk);
    return it < a.n_items ? (int)it : -1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int x0 = blockIdx.x % kXcds;
    int found = -1;
    for (int t = 0; t < kXcds && found < 0; ++t) {
      const int x = (x0 + t) % kXcds;
      if (__hip_atomic_load(&a.cursor[kXcds + x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) continue;
      const int64_t it = xcd_item(x, atomicAdd(&a.cursor[x], 1), a.chunk);
      if (it < a.n_items) found = (int)it;
      else __hip_atomic_store(&a.cursor[kXcds + x], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    *s_item = found;
  }
  __syncthreads();
  return *s_item;
}

// Output row of query position `pos` of (b, h) = bh: block order
// [B*H, n_pad, D], or with a.perm the raster row [b, perm[pos], h, :]; null
// for a pad position in raster order (nothing is written there).
template <typename T>
__device__ __forceinline__ T* out_row(const AttnArgs& a, int bh, int64_t pos, int D) {
  if (!a.perm) return (T*)a.o + ((int64_t)bh * a.n_pad + pos) * D;
  const int tok = a.perm[pos];
  if (tok < 0) return nullptr;
  const int b = bh / a.heads, h = bh - b * a.heads;
  return (T*)a.o + (((int64_t)b * a.n_tok + tok) * a.heads + h) * D;
}

// ------------------------------------------------------------------ bf16
// Workgroup = 2 waves = one 64-query block; wave w owns queries 32w..32w+31.
// A step is one 32-key half of a selected block:
//   S^T (32 keys x 32 queries) = K_half . Q^T     (D/16 MFMA 32x32x16 bf16)
//   online softmax in fp32 on the accumulators (each lane owns one query)
//   O^T (D x 32 queries) += V^T_half . P^T        (D/32 x 2 MFMA)
// P^T feeds the second product straight from the accumulators (the VT key
// slot order makes that consistent).  K and V^T halves stream from HBM into
// an NST-stage LDS ring with direct global->LDS loads (no register staging);
// each wave issues half of a stage's 1 KB loads, waits on its own vector
// memory counter, and one barrier per step publishes the stage to both waves
// and retires the stage the next load overwrites.  The LDS image of each
// stage is XOR-swizzled so the 16-byte operand reads are conflict free: the
// swizzle is applied by choosing each lane's source address, since a direct
// load writes lane i's 16 bytes at offset 16*i of its 1 KB destination.
// The running max is raised lazily: P may grow to 2^kLazy before O and l are
// rescaled, which skips most rescales once the row maximum is found.
// FOLD (the default inference form) takes the scale (1/sqrt(D) in log2
// units) into Q when it loads Q, rounding the scaled Q to bf16, and starts
// each S accumulator at minus the running max, so a weight is one exp2 of
// an accumulator with no multiply or shift per score.  The extra rounding
// of Q moves a logit by up to 2^-9 of |q . k| * scale, which grows with the
// logit range; without FOLD (the training form, and the inference form's
// exact-scale variant) S stays exact in fp32 and one fma applies the scale
// and the shift.

// G query blocks per workgroup (2G waves; wave w serves block w/2, queries
// 32*(w%2)..+31).  Steps walk the union of the G block lists half by half;
// a stage is loaded once and used by every wave pair whose list holds it.
// LSE: the training-forward form.  It sums the row in fp32 over the
// unrounded weights (the per-query log-sum-exp it writes is what the
// backward pass rebuilds P from, so it must be the softmax normaliser to
// fp32 accuracy), and writes lse and the fp32 output.  The inference form
// sums the bf16 weights PV uses, with dot instructions: half the adds, and
// O normalised by exactly the weights applied to V.
template <int D, int NST, int G, bool LSE, bool FOLD = !LSE>
__global__ __launch_bounds__(128 * G, 2) void k_attn_bf16(AttnArgs a) {
  static_assert(!(LSE && FOLD), "the training form keeps S exact");
  constexpr int NW = 2 * G;             // waves per workgroup
  constexpr int KS = D / 16;            // k-steps of S^T
  constexpr int DT = D / 32;            // d tiles of O^T
  constexpr int KCH = D / 8;            // 16-byte chunks per K row
  constexpr int HALF = 32 * D * 2;      // bytes of one K half (and of one V^T half)
  constexpr int STAGE = 2 * HALF;
  constexpr int NI = HALF / 1024;       // 1 KB direct loads per half per workgroup
  constexpr int LPW = NI / NW;          // loads per wave per half (K and V each)
  constexpr int PW = 2 * LPW;           // direct loads per wave per step
  constexpr float kLazy = 8.0f;
  static_assert(NI % NW == 0, "loads split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) uint4 ring[NST * STAGE / 16];
  __shared__ int s_item;
  __shared__ uint32_t s_bits[128 * G];  // per row of the group: 64 bitmap words of 64 bits
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int qg = w >> 1, w2 = w & 1;    // query block of the group, half of the block
  const int nw = (a.n_blk + 63) >> 6;   // bitmap words in use (n_blk <= 4096)
  // blocks with all 64 positions valid (no key mask needed), one word per lane
  const uint64_t fw = lane < nw ? a.blk_full[lane] : 0;
  const uint32_t full_lo = (uint32_t)fw, full_hi = (uint32_t)(fw >> 32);
  const int h = lane >> 5, l32 = lane & 31;
  const uint64_t t0 = wall_clock64();
  const float sl2 = a.scale * 1.44269504088896340736f;   // scores in log2 units
  // Source offset (bytes, within a K half / V^T half) of this lane's 16 bytes
  // for each of the wave's direct loads.  Load i writes LDS bytes
  // [1024 i, 1024 i + 1024) of the half; lane L lands at 1024 i + 16 L.
  // Physical chunk pc of K row r holds logical chunk pc ^ kswz(r); physical
  // chunk pc of V^T row d holds logical chunk pc ^ vswz(d).
  uint32_t koff[LPW], voff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int off = (NW * j + w) * 1024 + lane * 16;
    const int row = off / (KCH * 16), pc = (off / 16) % KCH;
    koff[j] = row * (D * 2) + ((pc ^ kswz<D>(row)) * 16);
    const int d = off / 64, pv = (off / 16) & 3;
    voff[j] = d * 64 + ((pv ^ vswz(d)) * 16);
  }
  const int ngh = (a.n_blk + G - 1) / G;   // groups per head
  for (int item = next_item(a, &s_item, true); item >= 0; item = next_item(a, &s_item, false)) {
    const int gid = sload(a.worklist, __builtin_amdgcn_readfirstlane(item));
    const int bh = gid / ngh;
    const int I0 = (gid - bh * ngh) * G;
    // this wave pair's query block, or -1: consecutive ids, or the pair
    // table (G = 2, groups paired by list overlap)
    int Iq = I0 + qg < a.n_blk ? I0 + qg : -1, Ifirst = I0;
    if (G == 2 && a.pairs) {
      const uint64_t pr = sload((const uint64_t*)a.pairs, gid);   // (x, y) of an int2
      const int px = (int)(uint32_t)pr, py = (int)(uint32_t)(pr >> 32);
      Iq = qg == 0 ? px : py;
      Ifirst = px;
    }
    const int64_t head = (int64_t)bh * a.n_pad;
    // The G rows' block sets as bitmaps: LDS words filled from the CSR
    // lists (ids outside the plan are dropped), then one 64-bit word per
    // lane for the union and for this wave's own row.
    s_bits[tid] = 0;
    __syncthreads();
    {
      const int64_t rr = (int64_t)bh * a.n_blk + Iq;
      if (Iq >= 0) {
        const int beg = sload(a.row_ptr, rr), end = sload(a.row_ptr, rr + 1);
        for (int j = beg + (tid & 127); j < end; j += 128) {
          const int J = a.col_idx[j];
          if ((unsigned)J < (unsigned)a.n_blk) atomicOr(&s_bits[128 * qg + (J >> 5)], 1u << (J & 31));
        }
      }
    }
    __syncthreads();
    uint32_t own_lo = s_bits[128 * qg + 2 * lane], own_hi = s_bits[128 * qg + 2 * lane + 1];
    uint32_t un_lo = 0, un_hi = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      un_lo |= s_bits[128 * g + 2 * lane];
      un_hi |= s_bits[128 * g + 2 * lane + 1];
    }
    // Two identical walks over the union: one issues loads NST-1 steps
    // ahead, the other follows the computation.  The step count (two
    // halves per union block) is known up front, so neither walk tests
    // for its end and the waits need no bookkeeping of what is in flight.
    BitWalk iw, cw;
    const int total = union_steps(un_lo, un_hi);
    const char* kbase = (const char*)(a.k + head * D);
    const char* vbase = (const char*)(a.vt + head * D);
    int curJ = 0;
    // Issue the direct loads of the next step into ring stage `stage`: half
    // u of block curJ (the walk advances on the first half).  Both arguments
    // are compile-time constants at every call site of the unrolled loop.
    auto issue_next = [&](int stage, int u) __attribute__((always_inline)) {
      if (u == 0) curJ = iw.next_known(un_lo, un_hi);
      const int J = curJ;
      const char* ksrc = kbase + ((int64_t)J * 64 + 32 * u) * D * 2;
      const char* vsrc = vbase + (int64_t)J * 64 * D * 2 + u * HALF;
      const uint32_t dst = lds_addr(ring) + stage * STAGE;
#pragma unroll
      for (int j = 0; j < LPW; ++j) {
        const int i = NW * j + w;
        dma16(ksrc, koff[j], dst + i * 1024);
        dma16(vsrc, voff[j], dst + HALF + i * 1024);
      }
    };

    const bool has_row = Iq >= 0;
    const int I = has_row ? Iq : Ifirst;
    bf16x8 qreg[KS];
    {
      const uint4* qrow = (const uint4*)(a.q + (head + (int64_t)I * 64 + 32 * w2 + l32) * D);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qreg[ks] = as_bf16x8(qrow[2 * ks + h]);
      if constexpr (FOLD) {   // Q . scale in log2 units, rounded to bf16
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          f32x8 qf = __builtin_convertvector(qreg[ks], f32x8);
          qf *= sl2;
          qreg[ks] = __builtin_convertvector(qf, bf16x8);
        }
      }
      // Settle the Q loads before any direct load is issued: a wait left to
      // the first use inside the step loop would also count, every step, the
      // direct loads in flight behind them.
      wait_vm<0>();
    }
    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f;
    // inference form: the accumulators start at -base; base is 0 until the
    // first step raises the running max, and equals it from then on
    f32x16 negm = {};
    float thr = -INFINITY;   // a lane raises its max once a score exceeds base + thr

#pragma unroll
    for (int st = 0; st < NST - 1; ++st)
      if (st < total) issue_next(st, st & 1);

    int J = 0;
    // valid-key mask of the current block for this wave: zero when the
    // wave's row does not list the block, all ones for a block without pads
    uint64_t kmask = 0;
    // Unrolled by the ring depth so each copy of the step reads a fixed
    // stage: the stage offset then folds into the LDS reads' immediate
    // offsets instead of costing address arithmetic every step.
    for (int st0 = 0; st0 < total; st0 += NST) {
#pragma unroll
    for (int kk = 0; kk < NST; ++kk) {
      const int st = st0 + kk;
      if (st >= total) break;
      const int u = NST % 2 == 0 ? (kk & 1) : (st & 1);   // half of the block
      if (u == 0) {
        J = cw.next_known(un_lo, un_hi);
        const bool mine = lane_word(own_lo, own_hi, J >> 6) >> (J & 63) & 1;
        const bool full = lane_word(full_lo, full_hi, J >> 6) >> (J & 63) & 1;
        kmask = !mine ? 0ull : (full ? ~0ull : sload(a.blk_mask, J));
      }
      // wait for this wave's loads of step st; the NST-2 steps issued after
      // it may stay in flight (fewer near the end of the walk)
      if (st + NST - 2 < total) wait_vm<(NST - 2) * PW>();
      else if (NST >= 4 && st + 2 < total) wait_vm<2 * PW>();
      else if (NST >= 3 && st + 1 < total) wait_vm<PW>();
      else wait_vm<0>();
      barrier_no_fence();
      if (st + NST - 1 < total)   // step st + NST - 1, into the stage retired by the barrier
        issue_next((kk + NST - 1) % NST, NST % 2 == 0 ? ((kk + NST - 1) & 1) : ((st + NST - 1) & 1));

      const uint32_t mh = (uint32_t)(kmask >> (32 * u));
      if (mh == 0) continue;   // not in this row's list, or a half of pad keys (uniform per wave)
      const uint4* kst = ring + kk * (STAGE / 16);
      const uint4* vst = kst + HALF / 16;

      f32x16 s;
      if constexpr (!FOLD) s = f32x16{};
      else s = negm;
      // All of the step's K operand reads are issued ahead of the products
      // (the scheduling fence keeps the compiler from trickling them in two
      // at a time, which left each product waiting out an LDS latency).
      bf16x8 kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[ks] = as_bf16x8(kst[l32 * KCH + ((2 * ks + h) ^ kswz<D>(l32))]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qreg[ks], s, 0, 0, 0);
      // s[i]: key 8*(i/4) + 4*h + i%4 of this half, query l32.  Pad keys get
      // -inf.  Without FOLD the scale (1/sqrt(D) in log2 units, > 0) is
      // applied after the max; with FOLD s is already scaled and shifted.
      if (mh != 0xFFFFFFFFu) {   // per register: a sign-extended bit, one three-input bit op
        const uint32_t ml = mh >> (4 * h);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t vm = (uint32_t)__builtin_amdgcn_sbfe((int)ml, 8 * (i >> 2) + (i & 3), 1);
          s[i] = __uint_as_float((__float_as_uint(s[i]) & vm) | (~vm & 0xFF800000u));   // else -inf
        }
      }
      // The V^T operands of the PV products are read now, so their LDS
      // latency passes under the softmax.
      bf16x8 vf[2 * DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 32 * dt + l32;
        const int sw = vswz(d);
        vf[2 * dt] = as_bf16x8(vst[d * 4 + ((0 + h) ^ sw)]);
        vf[2 * dt + 1] = as_bf16x8(vst[d * 4 + ((2 + h) ^ sw)]);
      }
      __builtin_amdgcn_sched_barrier(0);
      // From its softmax to the end of its PV products a wave runs at a
      // raised priority, so a wave finishing a step issues ahead of a
      // co-resident wave starting one (measured: 2.5% at the 720P shape,
      // neutral at 480P, bit-identical).
      __builtin_amdgcn_s_setprio(2);
      // The lazy test needs only this lane's 16 scores: some lane of the
      // wave exceeds the threshold exactly when some query's row does.  The
      // max over the other lane half (same query) is taken on a raise only.
      float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s[i]), s[i + 1]);
      mx = fmaxf(mx, s[15]);
      f32x8 p0, p1;
      if constexpr (!FOLD) {
        if (__ballot(mx * sl2 > m_run + kLazy)) {   // raise the running max (first step always)
          const float m_new = fmaxf(m_run, xhalf_max(mx) * sl2);
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
          m_run = m_new;
        }
        const float nm = -m_run;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p0[i] = __builtin_amdgcn_exp2f(fmaf(s[i], sl2, nm));
          p1[i] = __builtin_amdgcn_exp2f(fmaf(s[8 + i], sl2, nm));
        }
      } else {
        // scores are already less base
        if (__ballot(mx > thr)) {   // raise the running max (first step always)
          const float base = -negm[0];
          const float m_new = fmaxf(m_run, base + xhalf_max(mx));
          const float delta = m_new - base;
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
#pragma unroll
          for (int i = 0; i < 16; ++i) s[i] -= delta;
#pragma unroll
          for (int i = 0; i < 16; ++i) negm[i] = -m_new;
          m_run = m_new;
          thr = kLazy;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p0[i] = __builtin_amdgcn_exp2f(s[i]);
          p1[i] = __builtin_amdgcn_exp2f(s[8 + i]);
        }
      }
      const bf16x8 pb0 = __builtin_convertvector(p0, bf16x8);
      const bf16x8 pb1 = __builtin_convertvector(p1, bf16x8);
      if constexpr (LSE) {
#pragma unroll
        for (int i = 0; i < 8; ++i) l_run += p0[i] + p1[i];
      } else {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x2 a0 = {pb0[2 * i], pb0[2 * i + 1]}, a1 = {pb1[2 * i], pb1[2 * i + 1]};
          l_run = __builtin_amdgcn_fdot2_f32_bf16(a0, one2, l_run, false);
          l_run = __builtin_amdgcn_fdot2_f32_bf16(a1, one2, l_run, false);
        }
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[2 * dt], pb0, o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[2 * dt + 1], pb1, o[dt], 0, 0, 0);
      }
      __builtin_amdgcn_s_setprio(0);
    }
    }
    if (has_row) {
      const float l_tot = xhalf_sum(l_run);
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      const bool qvalid = sload(a.blk_mask, I) >> (32 * w2 + l32) & 1;
      uint16_t* orow = out_row<uint16_t>(a, bh, (int64_t)I * 64 + 32 * w2 + l32, D);
      if (LSE && h == 0)   // P_ij = exp2(s_ij * scale * log2(e) - lse_i) for the backward pass
        a.lse[head + (int64_t)I * 64 + 32 * w2 + l32] = qvalid && l_tot > 0.0f ? m_run + __log2f(l_tot) : 0.0f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          typedef float f32x4 __attribute__((ext_vector_type(4)));
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          f32x4 v = {o[dt][4 * g4] * inv, o[dt][4 * g4 + 1] * inv, o[dt][4 * g4 + 2] * inv, o[dt][4 * g4 + 3] * inv};
          if (!qvalid) v = f32x4{0.f, 0.f, 0.f, 0.f};
          const bf16x4 b = __builtin_convertvector(v, bf16x4);
          if (orow) *(uint2*)(orow + 32 * dt + 8 * g4 + 4 * h) = __builtin_bit_cast(uint2, b);
          if (LSE)
            *(f32x4*)(a.o32 + (head + (int64_t)I * 64 + 32 * w2 + l32) * D + 32 * dt + 8 * g4 + 4 * h) = v;
        }
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
  __shared__ uint32_t s_set[FVA_MAX_NBLK / 32];   // the row's blocks as a set
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
    // The row read as a set (an id listed twice counts once, ids outside the
    // plan are dropped), walked in ascending order.
    const int nwd = (a.n_blk + 31) >> 5;
    for (int i = tid; i < nwd; i += 256) s_set[i] = 0;
    __syncthreads();
    for (int e = a.row_ptr[r] + tid; e < a.row_ptr[r + 1]; e += 256) {
      const int J = a.col_idx[e];
      if ((unsigned)J < (unsigned)a.n_blk) atomicOr(&s_set[J >> 5], 1u << (J & 31));
    }
    __syncthreads();
    for (int wd = 0; wd < nwd; ++wd)
    for (uint32_t set = s_set[wd]; set; set &= set - 1) {
      const int J = 32 * wd + __builtin_ctz(set);
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
    float* orow = out_row<float>(a, bh, (int64_t)I * 64 + qi, D);
    if (orow) {
#pragma unroll
      for (int d = 0; d < DP; ++d) orow[part * DP + d] = qvalid ? o[d] * inv : 0.0f;
    }
  }
  if (a.wg_times && tid == 0) {
    a.wg_times[2 * blockIdx.x] = t0;
    a.wg_times[2 * blockIdx.x + 1] = wall_clock64();
  }
}

// ------------------------------------------------------------------ schedule
// Work list for the attention grid: heads in decreasing total cost (kept
// blocks, so the cheapest rows run last and the tail is short), each head's
// groups in id order (k_sched_lpt may then reorder them by cost inside the
// head).  Also clears the per-XCD cursors and exhaustion flags.  One
// workgroup.
__global__ __launch_bounds__(1024) void k_sched(const int32_t* __restrict__ row_ptr, int n_blk, int n_bh, int G,
                                                int32_t* __restrict__ worklist, int32_t* __restrict__ cursor) {
  __shared__ int cost[FVA_MAX_SCHED_HEADS];
  __shared__ int rank[FVA_MAX_SCHED_HEADS];
  const int tid = threadIdx.x;
  for (int bh = tid; bh < n_bh; bh += 1024)
    cost[bh] = row_ptr[(int64_t)(bh + 1) * n_blk] - row_ptr[(int64_t)bh * n_blk];
  if (tid < 2 * kXcds) cursor[tid] = 0;
  __syncthreads();
  for (int bh = tid; bh < n_bh; bh += 1024) {
    int rk = 0;
    const int c = cost[bh];
    for (int o = 0; o < n_bh; ++o) rk += (cost[o] > c) || (cost[o] == c && o < bh);
    rank[bh] = rk;
  }
  __syncthreads();
  // work items are groups of G consecutive query blocks of one head
  const int ngh = (n_blk + G - 1) / G;
  const int64_t n_items = (int64_t)n_bh * ngh;
  for (int64_t r = tid; r < n_items; r += 1024) {
    const int bh = (int)(r / ngh);
    const int k = (int)(r - (int64_t)bh * ngh);
    worklist[(int64_t)rank[bh] * ngh + k] = (int32_t)r;
  }
}

// Optional second pass over the work list: inside each head's segment,
// groups ordered by decreasing cost (sum of their rows' lengths; ties by
// id), so the persistent grid's last items are the short ones.  One
// workgroup per segment.
__global__ __launch_bounds__(1024) void k_sched_lpt(const int32_t* __restrict__ row_ptr, int n_blk, int G,
                                                    const int2* __restrict__ pairs, int32_t* __restrict__ worklist) {
  __shared__ int item[4096];
  __shared__ int cost[4096];
  const int ngh = (n_blk + G - 1) / G;
  int32_t* seg = worklist + (int64_t)blockIdx.x * ngh;
  for (int k = threadIdx.x; k < ngh; k += 1024) {
    const int r = seg[k];
    const int bh = r / ngh, g = r - bh * ngh;
    const int64_t hb = (int64_t)bh * n_blk;
    int c;
    if (pairs) {
      const int2 pr = pairs[r];
      c = row_ptr[hb + pr.x + 1] - row_ptr[hb + pr.x];
      if (pr.y >= 0) c += row_ptr[hb + pr.y + 1] - row_ptr[hb + pr.y];
    } else {
      const int64_t r0 = hb + (int64_t)g * G;
      const int r1 = min((g + 1) * G, n_blk) - g * G;
      c = row_ptr[r0 + r1] - row_ptr[r0];
    }
    item[k] = r;
    cost[k] = c;
  }
  __syncthreads();
  int pos[4];
  for (int k = threadIdx.x, i = 0; k < ngh; k += 1024, ++i) {
    int rk = 0;
    const int c = cost[k];
    for (int o = 0; o < ngh; ++o) rk += (cost[o] > c) || (cost[o] == c && o < k);
    pos[i] = rk;
  }
  __syncthreads();
  for (int k = threadIdx.x, i = 0; k < ngh; k += 1024, ++i) seg[pos[i]] = item[k];
}

// Query-block pairs for groups of two (one workgroup per head).  Candidate
// partners are spatial neighbours: in tile order the adjacent blocks along
// w, h and t; in Hilbert order the three blocks before and after along the
// curve.  Matching is by handshakes: in each round every unmatched block
// proposes its unmatched neighbour of largest list overlap (the keys a
// group's shared stages serve twice; ties to the lower id), and mutual
// proposals pair up.  Blocks left after the rounds are paired in id order.
// Pairs are listed by their lower id, so every head gets exactly
// ceil(n_blk / 2) groups in a deterministic order.
__device__ __forceinline__ int pair_nb(int I, int c, int n_blk, int nbw, int nbh, int hilbert) {
  // c in [0, 6): three forward then three backward neighbours, or -1
  const int dir = c < 3 ? 1 : -1, k = c % 3;
  if (hilbert) {
    const int J = I + dir * (k + 1);
    return J >= 0 && J < n_blk ? J : -1;
  }
  const int bw = I % nbw, bhh = (I / nbw) % nbh;
  if (k == 0) return (dir > 0 ? bw + 1 < nbw : bw > 0) ? I + dir : -1;
  if (k == 1) return (dir > 0 ? bhh + 1 < nbh : bhh > 0) ? I + dir * nbw : -1;
  const int J = I + dir * nbw * nbh;
  return J >= 0 && J < n_blk ? J : -1;
}

// exclusive prefix sum over x[0, n) in LDS (n <= 4096, 1024 threads);
// returns the total
__device__ int block_scan(int* x, int n, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  __syncthreads();
  int carry = 0;
  for (int base = 0; base < n; base += 1024) {
    const int i = base + tid;
    const int v = i < n ? x[i] : 0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int k = 0; k < 16; ++k) {
      before += k < wv ? wsum[k] : 0;
      total += wsum[k];
    }
    if (i < n) x[i] = carry + before + incl - v;
    carry += total;
    __syncthreads();
  }
  return carry;
}

__global__ __launch_bounds__(1024) void k_pair(const uint64_t* __restrict__ bits, int n_blk, int nw, int nbw,
                                               int nbh, int hilbert, int2* __restrict__ pairs) {
  __shared__ uint16_t ov[3 * 4096];   // overlap of forward edge 3I + k (I with its k-th forward neighbour)
  __shared__ int16_t prop[4096];      // proposal of each block this round, -1 none
  __shared__ int16_t mate[4096];      // matched partner, -1 unmatched
  __shared__ int pos[4096];
  __shared__ int wsum[16];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const uint64_t* hb = bits + (int64_t)bh * n_blk * nw;
  for (int e = tid; e < 3 * n_blk; e += 1024) {
    const int I = e / 3, J = pair_nb(I, e % 3, n_blk, nbw, nbh, hilbert);
    int o = 0;
    if (J >= 0)
      for (int w = 0; w < nw; ++w) o += __popcll(hb[(int64_t)I * nw + w] & hb[(int64_t)J * nw + w]);
    ov[e] = (uint16_t)o;
  }
  for (int I = tid; I < n_blk; I += 1024) mate[I] = -1;
  __syncthreads();
  // overlap of the edge between I and its c-th neighbour J (both directions)
  auto edge_ov = [&](int I, int c, int J) -> int { return c < 3 ? ov[3 * I + c] : ov[3 * J + (c - 3)]; };
  for (int round = 0; round < 8; ++round) {
    for (int I = tid; I < n_blk; I += 1024) {
      int best = -1, bo = -1;
      if (mate[I] < 0) {
        for (int c = 0; c < 6; ++c) {
          const int J = pair_nb(I, c, n_blk, nbw, nbh, hilbert);
          if (J < 0 || mate[J] >= 0) continue;
          const int o = edge_ov(I, c, J);
          if (o > bo || (o == bo && J < best)) { bo = o; best = J; }
        }
      }
      prop[I] = (int16_t)best;
    }
    __syncthreads();
    for (int I = tid; I < n_blk; I += 1024) {
      const int J = prop[I];
      if (J >= 0 && prop[J] == I) mate[I] = (int16_t)J;
    }
    __syncthreads();
  }
  // leftovers in id order: rank among unmatched blocks, then pair 2r with 2r+1
  for (int I = tid; I < n_blk; I += 1024) pos[I] = mate[I] < 0 ? 1 : 0;
  const int n_left = block_scan(pos, n_blk, wsum);
  // pos[I] = rank of unmatched I; find the unmatched block of each rank
  __shared__ int16_t left[4096];
  for (int I = tid; I < n_blk; I += 1024)
    if (mate[I] < 0) left[pos[I]] = (int16_t)I;
  __syncthreads();
  for (int r = tid; r + 1 < n_left; r += 1024)
    if ((r & 1) == 0) { mate[left[r]] = left[r + 1]; mate[left[r + 1]] = left[r]; }
  __syncthreads();
  // one entry per pair (or singleton), listed by its lower id
  for (int I = tid; I < n_blk; I += 1024) pos[I] = (mate[I] < 0 || mate[I] > I) ? 1 : 0;
  block_scan(pos, n_blk, wsum);
  int2* out = pairs + (int64_t)bh * ((n_blk + 1) / 2);
  for (int I = tid; I < n_blk; I += 1024)
    if (mate[I] < 0 || mate[I] > I) out[pos[I]] = make_int2(I, mate[I]);
}

// Groups of two: pair query blocks by list overlap (1, default) or take
// consecutive ids (0).  Pairing was 4.1% faster at the 720P Hilbert shape
// and 0.8% at the Wan-14B 480P tile-order one (measured, bitwise-equal
// outputs).  FVA_ATTN_PAIR overrides it.
int attn_pair() {
  const char* v = getenv("FVA_ATTN_PAIR");
  return v && atoi(v) == 0 ? 0 : 1;
}

// Work-list order inside a head: 1 = decreasing cost (default; 2% faster
// at the Wan-14B 480P shape, measured), 0 = group id.  FVA_ATTN_ORDER
// overrides it.
int attn_order() {
  const char* v = getenv("FVA_ATTN_ORDER");
  return v && atoi(v) == 0 ? 0 : 1;
}

// Groups per XCD chunk of the work list.  Persistent grid: one head's
// groups, so each XCD works through whole heads and a head's K/V is fetched
// into one L2, not eight (3.6% faster at the Wan-14B 480P shape and 10% at
// the Wan-1.3B one than chunks of 32, measured; the per-XCD cursors and
// stealing absorb heads of unequal cost).  When the head count is not a
// multiple of 8, heads are cut into 8 / gcd(heads, 8) equal chunks so every
// XCD gets the same number of them (12 heads: half-heads, 3 per XCD, 2.5%
// faster).  Plain grid: 32, since in-order dispatch would stall every XCD
// behind the one holding the heaviest head.  FVA_ATTN_CHUNK overrides it.
constexpr int kMaxChunk = 4096;
int attn_chunk(int groups_per_head, int n_heads, bool persistent) {
  int g = n_heads, b = kXcds;
  while (b) { const int t = g % b; g = b; b = t; }   // gcd(n_heads, 8)
  const int parts = kXcds / g;
  const int dflt = persistent ? (groups_per_head + parts - 1) / parts : 32;
  const char* v = getenv("FVA_ATTN_CHUNK");
  int n = v ? atoi(v) : dflt;
  // the plan sizes wg_times (max_wg) for plain grids rounded up to 8 chunks
  // of at most kMaxChunk groups
  if (n < 1 || n > kMaxChunk) n = dflt;
  return n;
}

// Query blocks per workgroup of the bf16 kernel (1, 2 or 4);
// FVA_ATTN_GROUP overrides it.
int attn_group() {
  const char* v = getenv("FVA_ATTN_GROUP");
  int n = v ? atoi(v) : 2;
  if (n != 1 && n != 2 && n != 4) n = 2;
  return n;
}

// LDS ring depth of the bf16 attention kernel (stages of 2*32*D*2 bytes).
// Two stages (loads one step ahead) measured 0.7% faster than four at the
// Wan-14B 480P shape, 1.4% at the 720P Hilbert one and 1.5% on the
// heterogeneous one (interleaved runs on one box; three stages were slower
// than either); FVA_ATTN_STAGES=2|3|4 overrides it for tuning.
int attn_stages() {
  const char* v = getenv("FVA_ATTN_STAGES");
  int n = v ? atoi(v) : 2;
  if (n < 2 || n > 4) n = 2;
  return n;
}

// FVA_ATTN_EXACT_SCALE=1: the inference form keeps S exact in fp32 and
// applies the scale with one fma per score instead of folding it into a bf16
// rounding of Q (for inputs whose logits span tens of log2 units, where that
// rounding moves outputs by more than the bf16 output error).  It runs the
// default launch shape: two query blocks per workgroup, a two-stage ring.
bool attn_exact_scale() {
  const char* v = getenv("FVA_ATTN_EXACT_SCALE");
  return v && atoi(v) == 1;
}

template <typename K>
int occupancy(K kernel, int threads) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, threads, 0) != hipSuccess || nb < 1) nb = 1;
  return nb;
}

}  // namespace

void fva_pair_blocks(fva_plan_t plan, const uint64_t* bits, int2* pairs, hipStream_t stream) {
  const fva_plan_desc& d = plan->desc;
  const fva_plan_info& in = plan->info;
  const int nbw = in.padded[2] / d.tile[2], nbh = in.padded[1] / d.tile[1];
  hipLaunchKernelGGL(k_pair, dim3(d.batch * d.heads), dim3(1024), 0, stream, bits, (int)in.n_blk, plan->nw, nbw, nbh,
                     d.order == FVA_ORDER_HILBERT ? 1 : 0, pairs);
}

static int attention_launch(fva_plan_t plan, const void* q_perm, const void* k_perm, const void* vt_perm,
                            const int32_t* row_ptr, const int32_t* col_idx, void* o_perm, int32_t sched_mode,
                            uint64_t* wg_times, float* lse, float* o32, bool raster, hipStream_t stream) {
  if (!plan) return fva_fail(FVA_EINVAL, "plan is NULL");
  if (!q_perm || !k_perm || !vt_perm || !o_perm) return fva_fail(FVA_EINVAL, "tensor pointer is NULL");
  if (!row_ptr || !col_idx) return fva_fail(FVA_EINVAL, "row_ptr / col_idx is NULL");
  if (sched_mode != FVA_SCHED_PERSISTENT && sched_mode != FVA_SCHED_PLAIN)
    return fva_fail(FVA_EINVAL, "unknown sched_mode %d", sched_mode);
  const fva_plan_desc& d = plan->desc;
  const fva_plan_info& in = plan->info;
  const int n_bh = d.batch * d.heads;
  const bool exact = d.dtype == FVA_DTYPE_BF16 && !lse && attn_exact_scale();
  // the training form and the exact-scale inference form are G = 2 only
  int G = d.dtype == FVA_DTYPE_BF16 ? (lse || exact ? 2 : attn_group()) : 1;
  if (d.head_dim == 64 && G > 2) G = 2;   // a 4 KB half splits over at most 4 waves
  const bool paired = G == 2 && attn_pair() == 1;
  const int64_t n_items = (int64_t)n_bh * ((in.n_blk + G - 1) / G);
  const int chunk = attn_chunk((in.n_blk + G - 1) / G, n_bh, sched_mode == FVA_SCHED_PERSISTENT);
  {  // a plain grid rounds up to 8 chunks; wg_times holds 2*max_wg stamps
    const int64_t deal = (int64_t)kXcds * chunk;
    if (sched_mode == FVA_SCHED_PLAIN && (n_items + deal - 1) / deal * deal > in.max_wg)
      return fva_fail(FVA_EINVAL, "plain grid exceeds max_wg %d", in.max_wg);
  }
  if (paired) {
    fva_csr_bits(plan, row_ptr, col_idx, plan->rowmask, stream);
    fva_pair_blocks(plan, plan->rowmask, plan->pairs, stream);
  }
  hipLaunchKernelGGL(k_sched, dim3(1), dim3(1024), 0, stream, row_ptr, in.n_blk, n_bh, G, plan->worklist,
                     plan->counters);
  if (attn_order() == 1)
    hipLaunchKernelGGL(k_sched_lpt, dim3(n_bh), dim3(1024), 0, stream, row_ptr, (int)in.n_blk, G,
                       paired ? (const int2*)plan->pairs : nullptr, plan->worklist);
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
  a.blk_full = plan->blk_full;
  a.o = o_perm;
  a.worklist = plan->worklist;
  a.pairs = paired ? plan->pairs : nullptr;
  a.cursor = plan->counters;
  a.wg_times = wg_times;
  a.lse = lse;
  a.o32 = o32;
  a.perm = raster ? plan->perm : nullptr;
  a.n_tok = in.n_tokens;
  a.heads = d.heads;
  a.n_pad = in.n_pad;
  a.n_items = (int)n_items;
  a.n_blk = in.n_blk;
  a.persistent = sched_mode == FVA_SCHED_PERSISTENT;
  a.chunk = chunk;
  a.scale = 1.0f / sqrtf((float)d.head_dim);

#define FVA_LAUNCH(KERNEL, THREADS)                                                              \
  do {                                                                                           \
    const int deal = kXcds * a.chunk;                                                            \
    int grid = (int)((a.n_items + deal - 1) / deal * deal);                                      \
    if (a.persistent)                                                                            \
      grid = (int)std::min<int64_t>(std::min<int64_t>(a.n_items, in.max_wg),                     \
                                    (int64_t)plan->num_cu * occupancy(KERNEL, THREADS));         \
    hipLaunchKernelGGL(KERNEL, dim3(grid), dim3(THREADS), 0, stream, a);                        \
  } while (0)
  if (d.dtype == FVA_DTYPE_BF16) {
    const int ns = attn_stages();
#define FVA_BF16_128(NS)                                                      \
    if (G == 1) FVA_LAUNCH((k_attn_bf16<128, NS, 1, false>), 128);            \
    else if (G == 2) FVA_LAUNCH((k_attn_bf16<128, NS, 2, false>), 256);       \
    else FVA_LAUNCH((k_attn_bf16<128, NS, 4, false>), 512);
#define FVA_BF16_64(NS)                                                       \
    if (G == 1) FVA_LAUNCH((k_attn_bf16<64, NS, 1, false>), 128);             \
    else FVA_LAUNCH((k_attn_bf16<64, NS, 2, false>), 256);
    if (lse) {   // training forward: the default shape only
      if (d.head_dim == 128) FVA_LAUNCH((k_attn_bf16<128, 2, 2, true>), 256);
      else FVA_LAUNCH((k_attn_bf16<64, 2, 2, true>), 256);
    } else if (exact) {
      if (d.head_dim == 128) FVA_LAUNCH((k_attn_bf16<128, 2, 2, false, false>), 256);
      else FVA_LAUNCH((k_attn_bf16<64, 2, 2, false, false>), 256);
    } else if (d.head_dim == 128) {
      if (ns == 2) { FVA_BF16_128(2) }
      else if (ns == 3) { FVA_BF16_128(3) }
      else { FVA_BF16_128(4) }
    } else {
      if (ns == 2) { FVA_BF16_64(2) }
      else if (ns == 3) { FVA_BF16_64(3) }
      else { FVA_BF16_64(4) }
    }
#undef FVA_BF16_128
#undef FVA_BF16_64
  } else {
    if (d.head_dim == 128) FVA_LAUNCH(k_attn_f32<128>, 256);
    else FVA_LAUNCH(k_attn_f32<64>, 256);
  }
#undef FVA_LAUNCH
  return fva_after_launch(stream, "fva_attention");

}

extern "C" int fva_attention(fva_plan_t plan, const void* q_perm, const void* k_perm, const void* vt_perm,
                             const int32_t* row_ptr, const int32_t* col_idx, void* o_perm, int32_t sched_mode,
                             uint64_t* wg_times, hipStream_t stream) {
  return attention_launch(plan, q_perm, k_perm, vt_perm, row_ptr, col_idx, o_perm, sched_mode, wg_times, nullptr,
                          nullptr, false, stream);
}

extern "C" int fva_attention_raster(fva_plan_t plan, const void* q_perm, const void* k_perm, const void* vt_perm,
                                    const int32_t* row_ptr, const int32_t* col_idx, void* o_raster,
                                    int32_t sched_mode, hipStream_t stream) {
  return attention_launch(plan, q_perm, k_perm, vt_perm, row_ptr, col_idx, o_raster, sched_mode, nullptr, nullptr,
                          nullptr, true, stream);
}

extern "C" int fva_attention_lse(fva_plan_t plan, const void* q_perm, const void* k_perm, const void* vt_perm,
                                 const int32_t* row_ptr, const int32_t* col_idx, void* o_perm, float* o32,
                                 float* lse, hipStream_t stream) {
  if (!plan) return fva_fail(FVA_EINVAL, "plan is NULL");
  if (!lse || !o32) return fva_fail(FVA_EINVAL, "lse / o32 is NULL");
  if (plan->desc.dtype != FVA_DTYPE_BF16) return fva_fail(FVA_EUNSUPPORTED, "the training path is bf16 only");
  return attention_launch(plan, q_perm, k_perm, vt_perm, row_ptr, col_idx, o_perm, FVA_SCHED_PERSISTENT, nullptr,
                          lse, o32, false, stream);
}

// ------------------------------------------------------ no-allocation entry
// fva_attention_static: fva_attention for callers that cannot allocate device
// memory (code under graph capture, serving loops, harnesses that forbid
// hipMalloc).  It takes the plan descriptor instead of a plan and keeps
// everything a plan would own for the call in one file-scope device array:
// the block validity tables, built by a kernel from the descriptor (tile
// order), and the scheduler's row bitmaps, pair table, work list and
// cursors.  Each device holds its own copy until the process ends; calls on
// one device share it, so calls that overlap on a device race.
namespace {

constexpr size_t kStaticScratchBytes = size_t(16) << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices];   // device address of `scratch` per device
int g_static_cus[kMaxDevices];     // compute units per device

// Validity tables of a tile-order plan: blk_mask[j] bit i set when local
// position i of block j lies inside the token grid; blk_full bit j set when
// block j has all 64 positions valid (64 words, blocks up to 4096).
__global__ __launch_bounds__(256) void k_static_tables(int GT, int GH, int GW, int tt, int th, int tw, int nbh,
                                                       int nbw, int n_blk, uint64_t* __restrict__ blk_mask,
                                                       uint64_t* __restrict__ blk_full) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  uint64_t m = 0;
  if (j < n_blk) {
    const int bt = j / (nbh * nbw), bh = (j / nbw) % nbh, bw = j % nbw;
    for (int loc = 0; loc < FVA_BLK; ++loc) {
      const int t = bt * tt + loc / (th * tw), h = bh * th + (loc / tw) % th, w = bw * tw + loc % tw;
      if (t < GT && h < GH && w < GW) m |= uint64_t(1) << loc;
    }
    blk_mask[j] = m;
  }
  // one bit per block; lanes of a wave cover 64 consecutive blocks = one word
  const uint64_t full = __ballot(j < n_blk && m == ~uint64_t(0));
  if ((threadIdx.x & 63) == 0 && j / 64 < 64) blk_full[j / 64] = full;
}

}  // namespace

extern "C" int fva_attention_static(const fva_plan_desc* desc, const void* q_perm, const void* k_perm,
                                    const void* vt_perm, const int32_t* row_ptr, const int32_t* col_idx,
                                    void* o_perm, hipStream_t stream) {
  if (!desc) return fva_fail(FVA_EINVAL, "desc is NULL");
  if (!q_perm || !k_perm || !vt_perm || !o_perm) return fva_fail(FVA_EINVAL, "tensor pointer is NULL");
  if (!row_ptr || !col_idx) return fva_fail(FVA_EINVAL, "row_ptr / col_idx is NULL");
  fva_plan_info in;
  int rc = fva_plan_dims(desc, &in);
  if (rc) return rc;
  if (desc->order != FVA_ORDER_TILE)
    return fva_fail(FVA_EUNSUPPORTED, "fva_attention_static supports tile order only");
  // scratch carve-up, 256-byte aligned regions
  const int nw = (in.n_blk + 63) / 64;
  auto up = [](size_t b) { return (b + 255) & ~size_t(255); };
  const size_t o_mask = 0, o_full = o_mask + up(sizeof(uint64_t) * in.n_blk), o_cnt = o_full + up(sizeof(uint64_t) * 64),
               o_bits = o_cnt + up(sizeof(int32_t) * 64), o_work = o_bits + up(sizeof(uint64_t) * in.n_rows * nw),
               o_pairs = o_work + up(sizeof(int32_t) * in.n_rows), need = o_pairs + up(sizeof(int2) * in.n_rows);
  if (need > kStaticScratchBytes)
    return fva_fail(FVA_EUNSUPPORTED, "fva_attention_static: this shape needs %zu bytes of scratch, the maximum is %zu",
                    need, kStaticScratchBytes);
  int dev = 0;
  if ((rc = fva_hip_check(hipGetDevice(&dev), "hipGetDevice"))) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fva_fail(FVA_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  void* base = nullptr;
  int cus = 0;
  {
    // once per device, with that device current: the device address of its
    // copy of `scratch` (the array's name is only a host-side stand-in)
    std::lock_guard<std::mutex> lock(g_static_mu);
    if (!g_static_ptr[dev]) {
      void* ptr = nullptr;
      if ((rc = fva_hip_check(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress"))) return rc;
      int n = 0;
      if ((rc = fva_hip_check(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev),
                              "hipDeviceGetAttribute")))
        return rc;
      g_static_cus[dev] = n > 0 ? n : 1;
      g_static_ptr[dev] = ptr;
    }
    base = g_static_ptr[dev];
    cus = g_static_cus[dev];
  }
  char* s = (char*)base;
  fva_plan_s p{};
  p.desc = *desc;
  p.info = in;
  p.esize = desc->dtype == FVA_DTYPE_BF16 ? 2 : 4;
  p.nw = nw;
  p.device = dev;
  p.num_cu = cus;
  p.stream = stream;
  p.blk_mask = (uint64_t*)(s + o_mask);
  p.blk_full = (uint64_t*)(s + o_full);
  p.counters = (int32_t*)(s + o_cnt);
  p.rowmask = (uint64_t*)(s + o_bits);
  p.worklist = (int32_t*)(s + o_work);
  p.pairs = (int2*)(s + o_pairs);
  const int nbh = in.padded[1] / desc->tile[1], nbw = in.padded[2] / desc->tile[2];
  // at least 16 workgroups so every blk_full word (64 of them) is written
  const unsigned tgrid = (unsigned)std::max((in.n_blk + 255) / 256, 16);
  hipLaunchKernelGGL(k_static_tables, dim3(tgrid), dim3(256), 0, stream, desc->grid[0], desc->grid[1], desc->grid[2],
                     desc->tile[0], desc->tile[1], desc->tile[2], nbh, nbw, (int)in.n_blk, p.blk_mask, p.blk_full);
  return attention_launch(&p, q_perm, k_perm, vt_perm, row_ptr, col_idx, o_perm, FVA_SCHED_PERSISTENT, nullptr,
                          nullptr, nullptr, false, stream);
}
