// Internal declarations shared by the libfva translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "fva.h"

#define FVA_BLK 64        // tokens per block (tile volume)
#define FVA_MAX_PHEAD 512 // per-head p values passed by value to the kernels
#define FVA_MAX_NBLK 4096 // blocks per head the selection kernels support
#define FVA_MAX_SCHED_HEADS 4096  // B*H the attention scheduler supports
#define FVA_MAX_SCORE_SPLIT 8     // key ranges the score grid may be split into

struct fva_plan_s {
  fva_plan_desc desc;
  fva_plan_info info;
  int esize;          // bytes per element: 2 (bf16) or 4 (fp32)
  int nw;             // 64-bit mask words per selection row = ceil(n_blk / 64)
  int device;
  int num_cu;
  hipStream_t stream; // stream the tables were uploaded on

  // device tables (uploaded once at creation)
  int32_t* perm;      // [n_pad] raster token or -1
  uint64_t* blk_mask; // [n_blk] valid-position bitmask
  uint64_t* blk_full; // [64] bit J set when block J has all 64 positions valid
  int32_t* blk_cnt;   // [n_blk] valid tokens
  uint8_t* sub_pos;   // [n_blk][8][8] local positions of each sub-block
  int32_t* sub_cnt;   // [n_blk][8] valid tokens per sub-block

  // workspace
  double* qbar;       // [B*H*n_blk*D] pooled Q, fp64
  double* kbar;       // [B*H*n_blk*(n_sub or 1)*D] pooled K (per sub-block), fp64
  double* ybuf;       // [B*H*n_blk*n_blk] block logits, fp64
  float* sbuf;        // [B*H*n_blk*n_blk] fp32 scores the selection read
  double* rowmax;     // [FVA_MAX_SCORE_SPLIT][n_rows] row max of the block logits per key range, fp64
  int score_split;    // key ranges of the latest score launch (rows of rowmax in use)
  int32_t* rowcnt;    // [n_rows] kept blocks per row
  uint64_t* rowmask;  // [n_rows*nw] kept-block bitmask per row
  int32_t* headcnt;   // [B*H]
  int32_t* deficit;   // [B*H] slack blocks to add per head
  int32_t* headoff;   // [B*H] first CSR entry of each head
  uint64_t* slack_thr;// [B*H] slack key threshold (radix prefix while it is built)
  uint32_t* slack_hist;// [B*H][256] digit histogram of the slack radix select (kept zero between calls)
  int32_t* slack_need; // [B*H] pairs still to place below the current prefix
  double2* rope_tab;  // [(T+H+W) * D/2] rotary (cos, sin) of the last fva_permute_rope call
  float* bwd_delta;   // [B*H*n_pad] backward: rowsum(dO * O) per query token
  uint64_t* bits_t;   // [n_rows][nw] backward: transposed per-head block bitmap (key block -> query blocks)
  int32_t* worklist;  // [n_rows] attention rows in schedule order
  int32_t* worklist_t;// [n_rows] backward: key-block groups in schedule order
  int2* pairs;        // [n_rows] attention: the two query blocks of each group of a head (second -1 if none)
  int2* pairs_t;      // [n_rows] backward: the two key blocks of each group of a head
  int32_t* counters;  // [64] work-queue cursor and misc counters

  // host state: bit 0 / bit 1 set once fva_permute_pool has enqueued the
  // pooled means of Q / K into qbar / kbar (cleared when fva_select pools
  // its own inputs there)
  int pooled;

  void* dev_base;     // single device allocation holding everything above
  size_t dev_bytes;
};

// Thread-local error text; returns `code` for convenient `return fva_fail(...)`.
int fva_fail(int code, const char* fmt, ...);
// Checks a HIP status; on failure records it and returns FVA_EHIP.
int fva_hip_check(hipError_t e, const char* what);
// After the launches of one call: with FVA_DEBUG=1, synchronise and check.
int fva_after_launch(hipStream_t s, const char* what);
// FVA_DEBUG=1 in the environment (read once).
int fva_debug_enabled();

struct SelectArgs {
  float p[FVA_MAX_PHEAD];
};

// Per-row id masks -> CSR (ascending ids) using the plan's selection
// workspace (row counts, head totals and offsets).
int fva_bits_to_csr(fva_plan_t plan, const uint64_t* bits, int32_t* row_ptr, int32_t* col_idx, hipStream_t stream);

// CSR -> per-row 64-bit-word bitmaps (rows as sets, out-of-range ids dropped).
void fva_csr_bits(fva_plan_t plan, const int32_t* row_ptr, const int32_t* col_idx, uint64_t* bits,
                  hipStream_t stream);

// Pairs of neighbouring blocks with overlapping bitmap rows, per head
// (ceil(n_blk / 2) entries per head; second -1 for a single block).
void fva_pair_blocks(fva_plan_t plan, const uint64_t* bits, int2* pairs, hipStream_t stream);
