/*
 * fva.h - training-free block-sparse spatiotemporal attention on AMD Instinct
 * MI355X (gfx950).  C ABI of libfva.so.
 *
 * The method (sources are the explainer/review pages, cited by title and
 * section):
 *   - "Video Sparse Attention" explainer, dialogue and section 3: tokens of
 *     the (t, h, w) latent grid are grouped into small (4,4,4) cubes; a light
 *     coarse stage pools each cube and predicts cube importance from the
 *     pooled tiles; a fine stage runs token-level attention only inside the
 *     chosen cubes, on a block layout that suits the hardware.
 *   - "FVAttn: Adaptive Sparse Attention with Runtime Load Balancing for Video
 *     Generation", sections 00-02: cubes are kept per query block by adaptive
 *     Top-p routing with a Top-k safety floor; per-head load is uneven and is
 *     balanced at run time; spare capacity buys extra high-value blocks.
 *   - "DFSAttn: Dynamic Fine-grained Sparse Attention for Efficient Video
 *     Generation", tricks 1-2: an optional 3D Hilbert-curve token order and
 *     block scores formed by summing finer sub-block scores.
 *
 * Call sequence for one attention call on one HIP stream:
 *   fva_permute(Q, rows) ; fva_permute(K, rows) ; fva_permute(V, vt)
 *   fva_select(...)      -> CSR block lists (row_ptr, col_idx)
 *   fva_attention(...)   -> O in block order
 *   fva_unpermute(O)     -> O in raster order
 * (fva_attention_raster does the last two steps in one pass;
 *  fva_permute_pool for Q and K with fva_select_pooled fold the pooling
 *  into the permutes.)
 *
 * Conventions shared by every call:
 *   - Raster tensors are [B, N, H, D] contiguous, token n = (t*GH + h)*GW + w
 *     (w fastest) on the unpadded grid (GT, GH, GW).
 *   - Block-order tensors are [B, H, N_pad, D] contiguous.  Position
 *     pos = blk*64 + local; pad positions hold zeros.
 *   - Element type is bfloat16 or float32 as fixed by the plan's dtype.
 *   - Every tensor pointer is a device pointer owned by the caller; it must
 *     stay valid until the stream has passed the call.
 *   - All calls are asynchronous on `stream` and never synchronise the host.
 *     Arguments are validated before anything is enqueued: on a non-zero
 *     status nothing was written.  A kernel fault surfaces at the caller's
 *     next synchronisation; with FVA_DEBUG=1 in the environment every call
 *     synchronises and checks after its launches (not while its stream is
 *     being captured into a graph).
 *   - Graph capture: the per-call entry points (everything except plan
 *     creation and destruction) only launch kernels on `stream`: no
 *     allocation, no memset or copy node, no host synchronisation, so a
 *     sequence of calls can be captured once and replayed.  Host-side
 *     arguments (p, k_min, modes) are fixed at capture; tensor contents
 *     are read at each replay.
 *   - A plan is not safe for concurrent calls on different streams: its
 *     workspace is shared.  No C++ exception crosses this interface.
 */
#ifndef FVA_H
#define FVA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  FVA_OK = 0,
  FVA_EINVAL = 1,        /* bad argument (null pointer, out-of-range value)  */
  FVA_EUNSUPPORTED = 2,  /* valid but not built: tile volume != 64, head_dim
                            not 64/128, unknown dtype, too many blocks ...   */
  FVA_EHIP = 3,          /* a HIP runtime call failed                        */
  FVA_ENOMEM = 4         /* device or host allocation failed                 */
};

enum { FVA_ORDER_TILE = 0, FVA_ORDER_HILBERT = 1 };
enum { FVA_DTYPE_BF16 = 0, FVA_DTYPE_F32 = 1 };
/* Block-order layouts written by fva_permute. */
enum {
  FVA_LAYOUT_ROWS = 0,   /* [B, H, N_pad, D]: used for Q and K               */
  FVA_LAYOUT_VT = 1      /* per 64-token block, two 32-key halves, each a
                            [D][32] matrix whose 32 key slots are ordered for
                            the matrix-core operand (see fva_permute): used
                            for V                                            */
};
enum { FVA_SLACK_NONE = 0, FVA_SLACK_MEDIAN = 1 };
/* Which tensor fva_permute_pool pools. */
enum { FVA_POOL_Q = 0, FVA_POOL_K = 1 };
enum { FVA_SCHED_PERSISTENT = 0, FVA_SCHED_PLAIN = 1 };

typedef struct fva_plan_s* fva_plan_t;

/* Problem statement: token grid, tile, heads, head_dim ("Video Sparse
 * Attention" section 3 for the (4,4,4) cubes; "DFSAttn" tricks 1-2 for the
 * Hilbert order and sub-blocks). */
typedef struct {
  int32_t batch;       /* B >= 1                                             */
  int32_t heads;       /* H >= 1                                             */
  int32_t head_dim;    /* D in {64, 128}                                     */
  int32_t grid[3];     /* (GT, GH, GW) token grid, each >= 1                 */
  int32_t tile[3];     /* cube shape; product must be 64                     */
  int32_t order;       /* FVA_ORDER_TILE or FVA_ORDER_HILBERT (needs
                          tile (4,4,4))                                      */
  int32_t sub[3];      /* sub-block shape for key-side sub-block scoring:
                          {0,0,0} = off, else divides tile with volume 8     */
  int32_t dtype;       /* FVA_DTYPE_BF16 or FVA_DTYPE_F32                    */
} fva_plan_desc;

typedef struct {
  int64_t n_tokens;        /* GT*GH*GW                                       */
  int64_t n_pad;           /* padded tokens = n_blk * 64                     */
  int32_t n_blk;           /* blocks per head                                */
  int32_t n_sub;           /* sub-blocks per block (0 or 8)                  */
  int32_t padded[3];       /* grid rounded up to tile multiples              */
  int64_t n_rows;          /* B*H*n_blk: rows of the block lists             */
  int64_t max_nnz;         /* n_rows*n_blk: capacity col_idx must have       */
  int64_t workspace_bytes; /* device bytes the plan owns                     */
  int32_t max_wg;          /* entries/2 that fva_attention's wg_times needs  */
} fva_plan_info;

/* Validate a descriptor and report sizes.  Host only: touches no device.
 * Returns FVA_EINVAL / FVA_EUNSUPPORTED on a bad descriptor. */
int fva_plan_dims(const fva_plan_desc* desc, fva_plan_info* info);

/* Build the plan's host tables into caller-owned host arrays (any may be
 * NULL).  Host only; for inspection and tests.
 *   perm[n_pad]      raster token index of each block-order position, or -1
 *                    for a pad position ("Video Sparse Attention" section 3;
 *                    with FVA_ORDER_HILBERT, positions are ranked by the 3D
 *                    Hilbert index of their padded-grid coordinate on the
 *                    enclosing 2^m cube, "DFSAttn" trick 1)
 *   blk_cnt[n_blk]   valid tokens per block
 *   blk_mask[n_blk]  bit i set when local position i of the block is valid
 *   sub_id[n_pad]    sub-block index within the block (raster order of the
 *                    sub-cube inside the tile), or -1 when sub-blocks are off
 */
int fva_plan_tables(const fva_plan_desc* desc, int32_t* perm, int32_t* blk_cnt,
                    uint64_t* blk_mask, int32_t* sub_id);

/* Create a plan: validate, build the tables, allocate the device tables and
 * the workspace (pooled Q/K, block logits and scores, selection scratch,
 * work list), and enqueue the table upload on `stream`.  *out receives the
 * handle.  The plan owns its device memory until fva_plan_destroy. */
int fva_plan_create(fva_plan_t* out, const fva_plan_desc* desc, hipStream_t stream);

/* The same call under the short name of the five-call sequence
 * (fva_plan, fva_permute, fva_select, fva_attention, fva_unpermute):
 * identical arguments, behaviour and status codes. */
int fva_plan(fva_plan_t* out, const fva_plan_desc* desc, hipStream_t stream);

/* Sizes of an existing plan. */
int fva_plan_query(fva_plan_t plan, fva_plan_info* info);

/* Synchronise the plan's creation stream and free everything it owns.
 * NULL is accepted. */
void fva_plan_destroy(fva_plan_t plan);

/* Gather a raster tensor [B, N, H, D] into block order ("Video Sparse
 * Attention" section 3: the tokens of a cube become contiguous so that the
 * fine stage works block by block).  Pad positions are written as zero.
 *   layout = FVA_LAYOUT_ROWS : x_perm is [B, H, N_pad, D].
 *   layout = FVA_LAYOUT_VT   : for block (b, h, j) at element offset
 *        ((b*H + h)*n_blk + j)*64*D, half u = key/32 occupies D*32 elements
 *        starting at u*D*32; inside it element [d*32 + s] holds x[key][d]
 *        with, for k = key%32, c = k/16, r = k%16:
 *        s = 16*c + 8*((r/4)%2) + (r%4) + 4*(r/8).
 * x_raster and x_perm must not overlap. */
int fva_permute(fva_plan_t plan, const void* x_raster, void* x_perm, int32_t layout,
                hipStream_t stream);

/* fva_permute (FVA_LAYOUT_ROWS) of Q or K that also computes the pooled means
 * the coarse stage scores ("Video Sparse Attention" section 3: the mean of
 * each (4,4,4) cube; "DFSAttn" trick 2: for K on a plan with sub-blocks, the
 * mean of each non-empty (2,2,2) sub-block instead), while the rows are at
 * hand, so fva_select_pooled need not read the block-order tensor again.
 *   which    FVA_POOL_Q or FVA_POOL_K.
 * x_perm receives exactly what fva_permute writes.  The means go to the
 * plan's workspace (fp64), where fva_select_pooled reads them; they are the
 * same bits fva_select's own pooling produces.  A later fva_select that pools
 * its own inputs overwrites them (fva_select_pooled then refuses until both
 * Q and K are pooled again). */
int fva_permute_pool(fva_plan_t plan, const void* x_raster, void* x_perm, int32_t which,
                     hipStream_t stream);

/* fva_permute (FVA_LAYOUT_ROWS) fused with a 3D rotary position encoding
 * that uses a global time index ("Accelerating Video Generation Inference
 * with Sequential-Parallel 3D Positional Encoding Using a Global Time Index",
 * section 2.2: a chunk of frames is encoded with t_global = t_local +
 * t_offset, so it needs no other chunk; section 2.3: the frequencies are
 * precomputed as one contiguous table).  For the raster token at grid
 * position (t, h, w) the D/2 dimension pairs (2p, 2p+1) are split over the
 * axes as evenly as possible, the remainder to t then h (D = 128: 22, 21,
 * 21 pairs; D = 64: 11, 11, 10); pair i of
 * an axis with P pairs turns by pos * base^(-i/P), pos being t + t_offset,
 * h or w.  The angles' cosines and sines are tabulated in fp64 on the device
 * for this call; the rotation runs in fp64 and is rounded once to the plan
 * dtype.  Use it for Q and K (V takes plain fva_permute).
 *   t_offset >= 0; base > 1.  Errors: FVA_EINVAL for bad arguments.
 * x_raster and x_perm must not overlap. */
int fva_permute_rope(fva_plan_t plan, const void* x_raster, void* x_perm, int32_t t_offset, double base,
                     hipStream_t stream);

/* Coarse stage and routing ("Video Sparse Attention" dialogue and section 3;
 * "FVAttn" sections 00 and 02; "DFSAttn" trick 2):
 *   pool   q_bar_I = mean of the valid rows of Q block I (k_bar likewise; with
 *          sub-blocks on, one k_bar per non-empty (J, s) pair), fp64;
 *   score  S_I. = softmax_J(q_bar_I . k_bar_J / sqrt(D)) computed in fp64
 *          and rounded once to fp32; with sub-blocks, the softmax runs over
 *          all non-empty (J, s) and S_IJ is the sum over s (computed as a
 *          log-sum-exp block logit);
 *   select per row, order J by (S desc, J asc) and keep the shortest prefix
 *          whose mass reaches p, then at least min(k_min, n_blk) blocks;
 *          p >= 1 keeps all blocks.  The mass is the exact integer sum of
 *          floor(clamp(S, 0, 1) * 2^47) against ceil(p * 2^47); NaN scores
 *          count as 0.  Kept ids are emitted ascending;
 *   slack  FVA_SLACK_MEDIAN: every (b, h) whose block count is below the
 *          lower median over the call's B*H heads gets the unselected (I, J)
 *          pairs of highest score (ties: lower I, then lower J) until its
 *          count equals that median ("FVAttn" section 02, one-GPU reading).
 * Arguments:
 *   q_perm, k_perm  block-order Q and K (FVA_LAYOUT_ROWS); ignored when
 *                   scores_in is given.
 *   p, p_count      host array: p_count == 1 (one p for all heads) or
 *                   p_count == B*H (per (b, h), b major); 0 < p; B*H <= 512
 *                   when per-head.
 *   k_min           >= 0.
 *   scores_in       optional device [B, H, n_blk, n_blk] fp32: skip pool and
 *                   score and select on these values instead.
 *   scores_out      optional device [B, H, n_blk, n_blk] fp32: receives the
 *                   scores selection used.
 *   row_ptr         device int32 [n_rows + 1], rows r = (b*H + h)*n_blk + I.
 *   col_idx         device int32, capacity max_nnz; only row_ptr[n_rows]
 *                   entries are written.
 *   head_nnz        optional device int32 [B*H]: kept blocks per (b, h). */
int fva_select(fva_plan_t plan, const void* q_perm, const void* k_perm, const float* p,
               int32_t p_count, int32_t k_min, int32_t slack_mode, const float* scores_in,
               float* scores_out, int32_t* row_ptr, int32_t* col_idx, int32_t* head_nnz,
               hipStream_t stream);

/* fva_select on the pooled means of the latest fva_permute_pool calls for Q
 * and K on this plan (same stream, or ordered before this call): pool is
 * skipped, score and select run as in fva_select, with the same results.
 * Arguments as for fva_select without q_perm, k_perm and scores_in.
 * FVA_EINVAL when Q or K has not been pooled since the plan was created or
 * since the last fva_select that pooled its own inputs. */
int fva_select_pooled(fva_plan_t plan, const float* p, int32_t p_count, int32_t k_min,
                      int32_t slack_mode, float* scores_out, int32_t* row_ptr, int32_t* col_idx,
                      int32_t* head_nnz, hipStream_t stream);

/* Fine stage ("Video Sparse Attention" section 3; load balancing of uneven
 * per-head work from "FVAttn" section 02, here across the compute units of
 * one GPU).  For every valid query token i of block I:
 *   o_i = sum_j softmax_j(q_i . k_j / sqrt(D)) v_j
 * over the valid key tokens j of the blocks listed in row (b, h, I).  Pad
 * query rows of o_perm are written as zero; a row with no blocks gives zero.
 *   q_perm, k_perm  FVA_LAYOUT_ROWS;  vt_perm  FVA_LAYOUT_VT.
 *   row_ptr, col_idx  any valid CSR over the plan's rows, e.g. from
 *                   fva_select: each row lists a set of block ids, in any
 *                   order; an id listed twice counts once and ids outside
 *                   [0, n_blk) are ignored.
 *   o_perm          [B, H, N_pad, D], plan dtype.
 *   sched_mode      FVA_SCHED_PERSISTENT: a persistent grid pops rows from a
 *                   device work list sorted by decreasing cost;
 *                   FVA_SCHED_PLAIN: one workgroup per row in list order.
 *   wg_times        optional device uint64 [2*max_wg]: per workgroup the
 *                   start and end of its busy time (100 MHz wall clock).
 * bf16: QK^T and PV run on bf16 matrix cores with fp32 accumulation, the
 * softmax in fp32, P rounded to bf16 before PV, O rounded to bf16 at the end.
 * By default Q enters the products multiplied by the softmax scale in log2
 * units (1/sqrt(D) * log2 e) and rounded to bf16 once more, which moves a
 * logit by up to 2^-9 of sum_d |q_d k_d| * scale: well inside the bf16 output
 * error for logits spanning a few log2 units, growing beyond it for rows
 * whose logits span tens.  With the environment variable
 * FVA_ATTN_EXACT_SCALE=1 set at the call, S stays exact in fp32 and the
 * scale is applied per score (about 6% slower).
 * fp32: fp32 throughout. */
int fva_attention(fva_plan_t plan, const void* q_perm, const void* k_perm, const void* vt_perm,
                  const int32_t* row_ptr, const int32_t* col_idx, void* o_perm,
                  int32_t sched_mode, uint64_t* wg_times, hipStream_t stream);

/* fva_attention followed by fva_unpermute in one pass: each output row is
 * written straight to its raster position, so the block-order O is never
 * stored and read back ("Video Sparse Attention" section 3: the gather to
 * blocks is undone after the fine stage).
 *   o_raster   [B, N, H, D], plan dtype.  Only valid tokens' rows are
 *              written; rows of other tokens are left as they are.
 * The other arguments are those of fva_attention (no wg_times).  The result
 * equals fva_attention + fva_unpermute bit for bit. */
int fva_attention_raster(fva_plan_t plan, const void* q_perm, const void* k_perm, const void* vt_perm,
                         const int32_t* row_ptr, const int32_t* col_idx, void* o_raster,
                         int32_t sched_mode, hipStream_t stream);

/* Forward pass of a training step: fva_attention that also keeps what the
 * backward pass needs.
 *   lse   device fp32 [B, H, N_pad], overwritten: per query token the
 *         log2-sum-exp2 of its scaled scores over the listed keys,
 *           lse[(b*H + h)*N_pad + t] = log2 sum_j exp(q_t . k_j / sqrt(D)),
 *         for valid tokens with a non-empty row, 0 otherwise (the softmax
 *         normaliser P is recomputed from);
 *   o32   device fp32 [B, H, N_pad, D], overwritten: o_perm before its
 *         rounding to bf16 (delta = rowsum(dO * O) is taken from it: the
 *         bf16 rounding of O would enter every dQ row multiplied by the
 *         mean of its listed keys).
 * Persistent schedule; bf16 plans only (FVA_EUNSUPPORTED otherwise).
 * Errors: FVA_EINVAL for NULL pointers. */
int fva_attention_lse(fva_plan_t plan, const void* q_perm, const void* k_perm, const void* vt_perm,
                      const int32_t* row_ptr, const int32_t* col_idx, void* o_perm, float* o32, float* lse,
                      hipStream_t stream);

/* Gradients of fva_attention for training ("Video Sparse Attention"
 * explainer, section 3: the same block lists drive the forward and the
 * backward kernels).  With s_ij = q_i . k_j / sqrt(D) and P the softmax of
 * row i over the valid keys of its listed blocks:
 *   dP = dO V^T,  delta_i = sum_d dO_id O_id,  dS = P * (dP - delta)
 *   dQ = dS K / sqrt(D),  dK = dS^T Q / sqrt(D),  dV = P^T dO
 * Arguments (block order, bf16, B*H heads of N_pad tokens):
 *   q_perm, k_perm, v_perm, do_perm   FVA_LAYOUT_ROWS (fva_permute);
 *   do_vt                             dO in FVA_LAYOUT_VT (K^T and Q^T are
 *                                     read from the row layouts);
 *                                     the pad rows of all of these must be
 *                                     zero, as fva_permute writes them;
 *   o32, lse                          outputs of fva_attention_lse on the
 *                                     same Q, K, V and lists;
 *   row_ptr, col_idx                  the forward pass's CSR (set semantics);
 *   dq_perm, dk_perm, dv_perm         FVA_LAYOUT_ROWS, overwritten; pad
 *                                     tokens and tokens no list reaches get 0.
 * All products on bf16 matrix cores with fp32 accumulation; P and dS are
 * rounded to bf16 as operands, the gradients to bf16 at the end.  Uses the
 * plan's workspace (not safe to overlap with other calls on the plan).
 * Errors: FVA_EINVAL for NULL pointers, FVA_EUNSUPPORTED for fp32 plans. */
int fva_attention_backward(fva_plan_t plan, const void* q_perm, const void* k_perm, const void* v_perm,
                           const float* o32, const float* lse, const void* do_perm, const void* do_vt,
                           const int32_t* row_ptr, const int32_t* col_idx, void* dq_perm, void* dk_perm,
                           void* dv_perm, hipStream_t stream);

/* Transposed block lists: row (b, h, J) of the output lists, ascending, the
 * query blocks I whose row (b, h, I) of the input lists holds J (input rows
 * read as sets).  These are the lists the backward pass walks for dK, dV.
 *   t_row_ptr   device int32 [n_rows + 1];
 *   t_col_idx   device int32, capacity >= the input's distinct in-range ids.
 * Errors: FVA_EINVAL for NULL pointers. */
int fva_mask_transpose(fva_plan_t plan, const int32_t* row_ptr, const int32_t* col_idx,
                       int32_t* t_row_ptr, int32_t* t_col_idx, hipStream_t stream);

/* Top-p for denoising step `step` (0-based) of `n_steps` ("DFSAttn"
 * explainer, trick 3: little is skipped while the latent is still noise and
 * more as the video sharpens).  The page gives no curve; this is the straight
 * line from p_first at the first step to p_last at the last, so a caller that
 * starts near 1 (almost dense) ends at its target sparsity.  n_steps == 1
 * gives p_last.  Host function: no device work, no plan.
 *   p_out  host float, written on success.
 * Errors: FVA_EINVAL for a NULL p_out, n_steps < 1, step outside
 * [0, n_steps), or p_first / p_last outside (0, 1]. */
int fva_p_schedule(int step, int n_steps, float p_first, float p_last, float* p_out);

/* Agreement of two block selections, for reusing a cached selection across
 * denoising steps ("DFSAttn" explainer, trick 3: blocks that mattered at an
 * earlier step are remembered instead of re-evaluated; fva_attention accepts
 * any cached CSR).  For every (b, h): counts[2*bh] = |A & B| and
 * counts[2*bh + 1] = |A | B| over its (I, J) block pairs, with each row read
 * as a set (repeated ids count once, ids outside [0, n_blk) are ignored).
 *   row_ptr_*, col_idx_*  device CSR over the plan's rows.
 *   counts                device int64 [2*B*H], overwritten.
 * Errors: FVA_EINVAL for NULL pointers. */
int fva_mask_overlap(fva_plan_t plan, const int32_t* row_ptr_a, const int32_t* col_idx_a,
                     const int32_t* row_ptr_b, const int32_t* col_idx_b, int64_t* counts,
                     hipStream_t stream);

/* Static calibrated selections ("Calibrated Sparse Attention" page: an
 * offline pass keeps the block patterns that stay stable across calibration
 * inputs, per layer, head and diffusion step; inference then computes only
 * those).  fva_mask_accumulate adds one selection to per-pair counts:
 * counts[r*n_blk + J] += 1 for every id J of row r (a row is read as a set
 * of plan blocks).  fva_mask_from_counts emits the CSR of the pairs counted
 * at least min_count times (ids ascending), usable by fva_attention at every
 * later call: min_count = 1 gives the union of the calibration runs,
 * min_count = runs their intersection.
 *   counts    device int32 [n_rows * n_blk], zeroed by the caller before the
 *             first run, owned by the caller.
 *   row_ptr, col_idx, head_nnz  as for fva_select (head_nnz nullable).
 * Errors: FVA_EINVAL for NULL pointers or min_count < 1. */
int fva_mask_accumulate(fva_plan_t plan, const int32_t* row_ptr, const int32_t* col_idx, int32_t* counts,
                        hipStream_t stream);
int fva_mask_from_counts(fva_plan_t plan, const int32_t* counts, int32_t min_count, int32_t* row_ptr,
                         int32_t* col_idx, int32_t* head_nnz, hipStream_t stream);

/* fva_attention for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It needs no plan: it takes the plan descriptor, and everything a plan
 * would own for the call (the block validity tables, built on the device
 * from the descriptor, and the scheduler's row bitmaps, pair table, work
 * list and cursors) lives in one static device array of 16 MiB that the
 * library holds on each device it runs on until the process ends.  It calls
 * no hipMalloc / hipFree and allocates nothing else.
 *   desc      as for fva_plan_create; FVA_ORDER_TILE only
 *             (FVA_EUNSUPPORTED otherwise).
 *   other arguments as for fva_attention with FVA_SCHED_PERSISTENT and no
 *             wg_times; o_perm is written in block order [B, H, N_pad, D].
 * The result equals fva_attention's on a plan of the same descriptor, bit
 * for bit (the same kernels).
 * Limit: the scratch must hold 8*n_blk + 8*n_rows*ceil(n_blk/64) +
 * 12*n_rows bytes plus alignment (Wan 480P at B*H = 80: 4.6 MiB; 720P at
 * 40 heads: 11.3 MiB); a larger shape returns FVA_EUNSUPPORTED with a
 * message before anything is enqueued.
 * Concurrency: every call on a device shares that device's array; calls
 * that overlap on one device (on different streams) race.  Calls in one
 * stream are ordered and safe.  The first call on a device looks up the
 * array's device address once (a host-side query, no allocation). */
int fva_attention_static(const fva_plan_desc* desc, const void* q_perm, const void* k_perm, const void* vt_perm,
                         const int32_t* row_ptr, const int32_t* col_idx, void* o_perm, hipStream_t stream);

/* Scatter block-order [B, H, N_pad, D] (FVA_LAYOUT_ROWS) back to raster
 * [B, N, H, D], dropping pad positions ("Video Sparse Attention" section 3:
 * the cube-contiguous token order exists only for the fine stage, and the
 * caller's sequence order is restored after it; "DFSAttn" trick 1: the
 * Hilbert reordering is undone after attention).  Inverse of fva_permute:
 * x_raster[b, perm[pos], h, :] = x_perm[b, h, pos, :] for every valid pos;
 * raster rows are written once each, nothing else is touched.
 * x_perm and x_raster must not overlap.  Errors: FVA_EINVAL for NULL
 * pointers or an unknown plan dtype. */
int fva_unpermute(fva_plan_t plan, const void* x_perm, void* x_raster, hipStream_t stream);

/* Message for the last non-zero status returned on this thread. */
const char* fva_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FVA_H */
