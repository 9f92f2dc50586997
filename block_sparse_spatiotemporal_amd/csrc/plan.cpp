// Plan: argument validation, host tables (tile or 3D Hilbert block order),
// device workspace, and the error plumbing of libfva.
//
// Block layout follows the "Video Sparse Attention" explainer, section 3
// (tokens grouped in (4,4,4) cubes, block-contiguous for the fine stage);
// the optional order is the 3D Hilbert curve of the "DFSAttn" explainer,
// trick 1, computed with J. Skilling's transpose construction ("Programming
// the Hilbert curve", AIP Conf. Proc. 707, 2004).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdlib>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "fva_internal.h"

static thread_local char g_err[512] = "";

int fva_fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int fva_hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return FVA_OK;
  return fva_fail(FVA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int fva_debug_enabled() {
  static int debug = -1;
  if (debug < 0) {
    const char* v = getenv("FVA_DEBUG");
    debug = (v && v[0] == '1') ? 1 : 0;
  }
  return debug;
}

int fva_after_launch(hipStream_t s, const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fva_fail(FVA_EHIP, "%s launch: %s", what, hipGetErrorString(e));
  if (fva_debug_enabled()) {
    // a stream being captured into a graph cannot be synchronised; its
    // launches are checked when the graph runs
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone) return FVA_OK;
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fva_fail(FVA_EHIP, "%s: %s", what, hipGetErrorString(e));
  }
  return FVA_OK;
}

extern "C" const char* fva_last_error(void) { return g_err; }

// ------------------------------------------------------------------ Hilbert
// Index of point (c[0], c[1], c[2]) on the 3D Hilbert curve of the 2^bits
// cube.  Level by level from the top bit: where the point's bit on an axis is
// set, the lower bits of axis 0 are complemented, otherwise the lower bits of
// axis 0 and that axis are exchanged (this removes the rotation the curve
// applies inside that sub-cube).  The three words are then Gray-encoded
// across axes, corrected by the parity pattern of the last axis, and their
// bits interleaved (axis 0 most significant within each level).
static uint64_t hilbert3(const uint32_t c[3], int bits) {
  uint32_t x[3] = {c[0], c[1], c[2]};
  for (uint32_t q = 1u << (bits - 1); q > 1; q >>= 1) {
    const uint32_t low = q - 1;
    for (int a = 0; a < 3; ++a) {
      if (x[a] & q) {
        x[0] ^= low;
      } else {
        const uint32_t t = (x[0] ^ x[a]) & low;
        x[0] ^= t;
        x[a] ^= t;
      }
    }
  }
  x[1] ^= x[0];
  x[2] ^= x[1];
  uint32_t fix = 0;
  for (uint32_t q = 1u << (bits - 1); q > 1; q >>= 1)
    if (x[2] & q) fix ^= q - 1;
  for (int a = 0; a < 3; ++a) x[a] ^= fix;
  uint64_t key = 0;
  for (int lev = bits - 1; lev >= 0; --lev)
    for (int a = 0; a < 3; ++a) key = (key << 1) | ((x[a] >> lev) & 1u);
  return key;
}

// ------------------------------------------------------------------ validation
static int validate(const fva_plan_desc* d, fva_plan_info* info) {
  if (!d) return fva_fail(FVA_EINVAL, "descriptor is NULL");
  if (d->batch < 1 || d->heads < 1) return fva_fail(FVA_EINVAL, "batch and heads must be >= 1");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fva_fail(FVA_EUNSUPPORTED, "head_dim %d unsupported (64 or 128)", d->head_dim);
  for (int a = 0; a < 3; ++a) {
    if (d->grid[a] < 1) return fva_fail(FVA_EINVAL, "grid[%d] = %d must be >= 1", a, d->grid[a]);
    if (d->tile[a] < 1) return fva_fail(FVA_EINVAL, "tile[%d] = %d must be >= 1", a, d->tile[a]);
  }
  if (d->tile[0] * d->tile[1] * d->tile[2] != FVA_BLK)
    return fva_fail(FVA_EUNSUPPORTED, "tile volume %d unsupported (must be 64)",
                    d->tile[0] * d->tile[1] * d->tile[2]);
  if (d->order != FVA_ORDER_TILE && d->order != FVA_ORDER_HILBERT)
    return fva_fail(FVA_EINVAL, "unknown order %d", d->order);
  if (d->order == FVA_ORDER_HILBERT && (d->tile[0] != 4 || d->tile[1] != 4 || d->tile[2] != 4))
    return fva_fail(FVA_EUNSUPPORTED, "Hilbert order needs tile (4,4,4)");
  const bool sub_on = d->sub[0] || d->sub[1] || d->sub[2];
  if (sub_on) {
    for (int a = 0; a < 3; ++a)
      if (d->sub[a] < 1 || d->tile[a] % d->sub[a])
        return fva_fail(FVA_EUNSUPPORTED, "sub[%d] = %d must divide tile", a, d->sub[a]);
    if (d->sub[0] * d->sub[1] * d->sub[2] != 8)
      return fva_fail(FVA_EUNSUPPORTED, "sub-block volume must be 8");
  }
  if (d->dtype != FVA_DTYPE_BF16 && d->dtype != FVA_DTYPE_F32)
    return fva_fail(FVA_EUNSUPPORTED, "unknown dtype %d", d->dtype);

  fva_plan_info in{};
  int64_t padded[3];
  for (int a = 0; a < 3; ++a) {
    padded[a] = (int64_t)(d->grid[a] + d->tile[a] - 1) / d->tile[a] * d->tile[a];
    in.padded[a] = (int32_t)padded[a];
  }
  in.n_tokens = (int64_t)d->grid[0] * d->grid[1] * d->grid[2];
  in.n_pad = padded[0] * padded[1] * padded[2];
  const int64_t n_blk = in.n_pad / FVA_BLK;
  if (n_blk > FVA_MAX_NBLK)
    return fva_fail(FVA_EUNSUPPORTED, "%lld blocks per head exceed %d", (long long)n_blk, FVA_MAX_NBLK);
  in.n_blk = (int32_t)n_blk;
  in.n_sub = sub_on ? 8 : 0;
  in.n_rows = (int64_t)d->batch * d->heads * n_blk;
  in.max_nnz = in.n_rows * n_blk;
  if (in.max_nnz >= (int64_t(1) << 31))
    return fva_fail(FVA_EUNSUPPORTED, "B*H*n_blk^2 = %lld exceeds int32 block lists", (long long)in.max_nnz);
  if ((int64_t)d->batch * d->heads * in.n_pad * d->head_dim >= (int64_t(1) << 40))
    return fva_fail(FVA_EUNSUPPORTED, "tensor too large");
  if ((int64_t)d->batch * d->heads > FVA_MAX_SCHED_HEADS)
    return fva_fail(FVA_EUNSUPPORTED, "B*H = %lld exceeds %d", (long long)d->batch * d->heads, FVA_MAX_SCHED_HEADS);
  // plain launches round the grid up to a multiple of 8 XCDs x 4096-row chunks at most
  in.max_wg = (int32_t)(std::max<int64_t>(in.n_rows, 4096) + 8 * 4096);
  if (info) *info = in;
  return FVA_OK;
}

// Workspace carve-up: every region 256-byte aligned inside one allocation.
struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  }
};

static void layout_workspace(const fva_plan_desc* d, const fva_plan_info& in, size_t* offs, size_t* total) {
  Carve c;
  const int64_t bh = (int64_t)d->batch * d->heads;
  const int nw = (in.n_blk + 63) / 64;
  offs[0] = c.take(sizeof(int32_t) * in.n_pad);                           // perm
  offs[1] = c.take(sizeof(uint64_t) * in.n_blk);                          // blk_mask
  offs[2] = c.take(sizeof(int32_t) * in.n_blk);                           // blk_cnt
  offs[3] = c.take(in.n_sub ? 64 * (size_t)in.n_blk : 0);                 // sub_pos
  offs[4] = c.take(in.n_sub ? sizeof(int32_t) * 8 * in.n_blk : 0);        // sub_cnt
  offs[5] = c.take(sizeof(double) * bh * in.n_blk * d->head_dim);        // qbar
  // kbar, plus 16 slack rows the score kernel's last key tile may read
  offs[6] = c.take(sizeof(double) * (bh * in.n_blk * (in.n_sub ? 8 : 1) + 16) * d->head_dim);
  offs[7] = c.take(sizeof(double) * bh * in.n_blk * in.n_blk);           // ybuf
  offs[8] = c.take(sizeof(double) * FVA_MAX_SCORE_SPLIT * in.n_rows);     // rowmax
  offs[9] = c.take(sizeof(int32_t) * in.n_rows);                         // rowcnt
  offs[10] = c.take(sizeof(uint64_t) * in.n_rows * nw);                  // rowmask
  offs[11] = c.take(sizeof(int32_t) * bh);                               // headcnt
  offs[12] = c.take(sizeof(int32_t) * bh);                               // deficit
  offs[13] = c.take(sizeof(uint64_t) * bh);                              // slack_thr
  offs[14] = c.take(sizeof(int32_t) * in.n_rows);                        // worklist
  offs[15] = c.take(sizeof(int32_t) * 64);                               // counters
  offs[16] = c.take(sizeof(float) * bh * in.n_blk * in.n_blk);           // sbuf
  offs[17] = c.take(sizeof(uint64_t) * 64);                              // blk_full
  offs[18] = c.take(sizeof(int32_t) * bh);                               // headoff
  offs[19] = c.take(sizeof(uint32_t) * 256 * bh);                        // slack_hist
  offs[20] = c.take(sizeof(int32_t) * bh);                               // slack_need
  offs[21] = c.take(sizeof(double2) * (d->grid[0] + d->grid[1] + d->grid[2]) * (d->head_dim / 2));  // rope_tab
  offs[22] = c.take(sizeof(float) * bh * in.n_pad);                      // bwd_delta
  offs[23] = c.take(sizeof(uint64_t) * in.n_rows * nw);                 // bits_t
  offs[24] = c.take(sizeof(int32_t) * in.n_rows);                        // worklist_t
  offs[25] = c.take(sizeof(int2) * in.n_rows);                           // pairs
  offs[26] = c.take(sizeof(int2) * in.n_rows);                           // pairs_t
  *total = c.off;
}

// ------------------------------------------------------------------ tables
struct HostTables {
  std::vector<int32_t> perm, cnt, sub_id, sub_cnt;
  std::vector<uint64_t> mask;
  std::vector<uint8_t> sub_pos;
};

static void build_tables(const fva_plan_desc* d, const fva_plan_info& in, HostTables& t) {
  const int GT = d->grid[0], GH = d->grid[1], GW = d->grid[2];
  const int PT = in.padded[0], PH = in.padded[1], PW = in.padded[2];
  const int tt = d->tile[0], th = d->tile[1], tw = d->tile[2];
  const int64_t n_pad = in.n_pad;
  // coordinate of every block-order position
  std::vector<int32_t> ct(n_pad), ch(n_pad), cw(n_pad);
  if (d->order == FVA_ORDER_TILE) {
    const int nh = PH / th, nw = PW / tw;
    for (int t = 0; t < PT; ++t)
      for (int h = 0; h < PH; ++h)
        for (int w = 0; w < PW; ++w) {
          const int64_t blk = ((int64_t)(t / tt) * nh + h / th) * nw + w / tw;
          const int loc = ((t % tt) * th + h % th) * tw + w % tw;
          const int64_t pos = blk * FVA_BLK + loc;
          ct[pos] = t, ch[pos] = h, cw[pos] = w;
        }
  } else {
    int bits = 1;
    while ((1 << bits) < std::max(PT, std::max(PH, PW))) ++bits;
    std::vector<std::pair<uint64_t, int64_t>> keyed;
    keyed.reserve(n_pad);
    for (int t = 0; t < PT; ++t)
      for (int h = 0; h < PH; ++h)
        for (int w = 0; w < PW; ++w) {
          const uint32_t c[3] = {(uint32_t)t, (uint32_t)h, (uint32_t)w};
          keyed.emplace_back(hilbert3(c, bits), ((int64_t)t * PH + h) * PW + w);
        }
    std::sort(keyed.begin(), keyed.end());
    for (int64_t pos = 0; pos < n_pad; ++pos) {
      const int64_t g = keyed[pos].second;
      ct[pos] = (int32_t)(g / ((int64_t)PH * PW));
      ch[pos] = (int32_t)((g / PW) % PH);
      cw[pos] = (int32_t)(g % PW);
    }
  }
  t.perm.assign(n_pad, -1);
  t.cnt.assign(in.n_blk, 0);
  t.mask.assign(in.n_blk, 0);
  for (int64_t pos = 0; pos < n_pad; ++pos) {
    if (ct[pos] < GT && ch[pos] < GH && cw[pos] < GW) {
      t.perm[pos] = (int32_t)(((int64_t)ct[pos] * GH + ch[pos]) * GW + cw[pos]);
      t.cnt[pos / FVA_BLK] += 1;
      t.mask[pos / FVA_BLK] |= uint64_t(1) << (pos % FVA_BLK);
    }
  }
  t.sub_id.assign(n_pad, -1);
  if (in.n_sub) {
    const int st = d->sub[0], sh = d->sub[1], sw = d->sub[2];
    const int ns_h = th / sh, ns_w = tw / sw;
    t.sub_pos.assign((size_t)in.n_blk * 64, 0);
    t.sub_cnt.assign((size_t)in.n_blk * 8, 0);
    std::vector<int> fill((size_t)in.n_blk * 8, 0);
    for (int64_t pos = 0; pos < n_pad; ++pos) {
      const int s = (((ct[pos] % tt) / st) * ns_h + (ch[pos] % th) / sh) * ns_w + (cw[pos] % tw) / sw;
      const int64_t blk = pos / FVA_BLK;
      t.sub_id[pos] = s;
      const int k = fill[blk * 8 + s]++;
      t.sub_pos[(blk * 8 + s) * 8 + k] = (uint8_t)(pos % FVA_BLK);
      if (t.perm[pos] >= 0) t.sub_cnt[blk * 8 + s] += 1;
    }
  }
}

extern "C" int fva_plan_dims(const fva_plan_desc* desc, fva_plan_info* info) {
  if (!info) return fva_fail(FVA_EINVAL, "info is NULL");
  int rc = validate(desc, info);
  if (rc) return rc;
  size_t offs[27], total;
  layout_workspace(desc, *info, offs, &total);
  info->workspace_bytes = (int64_t)total;
  return FVA_OK;
}

extern "C" int fva_plan_tables(const fva_plan_desc* desc, int32_t* perm, int32_t* blk_cnt,
                               uint64_t* blk_mask, int32_t* sub_id) {
  fva_plan_info in;
  int rc = validate(desc, &in);
  if (rc) return rc;
  HostTables t;
  build_tables(desc, in, t);
  if (perm) memcpy(perm, t.perm.data(), sizeof(int32_t) * in.n_pad);
  if (blk_cnt) memcpy(blk_cnt, t.cnt.data(), sizeof(int32_t) * in.n_blk);
  if (blk_mask) memcpy(blk_mask, t.mask.data(), sizeof(uint64_t) * in.n_blk);
  if (sub_id) memcpy(sub_id, t.sub_id.data(), sizeof(int32_t) * in.n_pad);
  return FVA_OK;
}

extern "C" int fva_plan_create(fva_plan_t* out, const fva_plan_desc* desc, hipStream_t stream) {
  if (!out) return fva_fail(FVA_EINVAL, "out is NULL");
  fva_plan_info in;
  int rc = validate(desc, &in);
  if (rc) return rc;
  size_t offs[27], total;
  layout_workspace(desc, in, offs, &total);
  in.workspace_bytes = (int64_t)total;

  HostTables t;
  build_tables(desc, in, t);

  fva_plan_s* p = new (std::nothrow) fva_plan_s();
  if (!p) return fva_fail(FVA_ENOMEM, "host allocation failed");
  p->desc = *desc;
  p->info = in;
  p->esize = desc->dtype == FVA_DTYPE_BF16 ? 2 : 4;
  p->nw = (in.n_blk + 63) / 64;
  p->stream = stream;
  if ((rc = fva_hip_check(hipGetDevice(&p->device), "hipGetDevice"))) { delete p; return rc; }
  hipDeviceProp_t prop;
  if ((rc = fva_hip_check(hipGetDeviceProperties(&prop, p->device), "hipGetDeviceProperties"))) {
    delete p;
    return rc;
  }
  p->num_cu = prop.multiProcessorCount;
  hipError_t e = hipMalloc(&p->dev_base, total);
  if (e != hipSuccess) {
    delete p;
    return fva_fail(FVA_ENOMEM, "hipMalloc(%zu): %s", total, hipGetErrorString(e));
  }
  p->dev_bytes = total;
  char* b = (char*)p->dev_base;
  p->perm = (int32_t*)(b + offs[0]);
  p->blk_mask = (uint64_t*)(b + offs[1]);
  p->blk_cnt = (int32_t*)(b + offs[2]);
  p->sub_pos = in.n_sub ? (uint8_t*)(b + offs[3]) : nullptr;
  p->sub_cnt = in.n_sub ? (int32_t*)(b + offs[4]) : nullptr;
  p->qbar = (double*)(b + offs[5]);
  p->kbar = (double*)(b + offs[6]);
  p->ybuf = (double*)(b + offs[7]);
  p->rowmax = (double*)(b + offs[8]);
  p->score_split = 1;
  p->rowcnt = (int32_t*)(b + offs[9]);
  p->rowmask = (uint64_t*)(b + offs[10]);
  p->headcnt = (int32_t*)(b + offs[11]);
  p->deficit = (int32_t*)(b + offs[12]);
  p->slack_thr = (uint64_t*)(b + offs[13]);
  p->worklist = (int32_t*)(b + offs[14]);
  p->counters = (int32_t*)(b + offs[15]);
  p->sbuf = (float*)(b + offs[16]);
  p->blk_full = (uint64_t*)(b + offs[17]);
  p->headoff = (int32_t*)(b + offs[18]);
  p->slack_hist = (uint32_t*)(b + offs[19]);
  p->slack_need = (int32_t*)(b + offs[20]);
  p->rope_tab = (double2*)(b + offs[21]);
  p->bwd_delta = (float*)(b + offs[22]);
  p->bits_t = (uint64_t*)(b + offs[23]);
  p->worklist_t = (int32_t*)(b + offs[24]);
  p->pairs = (int2*)(b + offs[25]);
  p->pairs_t = (int2*)(b + offs[26]);

  // Synchronous upload from pageable memory: the tables are small and this
  // happens once per plan, outside any timed path.
  rc = fva_hip_check(hipMemcpy(p->perm, t.perm.data(), sizeof(int32_t) * in.n_pad, hipMemcpyHostToDevice), "upload perm");
  if (!rc) rc = fva_hip_check(hipMemcpy(p->blk_mask, t.mask.data(), sizeof(uint64_t) * in.n_blk, hipMemcpyHostToDevice), "upload mask");
  if (!rc) rc = fva_hip_check(hipMemcpy(p->blk_cnt, t.cnt.data(), sizeof(int32_t) * in.n_blk, hipMemcpyHostToDevice), "upload cnt");
  if (!rc) {
    uint64_t full[64] = {};
    for (int64_t j = 0; j < in.n_blk; ++j)
      if (t.cnt[j] == FVA_BLK) full[j >> 6] |= 1ull << (j & 63);
    rc = fva_hip_check(hipMemcpy(p->blk_full, full, sizeof(full), hipMemcpyHostToDevice), "upload full");
  }
  if (!rc && in.n_sub) {
    rc = fva_hip_check(hipMemcpy(p->sub_pos, t.sub_pos.data(), t.sub_pos.size(), hipMemcpyHostToDevice), "upload sub_pos");
    if (!rc) rc = fva_hip_check(hipMemcpy(p->sub_cnt, t.sub_cnt.data(), sizeof(int32_t) * t.sub_cnt.size(), hipMemcpyHostToDevice), "upload sub_cnt");
  }
  if (!rc) rc = fva_hip_check(hipMemsetAsync(p->counters, 0, sizeof(int32_t) * 64, stream), "clear counters");
  if (!rc)
    rc = fva_hip_check(hipMemsetAsync(p->slack_hist, 0, sizeof(uint32_t) * 256 * (size_t)desc->batch * desc->heads, stream), "clear slack histogram");
  if (!rc) rc = fva_hip_check(hipStreamSynchronize(stream), "plan upload sync");
  if (rc) {
    (void)hipFree(p->dev_base);
    delete p;
    return rc;
  }
  *out = p;
  return FVA_OK;
}

extern "C" int fva_plan(fva_plan_t* out, const fva_plan_desc* desc, hipStream_t stream) {
  return fva_plan_create(out, desc, stream);
}

// Top-p for denoising step `step` of `n_steps`: linear from p_first at the
// first step to p_last at the last ("DFSAttn" explainer, trick 3: little is
// skipped while the latent is still noise, more as the video sharpens; the
// page gives no curve, and a straight line between the two end values is
// the plainest monotone one).  n_steps == 1 gives p_last.
extern "C" int fva_p_schedule(int step, int n_steps, float p_first, float p_last, float* p_out) {
  if (!p_out) return fva_fail(FVA_EINVAL, "p_out is NULL");
  if (n_steps < 1) return fva_fail(FVA_EINVAL, "n_steps = %d must be >= 1", n_steps);
  if (step < 0 || step >= n_steps) return fva_fail(FVA_EINVAL, "step %d outside [0, %d)", step, n_steps);
  if (!(p_first > 0.0f && p_first <= 1.0f) || !(p_last > 0.0f && p_last <= 1.0f))
    return fva_fail(FVA_EINVAL, "p_first %g and p_last %g must lie in (0, 1]", (double)p_first, (double)p_last);
  const double t = n_steps > 1 ? (double)step / (double)(n_steps - 1) : 1.0;
  *p_out = (float)((double)p_first + ((double)p_last - (double)p_first) * t);
  return FVA_OK;
}

extern "C" int fva_plan_query(fva_plan_t plan, fva_plan_info* info) {
  if (!plan || !info) return fva_fail(FVA_EINVAL, "plan or info is NULL");
  *info = plan->info;
  return FVA_OK;
}

extern "C" void fva_plan_destroy(fva_plan_t plan) {
  if (!plan) return;
  (void)hipStreamSynchronize(plan->stream);
  (void)hipDeviceSynchronize();
  (void)hipFree(plan->dev_base);
  delete plan;
}
