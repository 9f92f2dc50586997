// Host-only driver for the plan's validation and table builder, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_sanitize.py.
// Every descriptor of a sweep (ragged grids, every tile shape of volume 64
// over small grids, Hilbert order, sub-blocks, the video shapes, invalid
// fields) goes through fva_plan_dims and fva_plan_tables.  Valid plans must
// give a permutation of the tokens with -1 on pad positions, block masks and
// counts that agree with it, and sub-block ids in [0, 8); invalid ones must be
// rejected with an error code.  Exit status 0 and "ok <n>" when every check
// holds; the sanitizers abort on any memory or undefined-behaviour error.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "fva.h"

static int g_fail = 0;
#define CHECK(c, ...)                       \
  do {                                      \
    if (!(c)) {                             \
      std::printf("FAIL: " __VA_ARGS__);    \
      std::printf("\n");                    \
      ++g_fail;                             \
      return;                               \
    }                                       \
  } while (0)

static void check_plan(const fva_plan_desc& d) {
  fva_plan_info in{};
  const int rc = fva_plan_dims(&d, &in);
  CHECK(rc == FVA_OK, "dims rc %d for grid %d %d %d", rc, d.grid[0], d.grid[1], d.grid[2]);
  CHECK(in.n_tokens == (int64_t)d.grid[0] * d.grid[1] * d.grid[2], "n_tokens");
  CHECK(in.n_pad == (int64_t)in.n_blk * 64, "n_pad");
  std::vector<int32_t> perm(in.n_pad, -7), cnt(in.n_blk, -7), sub(in.n_pad, -7);
  std::vector<uint64_t> mask(in.n_blk, 0);
  CHECK(fva_plan_tables(&d, perm.data(), cnt.data(), mask.data(), sub.data()) == FVA_OK, "tables");
  std::vector<char> seen(in.n_tokens, 0);
  int64_t valid = 0;
  for (int64_t i = 0; i < in.n_pad; ++i) {
    const int32_t t = perm[i];
    const bool bit = mask[i / 64] >> (i % 64) & 1;
    CHECK(t >= -1 && t < in.n_tokens, "perm[%lld] = %d out of range", (long long)i, t);
    CHECK(bit == (t >= 0), "mask bit %lld disagrees with perm", (long long)i);
    if (t >= 0) {
      CHECK(!seen[t], "token %d listed twice", t);
      seen[t] = 1;
      ++valid;
    }
    if (in.n_sub) CHECK(sub[i] >= 0 && sub[i] < 8, "sub id %d at %lld", sub[i], (long long)i);
  }
  CHECK(valid == in.n_tokens, "valid positions %lld != tokens %lld", (long long)valid, (long long)in.n_tokens);
  for (int b = 0; b < in.n_blk; ++b)
    CHECK(cnt[b] == __builtin_popcountll(mask[b]), "block %d count %d", b, cnt[b]);
}

static void check_rejected(fva_plan_desc d, const char* what) {
  fva_plan_info in{};
  const int rc = fva_plan_dims(&d, &in);
  CHECK(rc == FVA_EINVAL || rc == FVA_EUNSUPPORTED, "%s accepted (rc %d)", what, rc);
  CHECK(fva_plan_tables(&d, nullptr, nullptr, nullptr, nullptr) == rc, "%s: tables rc differs", what);
}

int main() {
  int n = 0;
  fva_plan_desc d{};
  d.batch = 1, d.heads = 2, d.head_dim = 128, d.dtype = FVA_DTYPE_BF16;
  const int sizes[] = {1, 2, 3, 5, 8, 13};
  const int tiles[][3] = {{4, 4, 4}, {1, 8, 8}, {2, 4, 8}, {8, 8, 1}, {64, 1, 1}, {1, 1, 64}};
  const int subs[][3] = {{0, 0, 0}, {2, 2, 2}, {1, 2, 4}, {2, 1, 4}};
  for (const auto& tl : tiles)
    for (int order = 0; order < 2; ++order)
      for (const auto& sb : subs)
        for (int gt : sizes)
          for (int gh : sizes)
            for (int gw : sizes) {
              d.grid[0] = gt, d.grid[1] = gh, d.grid[2] = gw;
              for (int a = 0; a < 3; ++a) d.tile[a] = tl[a], d.sub[a] = sb[a];
              d.order = order ? FVA_ORDER_HILBERT : FVA_ORDER_TILE;
              const bool hil_ok = !order || (tl[0] == 4 && tl[1] == 4 && tl[2] == 4);
              bool sub_ok = true;
              if (sb[0])
                for (int a = 0; a < 3; ++a) sub_ok = sub_ok && tl[a] % sb[a] == 0;
              if (hil_ok && sub_ok) check_plan(d);
              else check_rejected(d, "tile/order/sub mismatch");
              ++n;
            }
  // the video shapes: Wan 480P in tile order, 720P in Hilbert order with sub-blocks
  d.tile[0] = d.tile[1] = d.tile[2] = 4;
  d.grid[0] = 21, d.grid[1] = 30, d.grid[2] = 52, d.order = FVA_ORDER_TILE, d.sub[0] = d.sub[1] = d.sub[2] = 0;
  check_plan(d), ++n;
  d.grid[0] = 21, d.grid[1] = 45, d.grid[2] = 80, d.order = FVA_ORDER_HILBERT, d.sub[0] = d.sub[1] = d.sub[2] = 2;
  check_plan(d), ++n;
  // invalid descriptors
  fva_plan_desc b = d;
  b.batch = 0; check_rejected(b, "batch 0"); b = d;
  b.heads = -1; check_rejected(b, "heads -1"); b = d;
  b.head_dim = 96; check_rejected(b, "head_dim 96"); b = d;
  b.grid[1] = 0; check_rejected(b, "grid 0"); b = d;
  b.tile[2] = 0; check_rejected(b, "tile 0"); b = d;
  b.tile[0] = 2; check_rejected(b, "tile volume 32"); b = d;
  b.order = 7; check_rejected(b, "order 7"); b = d;
  b.sub[0] = 3; check_rejected(b, "sub 3"); b = d;
  b.sub[0] = 1, b.sub[1] = 1, b.sub[2] = 4; check_rejected(b, "sub volume 4"); b = d;
  b.dtype = 9; check_rejected(b, "dtype 9"); b = d;
  b.grid[0] = 64, b.grid[1] = 64, b.grid[2] = 68; check_rejected(b, "more than 4096 blocks"); b = d;
  b.heads = 5000, b.grid[0] = 4, b.grid[1] = 4, b.grid[2] = 4; check_rejected(b, "B*H above 4096"); b = d;
  n += 12;
  if (fva_plan_dims(nullptr, nullptr) == FVA_OK) { std::printf("FAIL: null accepted\n"); ++g_fail; }
  if (g_fail) return 1;
  std::printf("ok %d\n", n);
  return 0;
}
