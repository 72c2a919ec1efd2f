// Host-side check of libfp8pa's planner and argument validation, built with
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py
// compiles it with host.cpp and runs it on the CPU).
//
// It calls fp8pa_plan and fp8pa_status_string over a grid of shapes around
// the supported limits and over seeded random shapes whose every field may
// take extreme values (INT32_MIN/MAX, zero, negatives, NaN/inf scales), and
// checks what a valid plan must satisfy.  A sanitizer report (signed
// overflow, out-of-bounds access, ...) aborts the run with a nonzero status.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>

#include "../include/fp8pa.h"

namespace {

int failures = 0;

void fail(const char* what, const fp8pa_shape& s) {
  ++failures;
  if (failures <= 20)
    std::fprintf(stderr, "FAIL %s: B=%d q_len=%d Hq=%d Hkv=%d D=%d bt=%d nb=%d stride=%d max=%d "
                 "window=%d splits=%d flags=%d kg=%d fmt=%d layout=%d page_stride=%lld\n",
                 what, s.batch, s.q_len, s.num_q_heads, s.num_kv_heads, s.head_dim, s.block_tokens,
                 s.num_blocks, s.block_table_stride, s.max_seq_len, s.window, s.num_splits, s.flags,
                 s.k_groups, s.kv_format, s.kv_layout, (long long)s.kv_page_stride);
}

fp8pa_shape base_shape() {
  fp8pa_shape s;
  std::memset(&s, 0, sizeof(s));
  s.batch = 16;
  s.q_len = 1;
  s.num_q_heads = 32;
  s.num_kv_heads = 8;
  s.head_dim = 128;
  s.block_tokens = 16;
  s.num_blocks = 8192;
  s.max_seq_len = 8192;
  s.block_table_stride = 512;
  s.k_scale_count = 8;
  s.v_scale_count = 8;
  s.sm_scale = 0.0884f;
  return s;
}

// What a plan that fp8pa_plan accepted must satisfy.
void check_plan(const fp8pa_shape& s, int cu, const fp8pa_plan_info& p) {
  if (p.grid_wgs < 1) fail("grid_wgs < 1", s);
  if (p.num_splits < 1) fail("num_splits < 1", s);
  if (p.tile_tokens != 32) fail("tile_tokens", s);
  if (p.variant != 0 && p.variant != 1) fail("variant", s);
  if (p.merge_launched != (p.num_splits > 1 ? 1 : 0) && p.split_mode != FP8PA_SPLIT_BALANCED)
    fail("merge_launched vs num_splits", s);
  if (p.merge_launched && p.workspace_bytes == 0) fail("merge without workspace", s);
  if (!p.merge_launched && p.workspace_bytes != 0) fail("workspace without merge", s);
  if (p.merge_launched) {
    const uint64_t rows = uint64_t(s.batch) * uint64_t(s.q_len) * uint64_t(s.num_q_heads);
    const uint64_t po = rows * uint64_t(p.num_splits) * uint64_t(s.head_dim) * 4u;
    const uint64_t pl = rows * uint64_t(p.num_splits) * 4u;
    if (p.workspace_lse_offset < po || p.workspace_lse_offset % 256 != 0) fail("lse offset", s);
    if (p.workspace_bytes < p.workspace_lse_offset + pl) fail("workspace size", s);
  }
  if (p.rows_per_group < 1 || p.row_groups < 1) fail("row groups", s);
  if (int64_t(p.rows_per_group) * p.row_groups <
      int64_t(s.num_q_heads / s.num_kv_heads) * s.q_len)
    fail("row groups cover the rows", s);
  if (p.max_tiles_per_split < 1) fail("max tiles", s);
  if (p.split_mode == FP8PA_SPLIT_FIXED &&
      int64_t(p.num_splits) * p.tiles_per_split * 32 < std::min<int64_t>(s.max_seq_len,
                                                                         s.window > 0 ? int64_t(s.window) + s.q_len - 1 : s.max_seq_len))
    fail("fixed splits cover the keys", s);
  (void)cu;
}

void run(const fp8pa_shape& s, int cu) {
  fp8pa_plan_info p;
  std::memset(&p, 0xAB, sizeof(p));
  const fp8pa_status st = fp8pa_plan(&s, cu, &p);
  if (std::strlen(fp8pa_status_string(st)) == 0) fail("empty status string", s);
  if (st == FP8PA_OK) check_plan(s, cu, p);
}

}  // namespace

int main() {
  long accepted = 0, total = 0;
  // 1. a grid around the supported shapes
  const int Ds[] = {32, 64, 128, 256, 512};
  const int bts[] = {1, 8, 16, 64, 1024, 3, 2048};
  const int qls[] = {1, 2, 4, 16, 128, 512};
  const int Gs[] = {1, 2, 3, 4, 8, 16};
  const int Bs[] = {1, 16, 255, 256, 257, 1024};
  const int maxs[] = {1, 512, 8192, 196608, 1 << 20};
  for (int D : Ds)
    for (int bt : bts)
      for (int ql : qls)
        for (int G : Gs)
          for (int B : Bs)
            for (int mx : maxs)
              for (int win : {0, 1, 4096})
                for (int fmt : {0, 1, 2}) {
                  fp8pa_shape s = base_shape();
                  s.head_dim = D;
                  s.block_tokens = bt;
                  s.q_len = ql;
                  s.num_kv_heads = 4;
                  s.num_q_heads = 4 * G;
                  s.batch = B;
                  s.max_seq_len = mx;
                  s.block_table_stride = bt > 0 ? (mx + bt - 1) / bt : 1;
                  s.window = win;
                  s.kv_format = fmt;
                  s.k_scale_count = 4;
                  s.v_scale_count = 1;
                  fp8pa_plan_info p;
                  ++total;
                  if (fp8pa_plan(&s, 256, &p) == FP8PA_OK) {
                    ++accepted;
                    check_plan(s, 256, p);
                  }
                  for (int cu : {1, 80, 304}) run(s, cu);
                }
  // 2. seeded random shapes with extreme values in every field
  std::mt19937_64 rng(12345);
  const int32_t extremes[] = {std::numeric_limits<int32_t>::min(), -1, 0, 1, 2, 3, 7, 16, 31, 32, 64,
                              128, 256, 1024, 65535, 65536, (1 << 30), std::numeric_limits<int32_t>::max()};
  auto pick = [&](int32_t typical_lo, int32_t typical_hi) -> int32_t {
    if (rng() % 4 == 0) return extremes[rng() % (sizeof(extremes) / sizeof(extremes[0]))];
    return int32_t(typical_lo + int64_t(rng() % uint64_t(int64_t(typical_hi) - typical_lo + 1)));
  };
  const float fext[] = {0.f, -0.f, 1e-30f, -0.1f, 0.0884f, 1e30f, INFINITY, -INFINITY, NAN};
  for (int it = 0; it < 400000; ++it) {
    fp8pa_shape s;
    s.batch = pick(1, 300);
    s.q_len = pick(1, 64);
    s.num_kv_heads = pick(1, 16);
    {
      const int64_t hq = int64_t(s.num_kv_heads) * pick(1, 16);
      s.num_q_heads = (rng() % 3 == 0 || hq > std::numeric_limits<int32_t>::max() ||
                       hq < std::numeric_limits<int32_t>::min())
                          ? pick(1, 128)
                          : int32_t(hq);
    }
    s.head_dim = pick(64, 256);
    s.block_tokens = pick(1, 1024);
    s.num_blocks = pick(1, 100000);
    s.max_seq_len = pick(1, 300000);
    s.block_table_stride = pick(1, 20000);
    s.k_scale_count = pick(1, 16);
    s.v_scale_count = pick(1, 16);
    s.k_groups = pick(0, 16);
    s.kv_layout = pick(0, 1);
    s.kv_format = pick(0, 2);
    s.window = pick(-5, 100000);
    s.sm_scale = (rng() % 8 == 0) ? fext[rng() % 9] : 0.0884f;
    s.num_splits = pick(0, 300);
    s.flags = pick(0, 7);
    s.kv_page_stride = (rng() % 4 == 0) ? int64_t(pick(0, 1 << 20)) * int64_t(rng() % 4096) : 0;
    const int cu = (rng() % 16 == 0) ? pick(-2, 2) : int(1 + rng() % 512);
    ++total;
    run(s, cu);
    fp8pa_plan_info p;
    if (fp8pa_plan(&s, cu, &p) == FP8PA_OK) ++accepted;
  }
  // 3. null arguments
  fp8pa_plan_info p;
  fp8pa_shape s = base_shape();
  if (fp8pa_plan(nullptr, 256, &p) == FP8PA_OK) fail("null shape accepted", s);
  if (fp8pa_plan(&s, 256, nullptr) == FP8PA_OK) fail("null info accepted", s);
  for (int st = -3; st < 12; ++st) (void)fp8pa_status_string(fp8pa_status(st));
  std::printf("plans: %ld accepted of %ld checked, %d failures\n", accepted, total, failures);
  return failures == 0 ? 0 : 1;
}
