// Host side of libfp8pa: argument validation and the split-KV launch plan.
// Pure C++ (no HIP headers), so the planner runs and is tested on any host.
//
// The plan follows the split-KV structure of FlashInfer PR #5591 (Summary:
// split producers plus one LSE reducer; split only as far as one wave of
// work needs) re-derived for MI355X: each wavefront owns one
// (sequence, kv head, row group, split) work item and walks 32-token tiles
// of its key range; the split count is raised until the grid holds about
// kTargetWavesPerCu wavefronts per compute unit, but a split keeps enough
// keys that its partial output stays small next to the KV bytes it reads.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "plan.h"

namespace fp8pa {
namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

int32_t log2i(int32_t x) {
  int32_t r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

}  // namespace

fp8pa_status make_plan(const fp8pa_shape* s, int32_t cu_count, Plan* plan) {
  if (!s || !plan) return FP8PA_ERR_INVALID_ARG;
  if (cu_count < 1) return FP8PA_ERR_INVALID_ARG;
  if (s->batch < 1 || s->q_len < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1)
    return FP8PA_ERR_INVALID_ARG;
  if (s->num_q_heads % s->num_kv_heads != 0) return FP8PA_ERR_INVALID_ARG;
  if (s->num_blocks < 1 || s->max_seq_len < 1 || s->block_table_stride < 1)
    return FP8PA_ERR_INVALID_ARG;
  if (s->max_seq_len < s->q_len) return FP8PA_ERR_INVALID_ARG;
  if (!is_pow2(s->block_tokens) || s->block_tokens > 1024) return FP8PA_ERR_INVALID_ARG;
  if (ceil_div(s->max_seq_len, s->block_tokens) > s->block_table_stride)
    return FP8PA_ERR_INVALID_ARG;
  if (s->k_scale_count != 1 && s->k_scale_count != s->num_kv_heads) return FP8PA_ERR_INVALID_ARG;
  if (s->v_scale_count != 1 && s->v_scale_count != s->num_kv_heads) return FP8PA_ERR_INVALID_ARG;
  if (!std::isfinite(s->sm_scale)) return FP8PA_ERR_INVALID_ARG;
  if (s->num_splits < 0) return FP8PA_ERR_INVALID_ARG;
  const int32_t known = FP8PA_FLAG_FORCE_DOT | FP8PA_FLAG_FORCE_MFMA;
  if (s->flags & ~known) return FP8PA_ERR_INVALID_ARG;
  if ((s->flags & known) == known) return FP8PA_ERR_INVALID_ARG;
  if (s->head_dim != 64 && s->head_dim != 128 && s->head_dim != 256) return FP8PA_ERR_UNSUPPORTED;

  Plan p;
  std::memset(&p, 0, sizeof(p));
  p.B = s->batch;
  p.q_len = s->q_len;
  p.Hq = s->num_q_heads;
  p.Hkv = s->num_kv_heads;
  p.D = s->head_dim;
  p.G = p.Hq / p.Hkv;
  p.bt = s->block_tokens;
  p.bt_shift = log2i(p.bt);

  // One page (all kv heads of bt tokens) must be addressable with 32-bit offsets.
  const int64_t page_bytes = int64_t(p.bt) * p.Hkv * p.D;
  if (page_bytes > (int64_t(1) << 30)) return FP8PA_ERR_UNSUPPORTED;
  const int64_t rows64 = int64_t(p.G) * p.q_len;
  if (rows64 > (int64_t(1) << 20)) return FP8PA_ERR_UNSUPPORTED;
  p.rows = int32_t(rows64);

  // Kernel variant: FP8 MFMA where a kv head has enough query rows to fill a
  // useful part of the 16-wide MFMA tile, VALU dot products otherwise (the
  // grouped-nf4-gemm selector's fp8-vs-f32 split, re-derived for gfx950).
  const bool mfma_ok = p.bt >= 16;
  if (s->flags & FP8PA_FLAG_FORCE_MFMA) {
    if (!mfma_ok) return FP8PA_ERR_UNSUPPORTED;
    p.variant = kVariantMfma;
  } else if (s->flags & FP8PA_FLAG_FORCE_DOT) {
    p.variant = kVariantDot;
  } else {
    p.variant = (mfma_ok && p.rows >= 3) ? kVariantMfma : kVariantDot;
  }
  p.rpg = p.variant == kVariantMfma ? kRowsMfma : kRowsDot;
  p.row_groups = int32_t(ceil_div(p.rows, p.rpg));
  const int32_t rows_eff = p.rows < p.rpg ? p.rows : p.rpg;

  // A workgroup takes adjacent kv heads (one wavefront each), so the bytes of
  // one token slot are read by one workgroup at about the same time.  The
  // MFMA kernel's register budget sets how many wavefronts share a SIMD
  // (4 at D = 64, 2 at D = 128, 1 at D = 256): groups of 8 at D = 64 and 4
  // otherwise let whole groups fill a compute unit.
  const int32_t max_hg = (p.variant == kVariantMfma && p.D != 64) ? 4 : 8;
  p.hg = 1;
  while (p.hg * 2 <= max_hg && p.Hkv % (p.hg * 2) == 0) p.hg *= 2;
  const int64_t units = int64_t(p.B) * (p.Hkv / p.hg) * p.row_groups;
  if (units > (int64_t(1) << 30)) return FP8PA_ERR_UNSUPPORTED;
  p.units = int32_t(units);

  // Tiles a sequence can span: its attended keys, plus one when a window
  // start need not fall on a tile boundary.
  int64_t max_keys = s->max_seq_len;
  if (s->window > 0) {
    const int64_t wk = int64_t(s->window) + s->q_len - 1;
    if (wk < max_keys) max_keys = wk;
  }
  const int64_t n_tiles = ceil_div(max_keys, kTileTokens) + (s->window > 0 ? 1 : 0);

  const int64_t waves_per_split = units * p.hg;
  int64_t tps;
  if (s->num_splits > 0) {
    tps = ceil_div(n_tiles, s->num_splits);
  } else {
    const int64_t target = int64_t(cu_count) * kTargetWavesPerCu;
    const int64_t want = ceil_div(target, waves_per_split);
    tps = ceil_div(n_tiles, want);
    // Keep each split's partial (rows * D floats) small next to the KV it
    // reads (2 * D bytes per key): at least ~64 keys per query row, as long
    // as that still leaves half the target parallelism.
    const int64_t min_tiles = ceil_div(int64_t(rows_eff) * 64, kTileTokens);
    int64_t cap = (n_tiles * waves_per_split) / (target / 2 > 0 ? target / 2 : 1);
    if (cap < 1) cap = 1;
    const int64_t lift = min_tiles < cap ? min_tiles : cap;
    if (tps < lift) tps = lift;
  }
  if (tps < 1) tps = 1;
  if (p.variant == kVariantMfma) {
    // the MFMA kernel holds a split's block-table entries in registers
    const int64_t max_tps = ((int64_t(kMaxSplitPages) - 1) * p.bt) / kTileTokens - 1;
    if (tps > max_tps) tps = max_tps;
  }
  int64_t splits = ceil_div(n_tiles, tps);
  if (splits < 1) splits = 1;
  if (splits * units > (int64_t(1) << 31) - 1) return FP8PA_ERR_UNSUPPORTED;
  p.tps = int32_t(tps);
  p.num_splits = int32_t(splits);
  p.grid_wgs = int32_t(splits * units);
  p.direct = splits == 1 ? 1 : 0;

  if (!p.direct) {
    const int64_t rows_total = int64_t(p.B) * p.q_len * p.Hq;
    const int64_t po = rows_total * splits * p.D * 4;
    const int64_t pl = rows_total * splits * 4;
    const int64_t off = ceil_div(po, kWorkspaceAlign) * kWorkspaceAlign;
    p.off_lse = size_t(off);
    p.ws_bytes = size_t(off + ceil_div(pl, kWorkspaceAlign) * kWorkspaceAlign);
  }
  *plan = p;
  return FP8PA_OK;
}

fp8pa_status check_merge_args(int32_t num_splits, int32_t num_rows, int32_t num_q_heads,
                              int32_t head_dim) {
  if (num_splits < 1 || num_rows < 0 || num_q_heads < 1) return FP8PA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return FP8PA_ERR_UNSUPPORTED;
  return FP8PA_OK;
}

}  // namespace fp8pa

extern "C" {

fp8pa_status fp8pa_plan(const fp8pa_shape* shape, int32_t cu_count, fp8pa_plan_info* out) {
  if (!out) return FP8PA_ERR_INVALID_ARG;
  fp8pa::Plan p;
  const fp8pa_status st = fp8pa::make_plan(shape, cu_count, &p);
  if (st != FP8PA_OK) return st;
  std::memset(out, 0, sizeof(*out));
  out->variant = p.variant;
  out->num_splits = p.num_splits;
  out->tiles_per_split = p.tps;
  out->tile_tokens = fp8pa::kTileTokens;
  out->heads_per_wg = p.hg;
  out->rows_per_group = p.rpg;
  out->row_groups = p.row_groups;
  out->grid_wgs = p.grid_wgs;
  out->merge_launched = p.direct ? 0 : 1;
  out->workspace_bytes = p.ws_bytes;
  out->workspace_lse_offset = p.off_lse;
  return FP8PA_OK;
}

const char* fp8pa_status_string(fp8pa_status status) {
  switch (status) {
    case FP8PA_OK: return "ok";
    case FP8PA_ERR_INVALID_ARG: return "invalid argument";
    case FP8PA_ERR_UNSUPPORTED: return "unsupported shape";
    case FP8PA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FP8PA_ERR_MISALIGNED: return "misaligned pointer";
    case FP8PA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

}  // extern "C"
