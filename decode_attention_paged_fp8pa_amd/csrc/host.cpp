// Host side of libfp8pa: argument validation and the split-KV launch plan.
// Pure C++ (no HIP headers), so the planner runs and is tested on any host.
//
// The plan follows the split-KV structure of FlashInfer PR #5591 (Summary:
// split producers plus one LSE reducer; split only as far as one wave of
// work needs) re-derived for MI355X: each wavefront owns one
// (sequence, kv head, row group, split) work item and walks 32-token tiles
// of its key range.  Splits are sized so that the busy wavefronts fill the
// compute units about once (as many as their registers let one hold); for
// batches of up to 256 sequences the kernel sizes them from the real
// seq_lens, which only the device holds.
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
  if (!is_pow2(s->block_tokens) || s->block_tokens > 1024) return FP8PA_ERR_INVALID_ARG;
  if (ceil_div(s->max_seq_len, s->block_tokens) > s->block_table_stride)
    return FP8PA_ERR_INVALID_ARG;
  if (!k_groups_ok(s->k_groups, s->head_dim)) return FP8PA_ERR_INVALID_ARG;
  if (s->kv_layout != FP8PA_LAYOUT_NHD && s->kv_layout != FP8PA_LAYOUT_HND) return FP8PA_ERR_INVALID_ARG;
  if (s->kv_format != FP8PA_KV_E4M3 && s->kv_format != FP8PA_KV_NVFP4 && s->kv_format != FP8PA_KV_MXFP8)
    return FP8PA_ERR_INVALID_ARG;
  if (s->kv_format != FP8PA_KV_E4M3 && s->k_groups > 1) return FP8PA_ERR_INVALID_ARG;
  if (s->kv_page_stride < 0) return FP8PA_ERR_INVALID_ARG;
  const int32_t kg = s->k_groups > 1 ? s->k_groups : 1;
  if (s->k_scale_count != kg && s->k_scale_count != s->num_kv_heads * kg)
    return FP8PA_ERR_INVALID_ARG;
  if (s->v_scale_count != 1 && s->v_scale_count != s->num_kv_heads) return FP8PA_ERR_INVALID_ARG;
  if (!std::isfinite(s->sm_scale)) return FP8PA_ERR_INVALID_ARG;
  if (s->num_splits < 0) return FP8PA_ERR_INVALID_ARG;
  const int32_t variants = FP8PA_FLAG_FORCE_DOT | FP8PA_FLAG_FORCE_MFMA;
  if (s->flags & ~(variants | FP8PA_FLAG_PARTIAL_ONLY)) return FP8PA_ERR_INVALID_ARG;
  if ((s->flags & variants) == variants) return FP8PA_ERR_INVALID_ARG;
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
  p.fmt = s->kv_format;
  p.page_stride = kv_page_stride_of(s->kv_page_stride, p.fmt, p.bt, p.Hkv, p.D);
  if (p.page_stride == 0) return FP8PA_ERR_INVALID_ARG;
  // block-scaled pages are read with 16-byte loads from each page's start
  if (p.fmt != FP8PA_KV_E4M3 && p.page_stride % 16 != 0) return FP8PA_ERR_MISALIGNED;
  if (p.page_stride > (int64_t(1) << 30)) return FP8PA_ERR_UNSUPPORTED;
  const int64_t rows64 = int64_t(p.G) * p.q_len;
  if (rows64 > (int64_t(1) << 20)) return FP8PA_ERR_UNSUPPORTED;
  p.rows = int32_t(rows64);

  // Kernel variant: FP8 MFMA where a kv head has enough query rows to fill a
  // useful part of the 16-wide MFMA tile, VALU dot products otherwise (the
  // grouped-nf4-gemm selector's fp8-vs-f32 split, re-derived for gfx950).
  // (NVFP4 pages: a bf16-MFMA kernel at head_dim 64 and 128; otherwise the
  // VALU kernel, whose lanes each take one 16-element block.)
  const bool mfma_ok = p.bt >= 16 && (p.fmt == FP8PA_KV_E4M3 || p.D <= 128);
  if (s->flags & FP8PA_FLAG_FORCE_MFMA) {
    if (!mfma_ok) return FP8PA_ERR_UNSUPPORTED;
    p.variant = kVariantMfma;
  } else if (s->flags & FP8PA_FLAG_FORCE_DOT) {
    p.variant = kVariantDot;
  } else {
    p.variant = (mfma_ok && p.rows >= 3) ? kVariantMfma : kVariantDot;
  }
  // A workgroup takes adjacent kv heads, up to 8 wavefronts: at 8 kv heads
  // per page token slot it reads whole token slots, so each page comes from
  // HBM in one pass (two workgroups reading halves of a page at different
  // times cost measurably more).  At D = 256 the MFMA kernel splits head_dim
  // over two wavefronts (they exchange partial scores through LDS), which
  // halves their registers.
  const bool fp8_mfma = p.variant == kVariantMfma && p.fmt == FP8PA_KV_E4M3;
  p.ds = (fp8_mfma && p.D == 256) ? 2 : 1;
  // At D = 64 with at most 8 query rows per kv head, the MFMA kernel runs
  // two kv heads per wavefront (one 128-byte line per token, all 16 MFMA
  // columns in use); hg then counts head pairs.
  p.pr = (fp8_mfma && p.D == 64 && p.rows <= 8 && p.Hkv % 2 == 0) ? 2 : 1;
  // More than 16 query rows per kv head (chunked prefill, wide MTP) at
  // head_dim 64: a wavefront carries two blocks of 16 rows over the same K/V
  // registers, so a tile's loads and V transposes serve both (32 rows:
  // 68 us against 92 us with one block).  At head_dim 128 two blocks spill
  // registers and measured slower (137 us against 170 us), and four blocks
  // need more than the 256 registers an MFMA operand can live in.
  p.nb = 1;
  if (fp8_mfma && p.D == 64 && p.ds == 1 && p.pr == 1 && p.rows > kRowsMfma) p.nb = 2;
  // Two, four or eight row groups of one kv head (wide MTP, chunked
  // prefill) share each K/V tile through LDS: the tile is fetched once per
  // workgroup instead of once per row group (prefill 1.35-1.5x faster at
  // head_dim 128; 32 rows 106 us against 137 us).  Two groups at head_dim
  // 64 stay with the two row blocks above, which need no LDS (68 us
  // against 85 us shared).
  // (not with head_dim scale groups: their third query part would not fit
  // the LDS-shared kernels' registers)
  p.lw = 0;
  if (fp8_mfma && p.ds == 1 && p.pr == 1 && p.D <= 128 && s->k_groups <= 1) {
    const int32_t rg1 = int32_t(ceil_div(p.rows, kRowsMfma));
    if (rg1 % 8 == 0) p.lw = 8;
    else if (rg1 % 4 == 0) p.lw = 4;
    else if (rg1 % 2 == 0 && p.D == 128) p.lw = 2;
    if (p.lw) p.nb = 1;
  }
  // (the VALU kernel carries one row per wavefront for one-row kv heads of
  // E4M3 pages, MHA decode: no FMAs on empty rows)
  p.rpg = p.variant == kVariantMfma ? kRowsMfma * p.nb
                                    : (p.rows == 1 && p.fmt == FP8PA_KV_E4M3 ? 1 : kRowsDot);
  p.row_groups = int32_t(ceil_div(p.rows, p.rpg));
  const int32_t rows_unit = p.variant == kVariantMfma ? kRowsMfma : p.rpg;
  const int32_t rows_eff = p.rows < rows_unit ? p.rows : rows_unit;
  // Non-temporal K/V loads keep streamed bytes from pushing reused ones out
  // of the caches; they pay only when no other wavefront reads the same
  // bytes (one row group) and a wavefront reads whole 128-byte lines.
  // (the VALU kernel: where one row per wavefront carries E4M3 pages)
  p.nt = (p.row_groups == 1 && p.D * p.pr / p.ds >= 128 &&
          (p.variant == kVariantMfma || (p.rpg == 1 && p.fmt == FP8PA_KV_E4M3)))
             ? 1
             : 0;

  const int32_t units = p.Hkv / p.pr;  // wavefront head units per sequence
  const int32_t max_hg = kMaxWgWaves / p.ds;
  p.hg = 1;
  while (p.hg * 2 <= max_hg && units % (p.hg * 2) == 0) p.hg *= 2;
  if (p.lw) p.hg = 1;
  p.upi = (units / p.hg) * (p.lw ? p.row_groups / p.lw : p.row_groups);
  const int64_t waves_per_item = int64_t(p.upi) * p.hg * p.ds * (p.lw ? p.lw : 1);

  // Tiles a sequence can span: its attended keys, plus one when a window
  // start need not fall on a tile boundary.
  int64_t max_keys = s->max_seq_len;
  if (s->window > 0) {
    const int64_t wk = int64_t(s->window) + s->q_len - 1;
    if (wk < max_keys) max_keys = wk;
  }
  const int64_t n_tiles = ceil_div(max_keys, kTileTokens) + (s->window > 0 ? 1 : 0);
  // Both kernels hold a split's block-table entries in registers, one
  // window of kMaxSplitTiles tiles; the LDS-shared kernels reload the window
  // as they go, so their splits may be longer.
  const int64_t tps_cap = p.lw ? kMaxSplitTilesLds : kMaxSplitTiles;
  p.tps_cap = int32_t(tps_cap < n_tiles ? tps_cap : n_tiles);

  // Splits: enough (sequence, split) items that the busy wavefronts fill the
  // device about once.  The host knows only max_seq_len, so for a batch of
  // up to kMaxBalancedBatch sequences the kernel itself reads seq_lens and
  // sizes one chunk for the batch's real tile count (BALANCED); longer
  // batches, or a caller's split count, get splits of a fixed size.
  // Wavefronts of the partial kernel one compute unit holds at once: the
  // MFMA kernel's registers allow 4 per SIMD at D = 64 and in the LDS-shared
  // kernels of 4 or 8 row groups (built for 128 registers), 2 otherwise
  // (head_dim 256 is split over two wavefronts); the dot kernel's 2.
  const int64_t waves_per_cu =
      ((fp8_mfma && p.D == 64 && p.pr == 1 && p.nb == 1) || p.lw >= 4) ? 16 : 8;
  const int64_t target_waves = int64_t(cu_count) * waves_per_cu;
  int64_t target_items = target_waves / waves_per_item;
  if (target_items < 1) target_items = 1;
  int64_t tps = 0, splits = 1, items = 0;
  // Each split writes rows * D floats of partial output (and the merge reads
  // them back) against 2 * D bytes of KV per key: at least ~64 keys per
  // query row keep that small, where parallelism allows.
  p.min_tiles = int32_t(ceil_div(int64_t(rows_eff) * 64, kTileTokens));
  p.split_mode = FP8PA_SPLIT_FIXED;
  if (s->num_splits > 0) {
    tps = ceil_div(n_tiles, s->num_splits);
  } else if (p.B <= kMaxBalancedBatch && target_items > 2 * int64_t(p.B) &&
             n_tiles > 1 && int64_t(p.B) * n_tiles < (int64_t(1) << 30)) {
    // (the kernel sums the batch's tiles in 32-bit integers)
    // Every sequence's last split may be short, so up to B items more than
    // T / c: aiming at target - B keeps all items in one round.
    p.split_mode = FP8PA_SPLIT_BALANCED;
    target_items -= p.B;
    // The kernel's chunk is at least min(min_tiles, 2 T / target_items) and
    // T / target_items: one tile at the least, so the slots must allow one
    // split per tile up to the target.
    tps = p.min_tiles;
    splits = n_tiles < target_items ? n_tiles : target_items;
    const int64_t need = ceil_div(n_tiles, int64_t(p.tps_cap));
    if (splits < need) splits = need;
    // sum_b max(1, ceil(n_b / c)) <= T / c + B, and the kernel's chunk c is at
    // least T / target_items unless the cap binds
    int64_t bound = ceil_div(int64_t(p.B) * n_tiles, int64_t(p.tps_cap));
    if (bound < target_items) bound = target_items;
    items = bound + p.B;
    if (items > int64_t(p.B) * splits) items = int64_t(p.B) * splits;
  } else {
    const int64_t want = ceil_div(target_items, int64_t(p.B));
    tps = ceil_div(n_tiles, want);
    // Keep each split's partial (rows * D floats) small next to the KV it
    // reads (2 * D bytes per key): at least ~64 keys per query row, as long
    // as that still leaves half the target parallelism.
    const int64_t min_tiles = p.min_tiles;
    const int64_t per_split = int64_t(p.B) * waves_per_item;
    int64_t cap = (n_tiles * per_split) / (target_waves / 2 > 0 ? target_waves / 2 : 1);
    if (cap < 1) cap = 1;
    const int64_t lift = min_tiles < cap ? min_tiles : cap;
    if (tps < lift) tps = lift;
  }
  if (p.split_mode == FP8PA_SPLIT_FIXED) {
    if (tps < 1) tps = 1;
    if (tps > p.tps_cap) tps = p.tps_cap;
    splits = ceil_div(n_tiles, tps);
    if (splits < 1) splits = 1;
    items = int64_t(p.B) * splits;
    if (splits == 1) p.split_mode = FP8PA_SPLIT_DIRECT;
  }
  if (items * p.upi > (int64_t(1) << 31) - 1) return FP8PA_ERR_UNSUPPORTED;
  p.tps = int32_t(tps);
  p.num_splits = int32_t(splits);
  p.target_items = p.split_mode == FP8PA_SPLIT_BALANCED ? int32_t(target_items) : 0;
  p.items = int32_t(items);
  p.grid_wgs = int32_t(items * p.upi);
  p.direct = p.split_mode == FP8PA_SPLIT_DIRECT ? 1 : 0;

  if (!p.direct) {
    const int64_t rows_total = int64_t(p.B) * p.q_len * p.Hq;
    const int64_t po = rows_total * splits * p.D * 4;  // splits = p.num_splits
    const int64_t pl = rows_total * splits * 4;
    const int64_t off = ceil_div(po, kWorkspaceAlign) * kWorkspaceAlign;
    p.off_lse = size_t(off);
    p.off_nsplit = size_t(off + ceil_div(pl, kWorkspaceAlign) * kWorkspaceAlign);
    p.ws_bytes = p.off_nsplit + size_t(ceil_div(int64_t(p.B) * 4, kWorkspaceAlign) * kWorkspaceAlign);
  }
  *plan = p;
  return FP8PA_OK;
}

fp8pa_status check_merge_args(int32_t num_splits, int32_t num_rows, int32_t num_q_heads,
                              int32_t head_dim) {
  if (num_splits < 1 || num_rows < 0 || num_q_heads < 1) return FP8PA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return FP8PA_ERR_UNSUPPORTED;
  // one merge wavefront per (row, 64 dims)
  if (int64_t(num_rows) * (head_dim / 64) > (int64_t(1) << 31) - 1) return FP8PA_ERR_UNSUPPORTED;
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
  out->split_mode = p.split_mode;
  out->num_splits = p.num_splits;
  out->tiles_per_split = p.tps;
  out->max_tiles_per_split = p.tps_cap;
  out->target_items = p.target_items;
  out->tile_tokens = fp8pa::kTileTokens;
  out->heads_per_wg = p.hg * p.pr;
  out->waves_per_head = p.ds;
  out->heads_per_wave = p.pr;
  out->row_blocks = p.variant == fp8pa::kVariantMfma ? p.nb : 1;
  out->nontemporal_kv = p.nt;
  out->row_groups_per_wg = p.lw ? p.lw : 1;
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
