// Internal launch plan shared by the host planner (host.cpp) and the kernel
// launcher (kernels.hip).  Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/fp8pa.h"

namespace fp8pa {

constexpr int kTileTokens = 32;      // tokens per tile: one PV MFMA k-step (16x16x32 fp8)
constexpr int kRowsMfma = 16;        // query rows per wavefront: the MFMA N dimension
constexpr int kRowsDot = 4;          // query rows per wavefront in the VALU dot kernel
constexpr size_t kWorkspaceAlign = 256;
constexpr int kMaxWgWaves = 8;       // wavefronts of a partial-kernel workgroup, at most
constexpr int kMaxSplitTiles = 128;  // tiles an MFMA split may span (64 two-tile steps, a lane each)
constexpr int kMaxSplitTilesLds = 1024;  // ... in the LDS-shared kernels, which reload the table window
constexpr int kMaxBalancedBatch = 256; // sequences a wavefront scans (4 per lane)

// K scale groups along head_dim: 0 and 1 both mean one group; otherwise 2, 4,
// 8 or 16 groups of at least 32 dims (so that every 16-byte slice a lane
// stages, of at most 32 dims at a 32-dim boundary, lies in one group).
inline bool k_groups_ok(int32_t k_groups, int32_t head_dim) {
  if (k_groups == 0 || k_groups == 1) return true;
  if (k_groups != 2 && k_groups != 4 && k_groups != 8 && k_groups != 16) return false;
  return head_dim / k_groups >= 32;
}

// log2 of the dims per K scale group.
inline int32_t k_group_shift(int32_t k_groups, int32_t head_dim) {
  const int32_t per = head_dim / (k_groups > 1 ? k_groups : 1);
  int32_t s = 0;
  while ((1 << s) < per) ++s;
  return s;
}

// Bytes of one page of one pool as the format lays it out (E4M3: bt * Hkv *
// D; NVFP4: a data region of bt * Hkv * D / 2 bytes, then a scale region of
// bt * Hkv * D / 16; MXFP8: bt * Hkv * D data bytes, then bt * Hkv * D / 32).
inline int64_t kv_page_bytes(int32_t kv_format, int32_t bt, int32_t hkv, int32_t d) {
  const int64_t rows = int64_t(bt) * hkv;
  if (kv_format == FP8PA_KV_NVFP4) return rows * (d / 2 + d / 16);
  if (kv_format == FP8PA_KV_MXFP8) return rows * (d + d / 32);
  return rows * d;
}
// The bytes of a row's data and scales in a block-scaled format.
inline int32_t kv_data_row(int32_t kv_format, int32_t d) { return kv_format == FP8PA_KV_NVFP4 ? d / 2 : d; }
inline int32_t kv_scale_row(int32_t kv_format, int32_t d) {
  return kv_format == FP8PA_KV_NVFP4 ? d / 16 : kv_format == FP8PA_KV_MXFP8 ? d / 32 : 0;
}

// The stride between a pool's pages: the caller's, or the dense page size.
// 0 when the caller's stride is shorter than a page or not a multiple of 16.
inline int64_t kv_page_stride_of(int64_t stride, int32_t kv_format, int32_t bt, int32_t hkv, int32_t d) {
  const int64_t dense = kv_page_bytes(kv_format, bt, hkv, d);
  if (stride == 0) return dense;
  if (stride < dense || stride % 16 != 0) return 0;
  return stride;
}

enum Variant : int32_t { kVariantDot = 0, kVariantMfma = 1 };

struct Plan {
  int32_t variant;
  int32_t B, q_len, Hq, Hkv, D, G;
  int32_t rows;            // G * q_len query rows per kv head
  int32_t rpg;             // rows per wavefront (row group)
  int32_t row_groups;
  int32_t hg;              // kv heads per workgroup
  int32_t ds;              // wavefronts per kv head (head_dim split; MFMA at D = 256: 2)
  int32_t pr;              // kv heads per wavefront (MFMA at D = 64 with <= 8 rows: 2)
  int32_t lw;              // LDS-shared tiles: row groups per workgroup (0: off)
  int32_t nb;              // 16-row blocks per wavefront (MFMA kernel; 1 or 2)
  int32_t nt;              // 1: non-temporal K/V loads (each byte read by one wavefront)
  int32_t fmt;             // FP8PA_KV_E4M3, FP8PA_KV_NVFP4 or FP8PA_KV_MXFP8
  int64_t page_stride;     // bytes between pages of a pool
  int32_t upi;             // workgroups per (sequence, split) item: (Hkv / hg) * row_groups
  int32_t split_mode;      // FP8PA_SPLIT_*
  int32_t num_splits;      // partial slots per query row
  int32_t tps;             // tiles per split (BALANCED: min_tiles, unused by the kernels)
  int32_t tps_cap;         // largest chunk
  int32_t target_items;    // BALANCED: items the chunk size aims at
  int32_t items;           // (sequence, split) items the grid covers
  int32_t bt, bt_shift;
  int32_t grid_wgs;        // items * upi
  int32_t direct;          // 1: the partial kernel writes the final output (one split)
  size_t ws_bytes;         // 0 when direct
  size_t off_lse;          // byte offset of partial_lse in the workspace
  size_t off_nsplit;       // byte offset of the per-sequence split counts (int32 [B])
  int32_t min_tiles;       // balanced plan: chunk floor (64 keys per query row)
};

// Validates `s` (host-known fields only) and fills `plan` for a device with
// `cu_count` compute units.
fp8pa_status make_plan(const fp8pa_shape* s, int32_t cu_count, Plan* plan);

// Validates fp8pa_merge's scalar arguments.
fp8pa_status check_merge_args(int32_t num_splits, int32_t num_rows, int32_t num_q_heads,
                              int32_t head_dim);

}  // namespace fp8pa
