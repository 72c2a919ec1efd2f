// libfp8pa device code for gfx950 (MI355X): paged flash-decode attention over
// an E4M3 KV cache, and the C-ABI entry points that launch it.
//
// Method (solution record "How do I run paged decode attention over an FP8
// KV cache for a quantized MoE serving path, with sliding windows, attention
// sinks and a custom scale?", fields `title`/`summary`): split-KV flash
// decode with the online softmax of FlashAttention v2/v3 (credited in the
// fish-scales-ops README, Acknowledgments), sink and window folded in, and a
// log-sum-exp reducer over the splits (FlashInfer PR #5591, Summary).
//
// MI355X design:
//  * One wavefront owns one work item (sequence b, kv head g, row group,
//    KV split) and walks 32-token tiles of its key range; a workgroup packs
//    1 to 8 wavefronts on adjacent kv heads, so a workgroup's loads of
//    one token slot are neighbouring bytes of the same page.
//  * Pages are read with raw buffer loads whose descriptor base is the page
//    (wave-uniform, from one scalar block-table load per 16 tokens); lanes
//    of tokens outside the attended range use an offset past the
//    descriptor's range, which the hardware turns into zeros.  So no page
//    outside the range is touched, no table entry of such a page is read,
//    and NaN bytes there cannot reach an MFMA.
//  * MFMA kernel: QK^T on v_mfma_f32_16x16x32_fp8_fp8 with keys on the M
//    side and the query rows of one kv head on the N side (heads on the N
//    side for small head groups: the SwapsAb choice of FlashInfer PR #5591).
//    The bf16 query row is split into two E4M3 parts, hi + lo, under a
//    per-row power-of-two scale, so the scores keep ~2^-8 relative
//    precision while the K codes go straight from HBM into the MFMA.
//    The fp32 score accumulator already holds, per lane, the 8 keys that the
//    PV MFMA's B operand needs, so P = 2^(s - m) is rounded to bf16 in place
//    (8 significant bits at any magnitude, so no weight underflows) and PV
//    runs on the bf16 16x16x32 MFMA; V is transposed to keys-along-K with
//    v_perm byte shuffles in registers (no LDS) and widened to bf16, which
//    holds every E4M3 value exactly.
//  * VALU kernel ("dot"): 16 bytes per lane, D/16 lanes per key, E4M3
//    decoded with v_cvt_pk_f32_fp8, fp32 FMAs and cross-lane reductions;
//    used for kv heads with one or two query rows and pages under 16 tokens.
//  * Merge kernel: one wavefront per output row.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <cmath>
#include <type_traits>
#include <cstdint>

#include "../../include/fp8pa.h"
#include "../../include/fp8pa_debug.h"
#include "plan.h"

namespace fp8pa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// An offset past any buffer range: raw buffer loads at it return zeros.
constexpr uint32_t kOob = 0x80000000u;
// Word 3 of a raw (untyped, unswizzled) buffer descriptor on gfx9 parts.
constexpr int kRsrcWord3 = 0x00020000;
// The online softmax keeps a reference max m that trails the true max by at
// most kLazy (log2 units): a tile moves m only when it exceeds m by more
// than that, so P = 2^(s - m) <= 2^kLazy, and most tiles skip rescaling O.
constexpr float kLazy = 8.0f;
constexpr float kMinNormal = 1.17549435e-38f;  // the least normal fp32 value
// f16 P is taken as 2^kPShift16 times its value: with P <= 2^kLazy before
// the shift it stays below 2^15 (under f16's 65504).
constexpr float kPShift16 = 7.0f;

// Division of 0 <= n < 2^31 by a divisor d >= 1 that the host knows: with
// 2^(l-1) < d <= 2^l, m = ceil(2^(31+l) / d) fits 32 bits and
// n / d = floor(n * m / 2^(31+l)) exactly (n * (m - 2^(31+l)/d) / 2^(31+l)
// < 2^-l <= 1/d never carries the quotient past the next integer).  A
// multiply and a shift instead of the ~25 instructions of a general
// division; the prologue's divisions sit on its critical path.
struct FastDiv {
  uint32_t m;
  uint32_t sh;  // 31 + l
};

struct Params {
  const uint16_t* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const float* k_scale;
  const float* v_scale;
  const float* sinks;
  uint16_t* out;
  float* lse;
  float* part_o;
  float* part_lse;
  int64_t page_bytes;  // bytes between pages of a pool (the page size when dense)
  int32_t tok_stride;  // bytes between token slots of a page: Hkv * D, or D head-major
  int32_t head_stride; // bytes between kv heads of a page: D, or bt * D head-major
  int32_t grp_bytes;   // bytes a 16-token group's descriptor spans from its base
  // NVFP4 pages (tok_stride / head_stride then count data-region bytes):
  int32_t sc_off;      // byte offset of a page's scale region
  int32_t sc_tok;      // scale bytes between token slots
  int32_t sc_head;     // scale bytes between kv heads
  int32_t B, q_len, Hq, Hkv, G, rows, row_groups, hg;
  int32_t upi;           // workgroups per (sequence, split) item
  int32_t num_splits;    // partial slots per query row
  int32_t tps;           // tiles per split; balanced plan: the least chunk
  int32_t tps_cap;       // the largest chunk
  int32_t balanced;      // 1: the chunk comes from the batch's seq_lens
  int32_t target_items;  // balanced plan: items the chunk size aims at
  int32_t min_tiles;     // balanced plan: chunk floor that keeps partials small
  int32_t* nsplit_out;   // per sequence: the splits it got (written by its first item), for the merge
  int32_t max_seq_len;
  int32_t bt_shift, bt_mask, table_stride, window;
  int32_t k_per_head, v_per_head, direct;
  int32_t k_groups;  // K scales per kv head (groups along head_dim), >= 1
  int32_t kg_shift;  // log2 of the dims per K scale group
  int32_t ds;  // wavefronts that split one kv head's head_dim (MFMA kernel, D = 256)
  int32_t pr;  // kv heads per wavefront (MFMA kernel: 2 pairs heads at D = 64)
  float sm_scale;
  // the same divisors for fdiv: upi, row_groups, G, num_splits, target_items
  // and target_items + B (1 where unused)
  FastDiv d_upi, d_rg, d_G, d_ns, d_ti, d_slots;
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float xor_shfl(float v, int mask) { return __shfl_xor(v, mask, 64); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return f32_to_bf16(a) | (f32_to_bf16(b) << 16);
}

// Cache policy of a K/V load: non-temporal (the gfx950 `nt` bit).  Each K/V
// byte is read once per call, so streaming it keeps the small data that is
// reused (seq_lens, block table, queries, split partials) in the caches.
// Only where a wavefront reads whole 128-byte lines: at head_dim 64 two kv
// heads share a line, and an early-evicted line would be fetched twice.
constexpr int kLoadNT = 2;

// Loads BYTES (1, 2, 4, 8 or a multiple of 16) at byte offset `off` of
// buffer `r` with cache policy AUX (1 and 2 bytes: zero-extended into dst[0]).
template <int BYTES, int AUX>
__device__ __forceinline__ void buf_load(Rsrc r, uint32_t off, uint32_t* dst) {
  if constexpr (BYTES == 1) {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, AUX);
  } else if constexpr (BYTES == 2) {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, AUX);
  } else if constexpr (BYTES == 4) {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
  } else if constexpr (BYTES == 8) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
    dst[0] = v.x;
    dst[1] = v.y;
  } else {
    static_assert(BYTES % 16 == 0, "load size");
#pragma unroll
    for (int i = 0; i < BYTES / 16; ++i) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16u * i, 0, AUX);
      dst[4 * i + 0] = v.x;
      dst[4 * i + 1] = v.y;
      dst[4 * i + 2] = v.z;
      dst[4 * i + 3] = v.w;
    }
  }
}


// ptr[i] (a wave-uniform index) through a vector-memory load.  A scalar load
// here would share the lgkm counter with the kernel-argument loads, so the
// first wait on those would also wait for this round trip.
__device__ __forceinline__ float uniform_vload(const float* ptr, int i) {
  const Rsrc r = __builtin_amdgcn_make_buffer_rsrc((void*)ptr, 0, 0x7fffffff, kRsrcWord3);
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, uint32_t(i) * 4u, 0, 0));
}
__device__ __forceinline__ int uniform_vload(const int32_t* ptr, int i) {
  const Rsrc r = __builtin_amdgcn_make_buffer_rsrc((void*)ptr, 0, 0x7fffffff, kRsrcWord3);
  return int(__builtin_amdgcn_raw_buffer_load_b32(r, uint32_t(i) * 4u, 0, 0));
}
// ptr[i] when `use` (wave-uniform), else 0.f without touching memory (a
// descriptor of size 0; ptr may then be null).  The value is left in flight:
// its first use, not this call, waits for it.
__device__ __forceinline__ float maybe_vload(const float* ptr, int i, bool use) {
  const Rsrc r = __builtin_amdgcn_make_buffer_rsrc((void*)ptr, 0, use ? 0x7fffffff : 0, kRsrcWord3);
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, use ? uint32_t(i) * 4u : 0u, 0, 0));
}

__device__ __forceinline__ int maybe_vload(const int32_t* ptr, int i, bool use) {
  const Rsrc r = __builtin_amdgcn_make_buffer_rsrc((void*)ptr, 0, use ? 0x7fffffff : 0, kRsrcWord3);
  return int(__builtin_amdgcn_raw_buffer_load_b32(r, use ? uint32_t(i) * 4u : 0u, 0, 0));
}

// Maximum of v over lanes l, l^16, l^32 and l^48 (the four lane groups that
// hold one MFMA column), with the gfx950 permlane swaps (no LDS round trip).
__device__ __forceinline__ float max_over_groups(float v) {
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
}

// Maxima of scores (MFMA sums or -inf, never NaN) as IEEE 754-2019
// `maximum`, which gfx950 executes as v_maximum3_f32 as it stands: fmaxf
// makes the compiler quiet every operand first in IEEE mode (one more
// instruction per operand).  For non-NaN inputs the two agree up to the sign
// of a zero maximum, which no caller can observe.
__device__ __forceinline__ float max_nn(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max3_nn(float a, float b, float c) { return max_nn(max_nn(a, b), c); }
// max_over_groups for values that are never NaN
__device__ __forceinline__ float max_over_groups_nn(float v) {
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max_nn(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max_nn(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
}

// Sum over the same four lanes (n, n + 16, n + 32, n + 48), the same in each.
__device__ __forceinline__ float sum_over_groups(float v) {
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
}

// 4x4 byte transpose: out[x] byte y = in[y] byte x.
__device__ __forceinline__ void transpose4x4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                             uint32_t* out) {
  const uint32_t t0 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);  // a0.b0 a1.b0 a0.b1 a1.b1
  const uint32_t t1 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);  // a2.b0 a3.b0 a2.b1 a3.b1
  const uint32_t t2 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);  // a0.b2 a1.b2 a0.b3 a1.b3
  const uint32_t t3 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);  // a2.b2 a3.b2 a2.b3 a3.b3
  out[0] = __builtin_amdgcn_perm(t1, t0, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(t1, t0, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(t3, t2, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(t3, t2, 0x07060302u);
}

// Eight E4M3 codes (two dwords, code 4i + b in byte b of dword i) times a
// power of two, as bf16: E4M3 has 4 significant bits, so the product is
// exact (the conversion applies the power of two itself).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1, float sc) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true);
  return bf16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__device__ __forceinline__ long as_long(uint32_t lo, uint32_t hi) {
  return (long)(((uint64_t)hi << 32) | (uint64_t)lo);
}

__device__ __forceinline__ int ceil_div_i(int a, int b) { return (a + b - 1) / b; }

__device__ __forceinline__ int fdiv(int n, FastDiv d) {
  return int(uint32_t((uint64_t(uint32_t(n)) * d.m) >> d.sh));
}

// Wavefront reductions without LDS: DPP within each row of 16 lanes (quad
// swaps, then half-row and row mirrors), then the gfx950 permlane swaps,
// which pair lane l with l ^ 32 and l ^ 16.  Every lane gets the result.
template <typename Op>
__device__ __forceinline__ int wave_reduce_i(int v, Op op) {
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = op(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));  // row_mirror
  const auto s32 = __builtin_amdgcn_permlane32_swap(uint32_t(v), uint32_t(v), false, false);
  v = op(int(s32[0]), int(s32[1]));
  const auto s16 = __builtin_amdgcn_permlane16_swap(uint32_t(v), uint32_t(v), false, false);
  return op(int(s16[0]), int(s16[1]));
}

template <typename Op>
__device__ __forceinline__ float wave_reduce_f(float v, Op op) {
  const auto as_i = [](float x) { return __float_as_int(x); };
  const auto as_f = [](int x) { return __int_as_float(x); };
  v = op(v, as_f(__builtin_amdgcn_update_dpp(0, as_i(v), 0xB1, 0xF, 0xF, false)));
  v = op(v, as_f(__builtin_amdgcn_update_dpp(0, as_i(v), 0x4E, 0xF, 0xF, false)));
  v = op(v, as_f(__builtin_amdgcn_update_dpp(0, as_i(v), 0x141, 0xF, 0xF, false)));
  v = op(v, as_f(__builtin_amdgcn_update_dpp(0, as_i(v), 0x140, 0xF, 0xF, false)));
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
}

__device__ __forceinline__ int wave_sum_i(int v) {
  return wave_reduce_i(v, [](int a, int b) { return a + b; });
}

__device__ __forceinline__ int wave_max_i(int v) {
  return wave_reduce_i(v, [](int a, int b) { return max(a, b); });
}

// Exclusive prefix sum over the 64 lanes of v, 0 <= v <= vmax, and the
// total (no LDS): an inclusive scan by DPP within each row of 16 lanes
// (shifts right by 1, 2, 4 and 8, zero-filled), then the row broadcasts that
// add row 0's total into row 1 and row 2's into row 3 (lane 15 of the row
// before), and lane 31's running total into rows 2 and 3.
__device__ __forceinline__ int wave_excl_prefix_i(int v, int vmax, int& total) {
  (void)vmax;
  int s = v;
  s += __builtin_amdgcn_update_dpp(0, s, 0x111, 0xF, 0xF, false);  // row_shr:1
  s += __builtin_amdgcn_update_dpp(0, s, 0x112, 0xF, 0xF, false);  // row_shr:2
  s += __builtin_amdgcn_update_dpp(0, s, 0x114, 0xF, 0xF, false);  // row_shr:4
  s += __builtin_amdgcn_update_dpp(0, s, 0x118, 0xF, 0xF, false);  // row_shr:8
  s += __builtin_amdgcn_update_dpp(0, s, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1 and 3
  s += __builtin_amdgcn_update_dpp(0, s, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2 and 3
  total = __builtin_amdgcn_readlane(s, 63);
  return s - v;
}

// Keys of sequence b that some query row attends: [ulo, uhi), covered by the
// 32-token tiles [tile0, tile1) (tiles are aligned to absolute positions).
struct Span {
  int ulo, uhi, tile0, tile1;
};

__device__ __forceinline__ Span span_of(int L, int q_len, int window) {
  Span sp;
  sp.uhi = L;
  sp.ulo = window > 0 ? max(0, L - q_len - window + 1) : 0;
  sp.tile0 = sp.ulo / kTileTokens;
  sp.tile1 = sp.uhi > sp.ulo ? (sp.uhi - 1) / kTileTokens + 1 : sp.tile0;
  return sp;
}

// Splits of a sequence with n tiles at chunk c (an empty sequence keeps one
// split, which writes LSE -inf), at most num_splits.
__device__ __forceinline__ int splits_of(int n, int c, int num_splits) {
  return n > 0 ? min(ceil_div_i(n, c), num_splits) : 1;
}

// seq_lens[b] limited to [0, max_seq_len], which bounds every table and page
// access of the kernels whatever the device array holds.
__device__ __forceinline__ int seq_len_of(const Params& p, int b) {
  return min(max(p.seq_lens[b], 0), p.max_seq_len);
}

// Work of one wavefront: (sequence b, kv head g, row group rg, split) and
// the split's tiles [ts, te).  Workgroup x takes item x / upi, an index into
// the batch's (sequence, split) pairs in sequence-major order, and kv head
// group and row group x % upi.
struct Work {
  int b, g, rg, split;
  int half;    // which part of head_dim this wavefront owns (0 unless head_dim is split)
  int nsplit;  // splits of sequence b; its slots [nsplit, num_splits) stay unused
  int L, ts, te;
  Span sp;
  bool active;  // false: the item index lies past the batch's last split
};

// The kv head, row group and head_dim part of this wavefront: these follow
// from the workgroup index alone, so loads that need only them can be issued
// before the (sequence, split) item is resolved.
// The workgroup's logical index.  Workgroups go to the 8 XCDs in turn
// (block i to XCD i % 8); with XCD each XCD's workgroups take one
// contiguous range of logical indices, so the workgroups of one item (which
// re-read the same K/V tiles when several row groups of a kv head share
// them) run on one XCD and meet those bytes in its L2.  (A compile-time
// choice: a branch on a kernel argument here would make the wavefront wait
// for that argument before it issues the loads of the others.)
template <bool XCD>
__device__ __forceinline__ int logical_block(int i) {
  if constexpr (!XCD) return i;
  const int n = gridDim.x, x = i & 7, q = n >> 3, r = n & 7;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + (i >> 3);
}

// The kernel arguments a partial kernel's prologue reads, requested in one
// batch of scalar loads before the first wait.  Left to itself the compiler
// issues them in two or three dependent rounds (the arguments behind one
// address are loaded only once that address is needed), and each round is a
// trip to memory before the first vector load can go out.  An empty asm that
// takes them all as scalar operands makes them all live at its point, and
// the workgroup index it passes through (and returns) makes every step of
// the work item come after it.
__device__ __forceinline__ int prologue_args(const Params& p) {
  int blk = blockIdx.x;
  asm volatile("" : "+s"(blk)
               : "s"(p.q), "s"(p.k_cache), "s"(p.v_cache), "s"(p.block_table), "s"(p.seq_lens),
                 "s"(p.k_scale), "s"(p.v_scale), "s"(p.sinks), "s"(p.B), "s"(p.q_len), "s"(p.G),
                 "s"(p.rows), "s"(p.row_groups), "s"(p.hg), "s"(p.upi), "s"(p.num_splits),
                 "s"(p.balanced), "s"(p.max_seq_len), "s"(p.k_per_head), "s"(p.v_per_head),
                 "s"(p.direct), "s"(p.k_groups), "s"(p.kg_shift), "s"(p.window), "s"(int(gridDim.x)));
  // (and no arithmetic on a loaded argument may be hoisted above it, where
  // its wait would split the batch)
  __builtin_amdgcn_sched_barrier(0);
  return blk;
}

template <bool XCD = false>
__device__ __forceinline__ Work work_head(const Params& p, int ds, int blk) {
  Work w;
  const int bid = logical_block<XCD>(blk);
  const int item = fdiv(bid, p.d_upi);
  const int unit = bid - item * p.upi;
  const int gg = fdiv(unit, p.d_rg);
  w.rg = unit - gg * p.row_groups;
  // the wavefront index is uniform across the wave; saying so keeps every
  // address derived from it (descriptor bases, table rows) in scalar registers
  const int wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  w.g = gg * p.hg + wv / ds;
  w.half = wv - (wv / ds) * ds;
  return w;
}

// seq_lens[l + 64 j], j < 4, for lane l (0 past the batch), requested first
// thing: the chain seq_lens -> work item -> block table -> K/V pages is the
// kernel's critical path, and everything else the prologue loads can wait.
// A descriptor sized to the batch returns 0 past it, so the four loads are
// branch-free and all in flight together.  The balanced plan reads them
// all; fixed plans read their own sequence's from them.
struct SeqLens {
  int v[4];
};

__device__ __forceinline__ SeqLens seq_lens_in_flight(const Params& p) {
  const int lane = threadIdx.x & 63;
  // (the size in bytes saturates: lanes read at most sequence 255)
  const Rsrc slr = __builtin_amdgcn_make_buffer_rsrc((void*)p.seq_lens, 0, min(p.B, 0x1fffffff) * 4, kRsrcWord3);
  SeqLens s;
#pragma unroll
  for (int j = 0; j < 4; ++j) s.v[j] = int(__builtin_amdgcn_raw_buffer_load_b32(slr, uint32_t(lane + 64 * j) * 4u, 0, 0));
  // (kept here: the scheduler would otherwise sink them below the other
  // prologue loads and the arithmetic that addresses those)
  __builtin_amdgcn_sched_barrier(0);
  return s;
}

template <bool XCD = false>
__device__ __forceinline__ void work_item(const Params& p, Work& w, int blk, const SeqLens& sl) {
  const int bid = logical_block<XCD>(blk);
  const int item = fdiv(bid, p.d_upi);
  w.active = true;

  if (!p.balanced) {
    w.b = fdiv(item, p.d_ns);
    w.split = item - w.b * p.num_splits;
    w.nsplit = p.num_splits;
    // (from the early loads for the first 256 sequences: lane b & 63 of load
    // b >> 6; a later sequence of a larger batch is loaded here)
    if (w.b < 256) {
      const int j = w.b >> 6;
      const int v = j == 0 ? sl.v[0] : j == 1 ? sl.v[1] : j == 2 ? sl.v[2] : sl.v[3];
      w.L = min(max(__builtin_amdgcn_readlane(v, w.b & 63), 0), p.max_seq_len);
    } else {
      w.L = seq_len_of(p, w.b);
    }
    w.sp = span_of(w.L, p.q_len, p.window);
    w.ts = w.sp.tile0 + w.split * p.tps;
    w.te = min(w.ts + p.tps, w.sp.tile1);
    if (p.nsplit_out && w.split == 0 && bid == item * p.upi && threadIdx.x == 0)
      p.nsplit_out[w.b] = w.nsplit;
    return;
  }

  // Balanced plan.  Every wavefront derives the same chunk c from the whole
  // batch: T tiles in all, M in the longest sequence.  c >= T / target_items
  // keeps the items near the target; c >= min(min_tiles, 2 T / target_items)
  // keeps each split's partial output small next to the KV bytes it reads
  // while leaving at least about half the target; c >= M / num_splits keeps
  // every sequence within its slots, and c <= tps_cap within the table
  // registers (the plan makes num_splits * tps_cap cover M).  Sequence b
  // then gets splits_of(n_b, c) splits.  Lane l holds sequences l + 64 j.
  const int lane = threadIdx.x & 63;
  int Lj[4], nj[4];
  int tsum = 0, tmax = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = lane + 64 * j;
    Lj[j] = b < p.B ? min(max(sl.v[j], 0), p.max_seq_len) : 0;
    const Span sp = span_of(Lj[j], p.q_len, p.window);
    nj[j] = b < p.B ? sp.tile1 - sp.tile0 : 0;
    tsum += nj[j];
    tmax = max(tmax, nj[j]);
  }
  // (reductions leave the same value in every lane; readfirstlane says so,
  // which keeps the tile range, and so every buffer descriptor, scalar)
  const int T = __builtin_amdgcn_readfirstlane(wave_sum_i(tsum));
  const int M = __builtin_amdgcn_readfirstlane(wave_max_i(tmax));
  const int floor_c = max(min(p.min_tiles, max(1, fdiv(2 * T, p.d_ti))), fdiv(M + p.num_splits - 1, p.d_ns));
  int c = min(max(fdiv(T + p.target_items - 1, p.d_ti), floor_c), p.tps_cap);
  // The grid holds target_items + B items, and sum_b ceil(n_b / c) <= T / c
  // + B is what keeps c >= T / target_items within it.  That bound is loose
  // (sequences of equal length reach T / c): a chunk of T / (target_items +
  // B) is taken instead when its items still fit, so that one round of
  // workgroups carries less per workgroup.
  const int slots = p.target_items + p.B;
  const int ct = min(max(fdiv(T + slots - 1, p.d_slots), floor_c), p.tps_cap);
  if (ct < c) {
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (64 * j >= p.B) break;  // (uniform: no lane holds a sequence)
      cnt += lane + 64 * j < p.B ? splits_of(nj[j], ct, p.num_splits) : 0;
    }
    if (__builtin_amdgcn_readfirstlane(wave_sum_i(cnt)) <= slots) c = ct;
  }
  int base = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (64 * j >= p.B) break;
    const int b = lane + 64 * j;
    const int ns = b < p.B ? splits_of(nj[j], c, p.num_splits) : 0;
    int tot;
    const int excl = wave_excl_prefix_i(ns, p.num_splits, tot);
    tot = __builtin_amdgcn_readfirstlane(tot);
    if (item < base + tot) {
      const uint64_t mask = __ballot(base + excl + ns > item);
      const int ln = __builtin_ctzll(mask);
      w.b = 64 * j + ln;
      w.nsplit = __builtin_amdgcn_readlane(ns, ln);
      w.split = item - base - __builtin_amdgcn_readlane(excl, ln);
      w.L = __builtin_amdgcn_readlane(Lj[j], ln);
      w.sp = span_of(w.L, p.q_len, p.window);
      w.ts = w.sp.tile0 + w.split * c;
      w.te = min(w.ts + c, w.sp.tile1);
      if (p.nsplit_out && w.split == 0 && bid == item * p.upi && threadIdx.x == 0)
        p.nsplit_out[w.b] = w.nsplit;
      return;
    }
    base += tot;
  }
  w.active = false;
  w.b = 0;
  w.split = 0;
  w.nsplit = 0;
  w.L = 0;
  w.sp = span_of(0, p.q_len, p.window);
  w.ts = w.te = 0;
}

__device__ __forceinline__ Work work_of(const Params& p, int ds, int blk) {
  const SeqLens sl = seq_lens_in_flight(p);
  Work w = work_head(p, ds, blk);
  work_item(p, w, blk, sl);
  return w;
}

// Query row `r` (0 <= r < rows) of kv head g: its token index, head and
// attended key range [klo, khi) for a sequence of L tokens.
struct Row {
  bool valid;
  int qi, h, klo, khi;
  size_t out_row;  // (b * q_len + qi) * Hq + h
};

__device__ __forceinline__ Row row_of(const Params& p, int b, int g, int r, int L) {
  Row o;
  o.valid = r < p.rows;
  const int rr = o.valid ? r : 0;
  o.qi = fdiv(rr, p.d_G);
  o.h = g * p.G + (rr - o.qi * p.G);
  const int pos = L - p.q_len + o.qi;
  o.khi = min(pos + 1, L);
  o.klo = p.window > 0 ? max(0, pos - p.window + 1) : 0;
  if (!o.valid || o.khi <= o.klo) {
    o.klo = 0;
    o.khi = 0;
  }
  o.out_row = ((size_t)b * p.q_len + o.qi) * p.Hq + o.h;
  return o;
}

// Tiles [ts, te) of a split clipped to the keys that some query position in
// qmin..qmax attends (positions L - q_len + q, each over its window).
struct TileRange {
  int ts, te;
};
__device__ __forceinline__ TileRange rows_tiles(const Params& p, int L, int qmin, int qmax, int ts,
                                                int te) {
  const int hi = L - p.q_len + qmax + 1;
  const int lo = p.window > 0 ? max(0, L - p.q_len + qmin - p.window + 1) : 0;
  TileRange r;
  r.ts = max(ts, lo / kTileTokens);
  r.te = min(te, (hi + kTileTokens - 1) / kTileTokens);
  return r;
}

// ---------------------------------------------------------------------------
// FP8-MFMA partial kernel.
//
// Lane l of a wavefront: n = l % 16 is the MFMA N column, i.e. the query row
// of the row group; qd = l / 16 is the lane group.  Per 32-token tile:
//   K, group A (tokens 0..15) and B (16..31): lane holds D/4 bytes of token n
//     of the group, bytes [D/4 * qd, D/4 * (qd + 1)) of its row;
//   V: lane holds D/16 bytes (d = D/16 * n ...) of the 8 tokens
//     kap(qd, j) = 4 qd + j (j < 4) and 16 + 4 qd + j - 4 (j >= 4), which are
//     exactly the tokens whose scores the QK accumulators give this lane.
// ---------------------------------------------------------------------------
//
// PR = 2 (head_dim 64, at most 8 query rows per kv head): a wavefront takes
// kv heads 2 g and 2 g + 1 as one problem of head_dim D = 128.  A token's two
// 64-byte head slices are one contiguous 128-byte line; MFMA rows 0-7 are
// the rows of head 2 g with the query in dims 0-63 and zeros in 64-127, rows
// 8-15 those of head 2 g + 1 the other way round, so each row's scores see
// only its own head's keys, and of the output only its own head's dims are
// kept.  All 16 MFMA columns do work and every load reads whole lines.
//
// NB = 2 (head_dim 64 with more than 16 query rows per kv head: chunked
// prefill, wide MTP): a wavefront takes two blocks of 16 rows over the same
// K/V registers, so each tile's loads and V transposes serve 32 rows.
//
// NT selects non-temporal K/V loads: right when each K/V byte is read by one
// wavefront (one row group), wrong when several row groups re-read it.
//
// LW = 2, 4 or 8: the workgroup is LW row groups of one kv head sharing each
// K/V tile through an LDS ring (chunked prefill, wide MTP).  With 4 or 8 the
// register budget is 128 (4 wavefronts per SIMD), so a compute unit holds
// more such workgroups, whose matrix, vector and LDS work then overlap (the
// 512-token chunk ~18% faster); with 2 the staging registers would spill.
template <int D, int DS, int PR, int NB, int NT, int LW>
__global__ __launch_bounds__(64 * kMaxWgWaves)
__attribute__((amdgpu_waves_per_eu((NB == 1 && D / DS == 64) || LW >= 4 ? 4 : D / DS <= 128 ? 2 : 1, 8))) void
partial_mfma_kernel(Params p) {
  static_assert(DS == 1 || DS == 2, "head_dim split");
  static_assert(PR == 1 || (PR == 2 && D == 128 && DS == 1), "paired heads");
  static_assert(NB == 1 || (DS == 1 && PR == 1), "row blocks need one whole head per wavefront");
  static_assert(LW == 0 || ((LW == 2 || LW == 4 || LW == 8) && DS == 1 && PR == 1 && NB == 1),
                "LDS-shared tiles");
  constexpr int DH = D / PR;       // head_dim of the output rows
  constexpr int DW = D / DS;       // head_dim slice of this wavefront
  constexpr int S = DW / 16;       // V bytes per lane per token
  constexpr int KB = DW / 4;       // K bytes per lane per token
  constexpr int KSTEPS = DW / 32;  // QK k-steps of 32 dims
  constexpr int KW = KB / 4;       // K dwords per lane per group
  constexpr int SW = S / 4;        // V dwords per lane per token
  constexpr int AUX = NT ? kLoadNT : 0;  // K/V load cache policy
  // Partial scores of the two wavefronts that share a kv head (DS = 2):
  // [wavefront][tile parity][lane][2 x f32x4], for the at most kMaxWgWaves
  // wavefronts of a workgroup.
  __shared__ f32x4 xch[DS == 2 ? kMaxWgWaves * 2 * 64 * 2 : 1];
  // LW > 0: the LW wavefronts of a workgroup are LW row groups of one kv
  // head and share each K/V tile through a two-slot LDS ring: per slot, K as
  // [32 tokens][D + 16 bytes] of E4M3, then V as [32 tokens][2 D + 32 bytes]
  // of bf16, widened once while staging instead of once per wavefront (rows
  // padded so that the transposing reads below hit distinct banks).
  constexpr int LROW = D + 16;
  constexpr int LROWV = 2 * D + 32;
  constexpr int LSLOT = kTileTokens * (LROW + LROWV);
  __shared__ __attribute__((aligned(16))) uint8_t ltile[LW ? 2 * LSLOT : 16];
  // With the ring, PV's V^T operands are built by transposing LDS reads
  // instead of byte permutes of each wavefront's own copy.
  constexpr bool TRV = LW > 0;

  const int blk = prologue_args(p);
  const SeqLens sl = seq_lens_in_flight(p);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int qd = lane >> 4;
  Work w = work_head<(LW > 0)>(p, DS, blk);
  if constexpr (LW > 0) {
    const int bid = logical_block<true>(blk);
    const int item = fdiv(bid, p.d_upi);
    const int unit = bid - item * p.upi;
    const int rgu = p.row_groups / LW;
    const int wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    w.rg = (unit % rgu) * LW + wv;
    w.g = unit / rgu;
    w.half = 0;
  }
  // This lane's rows: kv head kvh, row rlane[b] of that head's rows in block b.
  const int kvh = PR == 2 ? 2 * w.g + (n >> 3) : w.g;
  int rlane[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) rlane[b] = PR == 2 ? (n & 7) : (w.rg * NB + b) * kRowsMfma + n;
  // Loads that need only the kv head and the rows go first, so that their
  // round trips overlap the item's.
  // The K scale of the dims this lane stages: its kv head's (or the
  // tensor's), or with scale groups along head_dim the group's; a lane's KB
  // dims never straddle two groups.
  const int qdim = w.half * DW + KB * (PR == 2 ? (qd & 1) : qd);
  const float ks = p.k_scale[(p.k_per_head ? kvh * p.k_groups : 0) + (qdim >> p.kg_shift)];
  const float vs = uniform_vload(p.v_scale, p.v_per_head ? kvh : 0);
  // (the raw sink logits stay in flight until the softmax state is set up)
  float sink_raw[NB];
  bool has_sink[NB];
  const bool sinks_here = p.sinks && p.direct;  // uniform
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    has_sink[b] = sinks_here && rlane[b] < p.rows;
    const int rr = min(rlane[b], p.rows - 1);
    const int qi = fdiv(rr, p.d_G);
    sink_raw[b] = maybe_vload(p.sinks, kvh * p.G + (rr - qi * p.G), sinks_here);
  }
  work_item<(LW > 0)>(p, w, blk, sl);
  if (!w.active) return;  // uniform over the workgroup
  const int d0 = w.half * DW;      // first dim of this wavefront's slice
  const int L = w.L;
  const int ulo = w.sp.ulo, uhi = w.sp.uhi;
  // The wavefront's rows (the same for every wavefront of the workgroup) and
  // the query positions qmin..qmax they belong to.
  const int r0 = PR == 2 ? 0 : w.rg * NB * kRowsMfma;
  const int r1 = PR == 2 ? p.rows - 1 : min(r0 + NB * kRowsMfma, p.rows) - 1;
  const int qmin = fdiv(r0, p.d_G), qmax = fdiv(r1, p.d_G);
  // The split's tiles outside the keys some row attends are skipped: with
  // many query rows per sequence (chunked prefill) a row group's causal
  // range ends before the sequence does.
  // (LW > 0: the range of the workgroup's rows, the same for all its wavefronts)
  constexpr int kWgRows = (LW > 0 ? LW : 1) * NB * kRowsMfma;
  const int wg0 = (w.rg / (LW > 0 ? LW : 1)) * kWgRows;
  const int tq0 = LW ? fdiv(wg0, p.d_G) : qmin;
  const int tq1 = LW ? fdiv(min(wg0 + kWgRows, p.rows) - 1, p.d_G) : qmax;
  const TileRange tr = rows_tiles(p, L, tq0, tq1, w.ts, w.te);
  const int ts = tr.ts, te = tr.te;
  Row row[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) row[b] = row_of(p, w.b, kvh, rlane[b], L);
  // With paired heads a lane's 32 query / output dims (of the wavefront's
  // 128) belong to one head: `mine` says whether it is this lane's row's.
  const bool mine = PR == 1 || (qd >> 1) == (n >> 3);

  if (ts >= te && !p.direct) {
    if (w.half == 0 && qd == 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (row[b].valid) p.part_lse[row[b].out_row * p.num_splits + w.split] = -INFINITY;
    }
    return;
  }

  long qhi[NB][KSTEPS], qlo[NB][KSTEPS];  // query rows in E4M3 hi + lo parts (set below)
  // A third part where group K scales were folded into the query: q * ks is
  // an fp32 value, which hi + lo hold to ~8 bits only (a bf16 query they hold
  // almost exactly), too coarse for the LSE of rows with few keys.
  long qlo2[NB][KSTEPS];
  float cr[NB];                           // score scales into log2 units

  // ---- online softmax state (log2 units); the sink enters as a score whose
  // value vector is zero when this split writes the final output.  (The
  // denominator sums the fp32 weights: their bf16 roundings, which O gets,
  // would move the LSE of a row with one dominant key by up to 2^-9.)
  float m[NB], lsum[NB];
  f32x4 O[NB][S];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float sink2 = has_sink[b] ? sink_raw[b] * kLog2e : -INFINITY;
    m[b] = sink2;
    lsum[b] = (qd == 0 && sink2 > -INFINITY) ? 1.f : 0.f;
#pragma unroll
    for (int e = 0; e < S; ++e) O[b][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int tok = p.tok_stride;
  // (paired heads: the pair's first head; its partner's bytes follow it)
  const size_t hoff = (size_t)(PR == 2 ? 2 * w.g : w.g) * (size_t)p.head_stride + d0;
  const uint8_t* kbase_g = p.k_cache + hoff;
  const uint8_t* vbase_g = p.v_cache + hoff;
  const int32_t* btab = p.block_table + (size_t)w.b * p.table_stride;
  // K bytes of token n: KB * qd onwards in the wavefront's D-byte slice; with
  // paired heads lane groups 0-1 read the first head's 64 bytes and 2-3 the
  // second's, head_stride further on (adjacent in token-major pages).
  const uint32_t koff = PR == 2 ? uint32_t(n * tok + KB * (qd & 1) + (qd >> 1) * p.head_stride)
                                : uint32_t(n * tok + KB * qd);

  // Block-table entries of the split, read once before the loop: lane k of
  // tab[g] holds the page of 16-token group g & 1 of tile ts + 2 k + (g >> 1),
  // i.e. of the four groups that loop step k loads (0 for a group that holds
  // no attended token).  A split spans at most kMaxSplitTiles tiles (64
  // steps), so the loop reads each page number with one readlane from a
  // fixed register, and has no table loads and no waits on them.  (The
  // LDS-shared kernels take splits of up to kMaxSplitTilesLds tiles: each
  // staging wavefront loads the next window of entries into the same
  // registers just before it stages its first tile there, one wait per 128
  // tiles; fewer splits for long chunks, so fewer partial outputs to write
  // and merge and fewer workgroup rounds.)
  // (branch-free: a lane whose group holds no attended token reads at an
  // offset past the descriptor and gets 0, so the four loads issue back to
  // back with no wait between them)
  int tab[4];
  const Rsrc rtab = __builtin_amdgcn_make_buffer_rsrc((void*)btab, 0, p.table_stride * 4, kRsrcWord3);
  auto load_table = [&](int t0) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int tt = t0 + 2 * lane + (g >> 1);
      const int gk = tt * kTileTokens + 16 * (g & 1);
      const bool live = tt < te && gk < uhi && gk + 16 > ulo;
      tab[g] = int(__builtin_amdgcn_raw_buffer_load_b32(rtab, live ? uint32_t(gk >> p.bt_shift) * 4u : kOob,
                                                         0, 0));
    }
  };
  load_table(ts);
  // The query rows' raw bf16 bits; converted after the first tiles' loads
  // are issued, so the two round trips overlap.  Every lane loads (a row
  // past the last, or the other head's dims, reads row 0's valid bytes) and
  // keeps zeros where the row is not its own: no branch, no wait between.
  u32x4 qraw[NB][KB / 8];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint16_t* qrow = p.q + row[b].out_row * DH + d0 + KB * (PR == 2 ? (qd & 1) : qd);
    const bool qv = row[b].valid && mine;
#pragma unroll
    for (int i = 0; i < KB / 8; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 8 * i);
      qraw[b][i] = qv ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // Keys every row of this wavefront attends: [ilo, ihi).  A tile inside it
  // needs no score masks; only the others ("edge" tiles: at most the first
  // two and last two of a sequence) are masked.
  const int ihi = L - p.q_len + qmin + 1;
  const int ilo = p.window > 0 ? max(0, L - p.q_len + qmax - p.window + 1) : 0;

  // V bytes: S dims of the wavefront's slice per lane (paired heads: lanes
  // n < 8 the first head's, n >= 8 the second's)
  uint32_t voff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    voff[j] = PR == 2 ? uint32_t((4 * qd + j) * tok + S * (n & 7) + (n >> 3) * p.head_stride)
                      : uint32_t((4 * qd + j) * tok + S * n);

  // Loads of one 32-token tile into registers, without branches.  A tile at
  // or past `te`, or a 16-token group holding no attended token, gets a
  // descriptor of size 0: its loads return zeros and touch no memory.  A
  // group that holds some attended tokens is read whole from its page; the
  // bytes of its other tokens are cleared in the edge-tile path.
  struct TileRegs {
    uint32_t k[2][KW];
    uint32_t v[8][SW];
  };
  // `odd` is (tt - ts) & 1, a constant at every call site.
  auto load_tile = [&](int tt, TileRegs& r, int odd) {
    const int kb = tt * kTileTokens;
    const int step = ((tt - ts) >> 1) & 63;
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      const int gk = kb + 16 * grp;
      const bool live = tt < te && gk < uhi && gk + 16 > ulo;
      const int page = __builtin_amdgcn_readlane(tab[2 * odd + grp], step);
      const size_t base = (size_t)page * (size_t)p.page_bytes + (size_t)(gk & p.bt_mask) * tok;
      const int nrec = live ? p.grp_bytes : 0;
      const Rsrc rk = __builtin_amdgcn_make_buffer_rsrc((void*)(kbase_g + base), 0, nrec, kRsrcWord3);
      const Rsrc rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vbase_g + base), 0, nrec, kRsrcWord3);
      buf_load<KB, AUX>(rk, koff, r.k[grp]);
#pragma unroll
      for (int j = 0; j < 4; ++j) buf_load<S, AUX>(rv, voff[j], r.v[4 * grp + j]);
    }
  };

  // One tile: S^T = K Q^T, mask, online softmax with a lazy reference max,
  // P in bf16, O^T += V^T P^T, in three parts: qk_block (the MFMAs of one
  // row block's scores), soft_block (its softmax step, giving P) and the PV
  // MFMAs.  The V^T operands are built once and, with the K operands, serve
  // every row block.
  // Raw scores of row block b: lane (n, qd) gets tokens kap(qd, 0..3) in sa
  // and kap(qd, 4..7) in sb of row n.
  auto qk_block = [&](const TileRegs& r, int b, f32x4& sa, f32x4& sb) {
    sa = f32x4{0.f, 0.f, 0.f, 0.f};
    sb = f32x4{0.f, 0.f, 0.f, 0.f};
    // (the third query part exists only with head_dim scale groups, which
    // the LDS-shared kernels do not take)
    const bool third = LW == 0 && p.k_groups > 1;
    if constexpr (KSTEPS == 4) {
      // A 128-dim slice: one 16x16x128 FP8 MFMA per query part (gfx950's
      // full-rate form; unit E8M0 scales).  A lane's 32 K bytes and its 32
      // query bytes cover the same dims, which is all the sum needs.
      i32x8 ka, kbv, qh, ql;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ka[i] = int(r.k[0][i]);
        kbv[i] = int(r.k[1][i]);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        qh[2 * c] = int(uint32_t(qhi[b][c]));
        qh[2 * c + 1] = int(uint32_t(uint64_t(qhi[b][c]) >> 32));
        ql[2 * c] = int(uint32_t(qlo[b][c]));
        ql[2 * c + 1] = int(uint32_t(uint64_t(qlo[b][c]) >> 32));
      }
      sa = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qh, sa, 0, 0, 0, 127, 0, 127);
      sb = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kbv, qh, sb, 0, 0, 0, 127, 0, 127);
      sa = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, ql, sa, 0, 0, 0, 127, 0, 127);
      sb = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kbv, ql, sb, 0, 0, 0, 127, 0, 127);
      if (third) {
        i32x8 q3;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          q3[2 * c] = int(uint32_t(qlo2[b][c]));
          q3[2 * c + 1] = int(uint32_t(uint64_t(qlo2[b][c]) >> 32));
        }
        sa = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, q3, sa, 0, 0, 0, 127, 0, 127);
        sb = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kbv, q3, sb, 0, 0, 0, 127, 0, 127);
      }
    } else {
#pragma unroll
      for (int c = 0; c < KSTEPS; ++c) {
        const long ka = as_long(r.k[0][2 * c], r.k[0][2 * c + 1]);
        const long kbv = as_long(r.k[1][2 * c], r.k[1][2 * c + 1]);
        sa = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(ka, qhi[b][c], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(kbv, qhi[b][c], sb, 0, 0, 0);
        sa = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(ka, qlo[b][c], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(kbv, qlo[b][c], sb, 0, 0, 0);
        if (third) {
          sa = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(ka, qlo2[b][c], sa, 0, 0, 0);
          sb = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(kbv, qlo2[b][c], sb, 0, 0, 0);
        }
      }
    }
  };

  // The softmax step of row block b on tile tt's raw scores; returns P.
  auto soft_block = [&](int tt, int b, const f32x4& sa, const f32x4& sb) {
    const int kb = tt * kTileTokens;
    const bool edge = kb < ilo || kb + kTileTokens > ihi;  // uniform
    // Scores of this lane's 8 tokens: raw MFMA sums scaled later by csc
    // (one head_dim slice per wavefront), or, when two wavefronts split
    // head_dim, the sum of both slices' scaled scores exchanged through LDS.
    float sv[8];
    float csc = cr[b];
    if constexpr (DS == 2) {
      const int parity = (tt - ts) & 1;
      const int wv = int(threadIdx.x >> 6);
      f32x4* own = &xch[((wv * 2 + parity) * 64 + lane) * 2];
      own[0] = sa * csc;
      own[1] = sb * csc;
      __syncthreads();
      const f32x4* other = &xch[(((wv ^ 1) * 2 + parity) * 64 + lane) * 2];
      const f32x4 oa = other[0], ob = other[1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sv[j] = sa[j] * csc + oa[j];
        sv[j + 4] = sb[j] * csc + ob[j];
      }
      csc = 1.f;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sv[j] = sa[j];
        sv[j + 4] = sb[j];
      }
    }
    if (edge) {
      // a token this row does not attend scores -inf
      // (the barrier keeps this a branch: as selects it would run on every
      // tile, and only a sequence's first and last tiles need it)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = kb + (j < 4 ? 4 * qd + j : 16 + 4 * qd + (j - 4));
        sv[j] = (key >= row[b].klo && key < row[b].khi) ? sv[j] : -INFINITY;
      }
    }
    // Lazy reference max: move m only when this tile exceeds it by more
    // than kLazy (log2 units), so most tiles skip the O rescale; P stays
    // <= 2^kLazy.  Only then is the row's max over its four lane groups
    // needed (csc > 0, so the scaled max is the max of the scaled).
    const float ms = max3_nn(max3_nn(sv[0], sv[1], sv[2]), max3_nn(sv[3], sv[4], sv[5]), max_nn(sv[6], sv[7]));
    if (__builtin_amdgcn_ballot_w64(ms * csc > m[b] + kLazy) != 0) {
      const float mx = max_over_groups_nn(ms) * csc;
      const bool bump = mx > m[b] + kLazy;  // the same in the row's four lanes
      const float mnew = bump ? mx : m[b];
      const float alpha = bump ? exp2_fast(m[b] - mnew) : 1.f;
      lsum[b] *= alpha;
#pragma unroll
      for (int e = 0; e < S; ++e) O[b][e] *= alpha;
      m[b] = mnew;
    }
    const float noff = m[b] == -INFINITY ? 0.f : -m[b];
    float pj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pj[j] = exp2_fast(fmaf(sv[j], csc, noff));
    lsum[b] += ((pj[0] + pj[1]) + (pj[2] + pj[3])) + ((pj[4] + pj[5]) + (pj[6] + pj[7]));
    // P in bf16 (round to nearest even): 2^-9 relative error per weight at
    // any magnitude, so a weight far below the row's max still reaches O
    // (its mass is in lsum as well).
    bf16x8 P;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const bf16x2 h = __builtin_convertvector((f32x2{pj[j], pj[j + 1]}), bf16x2);
      P[j] = h.x;
      P[j + 1] = h.y;
    }
    return P;
  };

  // PV from the bf16 LDS tile in `slot` (LW > 0), with gfx950's 16-bit
  // transposing read: in each 16-lane group, lane r names an 8-byte row
  // (token 4 qd + r / 4, dims 16 e + 4 (r & 3) ...), and lane 4 h + c
  // receives element c of rows h, h + 4, h + 8, h + 12.  So element t of the
  // read = V[4 qd + t][16 e + n], and a second read 16 tokens on gives
  // elements 4..7: operand e holds V[kap(qd, j)][16 e + n], read once for
  // every row block.  (Tokens outside the span were written as zeros, so
  // nothing needs clearing.)
  auto pv_lds = [&](int slot, const bf16x8 (&Pb)[NB]) {
    const uint8_t* vrow = ltile + slot * LSLOT + kTileTokens * LROW + (4 * qd + (n >> 2)) * LROWV + 8 * (n & 3);
#pragma unroll
    for (int e = 0; e < S; ++e) {
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4*)(vrow + 32 * e));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4*)(vrow + 16 * LROWV + 32 * e));
      const bf16x8 vb = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int b = 0; b < NB; ++b) O[b][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, Pb[b], O[b][e], 0, 0, 0);
    }
  };

  // One whole tile from registers (LW = 0) or from LDS slot `slot`.
  auto compute_tile = [&](int tt, TileRegs& r, int slot) {
    const int kb = tt * kTileTokens;
    const bool edge = kb < ilo || kb + kTileTokens > ihi;  // uniform
    long vt[TRV ? 1 : S];
    if constexpr (!TRV) {
      if (edge) {
        // The V bytes of a token outside the sequence's attended span (read
        // whole with its group, possibly NaN codes) become 0, since P = 0
        // times NaN is NaN.
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = kb + (j < 4 ? 4 * qd + j : 16 + 4 * qd + (j - 4));
          const bool in_span = key >= ulo && key < uhi;
#pragma unroll
          for (int e = 0; e < SW; ++e) r.v[j][e] = in_span ? r.v[j][e] : 0u;
        }
      }
      // V^T operands: byte j of operand e = V[kap(qd, j)][S * n + e]
#pragma unroll
      for (int wd = 0; wd < SW; ++wd) {
        uint32_t lo4[4], hi4[4];
        transpose4x4(r.v[0][wd], r.v[1][wd], r.v[2][wd], r.v[3][wd], lo4);
        transpose4x4(r.v[4][wd], r.v[5][wd], r.v[6][wd], r.v[7][wd], hi4);
#pragma unroll
        for (int x4 = 0; x4 < 4; ++x4) vt[4 * wd + x4] = as_long(lo4[x4], hi4[x4]);
      }
    }
    // With two row blocks the V^T operands are widened to bf16 once and
    // serve both blocks.
    bf16x8 vtb[NB > 1 && !TRV ? S : 1];
    if constexpr (NB > 1 && !TRV) {
#pragma unroll
      for (int e = 0; e < S; ++e)
        vtb[e] = e4m3x8_to_bf16(uint32_t(vt[e]), uint32_t(uint64_t(vt[e]) >> 32), 1.0f);
    }
    bf16x8 Pb[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      f32x4 sa, sb;
      qk_block(r, b, sa, sb);
      Pb[b] = soft_block(tt, b, sa, sb);
      if constexpr (!TRV) {
#pragma unroll
        for (int e = 0; e < S; ++e) {
          const bf16x8 vb = NB > 1 ? vtb[e] : e4m3x8_to_bf16(uint32_t(vt[e]), uint32_t(uint64_t(vt[e]) >> 32), 1.0f);
          O[b][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, Pb[b], O[b][e], 0, 0, 0);
        }
        // keep the scheduler from interleaving blocks (their temporaries
        // would all be live at once)
        if constexpr (NB > 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (TRV) pv_lds(slot, Pb);
  };
  // Two register buffers in turn: while one tile computes, the next tile's
  // loads are in flight (8 KB per wavefront at D = 128).  Deeper pipelines
  // measured slower on MI355X: more than ~8 KB in flight per wavefront only
  // adds queueing in the memory system.
  TileRegs ta, tb;
  // LDS staging (LW > 0).  A tile is four regions (K group A, K group B, V
  // group A, V group B) of 16 tokens x D bytes.  The workgroup's wavefronts
  // form two halves that stage alternate tiles: half h loads the tiles t with
  // (t - ts) & 1 == h, each of its LW / 2 wavefronts RPW whole regions, a
  // lane CH = D / 4 bytes of one token per region.  A tile is loaded three
  // loop steps before it is computed and written into LDS one step before,
  // so the loads have two steps to arrive, and a wavefront never has more
  // than its own one set in flight (its waits are exact).
  constexpr int LWS = LW > 0 ? LW : 2;
  constexpr int RPW = 8 / LWS;  // regions per wavefront
  constexpr int CH = D / 4;
  // (uniform over the wavefront; saying so keeps the page choice and the
  // buffer descriptor in scalar registers)
  const int swv = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int shalf = swv / (LWS / 2);
  const int stok = lane >> 2, scol = (lane & 3) * CH;
  int sreg[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) sreg[rr] = (swv % (LWS / 2)) * RPW + rr;
  uint32_t sR[RPW][CH / 4];
  auto stage_load = [&](int t) {
    const int step = ((t - ts) >> 1) & 63;
    const int podd = (t - ts) & 1;
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int skv = sreg[rr] >> 1, sgrp = sreg[rr] & 1;
      const int ta0 = sgrp ? tab[1] : tab[0];
      const int ta2 = sgrp ? tab[3] : tab[2];
      const int pa = __builtin_amdgcn_readlane(ta0, step);
      const int pb = __builtin_amdgcn_readlane(ta2, step);
      const int page = podd ? pb : pa;
      const int gk = t * kTileTokens + 16 * sgrp;
      const bool live = t < te && gk < uhi && gk + 16 > ulo;
      const size_t base = (size_t)page * (size_t)p.page_bytes + (size_t)(gk & p.bt_mask) * tok;
      const Rsrc rs = __builtin_amdgcn_make_buffer_rsrc((void*)((skv ? vbase_g : kbase_g) + base), 0,
                                                        live ? 16 * tok : 0, kRsrcWord3);
      buf_load<CH, 0>(rs, uint32_t(stok * tok + scol), sR[rr]);
    }
  };
  // `t` is the tile the chunk belongs to: bytes of a token outside the
  // sequence's attended span (read whole with its 16-token group, possibly
  // NaN codes) go into LDS as zeros, since P = 0 times NaN is NaN.  V bytes
  // go in widened to bf16 (exact).
  auto stage_write = [&](int slot, int t) {
    // (uniform: a tile wholly inside the span needs no clearing)
    const bool whole = t * kTileTokens >= ulo && (t + 1) * kTileTokens <= uhi;
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int skv = sreg[rr] >> 1, sgrp = sreg[rr] & 1;  // uniform over the wavefront
      if (!whole) {
        const int key = t * kTileTokens + 16 * sgrp + stok;
        const bool in_span = key >= ulo && key < uhi;
#pragma unroll
        for (int i = 0; i < CH / 4; ++i) sR[rr][i] = in_span ? sR[rr][i] : 0u;
      }
      if (skv) {
        uint8_t* dst = ltile + slot * LSLOT + kTileTokens * LROW + (16 * sgrp + stok) * LROWV + 2 * scol;
#pragma unroll
        for (int i = 0; i < CH / 8; ++i)
          reinterpret_cast<bf16x8*>(dst)[i] = e4m3x8_to_bf16(sR[rr][2 * i], sR[rr][2 * i + 1], 1.0f);
      } else {
        uint8_t* dst = ltile + slot * LSLOT + (16 * sgrp + stok) * LROW + scol;
#pragma unroll
        for (int i = 0; i < CH / 16; ++i)
          reinterpret_cast<u32x4*>(dst)[i] = u32x4{sR[rr][4 * i], sR[rr][4 * i + 1], sR[rr][4 * i + 2], sR[rr][4 * i + 3]};
      }
    }
  };
  auto lds_read = [&](int slot, TileRegs& r) {
    const uint8_t* src = ltile + slot * LSLOT;
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      const uint8_t* kp = src + (16 * grp + n) * LROW + KB * qd;
#pragma unroll
      for (int i = 0; i < KB / 16; ++i) {
        const u32x4 v = reinterpret_cast<const u32x4*>(kp)[i];
        r.k[grp][4 * i] = v.x;
        r.k[grp][4 * i + 1] = v.y;
        r.k[grp][4 * i + 2] = v.z;
        r.k[grp][4 * i + 3] = v.w;
      }
    }
    // (V^T comes from transposing reads in compute_tile)
  };
  if constexpr (LW > 0) {
    stage_load(ts + shalf);
  } else {
    load_tile(ts, ta, 0);
    load_tile(ts + 1, tb, 1);
  }

  // ---- stage the query rows: per-row power-of-two scale, E4M3 hi + lo parts
  // One K scale per head goes into the score scale; group scales differ
  // along the row, so each lane folds its own into its query dims.
  const bool grouped = p.k_groups > 1;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float qf[KB];
#pragma unroll
    for (int i = 0; i < KB / 8; ++i) {
      const u32x4 v = qraw[b][i];
      qf[8 * i + 0] = bf16_lo(v.x);
      qf[8 * i + 1] = bf16_hi(v.x);
      qf[8 * i + 2] = bf16_lo(v.y);
      qf[8 * i + 3] = bf16_hi(v.y);
      qf[8 * i + 4] = bf16_lo(v.z);
      qf[8 * i + 5] = bf16_hi(v.z);
      qf[8 * i + 6] = bf16_lo(v.w);
      qf[8 * i + 7] = bf16_hi(v.w);
    }
    if (grouped) {
#pragma unroll
      for (int i = 0; i < KB; ++i) qf[i] *= ks;
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < KB; ++i) amax = fmaxf(amax, fabsf(qf[i]));
    amax = max_over_groups(amax);
    // 2^(7 - floor(log2 amax)) puts the largest element in [128, 256).
    int se = 0;
    if (amax > 0.f) {
      const int e = int((__float_as_uint(amax) >> 23) & 0xffu) - 127;
      se = min(max(7 - e, -120), 120);
    }
    const float qs = __uint_as_float(uint32_t(se + 127) << 23);
    float c0 = p.sm_scale * (grouped ? 1.f : ks) * kLog2e / qs;
    // Scores are scaled as fma(S, cr, .) with cr > 0, so a -inf mask stays
    // -inf: a negative scale's sign moves into the query, and a zero scale
    // becomes the least normal float (its scores stay ~0; any nonzero
    // scale, however small, is kept as it is).
    const float qsign = c0 < 0.f ? -qs : qs;
    cr[b] = fmaxf(fabsf(c0), kMinNormal);
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = qf[8 * c + j] * qsign;
      uint32_t h0 = 0, h1 = 0, l0 = 0, l1 = 0;
      h0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], h0, false);
      h0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], h0, true);
      h1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], h1, false);
      h1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], h1, true);
      const f32x2 d0 = __builtin_amdgcn_cvt_pk_f32_fp8(h0, false);
      const f32x2 d1 = __builtin_amdgcn_cvt_pk_f32_fp8(h0, true);
      const f32x2 d2 = __builtin_amdgcn_cvt_pk_f32_fp8(h1, false);
      const f32x2 d3 = __builtin_amdgcn_cvt_pk_f32_fp8(h1, true);
      l0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] - d0.x, x[1] - d0.y, l0, false);
      l0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] - d1.x, x[3] - d1.y, l0, true);
      l1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4] - d2.x, x[5] - d2.y, l1, false);
      l1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6] - d3.x, x[7] - d3.y, l1, true);
      qhi[b][c] = as_long(h0, h1);
      qlo[b][c] = as_long(l0, l1);
      uint32_t m0 = 0, m1 = 0;
      if (grouped) {
        const f32x2 e0 = __builtin_amdgcn_cvt_pk_f32_fp8(l0, false);
        const f32x2 e1 = __builtin_amdgcn_cvt_pk_f32_fp8(l0, true);
        const f32x2 e2 = __builtin_amdgcn_cvt_pk_f32_fp8(l1, false);
        const f32x2 e3 = __builtin_amdgcn_cvt_pk_f32_fp8(l1, true);
        m0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] - d0.x - e0.x, x[1] - d0.y - e0.y, m0, false);
        m0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] - d1.x - e1.x, x[3] - d1.y - e1.y, m0, true);
        m1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4] - d2.x - e2.x, x[5] - d2.y - e2.y, m1, false);
        m1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6] - d3.x - e3.x, x[7] - d3.y - e3.y, m1, true);
      }
      qlo2[b][c] = as_long(m0, m1);
    }
  }

  if constexpr (LW > 0) {
    // Tile t goes into LDS slot (t - ts) & 1: loaded by its half at step
    // t - 3, written at step t - 1, computed at step t.
    if (shalf == 0) {
      stage_write(0, ts);
      stage_load(ts + 2);
    }
    auto step = [&](int tt) {
      const int odd = (tt - ts) & 1;
      __syncthreads();  // tile tt is in its slot; the other slot's readers are done
      lds_read(odd, ta);
      if (shalf != odd) {
        stage_write(odd ^ 1, tt + 1);
        stage_load(tt + 3);
      }
      compute_tile(tt, ta, odd);
    };
    // Steps before w0 + 125 stage tiles of the table window that starts at
    // w0; both halves have staged their last one by then, so the next
    // window's entries load there, between two runs of the loop.
    int tt = ts;
#pragma unroll 1
    for (int w0 = ts;; w0 += kMaxSplitTiles) {
      const int tend = min(te, w0 + kMaxSplitTiles - 3);
      for (; tt < tend; ++tt) step(tt);
      if (tt >= te) break;
      load_table(w0 + kMaxSplitTiles);
    }
  } else {
  // two tiles in flight: tile t + 1 loads while tile t is computed
  for (int tt = ts; tt < te; tt += 2) {
    compute_tile(tt, ta, 0);
    if (tt + 1 >= te) break;
    load_tile(tt + 2, ta, 0);
    compute_tile(tt + 1, tb, 0);
    load_tile(tt + 3, tb, 1);
  }
  }

  // ---- epilogue: l over the 4 lane groups, normalise, write
  // O[b][e][i] is output dim S * (4 qd + i) + e of this lane's row in block
  // b (with paired heads: of the wavefront's 128, the row's own 64 start at
  // 64 * (n >> 3)); with V^T from transposing reads, dim 16 e + 4 qd + i.
  const int dlane = PR == 2 ? S * 4 * (qd & 1) : S * 4 * qd;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float l = sum_over_groups(lsum[b]);
    if (!row[b].valid) continue;
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : vs / l;
    const float lse = empty ? -INFINITY : (m[b] + log2_fast(l)) * kLn2;
    if (TRV && p.direct) {
      uint16_t* orow = p.out + row[b].out_row * DH + d0 + 4 * qd;
#pragma unroll
      for (int e = 0; e < S; ++e)
        *reinterpret_cast<u32x2*>(orow + 16 * e) =
            u32x2{pack_bf16x2(O[b][e][0] * inv, O[b][e][1] * inv), pack_bf16x2(O[b][e][2] * inv, O[b][e][3] * inv)};
      if (p.lse && qd == 0 && w.half == 0) p.lse[row[b].out_row] = lse;
    } else if (TRV) {
      const size_t slot = row[b].out_row * p.num_splits + w.split;
      if (!empty) {
        float* prow = p.part_o + slot * DH + d0 + 4 * qd;
#pragma unroll
        for (int e = 0; e < S; ++e) reinterpret_cast<f32x4*>(prow + 16 * e)[0] = O[b][e] * inv;
      }
      if (qd == 0 && w.half == 0) p.part_lse[slot] = lse;
    } else if (p.direct) {
      uint16_t* orow = p.out + row[b].out_row * DH + d0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t pk[S / 2];
#pragma unroll
        for (int e = 0; e < S; e += 2)
          pk[e / 2] = pack_bf16x2(O[b][e][i] * inv, O[b][e + 1][i] * inv);
        uint16_t* dst = orow + dlane + S * i;
        if (!mine) continue;
        if constexpr (S == 4) {
          *reinterpret_cast<u32x2*>(dst) = u32x2{pk[0], pk[1]};
        } else {
#pragma unroll
          for (int v = 0; v < S / 8; ++v)
            reinterpret_cast<u32x4*>(dst)[v] =
                u32x4{pk[4 * v], pk[4 * v + 1], pk[4 * v + 2], pk[4 * v + 3]};
        }
      }
      if (p.lse && qd == 0 && w.half == 0) p.lse[row[b].out_row] = lse;
    } else {
      const size_t slot = row[b].out_row * p.num_splits + w.split;
      if (!empty && mine) {
        float* prow = p.part_o + slot * DH + d0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float* dst = prow + dlane + S * i;
#pragma unroll
          for (int v = 0; v < S / 4; ++v)
            reinterpret_cast<f32x4*>(dst)[v] = f32x4{O[b][4 * v][i] * inv, O[b][4 * v + 1][i] * inv,
                                                     O[b][4 * v + 2][i] * inv, O[b][4 * v + 3][i] * inv};
        }
      }
      if (qd == 0 && w.half == 0) p.part_lse[slot] = lse;
    }
  }
}

// Eight NVFP4 elements (one data dword, element 2i in the low nibble of byte
// i) times a block scale, as bf16: E2M1 times an E4M3 scale has at most 6
// significant bits, so every step is exact.  (The conversion's own scale
// operand applies only a power of two, hence the fp32 multiply.)
// An E8M0 scale byte as the float 2^(s - 127) (0xFF: NaN; 0: 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __uint_as_float(s == 0xffu ? 0x7fc00000u : s == 0u ? 0x00400000u : s << 23);
}


// Eight NVFP4 elements times an E4M3 block scale (as an f16 pair {s, s}),
// in f16: an E2M1 value times an E4M3 scale has at most 6 significant bits
// and lies in [2^-10, 2688], so the conversion and the packed multiply are
// exact.
__device__ __forceinline__ f16x8 fp4x8_to_f16(uint32_t w, f16x2 sc) {
  const f16x2 a = f16x2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0)) * sc;
  const f16x2 b = f16x2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1)) * sc;
  const f16x2 c = f16x2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2)) * sc;
  const f16x2 d = f16x2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3)) * sc;
  return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w, float sc) {
  const f32x2 e[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0) * sc,
                      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1) * sc,
                      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2) * sc,
                      __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3) * sc};
  bf16x8 r;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const bf16x2 h = __builtin_convertvector(e[b], bf16x2);
    r[2 * b] = h.x;
    r[2 * b + 1] = h.y;
  }
  return r;
}

// ---------------------------------------------------------------------------
// Block-scaled pages on the matrix cores (head_dim 64 and 128, kv heads
// with at least 3 query rows).  The lane layout is the FP8-MFMA kernel's
// (keys on M, the 16 query rows of one kv head on N, V dims S n + e on M for
// PV), with 16x16x32 MFMAs on exactly dequantized K and V, so neither
// operand needs a hi + lo split: MXFP8 in bf16 (the bf16 query as it is, P
// rounded to bf16), NVFP4 in f16 (one conversion and one packed multiply
// per two elements; the query times a power of two, P rounded to f16).
//   K, per 16-token group: lane (n, qd) holds dims [D/4 qd, D/4 (qd + 1)) of
//     token n: D/8 data bytes and D/64 scale bytes (one per 16 dims); QK
//     k-step c uses dims D/4 qd + 8 c .. + 7, which lie in one block.
//   V: lane (n, qd) holds dims [S n, S n + S) (S = D/16, inside one block) of
//     the 8 tokens kap(qd, j): S/2 data bytes and one scale byte each.
// ---------------------------------------------------------------------------
template <int D, int FMT, int NT, bool HV = false>
__global__ __launch_bounds__(64 * kMaxWgWaves)
__attribute__((amdgpu_waves_per_eu(2, 8))) void
partial_mfma_nvfp4_kernel(Params p) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(FMT == FP8PA_KV_NVFP4 || FMT == FP8PA_KV_MXFP8, "block-scaled format");
  static_assert(!HV || D == 128, "whole-record V scale loads");
  constexpr bool MX = FMT == FP8PA_KV_MXFP8;
  constexpr int S = D / 16;        // V dims per lane
  constexpr int KD = D / 4;        // K dims per lane per token
  constexpr int KSTEPS = D / 32;   // QK k-steps of 32 dims (8 per lane)
  constexpr int KDB = MX ? KD : KD / 2;   // K data bytes per lane per token
  constexpr int KSB = MX ? 1 : KD / 16;   // K scale bytes per lane per token (one MX block)
  constexpr int VDB = MX ? S : S / 2;     // V data bytes per lane per token
  constexpr int VDW = VDB >= 4 ? VDB / 4 : 1;
  constexpr int BLK = MX ? 32 : 16;       // elements per scale
  constexpr int AUX = NT ? kLoadNT : 0;
  // Operand type of the MFMAs: bf16 for MXFP8 (the E8M0 scale applies in
  // the conversion), f16 for NVFP4 (the E4M3 scale applies with one packed
  // f16 multiply per two elements, exactly; P is taken as 2^kPShift16 times
  // its value, which keeps weights down to 2^-21 of the row's max normal in
  // f16, and the LSE takes the shift back out).
  using OpT = std::conditional_t<MX, bf16x8, f16x8>;
  // MXFP8 at head_dim 128: QK runs on the block-scaled FP8 MFMA
  // (v_mfma_scale_f32_16x16x128_f8f6f4) with the K codes as they are and
  // each 32-element block's E8M0 byte as an A scale; the query goes in as
  // E4M3 hi + lo parts under a per-row power of two, as in the E4M3 kernel.
  // That MFMA's operand layout (pinned by test_hw_mfma_block_scale_layout):
  // lane group g holds k = 16 g .. 16 g + 15 in bytes 0-15 and k = 64 + 16 g
  // .. in bytes 16-31, and the 32 k of block b take lane group b's scale.
  // So with k = head_dim, lane (n, g) loads dims [16 g, 16 g + 16) and
  // [64 + 16 g, 64 + 16 g + 16) of token n (and of the query), and block g's
  // scale byte.  (At head_dim 64 the kernel uses bf16 MFMAs.)
  constexpr bool MXQ = MX && D == 128;
  constexpr float kShift = MX ? 0.f : kPShift16;

  const int blk = prologue_args(p);
  const SeqLens sl = seq_lens_in_flight(p);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int qd = lane >> 4;
  Work w = work_head(p, 1, blk);
  const int kvh = w.g;
  const int rlane = w.rg * kRowsMfma + n;
  const float ks = uniform_vload(p.k_scale, p.k_per_head ? kvh : 0);
  const float vs = uniform_vload(p.v_scale, p.v_per_head ? kvh : 0);
  // (left in flight until the softmax state is set up; see the FP8 kernel)
  const bool sinks_here = p.sinks && p.direct;  // uniform
  const bool has_sink = sinks_here && rlane < p.rows;
  float sink_raw;
  {
    const int rr = min(rlane, p.rows - 1);
    const int qi = fdiv(rr, p.d_G);
    sink_raw = maybe_vload(p.sinks, kvh * p.G + (rr - qi * p.G), sinks_here);
  }
  work_item(p, w, blk, sl);
  if (!w.active) return;  // uniform over the workgroup
  const int L = w.L;
  const int ulo = w.sp.ulo, uhi = w.sp.uhi;
  const int r0 = w.rg * kRowsMfma;
  const int r1 = min(r0 + kRowsMfma, p.rows) - 1;
  const int qmin = fdiv(r0, p.d_G), qmax = fdiv(r1, p.d_G);
  const TileRange tr = rows_tiles(p, L, qmin, qmax, w.ts, w.te);
  const int ts = tr.ts, te = tr.te;
  const Row row = row_of(p, w.b, kvh, rlane, L);

  if (ts >= te && !p.direct && row.valid && qd == 0)
    p.part_lse[row.out_row * p.num_splits + w.split] = -INFINITY;
  if (ts >= te && !p.direct) return;

  // ---- online softmax state (log2 units); the sink enters as a score whose
  // value vector is zero when this split writes the final output.
  const float sink2 = has_sink ? sink_raw * kLog2e : -INFINITY;
  float m = sink2;
  float lsum = (qd == 0 && sink2 > -INFINITY) ? exp2f(kShift) : 0.f;
  f32x4 O[S];
#pragma unroll
  for (int e = 0; e < S; ++e) O[e] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int tok = p.tok_stride;   // data bytes between token slots
  const int stok = p.sc_tok;      // scale bytes between token slots
  const uint8_t* kd_g = p.k_cache + (size_t)kvh * (size_t)p.head_stride;
  const uint8_t* vd_g = p.v_cache + (size_t)kvh * (size_t)p.head_stride;
  const uint8_t* ks_g = p.k_cache + (size_t)p.sc_off + (size_t)kvh * (size_t)p.sc_head;
  const uint8_t* vs_g = p.v_cache + (size_t)p.sc_off + (size_t)kvh * (size_t)p.sc_head;
  const int32_t* btab = p.block_table + (size_t)w.b * p.table_stride;
  const uint32_t kdoff = uint32_t(n * tok + (MXQ ? 16 : KDB) * qd);
  const uint32_t ksoff = uint32_t(n * stok + (KD * qd) / BLK);
  uint32_t vdoff[4], vsoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    vdoff[j] = uint32_t((4 * qd + j) * tok + VDB * n);
    vsoff[j] = uint32_t((4 * qd + j) * stok + (S * n) / BLK);
  }
  // HV (scale records of consecutive tokens adjacent, RB bytes each, as in
  // head-major pages): a lane's four tokens of a group have one run of 4 RB
  // bytes of V scales, read with one 16-byte load (MXFP8) instead of four
  // one-byte loads; the lane takes its byte out of each record.  (The form
  // also holds for NVFP4's 8-byte records, two 16-byte loads, which measured
  // slower than the one-byte loads there; only MXFP8 takes it.)
  constexpr int RB = D / BLK;
  const uint32_t vsrun = uint32_t(4 * qd * RB);

  // Block-table entries of the split in registers, branch-free, as in the
  // FP8 kernel.
  int tab[4];
  {
    const Rsrc rt = __builtin_amdgcn_make_buffer_rsrc((void*)btab, 0, p.table_stride * 4, kRsrcWord3);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int tt = ts + 2 * lane + (g >> 1);
      const int gk = tt * kTileTokens + 16 * (g & 1);
      const bool live = tt < te && gk < uhi && gk + 16 > ulo;
      tab[g] = int(__builtin_amdgcn_raw_buffer_load_b32(rt, live ? uint32_t(gk >> p.bt_shift) * 4u : kOob,
                                                         0, 0));
    }
  }
  // the query row as bf16 operands: k-step c takes dims KD qd + 8 c .. + 7
  // (loaded by every lane, zeroed where the row is past the last)
  u32x4 qraw[KSTEPS];
  {
    const uint16_t* qrow = p.q + row.out_row * D + (MXQ ? 16 : KD) * qd;
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + (MXQ ? 8 * (c & 1) + 64 * (c >> 1) : 8 * c));
      qraw[c] = row.valid ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const int ihi = L - p.q_len + qmin + 1;
  const int ilo = p.window > 0 ? max(0, L - p.q_len + qmax - p.window + 1) : 0;

  struct TileRegs {
    uint32_t kd[2][KDB / 4];
    uint32_t ks[2];
    uint32_t vd[8][VDW];
    uint32_t vs[HV ? 2 * RB : 8];  // HV: the group's 4 records; else one byte per token
  };
  auto load_tile = [&](int tt, TileRegs& r, int odd) {
    const int kb = tt * kTileTokens;
    const int step = ((tt - ts) >> 1) & 63;
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
      const int gk = kb + 16 * grp;
      const bool live = tt < te && gk < uhi && gk + 16 > ulo;
      const int page = __builtin_amdgcn_readlane(tab[2 * odd + grp], step);
      const size_t pbase = (size_t)page * (size_t)p.page_bytes;
      const size_t slot = (size_t)(gk & p.bt_mask);
      const int nd = live ? 16 * tok : 0;
      const int ns = live ? 16 * stok : 0;
      const Rsrc rkd = __builtin_amdgcn_make_buffer_rsrc((void*)(kd_g + pbase + slot * tok), 0, nd, kRsrcWord3);
      const Rsrc rvd = __builtin_amdgcn_make_buffer_rsrc((void*)(vd_g + pbase + slot * tok), 0, nd, kRsrcWord3);
      const Rsrc rks = __builtin_amdgcn_make_buffer_rsrc((void*)(ks_g + pbase + slot * stok), 0, ns, kRsrcWord3);
      const Rsrc rvs = __builtin_amdgcn_make_buffer_rsrc((void*)(vs_g + pbase + slot * stok), 0, ns, kRsrcWord3);
      if constexpr (MXQ) {
        buf_load<16, AUX>(rkd, kdoff, r.kd[grp]);
        buf_load<16, AUX>(rkd, kdoff + 64u, r.kd[grp] + 4);
      } else {
        buf_load<KDB, AUX>(rkd, kdoff, r.kd[grp]);
      }
      buf_load<KSB, AUX>(rks, ksoff, &r.ks[grp]);
      if constexpr (HV) buf_load<4 * RB, AUX>(rvs, vsrun, &r.vs[RB * grp]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        buf_load<VDB, AUX>(rvd, vdoff[j], r.vd[4 * grp + j]);
        if constexpr (!HV) buf_load<1, AUX>(rvs, vsoff[j], &r.vs[4 * grp + j]);
      }
    }
  };

  float cr;  // score scale into log2 units (> 0; a negative one flips the query)
  OpT qb[KSTEPS];
  i32x8 qh8, ql8;  // (MXQ: the query's E4M3 hi and lo parts)
  auto compute_tile = [&](int tt, TileRegs& r) {
    const int kb = tt * kTileTokens;
    const bool edge = kb < ilo || kb + kTileTokens > ihi;  // uniform
    if (edge) {
      // bytes of tokens outside the sequence's attended span (possibly NaN
      // scale codes) become 0
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = kb + (j < 4 ? 4 * qd + j : 16 + 4 * qd + (j - 4));
        const bool in_span = key >= ulo && key < uhi;
#pragma unroll
        for (int w = 0; w < VDW; ++w) r.vd[j][w] = in_span ? r.vd[j][w] : 0u;
        if constexpr (!HV) r.vs[j] = in_span ? r.vs[j] : 0u;
      }
    }
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
    if constexpr (MXQ) {
      i32x8 ka, kbv;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ka[i] = int(r.kd[0][i]);
        kbv[i] = int(r.kd[1][i]);
      }
      const int sca = int(r.ks[0] & 0xff), scb = int(r.ks[1] & 0xff);
      sa = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qh8, sa, 0, 0, 0, sca, 0, 127);
      sb = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kbv, qh8, sb, 0, 0, 0, scb, 0, 127);
      sa = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, ql8, sa, 0, 0, 0, sca, 0, 127);
      sb = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kbv, ql8, sb, 0, 0, 0, scb, 0, 127);
    } else if constexpr (MX) {
      float kscale[2];
#pragma unroll
      for (int grp = 0; grp < 2; ++grp) kscale[grp] = e8m0_to_f32(r.ks[grp] & 0xff);
#pragma unroll
      for (int c = 0; c < KSTEPS; ++c) {
        const bf16x8 ka = e4m3x8_to_bf16(r.kd[0][2 * c], r.kd[0][2 * c + 1], kscale[0]);
        const bf16x8 kbv = e4m3x8_to_bf16(r.kd[1][2 * c], r.kd[1][2 * c + 1], kscale[1]);
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[c], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kbv, qb[c], sb, 0, 0, 0);
      }
    } else {
      // the lane's KSB (<= 2) E4M3 block scales of each group as f16
      f16x2 ksc[2];
#pragma unroll
      for (int grp = 0; grp < 2; ++grp) ksc[grp] = f16x2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.ks[grp], 1.0f, false));
#pragma unroll
      for (int c = 0; c < KSTEPS; ++c) {
        const int blk = (c * 8) / 16;  // the lane's block of k-step c
        const f16x2 sa2 = blk ? __builtin_shufflevector(ksc[0], ksc[0], 1, 1) : __builtin_shufflevector(ksc[0], ksc[0], 0, 0);
        const f16x2 sb2 = blk ? __builtin_shufflevector(ksc[1], ksc[1], 1, 1) : __builtin_shufflevector(ksc[1], ksc[1], 0, 0);
        const f16x8 ka = fp4x8_to_f16(r.kd[0][c], sa2);
        const f16x8 kbv = fp4x8_to_f16(r.kd[1][c], sb2);
        sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[c], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(kbv, qb[c], sb, 0, 0, 0);
      }
    }
    float sv[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sv[j] = sa[j];
      sv[j + 4] = sb[j];
    }
    if (edge) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = kb + (j < 4 ? 4 * qd + j : 16 + 4 * qd + (j - 4));
        sv[j] = (key >= row.klo && key < row.khi) ? sv[j] : -INFINITY;
      }
    }
    float ms = max3_nn(max3_nn(sv[0], sv[1], sv[2]), max3_nn(sv[3], sv[4], sv[5]), max_nn(sv[6], sv[7]));
    ms = max_over_groups_nn(ms);
    const float mx = ms * cr;
    const bool bump = mx > m + kLazy;
    if (__builtin_amdgcn_ballot_w64(bump) != 0) {
      const float mnew = bump ? mx : m;
      const float alpha = bump ? exp2_fast(m - mnew) : 1.f;
      lsum *= alpha;
#pragma unroll
      for (int e = 0; e < S; ++e) O[e] *= alpha;
      m = mnew;
    }
    const float noff = (m == -INFINITY ? 0.f : -m) + kShift;
    float pj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pj[j] = exp2_fast(fmaf(sv[j], cr, noff));
    lsum += ((pj[0] + pj[1]) + (pj[2] + pj[3])) + ((pj[4] + pj[5]) + (pj[6] + pj[7]));
    OpT P;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      if constexpr (MX) {
        const bf16x2 h = __builtin_convertvector((f32x2{pj[j], pj[j + 1]}), bf16x2);
        P[j] = h.x;
        P[j + 1] = h.y;
      } else {
        const f16x2 h = __builtin_convertvector((f32x2{pj[j], pj[j + 1]}), f16x2);
        P[j] = h.x;
        P[j + 1] = h.y;
      }
    }
    // This lane's V scale byte of token kap(qd, j) (in the low byte): with HV
    // out of the group's records (block (S n) / BLK of record j & 3), a token
    // outside the attended span taking 0 as its data bytes did.
    uint32_t vsj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (HV) {
        const int blk = (S * n) / BLK;
        const int wi = RB * (j >> 2) + (RB / 4) * (j & 3);
        const uint32_t wv = RB == 8 ? ((blk >> 2) ? r.vs[wi + 1] : r.vs[wi]) : r.vs[wi];
        vsj[j] = wv >> (8 * (blk & 3));
        if (edge) {
          const int key = kb + (j < 4 ? 4 * qd + j : 16 + 4 * qd + (j - 4));
          vsj[j] = key >= ulo && key < uhi ? vsj[j] : 0u;
        }
      } else {
        vsj[j] = r.vs[j];
      }
    }
    if constexpr (!MX) {
      // V^T operands in f16: token j's S dims as S/2 scaled f16 pairs, then
      // operand e takes element e of tokens kap(qd, 0..7), two tokens per
      // dword by a byte permute.
      uint32_t vh[8][S / 2];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f16x2 s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vsj[j], 1.0f, false);
        const f16x2 sc = __builtin_shufflevector(s2, s2, 0, 0);
        const uint32_t w = r.vd[j][0];
        vh[j][0] = __builtin_bit_cast(uint32_t, f16x2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0)) * sc);
        vh[j][1] = __builtin_bit_cast(uint32_t, f16x2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1)) * sc);
        if constexpr (S == 8) {
          vh[j][2] = __builtin_bit_cast(uint32_t, f16x2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2)) * sc);
          vh[j][3] = __builtin_bit_cast(uint32_t, f16x2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3)) * sc);
        }
      }
#pragma unroll
      for (int b = 0; b < S / 2; ++b) {
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          lo[j / 2] = __builtin_amdgcn_perm(vh[j + 1][b], vh[j][b], 0x05040100u);
          hi[j / 2] = __builtin_amdgcn_perm(vh[j + 1][b], vh[j][b], 0x07060302u);
        }
        O[2 * b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, (u32x4{lo[0], lo[1], lo[2], lo[3]})),
                                                          P, O[2 * b], 0, 0, 0);
        O[2 * b + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            __builtin_bit_cast(f16x8, (u32x4{hi[0], hi[1], hi[2], hi[3]})), P, O[2 * b + 1], 0, 0, 0);
      }
    } else {
      // V^T operands: element j of operand e = V[kap(qd, j)][S n + e]
      float vf[8][S];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // E4M3 times a power of two: the conversion applies it exactly
        const float sc = e8m0_to_f32(vsj[j] & 0xff);
        f32x2 e2[4];
        e2[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.vd[j][0], sc, false);
        e2[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.vd[j][0], sc, true);
        if constexpr (S == 8) {
          e2[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.vd[j][1], sc, false);
          e2[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.vd[j][1], sc, true);
        }
#pragma unroll
        for (int b = 0; b < S / 2; ++b) {
          vf[j][2 * b] = e2[b].x;
          vf[j][2 * b + 1] = e2[b].y;
        }
      }
#pragma unroll
      for (int e = 0; e < S; ++e) {
        bf16x8 vt;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const bf16x2 h = __builtin_convertvector((f32x2{vf[j][e], vf[j + 1][e]}), bf16x2);
          vt[j] = h.x;
          vt[j + 1] = h.y;
        }
        O[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, P, O[e], 0, 0, 0);
      }
    }
  };

  TileRegs ta, tb;
  load_tile(ts, ta, 0);
  load_tile(ts + 1, tb, 1);

  // ---- stage the query under a per-row power of two 2^se, which puts the
  // row's largest element in [2^T, 2^(T+1)): T = 7 for E4M3 hi + lo parts
  // (MXFP8 at head_dim 128, as in the E4M3 kernel), 14 for f16 (NVFP4: exact
  // for every element above 2^-24 of the largest), 0 for bf16 (MXFP8 at
  // head_dim 64: exact).  2^-se moves into the score scale, and the sign of
  // that scale into the query, so that fma(S, cr, .) keeps a -inf mask at
  // -inf; a zero scale becomes the least normal float (scores stay ~0).
  {
    constexpr int T = MXQ ? 7 : MX ? 0 : 14;
    const float c0 = p.sm_scale * ks * kLog2e;
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) {
      const uint32_t wv[4] = {qraw[c].x, qraw[c].y, qraw[c].z, qraw[c].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(wv[i])), fabsf(bf16_hi(wv[i]))));
    }
    amax = max_over_groups(amax);
    int se = 0;
    if (amax > 0.f) {
      const int e = int((__float_as_uint(amax) >> 23) & 0xffu) - 127;
      se = min(max(T - e, -120), 120);
    }
    const float qs = __uint_as_float(uint32_t(se + 127) << 23);
    cr = fmaxf(fabsf(c0) / qs, kMinNormal);
    const float sg = c0 < 0.f ? -qs : qs;
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) {
      const uint32_t wv[4] = {qraw[c].x, qraw[c].y, qraw[c].z, qraw[c].w};
      float x[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(wv[i]) * sg;
        x[2 * i + 1] = bf16_hi(wv[i]) * sg;
      }
      if constexpr (MXQ) {
        uint32_t h0 = 0, h1 = 0, l0 = 0, l1 = 0;
        h0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], h0, false);
        h0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], h0, true);
        h1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], h1, false);
        h1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], h1, true);
        const f32x2 d0 = __builtin_amdgcn_cvt_pk_f32_fp8(h0, false);
        const f32x2 d1 = __builtin_amdgcn_cvt_pk_f32_fp8(h0, true);
        const f32x2 d2 = __builtin_amdgcn_cvt_pk_f32_fp8(h1, false);
        const f32x2 d3 = __builtin_amdgcn_cvt_pk_f32_fp8(h1, true);
        l0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] - d0.x, x[1] - d0.y, l0, false);
        l0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] - d1.x, x[3] - d1.y, l0, true);
        l1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4] - d2.x, x[5] - d2.y, l1, false);
        l1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6] - d3.x, x[7] - d3.y, l1, true);
        qh8[2 * c] = int(h0);
        qh8[2 * c + 1] = int(h1);
        ql8[2 * c] = int(l0);
        ql8[2 * c + 1] = int(l1);
      } else {
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          if constexpr (MX) {
            const bf16x2 h = __builtin_convertvector((f32x2{x[i], x[i + 1]}), bf16x2);
            qb[c][i] = h.x;
            qb[c][i + 1] = h.y;
          } else {
            const f16x2 h = __builtin_convertvector((f32x2{x[i], x[i + 1]}), f16x2);
            qb[c][i] = h.x;
            qb[c][i + 1] = h.y;
          }
        }
      }
    }
  }

  for (int tt = ts; tt < te; tt += 2) {
    compute_tile(tt, ta);
    if (tt + 1 >= te) break;
    load_tile(tt + 2, ta, 0);
    compute_tile(tt + 1, tb);
    load_tile(tt + 3, tb, 1);
  }

  // ---- epilogue: l over the 4 lane groups, normalise, write
  lsum = sum_over_groups(lsum);
  if (!row.valid) return;
  const bool empty = !(lsum > 0.f);
  const float inv = empty ? 0.f : vs / lsum;
  const float lse = empty ? -INFINITY : (m - kShift + log2_fast(lsum)) * kLn2;
  // O[e][i] is output dim S * (4 qd + i) + e of this lane's row
  const int dlane = S * 4 * qd;
  if (p.direct) {
    uint16_t* orow = p.out + row.out_row * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t pk[S / 2];
#pragma unroll
      for (int e = 0; e < S; e += 2) pk[e / 2] = pack_bf16x2(O[e][i] * inv, O[e + 1][i] * inv);
      uint16_t* dst = orow + dlane + S * i;
      if constexpr (S == 4) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{pk[0], pk[1]};
      } else {
#pragma unroll
        for (int v = 0; v < S / 8; ++v)
          reinterpret_cast<u32x4*>(dst)[v] = u32x4{pk[4 * v], pk[4 * v + 1], pk[4 * v + 2], pk[4 * v + 3]};
      }
    }
    if (p.lse && qd == 0) p.lse[row.out_row] = lse;
  } else {
    const size_t slot = row.out_row * p.num_splits + w.split;
    if (!empty) {
      float* prow = p.part_o + slot * D;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float* dst = prow + dlane + S * i;
#pragma unroll
        for (int v = 0; v < S / 4; ++v)
          reinterpret_cast<f32x4*>(dst)[v] =
              f32x4{O[4 * v][i] * inv, O[4 * v + 1][i] * inv, O[4 * v + 2][i] * inv, O[4 * v + 3][i] * inv};
      }
    }
    if (qd == 0) p.part_lse[slot] = lse;
  }
}

// Sixteen NVFP4 elements (8 data bytes, element 2i in the low nibble of byte
// i) as floats: E2M1 decodes exactly, so the conversion's scale is 1.
__device__ __forceinline__ void fp4x16_to_f32(u32x2 w, float* f) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t x = h == 0 ? w.x : w.y;
    const f32x2 b0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, 0);
    const f32x2 b1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, 1);
    const f32x2 b2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, 2);
    const f32x2 b3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, 3);
    f[8 * h + 0] = b0.x;
    f[8 * h + 1] = b0.y;
    f[8 * h + 2] = b1.x;
    f[8 * h + 3] = b1.y;
    f[8 * h + 4] = b2.x;
    f[8 * h + 5] = b2.y;
    f[8 * h + 6] = b3.x;
    f[8 * h + 7] = b3.y;
  }
}

// ---------------------------------------------------------------------------
// VALU dot-product partial kernel: D/16 lanes per token, 16 elements per
// lane, RPG query rows per wavefront (1 for one-row kv heads, MHA decode;
// else 4).  Lane l: token kk = l / (D/16) of a round, chunk c = l % (D/16),
// dims [16 c, 16 c + 16).
//
// FMT = FP8PA_KV_NVFP4: a lane's 16 elements of a token are one NVFP4 block
// (8 data bytes and one E4M3 scale byte), so the block scale multiplies the
// lane's partial q.K before the cross-lane sum, and P before it meets V.
//
// Pages of at least 16 tokens: the split's block-table entries are read
// once into registers (as in the MFMA kernel), each 16-token group's page
// is a wave-uniform readlane, and every load goes through a buffer
// descriptor on that group (a key outside the span reads at an offset past
// it and gets zeros), with two tiles in flight.  Smaller pages read each
// key's page per lane.
// ---------------------------------------------------------------------------
template <int D, int FMT, int RPG, int NT = 0>
__global__ __launch_bounds__(512) void partial_dot_kernel(Params p) {
  constexpr int LPK = D / 16;    // lanes per token
  constexpr int KPI = 64 / LPK;  // tokens per round
  constexpr int R = kTileTokens / KPI;
  constexpr bool NV = FMT == FP8PA_KV_NVFP4;
  constexpr bool MX = FMT == FP8PA_KV_MXFP8;
  constexpr int KWB = NV ? 8 : 16;  // data bytes a lane reads per token
  constexpr int AUX = NT ? kLoadNT : 0;  // K/V load cache policy (NT: one wave reads each line)

  const int blk = prologue_args(p);
  const int lane = threadIdx.x & 63;
  const int kk = lane / LPK;
  const int c = lane % LPK;
  const Work w = work_of(p, 1, blk);
  if (!w.active) return;  // uniform over the workgroup
  const int L = w.L;
  const int ulo = w.sp.ulo, uhi = w.sp.uhi;
  const int r0 = w.rg * RPG, r1 = min(r0 + RPG, p.rows) - 1;
  const TileRange tr = rows_tiles(p, L, fdiv(r0, p.d_G), fdiv(r1, p.d_G), w.ts, w.te);
  const int ts = tr.ts, te = tr.te;

  Row rows[RPG];
#pragma unroll
  for (int rr = 0; rr < RPG; ++rr) rows[rr] = row_of(p, w.b, w.g, w.rg * RPG + rr, L);

  if (ts >= te && !p.direct) {
    if (lane == 0) {
#pragma unroll
      for (int rr = 0; rr < RPG; ++rr)
        if (rows[rr].valid) p.part_lse[rows[rr].out_row * p.num_splits + w.split] = -INFINITY;
    }
    return;
  }

  const int tok = p.tok_stride;
  // a lane's bytes of a token: 16 E4M3 codes, or 8 NVFP4 data bytes and one scale byte
  const size_t lane_off = (size_t)w.g * (size_t)p.head_stride + KWB * c;
  const uint8_t* kbase_g = p.k_cache + lane_off;
  const uint8_t* vbase_g = p.v_cache + lane_off;
  // (the lane's block: NVFP4's are its 16 elements, MXFP8's 32 span two lanes)
  const size_t sc_lane = (size_t)p.sc_off + (size_t)w.g * (size_t)p.sc_head + (MX ? c / 2 : c);
  const int32_t* btab = p.block_table + (size_t)w.b * p.table_stride;
  // pages of at least 16 tokens: every 16-token group lies in one page (MXFP8
  // at head_dim 256 keeps the per-lane path: the grouped scale loads would
  // spill registers there)
  const bool grouped_pages = p.bt_shift >= 4 && !(MX && D == 256);  // uniform

  // Block-table entries of the split (pages of 16 or more tokens): lane k of
  // tab[g] holds the page of 16-token group g & 1 of tile ts + 2 k + (g >> 1);
  // a split spans at most kMaxSplitTiles tiles.  Branch-free, as in the MFMA
  // kernel.
  int tab[4] = {0, 0, 0, 0};
  if (grouped_pages) {
    const Rsrc rt = __builtin_amdgcn_make_buffer_rsrc((void*)btab, 0, p.table_stride * 4, kRsrcWord3);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int tt = ts + 2 * lane + (g >> 1);
      const int gk = tt * kTileTokens + 16 * (g & 1);
      const bool live = tt < te && gk < uhi && gk + 16 > ulo;
      tab[g] = int(__builtin_amdgcn_raw_buffer_load_b32(rt, live ? uint32_t(gk >> p.bt_shift) * 4u : kOob,
                                                         0, 0));
    }
  }

  // this lane's 16 dims lie in one K scale group
  const float ks = p.k_scale[(p.k_per_head ? w.g * p.k_groups : 0) + ((16 * c) >> p.kg_shift)];
  const float cq = p.sm_scale * ks * kLog2e;
  float qf[RPG][16];
#pragma unroll
  for (int rr = 0; rr < RPG; ++rr) {
    // (every lane loads a valid row, the first one past the last, and
    // keeps zeros: no branch between the loads)
    const uint16_t* qrow = p.q + rows[rr].out_row * D + 16 * c;
    const u32x4 a = reinterpret_cast<const u32x4*>(qrow)[0];
    const u32x4 b = reinterpret_cast<const u32x4*>(qrow)[1];
    const uint32_t wv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    const float qs = rows[rr].valid ? cq : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qf[rr][2 * j] = bf16_lo(wv[j]) * qs;
      qf[rr][2 * j + 1] = bf16_hi(wv[j]) * qs;
    }
  }

  float m[RPG], lsum[RPG], acc[RPG][16];
  const bool sinks_here = p.sinks && p.direct;  // uniform
#pragma unroll
  for (int rr = 0; rr < RPG; ++rr) {
    const float raw = maybe_vload(p.sinks, rows[rr].h, sinks_here);
    const float sink2 = (sinks_here && rows[rr].valid) ? raw * kLog2e : -INFINITY;
    m[rr] = sink2;
    lsum[rr] = (kk == 0 && sink2 > -INFINITY) ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[rr][j] = 0.f;
  }

  // One tile's K/V (and block-scale) bytes of this lane's tokens.
  struct TileRegs {
    u32x4 kr[R], vr[R];
    // the block scale bytes of the lane's block of each token, four per word
    // (decoded where used: fewer live registers than one float per token)
    uint32_t ksw[(R + 3) / 4], vsw[(R + 3) / 4];
  };
  // (descriptor bases are wave-uniform: the page and the kv head; the lane's
  // token and chunk go into the per-lane offset)
  const uint8_t* khead = p.k_cache + (size_t)w.g * (size_t)p.head_stride;
  const uint8_t* vhead = p.v_cache + (size_t)w.g * (size_t)p.head_stride;
  auto load_grouped = [&](int tt, TileRegs& r, int odd) {
    const int kb = tt * kTileTokens;
    const int step = ((tt - ts) >> 1) & 63;
#pragma unroll
    for (int i = 0; i < (R + 3) / 4; ++i) r.ksw[i] = r.vsw[i] = 0u;
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
      const int grp = (rho * KPI) / 16;  // 16-token group of this round (constant)
      const int gk = kb + 16 * grp;
      const bool live = tt < te && gk < uhi && gk + 16 > ulo;
      const int page = __builtin_amdgcn_readlane(tab[2 * odd + grp], step);
      const size_t pbase = (size_t)page * (size_t)p.page_bytes;
      const size_t gbase = pbase + (size_t)(gk & p.bt_mask) * tok;
      const int key = kb + rho * KPI + kk;
      const bool in_span = key >= ulo && key < uhi;
      const uint32_t off = in_span ? uint32_t((key - gk) * tok + KWB * c) : kOob;
      const int nrec = live ? 16 * tok : 0;
      const Rsrc rk = __builtin_amdgcn_make_buffer_rsrc((void*)(khead + gbase), 0, nrec, kRsrcWord3);
      const Rsrc rv = __builtin_amdgcn_make_buffer_rsrc((void*)(vhead + gbase), 0, nrec, kRsrcWord3);
      if constexpr (NV) {
        uint32_t kd[2], vd[2];
        buf_load<8, AUX>(rk, off, kd);
        buf_load<8, AUX>(rv, off, vd);
        r.kr[rho] = u32x4{kd[0], kd[1], 0u, 0u};
        r.vr[rho] = u32x4{vd[0], vd[1], 0u, 0u};
      } else {
        uint32_t kd[4], vd[4];
        buf_load<16, AUX>(rk, off, kd);
        buf_load<16, AUX>(rv, off, vd);
        r.kr[rho] = u32x4{kd[0], kd[1], kd[2], kd[3]};
        r.vr[rho] = u32x4{vd[0], vd[1], vd[2], vd[3]};
      }
      if constexpr (NV || MX) {
        const int snrec = live ? 16 * p.sc_tok : 0;
        const size_t sbase = pbase + (size_t)p.sc_off + (size_t)w.g * (size_t)p.sc_head +
                             (size_t)(gk & p.bt_mask) * p.sc_tok;
        const Rsrc rks = __builtin_amdgcn_make_buffer_rsrc((void*)(p.k_cache + sbase), 0, snrec, kRsrcWord3);
        const Rsrc rvs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.v_cache + sbase), 0, snrec, kRsrcWord3);
        const uint32_t soff = in_span ? uint32_t((key - gk) * p.sc_tok + (MX ? c / 2 : c)) : kOob;
        uint32_t kb8, vb8;
        buf_load<1, 0>(rks, soff, &kb8);
        buf_load<1, 0>(rvs, soff, &vb8);
        r.ksw[rho / 4] |= (kb8 & 0xffu) << (8 * (rho % 4));
        r.vsw[rho / 4] |= (vb8 & 0xffu) << (8 * (rho % 4));
      }
    }
  };
  auto load_per_lane = [&](int tt, TileRegs& r) {
    const int kb = tt * kTileTokens;
#pragma unroll
    for (int i = 0; i < (R + 3) / 4; ++i) r.ksw[i] = r.vsw[i] = 0u;
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
      const int key = kb + rho * KPI + kk;
      r.kr[rho] = u32x4{0u, 0u, 0u, 0u};
      r.vr[rho] = u32x4{0u, 0u, 0u, 0u};
      if (tt < te && key >= ulo && key < uhi) {
        const int page = btab[key >> p.bt_shift];
        const size_t pbase = (size_t)page * (size_t)p.page_bytes;
        const size_t off = pbase + (size_t)(key & p.bt_mask) * tok;
        if constexpr (NV) {
          const u32x2 kd = *reinterpret_cast<const u32x2*>(kbase_g + off);
          const u32x2 vd = *reinterpret_cast<const u32x2*>(vbase_g + off);
          r.kr[rho] = u32x4{kd.x, kd.y, 0u, 0u};
          r.vr[rho] = u32x4{vd.x, vd.y, 0u, 0u};
        } else {
          r.kr[rho] = *reinterpret_cast<const u32x4*>(kbase_g + off);
          r.vr[rho] = *reinterpret_cast<const u32x4*>(vbase_g + off);
        }
        if constexpr (NV || MX) {
          const size_t soff = pbase + sc_lane + (size_t)(key & p.bt_mask) * p.sc_tok;
          r.ksw[rho / 4] |= uint32_t(p.k_cache[soff]) << (8 * (rho % 4));
          r.vsw[rho / 4] |= uint32_t(p.v_cache[soff]) << (8 * (rho % 4));
        }
      }
    }
  };
  auto scale_of = [&](const uint32_t* sw, int rho) {
    const uint32_t b = (sw[rho / 4] >> (8 * (rho % 4))) & 0xffu;
    return MX ? e8m0_to_f32(b) : __builtin_amdgcn_cvt_f32_fp8(int(b), 0);
  };
  auto compute_tile = [&](int tt, const TileRegs& r) {
    const int kb = tt * kTileTokens;
    float x[R][RPG];
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
      float kf[16];
      if constexpr (NV) {
        fp4x16_to_f32(u32x2{r.kr[rho].x, r.kr[rho].y}, kf);
      } else {
        const uint32_t kw[4] = {r.kr[rho].x, r.kr[rho].y, r.kr[rho].z, r.kr[rho].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(kw[j], false);
          const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(kw[j], true);
          kf[4 * j + 0] = lo.x;
          kf[4 * j + 1] = lo.y;
          kf[4 * j + 2] = hi.x;
          kf[4 * j + 3] = hi.y;
        }
      }
      const int key = kb + rho * KPI + kk;
#pragma unroll
      for (int rr = 0; rr < RPG; ++rr) {
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) d = fmaf(kf[j], qf[rr][j], d);
        if constexpr (NV || MX) d *= scale_of(r.ksw, rho);
#pragma unroll
        for (int s = 1; s < LPK; s <<= 1) d += xor_shfl(d, s);
        x[rho][rr] = (key >= rows[rr].klo && key < rows[rr].khi) ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int rr = 0; rr < RPG; ++rr) {
      float mx = x[0][rr];
#pragma unroll
      for (int rho = 1; rho < R; ++rho) mx = fmaxf(mx, x[rho][rr]);
#pragma unroll
      for (int s = LPK; s < 64; s <<= 1) mx = fmaxf(mx, xor_shfl(mx, s));
      const float mnew = fmaxf(m[rr], mx);
      const float muse = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = exp2_fast(m[rr] - muse);
      m[rr] = mnew;
      lsum[rr] *= alpha;
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[rr][j] *= alpha;
#pragma unroll
      for (int rho = 0; rho < R; ++rho) x[rho][rr] = exp2_fast(x[rho][rr] - muse);
    }
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
      float vf[16];
      if constexpr (NV) {
        fp4x16_to_f32(u32x2{r.vr[rho].x, r.vr[rho].y}, vf);
      } else {
        const uint32_t vw[4] = {r.vr[rho].x, r.vr[rho].y, r.vr[rho].z, r.vr[rho].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(vw[j], false);
          const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(vw[j], true);
          vf[4 * j + 0] = lo.x;
          vf[4 * j + 1] = lo.y;
          vf[4 * j + 2] = hi.x;
          vf[4 * j + 3] = hi.y;
        }
      }
#pragma unroll
      for (int rr = 0; rr < RPG; ++rr) {
        const float pp = x[rho][rr];
        lsum[rr] += pp;
        // (NVFP4: the block scale of V joins P; a key outside the span has
        // P = 0 and scale 0)
        const float pv = (NV || MX) ? pp * scale_of(r.vsw, rho) : pp;
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[rr][j] = fmaf(pv, vf[j], acc[rr][j]);
      }
    }
  };

  // Two tiles in flight where the registers allow (one query row, or head_dim
  // 64); with four rows at head_dim 128 or 256 a second tile's registers
  // would spill, so those load each tile before computing it.
  constexpr bool kTwoTiles = RPG == 1 || D == 64;
  if (grouped_pages && !kTwoTiles) {
    TileRegs ta;
    for (int tt = ts; tt < te; ++tt) {
      load_grouped(tt, ta, (tt - ts) & 1);
      compute_tile(tt, ta);
    }
  } else if (grouped_pages) {
    // two tiles in flight: tile t + 1 loads while tile t is computed
    TileRegs ta, tb;
    load_grouped(ts, ta, 0);
    load_grouped(ts + 1, tb, 1);
    for (int tt = ts; tt < te; tt += 2) {
      compute_tile(tt, ta);
      if (tt + 1 >= te) break;
      load_grouped(tt + 2, ta, 0);
      compute_tile(tt + 1, tb);
      load_grouped(tt + 3, tb, 1);
    }
  } else {
    TileRegs ta;
    for (int tt = ts; tt < te; ++tt) {
      load_per_lane(tt, ta);
      compute_tile(tt, ta);
    }
  }

  // reduce over the tokens of a round (lanes with equal c)
#pragma unroll
  for (int rr = 0; rr < RPG; ++rr) {
#pragma unroll
    for (int s = LPK; s < 64; s <<= 1) {
      lsum[rr] += xor_shfl(lsum[rr], s);
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[rr][j] += xor_shfl(acc[rr][j], s);
    }
  }
  if (kk != 0) return;
  const float vs = p.v_scale[p.v_per_head ? w.g : 0];
#pragma unroll
  for (int rr = 0; rr < RPG; ++rr) {
    if (!rows[rr].valid) continue;
    const bool empty = !(lsum[rr] > 0.f);
    const float inv = empty ? 0.f : vs / lsum[rr];
    const float lse = empty ? -INFINITY : (m[rr] + log2_fast(lsum[rr])) * kLn2;
    if (p.direct) {
      uint16_t* dst = p.out + rows[rr].out_row * D + 16 * c;
      uint32_t pk[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pk[j] = pack_bf16x2(acc[rr][2 * j] * inv, acc[rr][2 * j + 1] * inv);
      reinterpret_cast<u32x4*>(dst)[0] = u32x4{pk[0], pk[1], pk[2], pk[3]};
      reinterpret_cast<u32x4*>(dst)[1] = u32x4{pk[4], pk[5], pk[6], pk[7]};
      if (p.lse && c == 0) p.lse[rows[rr].out_row] = lse;
    } else {
      const size_t slot = rows[rr].out_row * p.num_splits + w.split;
      if (!empty) {
        float* dst = p.part_o + slot * D + 16 * c;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          reinterpret_cast<f32x4*>(dst)[v] = f32x4{acc[rr][4 * v] * inv, acc[rr][4 * v + 1] * inv,
                                                   acc[rr][4 * v + 2] * inv, acc[rr][4 * v + 3] * inv};
      }
      if (c == 0) p.part_lse[slot] = lse;
    }
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge: one wavefront per row, D/64 dims per lane.  Lane s
// loads the LSE of split s (64 splits per pass), the wave reduces their
// maximum, and each lane then accumulates its dims of the partial outputs,
// sixteen splits per step with the weights read from the owning lanes.  A split
// whose weight is 0 (LSE = -inf) is skipped by a select, so whatever its
// partial output holds (never written, possibly NaN) cannot leak.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

struct MergeArgs {
  int num_splits, num_rows, Hq;
  int rows_per_seq;  // B * q_len * Hq rows, q_len * Hq per sequence
  const float* po;
  const float* pl;
  const float* sinks;
  uint16_t* out;
  float* lse_out;
  // Optional: the splits each sequence got (slots 0 .. n - 1 of its rows hold
  // partials), written by the partial pass; nullptr: every row has num_splits.
  const int32_t* nsplit;
  FastDiv d_rps;  // rows_per_seq for fdiv
};

// The merge's kernel arguments in one batch of scalar loads, as for the
// partial kernels: the returned workgroup index orders the rest after them.
__device__ __forceinline__ int merge_args(const MergeArgs& a) {
  int blk = blockIdx.x;
  asm volatile("" : "+s"(blk)
               : "s"(a.num_splits), "s"(a.num_rows), "s"(a.Hq), "s"(a.po), "s"(a.pl), "s"(a.sinks),
                 "s"(a.out), "s"(a.lse_out), "s"(a.nsplit), "s"(a.rows_per_seq), "s"(a.d_rps.m),
                 "s"(a.d_rps.sh));
  __builtin_amdgcn_sched_barrier(0);
  return blk;
}

// One workgroup per (query row, 64 dims of head_dim); lane l owns dim
// 64 c + l.  Its W wavefronts take the splits in turn (wavefront w: splits
// w, w + W, ...) and reduce them to a local (max, sum, weighted sum), which
// LDS combines when W > 1: rows with many splits so need few dependent
// round trips.  Each wavefront issues the load of its row's split count,
// its first LSEs and its first 16 / W partial outputs together, before any
// of them is known (the plans fill slots from 0 upwards): rows of up to 16
// splits take one round trip; further splits are read only where their
// weight is nonzero (a ballot over the weights gives their indices, 16 at a
// time).
template <int D, int W>
__global__ __launch_bounds__(64 * W) void merge_kernel(MergeArgs a) {
  constexpr int C = D / 64;  // workgroups per row
  constexpr int U = 16;      // partial outputs in flight together per wavefront
  constexpr int U0 = 16 / W; // loaded before the split count and the weights are known
  __shared__ float red_acc[W][64];
  __shared__ float red_ml[W][2];
  const int blk = merge_args(a);
  const int row = blk / C;
  const int chunk = blk - row * C;
  const int lane = threadIdx.x & 63;
  const int wv = W == 1 ? 0 : __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int S = a.num_splits;
  // (issued first: the split count is the one value everything else waits
  // on; branch-free, so that no wait for it lands before the loads below)
  const bool has_ns = a.nsplit != nullptr;
  const int ns_raw = maybe_vload(a.nsplit, fdiv(row, a.d_rps), has_ns);
  const float* lrow = a.pl + (size_t)row * S;
  const float* obase = a.po + (size_t)row * S * D + 64 * chunk + lane;
  // lane i of this wavefront stands for split wv + W * (i0 + i).  The first
  // loads are branch-free (indices clamped to the row's slots, results
  // selected below), so they all issue before the first wait.
  const int sl0 = wv + W * lane;
  float l0 = lrow[min(sl0, S - 1)];
  float o0[U0];
#pragma unroll
  for (int u = 0; u < U0; ++u) o0[u] = obase[(size_t)min(wv + W * u, S - 1) * D];
  // (nothing below may be scheduled above this point: the split count is
  // the first value waited for)
  __builtin_amdgcn_sched_barrier(0);
  l0 = sl0 < S ? l0 : -INFINITY;
  // (the count is first touched here: without the asm the compiler would
  // clamp it above the loads, and wait for it there)
  int ns_v = ns_raw;
  asm volatile("" : "+v"(ns_v));
  // (clamped: a sequence's split count is at least 1 and at most num_splits)
  const int ns = __builtin_amdgcn_readfirstlane(has_ns ? min(max(ns_v, 1), S) : S);
  // this wavefront's splits: wv + W * i for i < nw
  const int nw = ns > wv ? (ns - wv + W - 1) / W : 0;
  float M = lane < nw ? l0 * kLog2e : -INFINITY;
  for (int i = 64 + lane; i < nw; i += 64) M = fmaxf(M, lrow[wv + W * i] * kLog2e);
  M = wave_reduce_f(M, [](float x, float y) { return fmaxf(x, y); });
  const float Mu = M == -INFINITY ? 0.f : M;  // every weight is 0 then
  float acc = 0.f, lpart = 0.f;
  for (int i0 = 0; i0 < nw; i0 += 64) {
    const int i = i0 + lane;
    const float ls = i0 == 0 ? l0 : (i < nw ? lrow[wv + W * i] : -INFINITY);
    const float w = i < nw ? exp2_fast(ls * kLog2e - Mu) : 0.f;
    lpart += w;
    uint64_t mask = __ballot(w > 0.f);
    if (i0 == 0) {
#pragma unroll
      for (int u = 0; u < U0; ++u) {
        const float wu = lane_value(w, u);
        acc = wu > 0.f ? fmaf(wu, o0[u], acc) : acc;
      }
      mask &= ~((uint64_t(1) << U0) - 1);
    }
    while (mask) {
      int idx[U];
      float o[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        idx[u] = mask ? __builtin_ctzll(mask) : -1;
        mask &= mask - 1;
        o[u] = idx[u] >= 0 ? obase[(size_t)(wv + W * (i0 + idx[u])) * D] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (idx[u] >= 0) acc = fmaf(lane_value(w, idx[u]), o[u], acc);
    }
  }
  lpart = wave_reduce_f(lpart, [](float x, float y) { return x + y; });
  if constexpr (W > 1) {
    red_acc[wv][lane] = acc;
    if (lane == 0) {
      red_ml[wv][0] = M;
      red_ml[wv][1] = lpart;
    }
    __syncthreads();
    if (wv != 0) return;
  }
  // combine: the sink joins once, in log2 units like the partial maxima
  const float sink2 = a.sinks ? a.sinks[row % a.Hq] * kLog2e : -INFINITY;
  float Mt = sink2, Lsum = 0.f, o = 0.f;
  if constexpr (W > 1) {
#pragma unroll
    for (int k = 0; k < W; ++k) Mt = fmaxf(Mt, red_ml[k][0]);
  } else {
    Mt = fmaxf(Mt, M);
  }
  const float Mtu = Mt == -INFINITY ? 0.f : Mt;
  if (sink2 > -INFINITY) Lsum = exp2_fast(sink2 - Mtu);
#pragma unroll
  for (int k = 0; k < W; ++k) {
    const float mk = W > 1 ? red_ml[k][0] : M;
    const float f = mk > -INFINITY ? exp2_fast(mk - Mtu) : 0.f;
    Lsum = fmaf(f, W > 1 ? red_ml[k][1] : lpart, Lsum);
    o = fmaf(f, W > 1 ? red_acc[k][lane] : acc, o);
  }
  const bool empty = !(Lsum > 0.f);
  const float inv = empty ? 0.f : 1.f / Lsum;
  a.out[(size_t)row * D + 64 * chunk + lane] = uint16_t(f32_to_bf16(o * inv));
  if (a.lse_out && chunk == 0 && lane == 0)
    a.lse_out[row] = empty ? -INFINITY : (Mtu + log2_fast(Lsum)) * kLn2;
}

// The same merge for many rows with few splits each (chunked prefill: tens
// of thousands of rows of 2-8 splits), where one wavefront per (row, 64
// dims) would need several dependent rounds of tiny workgroups: a wavefront
// takes 4 whole rows, 16 lanes each (D / 16 dims per lane), and issues the
// LSEs and partial outputs of a row's first U splits together with its
// split count, so a row of up to U splits takes one round trip; further
// splits follow in batches of U.  Splits past a row's count, read before the
// count is known, are dropped, and a zero weight never multiplies a partial
// (an empty split's payload may be anything).
template <int D>
__global__ __launch_bounds__(64) void merge_rows_kernel(MergeArgs a) {
  constexpr int VPL = D / 16;          // dims per lane
  constexpr int NV = VPL / 4;          // their float4s
  constexpr int U = D == 256 ? 4 : 8;  // splits per batch
  const int blk = merge_args(a);
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int row0 = blk * 4 + (lane >> 4);
  const bool valid = row0 < a.num_rows;
  const int row = valid ? row0 : a.num_rows - 1;
  const int S = a.num_splits;
  // (issued first: the split count is the one value everything else waits
  // on; branch-free, so that no wait for it lands before the loads below)
  const bool has_ns = a.nsplit != nullptr;
  const int ns_raw = maybe_vload(a.nsplit, fdiv(row, a.d_rps), has_ns);
  const float* lrow = a.pl + (size_t)row * S;
  const f32x4* orow = reinterpret_cast<const f32x4*>(a.po + (size_t)row * S * D + l16 * VPL);
  float lv[U];
  f32x4 ov[U][NV];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int sl = min(u, S - 1);
    lv[u] = lrow[sl];
#pragma unroll
    for (int v = 0; v < NV; ++v) ov[u][v] = orow[(size_t)sl * (D / 4) + v];
  }
  __builtin_amdgcn_sched_barrier(0);
  // (first touched here, as in merge_kernel)
  int ns_v = ns_raw;
  asm volatile("" : "+v"(ns_v));
  const int ns = has_ns ? min(max(ns_v, 1), S) : S;
  float M = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u) M = u < ns ? fmaxf(M, lv[u] * kLog2e) : M;
  for (int sl = U; sl < ns; ++sl) M = fmaxf(M, lrow[sl] * kLog2e);
  const float Mu = M == -INFINITY ? 0.f : M;  // every weight is 0 then
  float lpart = 0.f;
  f32x4 acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto take = [&](const float (&l)[U], const f32x4 (&o)[U][NV], int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = base + u < ns ? exp2_fast(l[u] * kLog2e - Mu) : 0.f;
      lpart += w;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[v][i] = w > 0.f ? fmaf(w, o[u][v][i], acc[v][i]) : acc[v][i];
      }
    }
  };
  take(lv, ov, 0);
  for (int base = U; base < ns; base += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sl = min(base + u, ns - 1);
      lv[u] = lrow[sl];
#pragma unroll
      for (int v = 0; v < NV; ++v) ov[u][v] = orow[(size_t)sl * (D / 4) + v];
    }
    take(lv, ov, base);
  }
  // combine: the sink joins once, in log2 units like the partial maxima
  const float sink2 = a.sinks ? a.sinks[row % a.Hq] * kLog2e : -INFINITY;
  const float Mt = fmaxf(sink2, M);
  const float Mtu = Mt == -INFINITY ? 0.f : Mt;
  const float f = M > -INFINITY ? exp2_fast(M - Mtu) : 0.f;
  const float Lsum = fmaf(f, lpart, sink2 > -INFINITY ? exp2_fast(sink2 - Mtu) : 0.f);
  const bool empty = !(Lsum > 0.f);
  const float inv = empty ? 0.f : 1.f / Lsum;
  if (!valid) return;
  uint32_t packed[VPL / 2];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    packed[2 * v] = pack_bf16x2(f * acc[v][0] * inv, f * acc[v][1] * inv);
    packed[2 * v + 1] = pack_bf16x2(f * acc[v][2] * inv, f * acc[v][3] * inv);
  }
  uint32_t* orow_out = reinterpret_cast<uint32_t*>(a.out + (size_t)row * D + l16 * VPL);
  if constexpr (VPL == 4) {
    *reinterpret_cast<u32x2*>(orow_out) = u32x2{packed[0], packed[1]};
  } else {
#pragma unroll
    for (int v = 0; v < VPL / 8; ++v)
      reinterpret_cast<u32x4*>(orow_out)[v] =
          u32x4{packed[4 * v], packed[4 * v + 1], packed[4 * v + 2], packed[4 * v + 3]};
  }
  if (a.lse_out && l16 == 0)
    a.lse_out[row] = empty ? -INFINITY : (Mtu + log2_fast(Lsum)) * kLn2;
}

// ---------------------------------------------------------------------------
// Diagnostics: the conversion instruction and the MFMA operand layout the
// kernels rely on.
// ---------------------------------------------------------------------------
__global__ void debug_e4m3_kernel(const uint8_t* codes, float* out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8(uint32_t(codes[i]), false);
  out[i] = v.x;
}

__global__ void debug_nvfp4_kernel(const uint8_t* data, const uint8_t* scales, float* out, int n) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  float f[16];
  fp4x16_to_f32(*reinterpret_cast<const u32x2*>(data + 8 * size_t(k)), f);
  const float sc = __builtin_amdgcn_cvt_f32_fp8(int(scales[k]), 0);
#pragma unroll
  for (int j = 0; j < 16; ++j) out[16 * size_t(k) + j] = f[j] * sc;
}

// MXFP8 block k (32 E4M3 codes and one E8M0 scale) as the bf16 operands the
// block-scaled MFMA kernel builds from it, widened back to float.
__global__ void debug_mxfp8_kernel(const uint8_t* data, const uint8_t* scales, float* out, int n) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= n) return;
  const float sc = e8m0_to_f32(scales[k]);
  const uint32_t* w = reinterpret_cast<const uint32_t*>(data + 32 * size_t(k));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x8 v = e4m3x8_to_bf16(w[2 * q], w[2 * q + 1], sc);
#pragma unroll
    for (int j = 0; j < 8; ++j) out[32 * size_t(k) + 8 * q + j] = float(v[j]);
  }
}

__global__ void debug_wave_ops_kernel(const int32_t* in, int vmax, int32_t* out) {
  const int lane = threadIdx.x & 63;
  const int v = in[lane];
  int tot = 0;
  out[lane] = wave_excl_prefix_i(v, vmax, tot);
  out[64 + lane] = wave_sum_i(v);
  out[128 + lane] = wave_max_i(v);
  out[192 + lane] = tot;
}

// One transposing LDS read per lane over a 4 KB copy of `src`; row
// addresses are clamped to 8-byte-aligned offsets inside the copy.
__global__ void debug_lds_tr8_kernel(const uint8_t* src, const int32_t* addr, uint8_t* out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4096];
  const int lane = threadIdx.x & 63;
  for (int i = lane; i < 4096 / 16; i += 64)
    reinterpret_cast<u32x4*>(lds)[i] = reinterpret_cast<const u32x4*>(src)[i];
  __syncthreads();
  const int a = min(max(addr[lane], 0), 4096 - 8) & ~7;
  const i32x2 t = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(lds + a));
  reinterpret_cast<u32x2*>(out)[lane] = u32x2{uint32_t(t.x), uint32_t(t.y)};
}

// One transposing 16-bit LDS read per lane over a 4 KB copy of `src`; row
// addresses are clamped to 8-byte-aligned offsets inside the copy.
__global__ void debug_lds_tr16_kernel(const uint8_t* src, const int32_t* addr, uint8_t* out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[4096];
  const int lane = threadIdx.x & 63;
  for (int i = lane; i < 4096 / 16; i += 64)
    reinterpret_cast<u32x4*>(lds)[i] = reinterpret_cast<const u32x4*>(src)[i];
  __syncthreads();
  const int a = min(max(addr[lane], 0), 4096 - 8) & ~7;
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(lds + a));
  reinterpret_cast<u32x2*>(out)[lane] =
      u32x2{uint32_t(uint16_t(t.x)) | (uint32_t(uint16_t(t.y)) << 16), uint32_t(uint16_t(t.z)) | (uint32_t(uint16_t(t.w)) << 16)};
}

// Streaming read of n16 16-byte units: workgroup x reads units
// [x per_wg, (x + 1) per_wg), four loads in flight per lane; the XOR of
// everything read is stored only in the impossible case that it equals a
// fixed word, which keeps the loads alive.
// W-byte loads (4, 8 or 16): the buffer is n W-byte words; a workgroup
// streams per_wg of them, 64 bytes per lane in flight whatever W is.
template <int W>
__global__ __launch_bounds__(256) void debug_read_kernel(const uint8_t* __restrict__ buf, uint64_t n,
                                                         uint64_t per_wg, uint32_t* sink) {
  using T = std::conditional_t<W == 16, u32x4, std::conditional_t<W == 8, u32x2, uint32_t>>;
  constexpr int U = 64 / W;
  const T* words = reinterpret_cast<const T*>(buf);
  const uint64_t base = uint64_t(blockIdx.x) * per_wg;
  const uint64_t end = base + per_wg < n ? base + per_wg : n;
  uint32_t acc = 0;
  for (uint64_t i = base + threadIdx.x; i < end; i += U * 256) {
    T v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t idx = i + uint64_t(u) * 256;
      v[u] = idx < end ? __builtin_nontemporal_load(&words[idx]) : T{};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (W == 16) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      else if constexpr (W == 8) acc ^= v[u].x ^ v[u].y;
      else acc ^= v[u];
    }
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

__global__ void debug_mfma_kernel(const uint8_t* a, const uint8_t* b, float* c) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, qd = lane >> 4;
  uint32_t aw[2], bw[2];
  for (int h = 0; h < 2; ++h) {
    uint32_t va = 0, vb = 0;
    for (int j = 0; j < 4; ++j) {
      va |= uint32_t(a[n * 32 + 8 * qd + 4 * h + j]) << (8 * j);   // A[m = n][k]
      vb |= uint32_t(b[(8 * qd + 4 * h + j) * 16 + n]) << (8 * j);  // B[k][n]
    }
    aw[h] = va;
    bw[h] = vb;
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(as_long(aw[0], aw[1]), as_long(bw[0], bw[1]), acc,
                                                   0, 0, 0);
  for (int i = 0; i < 4; ++i) c[(4 * qd + i) * 16 + n] = acc[i];
}

// One block-scaled 16x16x128 FP8 MFMA: lane (n, qd) = (l % 16, l / 16) holds
// bytes a[n][32 qd .. 32 qd + 31] of A, b[32 qd .. 32 qd + 31][n] of B, and
// the E8M0 byte a_scale[n][qd] as its A scale (B's scale is 1).
__global__ void debug_mfma_scale_kernel(const uint8_t* a, const uint8_t* a_scale, const uint8_t* b, float* c) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, qd = lane >> 4;
  i32x8 av, bv;
  for (int w = 0; w < 8; ++w) {
    uint32_t x = 0, y = 0;
    for (int j = 0; j < 4; ++j) {
      x |= uint32_t(a[n * 128 + 32 * qd + 4 * w + j]) << (8 * j);
      y |= uint32_t(b[(32 * qd + 4 * w + j) * 16 + n]) << (8 * j);
    }
    av[w] = int(x);
    bv[w] = int(y);
  }
  const int sa = int(a_scale[n * 4 + qd]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, sa, 0, 127);
  for (int i = 0; i < 4; ++i) c[(4 * qd + i) * 16 + n] = acc[i];
}

// ---------------------------------------------------------------------------
// Host helpers
// ---------------------------------------------------------------------------
std::atomic<int> g_cu_count[64];

int cu_count_of(int dev) {
  if (dev >= 0 && dev < 64) {
    const int v = g_cu_count[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1)
    return -1;
  if (dev >= 0 && dev < 64) g_cu_count[dev].store(c, std::memory_order_relaxed);
  return c;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

template <int D>
hipError_t launch_partial(const Plan& pl, const Params& prm, hipStream_t st) {
  const dim3 grid(pl.grid_wgs), block(64 * pl.hg * pl.ds);
  if (pl.variant == kVariantMfma && pl.fmt == FP8PA_KV_NVFP4) {
    if constexpr (D == 64)
      partial_mfma_nvfp4_kernel<64, FP8PA_KV_NVFP4, 0><<<grid, block, 0, st>>>(prm);
    else if constexpr (D == 128) {
      // (one-byte V scale loads: the whole-record form measured slower with
      // NVFP4's 8-byte records)
      if (pl.nt)
        partial_mfma_nvfp4_kernel<128, FP8PA_KV_NVFP4, 1><<<grid, block, 0, st>>>(prm);
      else
        partial_mfma_nvfp4_kernel<128, FP8PA_KV_NVFP4, 0><<<grid, block, 0, st>>>(prm);
    }
  } else if (pl.variant == kVariantMfma && pl.fmt == FP8PA_KV_MXFP8) {
    if constexpr (D == 64)
      partial_mfma_nvfp4_kernel<64, FP8PA_KV_MXFP8, 0><<<grid, block, 0, st>>>(prm);
    else if constexpr (D == 128) {
      // whole-record V scale loads where the records of consecutive tokens
      // are adjacent (head-major pages, or one kv head)
      const bool hv = prm.sc_tok == 128 / 32;
      if (pl.nt && hv)
        partial_mfma_nvfp4_kernel<128, FP8PA_KV_MXFP8, 1, true><<<grid, block, 0, st>>>(prm);
      else if (pl.nt)
        partial_mfma_nvfp4_kernel<128, FP8PA_KV_MXFP8, 1><<<grid, block, 0, st>>>(prm);
      else if (hv)
        partial_mfma_nvfp4_kernel<128, FP8PA_KV_MXFP8, 0, true><<<grid, block, 0, st>>>(prm);
      else
        partial_mfma_nvfp4_kernel<128, FP8PA_KV_MXFP8, 0><<<grid, block, 0, st>>>(prm);
    }
  } else if (pl.variant != kVariantMfma) {
    if (pl.fmt == FP8PA_KV_NVFP4)
      partial_dot_kernel<D, FP8PA_KV_NVFP4, kRowsDot><<<grid, block, 0, st>>>(prm);
    else if (pl.fmt == FP8PA_KV_MXFP8)
      partial_dot_kernel<D, FP8PA_KV_MXFP8, kRowsDot><<<grid, block, 0, st>>>(prm);
    else if (pl.rpg == 1 && pl.nt)
      partial_dot_kernel<D, FP8PA_KV_E4M3, 1, 1><<<grid, block, 0, st>>>(prm);
    else if (pl.rpg == 1)
      partial_dot_kernel<D, FP8PA_KV_E4M3, 1><<<grid, block, 0, st>>>(prm);
    else
      partial_dot_kernel<D, FP8PA_KV_E4M3, kRowsDot><<<grid, block, 0, st>>>(prm);
  } else if constexpr (D == 64) {
    // non-temporal loads only where a wavefront reads whole lines (paired heads)
    if (pl.lw == 8)
      partial_mfma_kernel<64, 1, 1, 1, 0, 8><<<grid, dim3(512), 0, st>>>(prm);
    else if (pl.lw == 4)
      partial_mfma_kernel<64, 1, 1, 1, 0, 4><<<grid, dim3(256), 0, st>>>(prm);
    else if (pl.lw == 2)
      partial_mfma_kernel<64, 1, 1, 1, 0, 2><<<grid, dim3(128), 0, st>>>(prm);
    else if (pl.pr == 2)
      partial_mfma_kernel<128, 1, 2, 1, 1, 0><<<grid, block, 0, st>>>(prm);
    else if (pl.nb == 2)
      partial_mfma_kernel<64, 1, 1, 2, 0, 0><<<grid, block, 0, st>>>(prm);
    else
      partial_mfma_kernel<64, 1, 1, 1, 0, 0><<<grid, block, 0, st>>>(prm);
  } else if constexpr (D == 128) {
    if (pl.lw == 8)
      partial_mfma_kernel<128, 1, 1, 1, 0, 8><<<grid, dim3(512), 0, st>>>(prm);
    else if (pl.lw == 4)
      partial_mfma_kernel<128, 1, 1, 1, 0, 4><<<grid, dim3(256), 0, st>>>(prm);
    else if (pl.lw == 2)
      partial_mfma_kernel<128, 1, 1, 1, 0, 2><<<grid, dim3(128), 0, st>>>(prm);
    else if (pl.nt)
      partial_mfma_kernel<128, 1, 1, 1, 1, 0><<<grid, block, 0, st>>>(prm);
    else
      partial_mfma_kernel<128, 1, 1, 1, 0, 0><<<grid, block, 0, st>>>(prm);
  } else {
    if (pl.nt)
      partial_mfma_kernel<256, 2, 1, 1, 1, 0><<<grid, block, 0, st>>>(prm);
    else
      partial_mfma_kernel<256, 2, 1, 1, 0, 0><<<grid, block, 0, st>>>(prm);
  }
  return hipGetLastError();
}

// Wavefronts per merge workgroup: one while the rows alone give each compute
// unit a few workgroups, four (splits of a row in parallel) for few rows.
// Wavefronts per (row, 64 dims) workgroup: 4 when the rows give fewer than 4
// workgroups per CU, 1 up to 32 per CU (one resident round), and beyond that
// 0: the many-rows kernel (4 whole rows per wavefront).
// The multiplier and shift for fdiv by d (d < 1 is taken as 1: such a
// divisor is never used).
FastDiv fast_div(int64_t d) {
  if (d < 1) d = 1;
  uint32_t l = 0;
  while ((int64_t(1) << l) < d) ++l;
  FastDiv f;
  f.sh = 31 + l;
  f.m = uint32_t(((uint64_t(1) << f.sh) + uint64_t(d) - 1) / uint64_t(d));
  return f;
}

int merge_waves(int64_t workgroups, int cu) {
  if (workgroups > 32 * int64_t(cu)) return 0;
  return workgroups >= 4 * int64_t(cu) ? 1 : 4;
}

template <int D>
void launch_merge_d(const MergeArgs& a, int waves, hipStream_t st) {
  const dim3 grid(unsigned(int64_t(a.num_rows) * (D / 64)));
  if (waves == 0)
    merge_rows_kernel<D><<<dim3(unsigned((a.num_rows + 3) / 4)), dim3(64), 0, st>>>(a);
  else if (waves == 1)
    merge_kernel<D, 1><<<grid, dim3(64), 0, st>>>(a);
  else
    merge_kernel<D, 4><<<grid, dim3(256), 0, st>>>(a);
}

hipError_t launch_merge(int D, const MergeArgs& a, int cu, hipStream_t st) {
  if (a.num_rows == 0) return hipSuccess;
  const int waves = merge_waves(int64_t(a.num_rows) * (D / 64), cu);
  switch (D) {
    case 64: launch_merge_d<64>(a, waves, st); break;
    case 128: launch_merge_d<128>(a, waves, st); break;
    default: launch_merge_d<256>(a, waves, st); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The allocation-free entry point's workspace: one static array per device,
// kScratchBytes long, that the code object brings with it.  Its name is a
// host-side stand-in in host code; the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever handed to a kernel.  Calls on one device share
// the array, so calls that overlap on one device race.  Nothing in it must
// start at zero: every byte a merge reads was written by the partial pass
// before it, in stream order.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(FP8PA_NOALLOC_SCRATCH_BYTES);
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// The device address of `dev`'s scratch array (dev must be current), or null
// when the runtime cannot give it.
void* scratch_of(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// Both decode entry points: `scratch_ptr` non-null means the workspace is
// the device's static scratch array (fp8pa_decode_noalloc), of which the
// plan may use at most kScratchBytes.
fp8pa_status decode_impl(const fp8pa_shape* shape, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_table,
                         const int32_t* seq_lens, const float* k_scale, const float* v_scale,
                         const float* sinks, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream, bool use_scratch) {
  if (!shape) return FP8PA_ERR_INVALID_ARG;
  Plan pl;
  fp8pa_status st = make_plan(shape, 1, &pl);  // shape checks before touching the GPU
  if (st != FP8PA_OK) return st;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !k_scale || !v_scale || !out)
    return FP8PA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(k_scale, 4) ||
      !aligned(v_scale, 4) || (sinks && !aligned(sinks, 4)) || (lse && !aligned(lse, 4)) ||
      (workspace && !aligned(workspace, kWorkspaceAlign)))
    return FP8PA_ERR_MISALIGNED;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8PA_ERR_HIP;
  const int cu = cu_count_of(dev);
  if (cu < 1) return FP8PA_ERR_HIP;
  st = make_plan(shape, cu, &pl);
  if (st != FP8PA_OK) return st;
  if (use_scratch) {
    if (pl.ws_bytes > kScratchBytes) return FP8PA_ERR_WORKSPACE_TOO_SMALL;
    if (pl.ws_bytes > 0) {
      workspace = scratch_of(dev);
      if (!workspace) return FP8PA_ERR_HIP;
      workspace_bytes = kScratchBytes;
    }
  }
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes))
    return FP8PA_ERR_WORKSPACE_TOO_SMALL;

  Params prm;
  prm.q = static_cast<const uint16_t*>(q);
  prm.k_cache = static_cast<const uint8_t*>(k_cache);
  prm.v_cache = static_cast<const uint8_t*>(v_cache);
  prm.block_table = block_table;
  prm.seq_lens = seq_lens;
  prm.k_scale = k_scale;
  prm.v_scale = v_scale;
  prm.sinks = sinks;
  prm.out = static_cast<uint16_t*>(out);
  prm.lse = lse;
  prm.part_o = pl.direct ? nullptr : static_cast<float*>(workspace);
  prm.part_lse =
      pl.direct ? nullptr : reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.off_lse);
  prm.page_bytes = pl.page_stride;
  const bool hnd = shape->kv_layout == FP8PA_LAYOUT_HND;
  // bytes per element row of a head: D codes, or D / 2 NVFP4 data bytes; and
  // the scale region's rows (NVFP4: D / 16 bytes, MXFP8: D / 32)
  const int32_t row = kv_data_row(pl.fmt, pl.D);
  const int32_t srow = kv_scale_row(pl.fmt, pl.D);
  prm.tok_stride = hnd ? row : pl.Hkv * row;
  prm.head_stride = hnd ? pl.bt * row : row;
  prm.sc_off = pl.Hkv * pl.bt * row;
  prm.sc_tok = hnd ? srow : pl.Hkv * srow;
  prm.sc_head = hnd ? pl.bt * srow : srow;
  // a group's tokens, plus with paired head-major heads the second head's
  prm.grp_bytes = (pl.pr == 2 && hnd) ? prm.head_stride + 16 * pl.D : 16 * prm.tok_stride;
  prm.q_len = pl.q_len;
  prm.Hq = pl.Hq;
  prm.Hkv = pl.Hkv;
  prm.G = pl.G;
  prm.rows = pl.rows;
  prm.row_groups = pl.row_groups;
  prm.B = pl.B;
  prm.hg = pl.hg;
  prm.upi = pl.upi;
  prm.num_splits = pl.num_splits;
  prm.tps = pl.tps;
  prm.tps_cap = pl.tps_cap;
  prm.balanced = pl.split_mode == FP8PA_SPLIT_BALANCED ? 1 : 0;
  prm.target_items = pl.target_items > 0 ? pl.target_items : 1;
  prm.max_seq_len = shape->max_seq_len;
  prm.min_tiles = pl.min_tiles;
  prm.nsplit_out =
      pl.direct ? nullptr : reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + pl.off_nsplit);
  prm.bt_shift = pl.bt_shift;
  prm.bt_mask = pl.bt - 1;
  prm.table_stride = shape->block_table_stride;
  prm.window = shape->window > 0 ? shape->window : 0;
  prm.k_groups = shape->k_groups > 1 ? shape->k_groups : 1;
  prm.kg_shift = k_group_shift(prm.k_groups, shape->head_dim);
  prm.k_per_head = shape->k_scale_count > prm.k_groups ? 1 : 0;
  prm.v_per_head = shape->v_scale_count > 1 ? 1 : 0;
  prm.direct = pl.direct;
  prm.ds = pl.ds;
  prm.pr = pl.pr;
  prm.sm_scale = shape->sm_scale;
  prm.d_upi = fast_div(prm.upi);
  prm.d_rg = fast_div(prm.row_groups);
  prm.d_G = fast_div(prm.G);
  prm.d_ns = fast_div(prm.num_splits);
  prm.d_ti = fast_div(prm.target_items);
  prm.d_slots = fast_div(int64_t(prm.target_items) + prm.B);

  const hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (pl.D) {
    case 64: e = launch_partial<64>(pl, prm, hs); break;
    case 128: e = launch_partial<128>(pl, prm, hs); break;
    default: e = launch_partial<256>(pl, prm, hs); break;
  }
  if (e != hipSuccess) return FP8PA_ERR_HIP;
  if (!pl.direct && !(shape->flags & FP8PA_FLAG_PARTIAL_ONLY)) {
    MergeArgs ma;
    ma.num_splits = pl.num_splits;
    ma.num_rows = pl.B * pl.q_len * pl.Hq;
    ma.Hq = pl.Hq;
    ma.po = prm.part_o;
    ma.pl = prm.part_lse;
    ma.sinks = sinks;
    ma.out = prm.out;
    ma.lse_out = lse;
    ma.nsplit = prm.nsplit_out;
    ma.rows_per_seq = pl.q_len * pl.Hq;
    ma.d_rps = fast_div(ma.rows_per_seq);
    e = launch_merge(pl.D, ma, cu, hs);
    if (e != hipSuccess) return FP8PA_ERR_HIP;
  }
  return FP8PA_OK;
}

}  // namespace
}  // namespace fp8pa

using namespace fp8pa;

extern "C" {

fp8pa_status fp8pa_workspace_bytes(const fp8pa_shape* shape, int device, size_t* bytes) {
  if (!shape || !bytes) return FP8PA_ERR_INVALID_ARG;
  Plan pl;
  fp8pa_status st = make_plan(shape, 1, &pl);
  if (st != FP8PA_OK) return st;
  const int cu = cu_count_of(device);
  if (cu < 1) return FP8PA_ERR_HIP;
  st = make_plan(shape, cu, &pl);
  if (st != FP8PA_OK) return st;
  *bytes = pl.ws_bytes;
  return FP8PA_OK;
}

fp8pa_status fp8pa_decode(const fp8pa_shape* shape, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* block_table,
                          const int32_t* seq_lens, const float* k_scale, const float* v_scale,
                          const float* sinks, void* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return decode_impl(shape, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, sinks,
                     out, lse, workspace, workspace_bytes, stream, false);
}

fp8pa_status fp8pa_decode_noalloc(const fp8pa_shape* shape, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const int32_t* seq_lens, const float* k_scale,
                                  const float* v_scale, const float* sinks, void* out, float* lse,
                                  void* stream) {
  return decode_impl(shape, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, sinks,
                     out, lse, nullptr, 0, stream, true);
}

fp8pa_status fp8pa_merge(int32_t num_splits, int32_t num_rows, int32_t num_q_heads,
                         int32_t head_dim, const float* partial_o, const float* partial_lse,
                         const float* sinks, void* out, float* lse, void* stream) {
  const fp8pa_status st = check_merge_args(num_splits, num_rows, num_q_heads, head_dim);
  if (st != FP8PA_OK) return st;
  if (!partial_o || !partial_lse || !out) return FP8PA_ERR_INVALID_ARG;
  if (!aligned(partial_o, 16) || !aligned(out, 16) || !aligned(partial_lse, 4) ||
      (sinks && !aligned(sinks, 4)) || (lse && !aligned(lse, 4)))
    return FP8PA_ERR_MISALIGNED;
  MergeArgs ma{};
  ma.num_splits = num_splits;
  ma.num_rows = num_rows;
  ma.Hq = num_q_heads;
  ma.po = partial_o;
  ma.pl = partial_lse;
  ma.sinks = sinks;
  ma.out = static_cast<uint16_t*>(out);
  ma.lse_out = lse;
  ma.nsplit = nullptr;  // every row merges all num_splits slots
  ma.rows_per_seq = 1;
  ma.d_rps = fast_div(1);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8PA_ERR_HIP;
  const int cu = cu_count_of(dev);
  if (cu < 1) return FP8PA_ERR_HIP;
  const hipError_t e = launch_merge(head_dim, ma, cu, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8PA_OK : FP8PA_ERR_HIP;
}

fp8pa_status fp8pa_debug_e4m3_to_f32(const uint8_t* codes, float* out, int32_t n, void* stream) {
  if (n < 0 || (n > 0 && (!codes || !out))) return FP8PA_ERR_INVALID_ARG;
  if (n == 0) return FP8PA_OK;
  debug_e4m3_kernel<<<dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      codes, out, n);
  return hipGetLastError() == hipSuccess ? FP8PA_OK : FP8PA_ERR_HIP;
}

fp8pa_status fp8pa_debug_mxfp8(const uint8_t* data, const uint8_t* scales, float* out, int32_t n,
                               void* stream) {
  if (n < 0 || (n > 0 && (!data || !scales || !out))) return FP8PA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(data) % 4 != 0) return FP8PA_ERR_MISALIGNED;
  if (n == 0) return FP8PA_OK;
  debug_mxfp8_kernel<<<dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      data, scales, out, n);
  return hipGetLastError() == hipSuccess ? FP8PA_OK : FP8PA_ERR_HIP;
}

fp8pa_status fp8pa_debug_nvfp4(const uint8_t* data, const uint8_t* scales, float* out, int32_t n,
                               void* stream) {
  if (n < 0 || (n > 0 && (!data || !scales || !out))) return FP8PA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(data) % 8 != 0) return FP8PA_ERR_MISALIGNED;
  if (n == 0) return FP8PA_OK;
  debug_nvfp4_kernel<<<dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      data, scales, out, n);
  return hipGetLastError() == hipSuccess ? FP8PA_OK : FP8PA_ERR_HIP;
}

fp8pa_status fp8pa_debug_fast_div(int64_t d, uint32_t* m, uint32_t* shift) {
  if (!m || !shift) return FP8PA_ERR_INVALID_ARG;
  const FastDiv f = fast_div(d);
  *m = f.m;
  *shift = f.sh;
  return FP8PA_OK;
}

fp8pa_status fp8pa_debug_wave_ops(const int32_t* in, int32_t vmax, int32_t* out, void* stream) {
  if (!in || !out || vmax < 0) return FP8PA_ERR_INVALID_ARG;
  debug_wave_ops_kernel<<<dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream)>>>(in, vmax, out);
  return hipGetLastError() == hipSuccess ? FP8PA_OK : FP8PA_ERR_HIP;
}

fp8pa_status fp8pa_debug_lds_tr8(const uint8_t* lds_bytes, const int32_t* row_addr, uint8_t* out,
                                 void* stream) {
  if (!lds_bytes || !row_addr || !out) return FP8PA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(lds_bytes) | reinterpret_cast<uintptr_t>(out)) & 15)
    return FP8PA_ERR_MISALIGNED;
  debug_lds_tr8_kernel<<<dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream)>>>(lds_bytes, row_addr, out);
  return hipGetLastError() == hipSuccess ? FP8PA_OK : FP8PA_ERR_HIP;
}

fp8pa_status fp8pa_debug_stream_read(const void* buf, uint64_t bytes, int32_t load_bytes, uint32_t* sink,
                                     void* stream) {
  if (!sink || (bytes > 0 && !buf)) return FP8PA_ERR_INVALID_ARG;
  if (bytes % 16 != 0) return FP8PA_ERR_INVALID_ARG;
  if (load_bytes != 4 && load_bytes != 8 && load_bytes != 16) return FP8PA_ERR_INVALID_ARG;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return FP8PA_ERR_MISALIGNED;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8PA_ERR_HIP;
  const int cu = cu_count_of(dev);
  if (cu < 1) return FP8PA_ERR_HIP;
  const uint64_t n = bytes / uint64_t(load_bytes);
  const unsigned grid = bytes == 0 ? 1u : unsigned(2 * cu);
  const uint64_t per_wg = (n + grid - 1) / grid;
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (load_bytes == 16)
    debug_read_kernel<16><<<dim3(grid), dim3(256), 0, st>>>(b, n, per_wg, sink);
  else if (load_bytes == 8)
    debug_read_kernel<8><<<dim3(grid), dim3(256), 0, st>>>(b, n, per_wg, sink);
  else
    debug_read_kernel<4><<<dim3(grid), dim3(256), 0, st>>>(b, n, per_wg, sink);
  return hipGetLastError() == hipSuccess ? FP8PA_OK : FP8PA_ERR_HIP;
}

fp8pa_status fp8pa_debug_lds_tr16(const uint8_t* lds_bytes, const int32_t* row_addr, uint8_t* out,
                                  void* stream) {
  if (!lds_bytes || !row_addr || !out) return FP8PA_ERR_INVALID_ARG;
  if (!aligned(lds_bytes, 16) || !aligned(out, 16) || !aligned(row_addr, 4)) return FP8PA_ERR_MISALIGNED;
  debug_lds_tr16_kernel<<<dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream)>>>(lds_bytes, row_addr, out);
  return hipGetLastError() == hipSuccess ? FP8PA_OK : FP8PA_ERR_HIP;
}

fp8pa_status fp8pa_debug_mfma_fp8(const uint8_t* a, const uint8_t* b, float* c, void* stream) {
  if (!a || !b || !c) return FP8PA_ERR_INVALID_ARG;
  debug_mfma_kernel<<<dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream)>>>(a, b, c);
  return hipGetLastError() == hipSuccess ? FP8PA_OK : FP8PA_ERR_HIP;
}

fp8pa_status fp8pa_debug_mfma_scale_fp8(const uint8_t* a, const uint8_t* a_scale, const uint8_t* b, float* c,
                                        void* stream) {
  if (!a || !a_scale || !b || !c) return FP8PA_ERR_INVALID_ARG;
  debug_mfma_scale_kernel<<<dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream)>>>(a, a_scale, b, c);
  return hipGetLastError() == hipSuccess ? FP8PA_OK : FP8PA_ERR_HIP;
}

const char* fp8pa_version(void) {
  return "fp8pa 0.1.0 (HIP, gfx950; FP8-MFMA and VALU partial kernels, E4M3, NVFP4 and MXFP8 pages, LSE merge)";
}

}  // extern "C"
