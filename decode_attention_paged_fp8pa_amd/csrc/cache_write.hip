// KV-cache writer: bf16 keys / values of new tokens -> E4M3 pages.
//
// The cache writer of the gist "Qwen3.8-27B ... 451K tokens of KV on a single
// RTX 5090" (kernel reshape_and_cache_nvfp4_kernel) takes a token's slot from
// slot_mapping (a negative slot is skipped), splits it into page and place in
// the page, and multiplies each element by the fp32 reciprocal of its scale
// before encoding; here the encoding is OCP E4M3 ("e4m3fn", the type the
// FlashInfer page `flashinfer.gemm.fp8_qkv_qknorm_rope` names), the format
// the decode kernels read.
//
// One thread converts 8 consecutive elements of one token row: a 16-byte
// bf16 load, four gfx950 v_cvt_pk_fp8_f32 conversions (round to nearest
// even), one 8-byte store.  Consecutive threads take consecutive chunks of a
// row, so both the reads and the writes of a token are contiguous.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/fp8pa.h"
#include "plan.h"

namespace fp8pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.f;
// fp32(1 / 6): the quantizer multiplies the block maximum by it.
constexpr float kSixth = 1.0f / 6.0f;

struct WriteParams {
  const uint16_t* src[2];   // key, value
  int64_t stride[2];        // elements between token rows
  const float* scale[2];
  int32_t per_head[2];      // 1: one set of scales per kv head
  int32_t groups[2];        // scales per head (K: k_groups along head_dim; V: 1)
  int32_t group_shift[2];   // log2 of the 8-element chunks per group
  uint8_t* cache[2];
  const int64_t* slots;
  int64_t num_tokens;
  int64_t chunks;           // num_tokens * chunks_per_token
  int64_t num_slots;        // num_blocks * bt
  int64_t page_bytes;       // bytes between pages of a pool
  int32_t chunks_per_token; // Hkv * D / 8
  int32_t chunks_per_head;  // D / 8
  int32_t token_bytes;      // bytes between token slots of a page: Hkv * D, or D head-major
  int32_t head_bytes;       // bytes between kv heads of a page: D, or bt * D head-major
  // NVFP4 / MXFP8 pages (token_bytes / head_bytes then count data-region bytes):
  int32_t sc_off;           // byte offset of a page's scale region
  int32_t sc_tok, sc_head;  // scale bytes between token slots / kv heads
  int64_t fp4_blocks;       // scale blocks to write: num_tokens * Hkv * D / (16 or 32)
  int32_t blocks_per_token; // Hkv * D / (16 or 32)
  int32_t blocks_per_head;  // D / (16 or 32)
  int32_t bt_shift, bt_mask;
};

// x * inv in fp32, kept NaN but saturated to +-448 (the encoding has no
// infinity; fminf / fmaxf would turn a NaN into a bound).
__device__ __forceinline__ float clamp_e4m3(float v) {
  return fabsf(v) > kE4M3Max ? copysignf(kE4M3Max, v) : v;
}
__device__ __forceinline__ float scaled(uint32_t bf16_bits, float inv) {
  return clamp_e4m3(__uint_as_float(bf16_bits << 16) * inv);
}

// Eight bf16 values (four dwords) -> eight E4M3 codes (two dwords).
__device__ __forceinline__ u32x2 encode8(u32x4 x, float inv) {
  uint32_t lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(scaled(x.x & 0xffffu, inv), scaled(x.x >> 16, inv), lo, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(scaled(x.y & 0xffffu, inv), scaled(x.y >> 16, inv), lo, true);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(scaled(x.z & 0xffffu, inv), scaled(x.z >> 16, inv), hi, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(scaled(x.w & 0xffffu, inv), scaled(x.w >> 16, inv), hi, true);
  return u32x2{lo, hi};
}

// blockIdx.y: 0 keys, 1 values.  Grid-stride over (token, 8-element chunk).
__global__ __launch_bounds__(256) void cache_write_kernel(WriteParams p) {
  const int kv = blockIdx.y;
  const uint16_t* src = p.src[kv];
  uint8_t* cache = p.cache[kv];
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < p.chunks;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t t = i / p.chunks_per_token;
    const int c = int(i - t * p.chunks_per_token);
    const int64_t slot = p.slots[t];
    if (slot < 0 || slot >= p.num_slots) continue;
    const int h = c / p.chunks_per_head;
    const int grp = (c - h * p.chunks_per_head) >> p.group_shift[kv];
    const float inv = 1.f / p.scale[kv][(p.per_head[kv] ? h * p.groups[kv] : 0) + grp];
    const u32x4 x = *reinterpret_cast<const u32x4*>(src + t * p.stride[kv] + 8 * int64_t(c));
    uint8_t* dst = cache + (slot >> p.bt_shift) * p.page_bytes +
                   int64_t(slot & p.bt_mask) * p.token_bytes + int64_t(h) * p.head_bytes +
                   8 * (c - h * p.chunks_per_head);
    *reinterpret_cast<u32x2*>(dst) = encode8(x, inv);
  }
}

// E2M1 code of t: nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 with ties to the
// even code (the midpoints 0.25, 1.25, 2.5, 5 go down, 0.75, 1.75, 3.5 up),
// saturating at 6, with t's sign bit.
__device__ __forceinline__ uint32_t e2m1_code(float t) {
  const float a = fabsf(t);
  const uint32_t c = a <= 0.25f   ? 0u
                     : a < 0.75f  ? 1u
                     : a <= 1.25f ? 2u
                     : a < 1.75f  ? 3u
                     : a <= 2.5f  ? 4u
                     : a < 3.5f   ? 5u
                     : a <= 5.0f  ? 6u
                                  : 7u;
  return c | ((__float_as_uint(t) >> 28) & 8u);
}

// NVFP4 writer: one thread per 16-element block of a head's row; blockIdx.y
// 0 keys, 1 values.  The steps of the quantizer the gist prints
// (nvfp4_utils.cuh, cvt_warp_fp16_to_fp4, NVFP4 path) with the global scale
// g = 1 / scale that reshape_and_cache_nvfp4_kernel gives it: block scale
// s = g * (max|x| * (1/6)), its E4M3 byte (saturating), then the codes E2M1
// of x * (1 / (E4M3(byte) * (1 / g))).  Every reciprocal here is the
// correctly rounded fp32 quotient (the page uses an approximate one).
__global__ __launch_bounds__(256) void cache_write_nvfp4_kernel(WriteParams p) {
  const int kv = blockIdx.y;
  const uint16_t* src = p.src[kv];
  uint8_t* cache = p.cache[kv];
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < p.fp4_blocks;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t t = i / p.blocks_per_token;
    const int bi = int(i - t * p.blocks_per_token);
    const int64_t slot = p.slots[t];
    if (slot < 0 || slot >= p.num_slots) continue;
    const int h = bi / p.blocks_per_head;
    const int blk = bi - h * p.blocks_per_head;
    const float g = __fdiv_rn(1.f, p.scale[kv][p.per_head[kv] ? h : 0]);
    const float inv_g = __fdiv_rn(1.f, g);
    const u32x4* x = reinterpret_cast<const u32x4*>(src + t * p.stride[kv] + 16 * int64_t(bi));
    const u32x4 x0 = x[0], x1 = x[1];
    const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    float y[16];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      y[2 * j] = __uint_as_float(w[j] << 16);
      y[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      amax = fmaxf(amax, fmaxf(fabsf(y[2 * j]), fabsf(y[2 * j + 1])));
    }
    // two separate fp32 products, in the page's order (s >= 0, so the clamp
    // at 448 is the saturating conversion)
    const float sc = fminf(__fmul_rn(g, __fmul_rn(amax, kSixth)), kE4M3Max);
    const uint32_t sbyte = __builtin_amdgcn_cvt_pk_fp8_f32(sc, 0.f, 0u, false) & 0xffu;
    const float sv = __builtin_amdgcn_cvt_f32_fp8(int(sbyte), 0);
    const float r = sv > 0.f ? __fdiv_rn(1.f, __fmul_rn(sv, inv_g)) : 0.f;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lo |= e2m1_code(__fmul_rn(y[j], r)) << (4 * j);
      hi |= e2m1_code(__fmul_rn(y[8 + j], r)) << (4 * j);
    }
    uint8_t* page = cache + (slot >> p.bt_shift) * p.page_bytes;
    const int64_t off = slot & p.bt_mask;
    *reinterpret_cast<u32x2*>(page + off * p.token_bytes + int64_t(h) * p.head_bytes + 8 * blk) =
        u32x2{lo, hi};
    page[p.sc_off + off * p.sc_tok + int64_t(h) * p.sc_head + blk] = uint8_t(sbyte);
  }
}

// MXFP8 writer: one thread per 32-element block of a head's row; blockIdx.y
// 0 keys, 1 values.  Per block (the OCP MX rule): y = x * (1 / scale); the
// shared exponent X = floor(log2(max|y|)) - 8 (E4M3's largest exponent),
// clamped to [-127, 127]; the scale byte X + 127; the codes E4M3(y * 2^-X),
// nearest with ties to even, saturated to +-448.
__global__ __launch_bounds__(256) void cache_write_mxfp8_kernel(WriteParams p) {
  const int kv = blockIdx.y;
  const uint16_t* src = p.src[kv];
  uint8_t* cache = p.cache[kv];
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < p.fp4_blocks;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t t = i / p.blocks_per_token;
    const int bi = int(i - t * p.blocks_per_token);
    const int64_t slot = p.slots[t];
    if (slot < 0 || slot >= p.num_slots) continue;
    const int h = bi / p.blocks_per_head;
    const int blk = bi - h * p.blocks_per_head;
    const float g = __fdiv_rn(1.f, p.scale[kv][p.per_head[kv] ? h : 0]);
    const u32x4* x = reinterpret_cast<const u32x4*>(src + t * p.stride[kv] + 32 * int64_t(bi));
    float y[32];
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 v = x[q];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[8 * q + 2 * j] = __uint_as_float(w[j] << 16) * g;
        y[8 * q + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u) * g;
        amax = fmaxf(amax, fmaxf(fabsf(y[8 * q + 2 * j]), fabsf(y[8 * q + 2 * j + 1])));
      }
    }
    // floor(log2(amax)) is amax's unbiased exponent (zero and subnormal
    // maxima fall below -126 and clamp to -127 with it)
    const int e = int((__float_as_uint(amax) >> 23) & 0xffu) - 127;
    const int X = min(max(e - 8, -127), 127);
    const float m = ldexpf(1.f, -X);  // an exact power of two
    uint32_t code[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t c = 0;
      c = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(y[4 * j] * m), clamp_e4m3(y[4 * j + 1] * m), c, false);
      c = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(y[4 * j + 2] * m), clamp_e4m3(y[4 * j + 3] * m), c, true);
      code[j] = c;
    }
    uint8_t* page = cache + (slot >> p.bt_shift) * p.page_bytes;
    const int64_t off = slot & p.bt_mask;
    u32x4* dst = reinterpret_cast<u32x4*>(page + off * p.token_bytes + int64_t(h) * p.head_bytes + 32 * blk);
    dst[0] = u32x4{code[0], code[1], code[2], code[3]};
    dst[1] = u32x4{code[4], code[5], code[6], code[7]};
    page[p.sc_off + off * p.sc_tok + int64_t(h) * p.sc_head + blk] = uint8_t(X + 127);
  }
}

bool aligned_to(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

int log2_exact(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return (1 << s) == v ? s : -1;
}

}  // namespace
}  // namespace fp8pa

using namespace fp8pa;

extern "C" fp8pa_status fp8pa_cache_write(const fp8pa_write_shape* s, const void* key,
                                          const void* value, const int64_t* slot_mapping,
                                          const float* k_scale, const float* v_scale,
                                          void* k_cache, void* v_cache, void* stream) {
  if (!s) return FP8PA_ERR_INVALID_ARG;
  if (s->num_tokens < 0 || s->num_kv_heads < 1 || s->num_blocks < 1) return FP8PA_ERR_INVALID_ARG;
  if (s->head_dim != 64 && s->head_dim != 128 && s->head_dim != 256) return FP8PA_ERR_UNSUPPORTED;
  const int bt_shift = log2_exact(s->block_tokens);
  if (s->block_tokens < 1 || s->block_tokens > 1024 || bt_shift < 0) return FP8PA_ERR_INVALID_ARG;
  const int64_t row = int64_t(s->num_kv_heads) * s->head_dim;
  if (s->key_stride < row || s->value_stride < row) return FP8PA_ERR_INVALID_ARG;
  if (s->key_stride % 8 != 0 || s->value_stride % 8 != 0) return FP8PA_ERR_MISALIGNED;
  if (!k_groups_ok(s->k_groups, s->head_dim)) return FP8PA_ERR_INVALID_ARG;
  if (s->kv_layout != FP8PA_LAYOUT_NHD && s->kv_layout != FP8PA_LAYOUT_HND) return FP8PA_ERR_INVALID_ARG;
  if (s->kv_format != FP8PA_KV_E4M3 && s->kv_format != FP8PA_KV_NVFP4 && s->kv_format != FP8PA_KV_MXFP8)
    return FP8PA_ERR_INVALID_ARG;
  const bool nv = s->kv_format == FP8PA_KV_NVFP4;
  const bool mx = s->kv_format == FP8PA_KV_MXFP8;
  if ((nv || mx) && s->k_groups > 1) return FP8PA_ERR_INVALID_ARG;
  if (s->kv_page_stride < 0) return FP8PA_ERR_INVALID_ARG;
  const int64_t page_stride =
      kv_page_stride_of(s->kv_page_stride, s->kv_format, s->block_tokens, s->num_kv_heads, s->head_dim);
  if (page_stride == 0) return FP8PA_ERR_INVALID_ARG;
  // block-scaled pages take 8- and 16-byte stores from each page's start
  if ((nv || mx) && page_stride % 16 != 0) return FP8PA_ERR_MISALIGNED;
  const int32_t kg = s->k_groups > 1 ? s->k_groups : 1;
  if ((s->k_scale_count != kg && s->k_scale_count != s->num_kv_heads * kg) ||
      (s->v_scale_count != 1 && s->v_scale_count != s->num_kv_heads))
    return FP8PA_ERR_INVALID_ARG;
  if (s->num_tokens == 0) return FP8PA_OK;
  if (!key || !value || !slot_mapping || !k_scale || !v_scale || !k_cache || !v_cache)
    return FP8PA_ERR_INVALID_ARG;
  if (!aligned_to(key, 16) || !aligned_to(value, 16) || !aligned_to(k_cache, 8) ||
      !aligned_to(v_cache, 8) || !aligned_to(slot_mapping, 8) || !aligned_to(k_scale, 4) ||
      !aligned_to(v_scale, 4))
    return FP8PA_ERR_MISALIGNED;
  const int64_t cpt = row / 8;
  if (s->num_tokens > (int64_t(1) << 40) / cpt) return FP8PA_ERR_UNSUPPORTED;

  WriteParams p;
  p.src[0] = static_cast<const uint16_t*>(key);
  p.src[1] = static_cast<const uint16_t*>(value);
  p.stride[0] = s->key_stride;
  p.stride[1] = s->value_stride;
  p.scale[0] = k_scale;
  p.scale[1] = v_scale;
  p.per_head[0] = s->k_scale_count > kg ? 1 : 0;
  p.per_head[1] = s->v_scale_count > 1 ? 1 : 0;
  p.groups[0] = kg;
  p.groups[1] = 1;
  p.group_shift[0] = k_group_shift(kg, s->head_dim) - 3;
  p.group_shift[1] = k_group_shift(1, s->head_dim) - 3;
  p.cache[0] = static_cast<uint8_t*>(k_cache);
  p.cache[1] = static_cast<uint8_t*>(v_cache);
  p.slots = slot_mapping;
  p.num_tokens = s->num_tokens;
  p.chunks = s->num_tokens * cpt;
  p.num_slots = int64_t(s->num_blocks) * s->block_tokens;
  p.page_bytes = page_stride;
  p.chunks_per_token = int32_t(cpt);
  p.chunks_per_head = s->head_dim / 8;
  const bool hnd = s->kv_layout == FP8PA_LAYOUT_HND;
  // bytes per element row of a head: D codes, or D / 2 NVFP4 data bytes; and
  // the scale region's rows (NVFP4: D / 16 bytes, MXFP8: D / 32)
  const int32_t erow = kv_data_row(s->kv_format, s->head_dim);
  const int32_t srow = kv_scale_row(s->kv_format, s->head_dim);
  p.token_bytes = hnd ? erow : s->num_kv_heads * erow;
  p.head_bytes = hnd ? s->block_tokens * erow : erow;
  p.sc_off = s->num_kv_heads * s->block_tokens * erow;
  p.sc_tok = hnd ? srow : s->num_kv_heads * srow;
  p.sc_head = hnd ? s->block_tokens * srow : srow;
  p.blocks_per_head = mx ? s->head_dim / 32 : s->head_dim / 16;
  p.blocks_per_token = s->num_kv_heads * p.blocks_per_head;
  p.fp4_blocks = s->num_tokens * p.blocks_per_token;
  p.bt_shift = bt_shift;
  p.bt_mask = s->block_tokens - 1;

  const int64_t work = (nv || mx) ? p.fp4_blocks : p.chunks;
  const int64_t blocks = (work + 255) / 256;
  const dim3 grid(unsigned(blocks < 4096 ? blocks : 4096), 2), block(256);
  if (nv)
    cache_write_nvfp4_kernel<<<grid, block, 0, static_cast<hipStream_t>(stream)>>>(p);
  else if (mx)
    cache_write_mxfp8_kernel<<<grid, block, 0, static_cast<hipStream_t>(stream)>>>(p);
  else
    cache_write_kernel<<<grid, block, 0, static_cast<hipStream_t>(stream)>>>(p);
  return hipGetLastError() == hipSuccess ? FP8PA_OK : FP8PA_ERR_HIP;
}
