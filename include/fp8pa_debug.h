/*
 * fp8pa_debug.h: diagnostic entry points of libfp8pa.  They expose the
 * hardware behaviour the decode kernels rely on, so a test can check it
 * against the definitions directly:
 *
 *  - the E4M3 decode done by gfx950's v_cvt_pk_f32_fp8, which must be the
 *    OCP "e4m3fn" variant named on the FlashInfer page
 *    `flashinfer.gemm.fp8_qkv_qknorm_rope` (Parameters: torch.float8_e4m3fn),
 *    not the FNUZ variant of earlier CDNA parts;
 *  - the operand and result lane layout of v_mfma_f32_16x16x32_fp8_fp8 that
 *    the decode kernels assume;
 *  - the wavefront-wide integer sum, maximum and prefix sum (DPP row ops,
 *    permlane swaps, ballot + mbcnt) with which the kernels size a batch's
 *    KV splits on the device;
 *  - the lane mapping of gfx950's transposing LDS read ds_read_b64_tr_b8,
 *    from which the kernels that share K/V tiles through LDS build PV's
 *    V^T operands.
 *
 * Same conventions as fp8pa.h: device pointers owned by the caller, work
 * queued on `stream` (a hipStream_t passed as void*), a status returned.
 */
#ifndef FP8PA_DEBUG_H_
#define FP8PA_DEBUG_H_

#include <stdint.h>

#include "fp8pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* out[i] = value of E4M3 code codes[i] as decoded by the hardware conversion
 * instruction, for i < n.  codes: uint8 [n]; out: float [n]. */
fp8pa_status fp8pa_debug_e4m3_to_f32(const uint8_t* codes, float* out, int32_t n, void* stream);

/* out[16 k + j] = element j of NVFP4 block k times its scale, for k < n, as
 * the VALU kernel decodes them: data is uint8 [n][8] (8-byte aligned; element
 * 2i in the low nibble of byte i), scales uint8 [n] E4M3, out float [16 n]. */
fp8pa_status fp8pa_debug_nvfp4(const uint8_t* data, const uint8_t* scales, float* out, int32_t n,
                               void* stream);

/* out[32 k + j] = element j of MXFP8 block k as the block-scaled MFMA kernel
 * dequantizes it (E4M3 code times 2^(scale - 127), rounded to bf16, which is
 * exact), for k < n: data is uint8 [n][32] (4-byte aligned), scales uint8
 * [n] E8M0, out float [32 n]. */
fp8pa_status fp8pa_debug_mxfp8(const uint8_t* data, const uint8_t* scales, float* out, int32_t n,
                               void* stream);

/* c = a x b for one 16x16x32 FP8 MFMA: a is E4M3 [16][32] (row-major, M x K),
 * b is E4M3 [32][16] (K x N), c is float [16][16] row-major.  The kernel
 * loads the operands and stores the result with the lane layout the decode
 * kernels use (lane l: A row l%16 and B column l%16, k = 8*(l/16) .. +7;
 * result rows 4*(l/16) + i, column l%16), so c equals the exact product only
 * if that layout is the hardware's. */
fp8pa_status fp8pa_debug_mfma_fp8(const uint8_t* a, const uint8_t* b, float* c, void* stream);

/* c = (a scaled) x b for one block-scaled 16x16x128 FP8 MFMA
 * (v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 operands): a is E4M3 [16][128]
 * (M x K), b is E4M3 [128][16] (K x N), a_scale is E8M0 [16][4], c is float
 * [16][16] row-major.  Lane l = 16 qd + n loads A row n, bytes 32 qd .. +31,
 * B column n, rows 32 qd .. +31, and a_scale[n][qd] as its A scale byte (B's
 * scale is 1); the result is stored with rows 4 qd + i, column n.  The GPU
 * test states which A elements each lane's scale multiplies. */
fp8pa_status fp8pa_debug_mfma_scale_fp8(const uint8_t* a, const uint8_t* a_scale, const uint8_t* b, float* c,
                                        void* stream);

/* The multiplier and shift the kernels divide by a host-known divisor with
 * (host only, no GPU): for d >= 1 (d < 1 is taken as 1), *m and *shift such
 * that n / d == (uint64_t)n * *m >> *shift for every 0 <= n < 2^31.  The
 * kernels take them for the workgroups per item, the row groups, the query
 * heads per kv head, the split slots and the merge's rows per sequence.
 * Returns FP8PA_ERR_INVALID_ARG for null outputs. */
fp8pa_status fp8pa_debug_fast_div(int64_t d, uint32_t* m, uint32_t* shift);

/* One wavefront of 64 lanes, lane l holding in[l] (int32 [64], each in
 * [0, vmax], vmax >= 0): out[l] = the exclusive prefix sum in[0] + ... +
 * in[l-1], out[64 + l] = the wavefront sum, out[128 + l] = the wavefront
 * maximum, out[192 + l] = the total the prefix routine reports.  out: int32
 * [256]. */
fp8pa_status fp8pa_debug_wave_ops(const int32_t* in, int32_t vmax, int32_t* out, void* stream);

/* One wavefront of 64 lanes over a 4 KB LDS copy of lds_bytes (uint8
 * [4096], 16-byte aligned): lane l performs one ds_read_b64_tr_b8 at LDS
 * offset row_addr[l] (int32 [64]; clamped to [0, 4088] and rounded down to a
 * multiple of 8) and stores its 8 result bytes at out[8 l .. 8 l + 7] (uint8
 * [512], 16-byte aligned).  The mapping the kernels rely on: with
 * l = 16 g + 8 h + c (c < 8, h < 2), out[8 l + t] =
 * lds_bytes[row_addr[16 g + 2 t + h] + c] for t < 8, i.e. each 16-lane group
 * transposes the 16 x 8-byte rows its lanes name. */
fp8pa_status fp8pa_debug_lds_tr8(const uint8_t* lds_bytes, const int32_t* row_addr, uint8_t* out,
                                 void* stream);

/* As fp8pa_debug_lds_tr8, with one ds_read_b64_tr_b16 per lane (16-bit
 * elements, four per lane): out[8 l .. 8 l + 7] holds lane l's four result
 * elements, little-endian.  The mapping the kernels rely on: with
 * l = 16 g + 4 h + c (c < 4, h < 4), element t of lane l is element c of the
 * 8-byte row named by lane 16 g + 4 t + h, for t < 4. */
fp8pa_status fp8pa_debug_lds_tr16(const uint8_t* lds_bytes, const int32_t* row_addr, uint8_t* out,
                                  void* stream);

/* One launch that reads `bytes` bytes of `buf` (16-byte aligned, bytes a
 * multiple of 16) and nothing else: two workgroups of 256 lanes per compute
 * unit, each streaming one contiguous chunk with non-temporal loads of
 * load_bytes (4, 8 or 16; else FP8PA_ERR_INVALID_ARG) each, 64 bytes in
 * flight per lane.  It is the practical ceiling of a kernel that must read
 * that many bytes from HBM in one launch (the benchmark times it at each
 * workload's KV byte count, and at each load width); bytes = 0 launches one
 * empty workgroup, the launch's own cost.  sink: one device uint32 the kernel
 * may write. */
fp8pa_status fp8pa_debug_stream_read(const void* buf, uint64_t bytes, int32_t load_bytes, uint32_t* sink,
                                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8PA_DEBUG_H_ */
