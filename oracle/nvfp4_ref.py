"""Plain definition of the NVFP4 KV-cache format: read side and writer.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Reference passages:

* [P4] Gist "Qwen3.8-27B ... 451K tokens of KV on a single RTX 5090": its
  stack table runs an NVFP4 KV cache in the head-major layout; the writer
  kernel `reshape_and_cache_nvfp4_kernel` stores each side of a page as a
  data region followed by a scale region ([K_data | K_scale | V_data |
  V_scale]); a head's row holds head_size / 2 data bytes (two 4-bit codes per
  byte) and head_size / 16 scale bytes (one per 16 elements); the elements
  are multiplied by fp32(1 / k_scale) (resp. v_scale) before quantization;
  the layout is head-major (head stride block_size * dim, token stride dim)
  or token-major (dim, num_heads * dim) in both regions.
* The 4-bit element code is OCP FP4 E2M1 (sign, two exponent bits with bias
  1, one mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6); the block scale is an
  E4M3 byte, decoded as in the decode oracle.

Readings of what the pages leave open, each the plainest one the rest supports:
* element 2 i of a block sits in the low nibble of its byte, 2 i + 1 in the
  high nibble;
* a value reads as E2M1(code) * E4M3(scale byte) * tensor scale (k_scale or
  v_scale, one per tensor or per kv head);
* the writer follows the quantizer the gist prints (`nvfp4_utils.cuh`,
  `cvt_warp_fp16_to_fp4`, NVFP4 path) with the global scale g = fp32(1 /
  scale) that `reshape_and_cache_nvfp4_kernel` passes it.  Per 16-element
  block of bf16 inputs x: the block maximum a = max|x| (of the inputs
  themselves); the block scale s = fp32(g * fp32(a * fp32(1 / 6))); the scale
  byte = E4M3 of s rounded to nearest even, saturating at 448 (s is never
  negative); the output factor r = fp32(1 / fp32(E4M3(byte) * fp32(1 / g)))
  when the byte decodes to a nonzero value, else 0; the codes = E2M1 of
  fp32(x * r), nearest with ties to the even code, saturating at 6 and
  keeping the sign bit of their fp32 value.  The page forms its reciprocals
  (of 6, of g and of the product) with an approximate instruction; here each
  is the correctly rounded fp32 quotient.  NaN inputs are outside the format.
"""

from __future__ import annotations

import numpy as np

from .fp8pa_ref import E4M3_TABLE
from .fp8pa_write_ref import e4m3_encode

#: fp32(1 / 6), the reciprocal the quantizer multiplies the block maximum by.
SIXTH = np.float32(np.float32(1.0) / np.float32(6.0))

__all__ = ["E2M1_TABLE", "e2m1_decode_code", "e2m1_encode", "nvfp4_side_bytes",
           "nvfp4_gather", "nvfp4_cache_write"]


def e2m1_decode_code(c: int) -> float:
    """Value of one E2M1 code: bit 3 sign, bits 2..1 exponent (bias 1), bit 0
    mantissa; exponent 0 is subnormal (m / 2)."""
    c = int(c) & 0xF
    sign = -1.0 if c & 0x8 else 1.0
    e = (c >> 1) & 0x3
    m = c & 0x1
    if e == 0:
        return sign * (m / 2.0)
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


#: float64 value of every E2M1 code, indexed by the 4-bit code.
E2M1_TABLE = np.array([e2m1_decode_code(c) for c in range(16)], dtype=np.float64)


def e2m1_encode(t) -> np.ndarray:
    """E2M1 codes of float64 numbers: the nearest of the 8 magnitudes, ties to
    the even code, saturating at 6; the code takes the sign bit of t."""
    t = np.asarray(t, dtype=np.float64)
    mags = E2M1_TABLE[:8]
    a = np.minimum(np.abs(t), 6.0)
    dist = np.abs(a[..., None] - mags)              # [..., 8]
    best = dist.min(axis=-1, keepdims=True)
    ties = dist == best
    # among the nearest codes pick the even one (at most two are nearest)
    idx = np.where(ties[..., ::2].any(axis=-1),
                   2 * np.argmax(ties[..., ::2], axis=-1),
                   2 * np.argmax(ties[..., 1::2], axis=-1) + 1)
    return (idx | np.where(np.signbit(t), 8, 0)).astype(np.uint8)


def nvfp4_side_bytes(num_kv_heads: int, block_tokens: int, head_dim: int) -> int:
    """Bytes of one side (K or V) of one page: data region then scale region."""
    return num_kv_heads * block_tokens * (head_dim // 2 + head_dim // 16)


def _offsets(pages, slots, g, num_kv_heads, block_tokens, head_dim, kv_layout):
    """(data row offset, scale row offset) inside the pool for each position."""
    data_row = head_dim // 2
    sc_row = head_dim // 16
    data_bytes = num_kv_heads * block_tokens * data_row
    if kv_layout == "HND":
        r = g * block_tokens + slots
    else:
        r = slots * num_kv_heads + g
    return r * data_row, data_bytes + r * sc_row


def nvfp4_gather(pool, block_table_row, g, ts, scale, num_kv_heads, block_tokens, head_dim,
                 kv_layout="NHD"):
    """Dequantised rows [len(ts), D] of kv head g of an NVFP4 pool (uint8
    [num_blocks, page_stride], each page beginning with its data region) at
    logical positions ts, times `scale` (one number or one per dim)."""
    pool = np.asarray(pool, dtype=np.uint8)
    ts = np.asarray(ts, dtype=np.int64)
    pages = np.asarray(block_table_row)[ts // block_tokens].astype(np.int64)
    slots = ts % block_tokens
    doff, soff = _offsets(pages, slots, g, num_kv_heads, block_tokens, head_dim, kv_layout)
    d = np.arange(head_dim)
    data = pool[pages[:, None], doff[:, None] + d // 2]             # [n, D] bytes
    codes = np.where(d % 2 == 0, data & 0xF, data >> 4)
    sc = pool[pages[:, None], soff[:, None] + d // 16]              # [n, D] scale bytes
    return E2M1_TABLE[codes] * E4M3_TABLE[sc] * np.asarray(scale, dtype=np.float64)


def nvfp4_cache_write(key_bits, value_bits, slot_mapping, k_scale, v_scale, k_pool, v_pool,
                      num_kv_heads, block_tokens, head_dim, kv_layout="NHD"):
    """Copies of the two NVFP4 pools (uint8 [num_blocks, page_stride]) with
    every token whose slot lies in [0, num_blocks * block_tokens) written
    (negative and larger slots are skipped); key_bits / value_bits are bf16
    bit patterns [T, Hkv, D]."""
    outs = []
    nb = np.asarray(k_pool).shape[0]
    for src_bits, scales, pool in ((key_bits, k_scale, k_pool), (value_bits, v_scale, v_pool)):
        out = np.array(pool, dtype=np.uint8, copy=True)
        sc = np.asarray(scales, dtype=np.float32).reshape(-1)
        vals = (np.asarray(src_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
        for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64).reshape(-1)):
            if slot < 0 or slot >= nb * block_tokens:
                continue
            page, off = int(slot) // block_tokens, int(slot) % block_tokens
            for h in range(num_kv_heads):
                g = np.float32(np.float32(1.0) / sc[h if sc.size > 1 else 0])  # the global scale
                inv_g = np.float32(np.float32(1.0) / g)
                x = vals[t, h, :]                                                 # [D] float32
                doff, soff = _offsets(np.array([page]), np.array([off]), h, num_kv_heads,
                                      block_tokens, head_dim, kv_layout)
                for blk in range(head_dim // 16):
                    xb = x[16 * blk: 16 * blk + 16]
                    a = np.float32(np.max(np.abs(xb)))
                    s = np.float32(g * np.float32(a * SIXTH))
                    sbyte = int(e4m3_encode(np.float64(s)))
                    sval = np.float32(E4M3_TABLE[sbyte])
                    r = np.float32(np.float32(1.0) / np.float32(sval * inv_g)) if sval != 0 else np.float32(0.0)
                    codes = e2m1_encode((xb * r).astype(np.float32).astype(np.float64))
                    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
                    out[page, int(doff[0]) + 8 * blk: int(doff[0]) + 8 * blk + 8] = packed
                    out[page, int(soff[0]) + blk] = sbyte
        outs.append(out)
    return outs[0], outs[1]
