"""Plain definition of the MXFP8 KV-cache format: read side and writer.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Reference passages:

* The `fish-scales-ops` README ("Rules worth knowing up front" and the
  feature table): its attention kernels take MXFP8 queries, keys and values
  with separate scale tensors, MXFP8 meaning blocks of 1 x 32 elements that
  share one power-of-two (UE8M0) scale, and its paged decode needs pages of a
  multiple of 32 tokens.
* The OCP Microscaling (MX) formats: an MXFP8 block is 32 E4M3 elements and
  one E8M0 scale byte s, which reads as 2^(s - 127) (0xFF is NaN); a block's
  shared exponent is floor(log2(max |x|)) minus the element format's largest
  exponent (8 for E4M3), and its elements are x / 2^exponent rounded to the
  element format.

Readings of what the pages leave open, each the plainest one the rest supports:
* K and V alike: blocks of 32 consecutive head_dim elements of one token and
  kv head (a cache receives a token's row at a time, so a block never spans
  tokens that are written apart);
* each side of a page is a data region (the E4M3 codes, in the head-major or
  token-major row order of the NVFP4 pages of the gist "Qwen3.8-27B ... on a
  single RTX 5090") followed by a scale region (D / 32 E8M0 bytes per row, in
  the same row order);
* a value reads as E4M3(code) * 2^(s - 127) * tensor scale (k_scale or
  v_scale, one per tensor or per kv head);
* the writer takes y = fp32(x * fp32(1 / scale)) per element; per block the
  shared exponent X = floor(log2(max |y|)) - 8, clamped to [-127, 127]
  (X = -127 for an all-zero block), the scale byte X + 127, and the codes
  E4M3(y * 2^-X) rounded to nearest even and saturated at +-448 (a block's
  largest element can reach 2^9 before saturation, as the MX rule allows).
  NaN inputs are outside the format.
"""

from __future__ import annotations

import math

import numpy as np

from .fp8pa_ref import E4M3_TABLE
from .fp8pa_write_ref import e4m3_encode

__all__ = ["e8m0_decode", "mxfp8_side_bytes", "mxfp8_gather", "mxfp8_cache_write"]

MX_BLOCK = 32
E4M3_EMAX = 8


def e8m0_decode(s) -> np.ndarray:
    """Value of E8M0 scale bytes: 2^(s - 127), NaN for 0xFF."""
    s = np.asarray(s, dtype=np.int64)
    v = np.ldexp(1.0, s - 127)
    return np.where(s == 0xFF, np.nan, v)


def mxfp8_side_bytes(num_kv_heads: int, block_tokens: int, head_dim: int) -> int:
    """Bytes of one side (K or V) of one page: data region then scale region."""
    return num_kv_heads * block_tokens * (head_dim + head_dim // MX_BLOCK)


def _offsets(slots, g, num_kv_heads, block_tokens, head_dim, kv_layout):
    """(data row offset, scale row offset) inside a page for each position."""
    sc_row = head_dim // MX_BLOCK
    data_bytes = num_kv_heads * block_tokens * head_dim
    if kv_layout == "HND":
        r = g * block_tokens + slots
    else:
        r = slots * num_kv_heads + g
    return r * head_dim, data_bytes + r * sc_row


def mxfp8_gather(pool, block_table_row, g, ts, scale, num_kv_heads, block_tokens, head_dim,
                 kv_layout="NHD"):
    """Dequantised rows [len(ts), D] of kv head g of an MXFP8 pool (uint8
    [num_blocks, page_stride], each page beginning with its data region) at
    logical positions ts, times `scale` (one number or one per dim)."""
    pool = np.asarray(pool, dtype=np.uint8)
    ts = np.asarray(ts, dtype=np.int64)
    pages = np.asarray(block_table_row)[ts // block_tokens].astype(np.int64)
    slots = ts % block_tokens
    doff, soff = _offsets(slots, g, num_kv_heads, block_tokens, head_dim, kv_layout)
    d = np.arange(head_dim)
    codes = pool[pages[:, None], doff[:, None] + d]                       # [n, D]
    sc = pool[pages[:, None], soff[:, None] + d // MX_BLOCK]              # [n, D]
    return E4M3_TABLE[codes] * e8m0_decode(sc) * np.asarray(scale, dtype=np.float64)


def shared_exponent(amax: float) -> int:
    """floor(log2(amax)) - 8, clamped to [-127, 127]; -127 for amax = 0."""
    if amax == 0.0:
        return -127
    x = math.floor(math.log2(amax))
    # log2 of a float64 can round up to the next integer just below a power of two
    if 2.0 ** x > amax:
        x -= 1
    elif 2.0 ** (x + 1) <= amax:
        x += 1
    return int(min(max(x - E4M3_EMAX, -127), 127))


def mxfp8_cache_write(key_bits, value_bits, slot_mapping, k_scale, v_scale, k_pool, v_pool,
                      num_kv_heads, block_tokens, head_dim, kv_layout="NHD"):
    """Copies of the two MXFP8 pools (uint8 [num_blocks, page_stride]) with
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
                g = np.float32(1.0) / sc[h if sc.size > 1 else 0]
                y = (vals[t, h, :] * g).astype(np.float32)                      # [D]
                doff, soff = _offsets(np.array([off]), h, num_kv_heads, block_tokens, head_dim,
                                      kv_layout)
                for blk in range(head_dim // MX_BLOCK):
                    yb = y[MX_BLOCK * blk: MX_BLOCK * (blk + 1)].astype(np.float64)
                    x = shared_exponent(float(np.max(np.abs(yb))))
                    scaled = np.clip(yb * 2.0 ** (-x), -448.0, 448.0)          # exact power of two
                    codes = e4m3_encode(scaled)
                    out[page, int(doff[0]) + MX_BLOCK * blk: int(doff[0]) + MX_BLOCK * (blk + 1)] = codes
                    out[page, int(soff[0]) + blk] = x + 127
        outs.append(out)
    return outs[0], outs[1]
