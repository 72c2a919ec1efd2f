"""Plain definition of the FP8 KV-cache writer: bf16 K/V -> E4M3 pages.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Reference passage:

* [P4] Gist "Qwen3.8-27B ... 451K tokens of KV on a single RTX 5090",
  kernel `reshape_and_cache_nvfp4_kernel`: one token at a time, the token's
  slot comes from `slot_mapping` and a negative slot means "skip"; the slot
  splits into `slot / block_size` (the page) and `slot % block_size` (the
  token's place in it); the kernel forms `1 / k_scale` (resp. `v_scale`) in
  fp32 and multiplies each key (value) element by it before encoding.  That
  page stores NVFP4; the same steps with an E4M3 encoding give the writer of
  the E4M3 cache the decode path reads (value = decode(code) * scale, the
  reading R2 of the decode oracle).
* [P2] FlashInfer API page `flashinfer.gemm.fp8_qkv_qknorm_rope`,
  Parameters: the FP8 type is `torch.float8_e4m3fn` (OCP E4M3 "FN": bias 7,
  largest finite value 448, no infinities, S.1111.111 is NaN).

Readings of what the pages leave open, each the plainest one the rest supports:
* rounding is to nearest, ties to even (the OCP default), and a finite
  value beyond the largest magnitude saturates to +-448 (the FN format has
  no infinity to round to); an infinite input saturates the same way; a NaN
  input gives a NaN code;
* the product x * (1 / scale) is formed in fp32 from the exact bf16 value,
  as the page's kernel does, and the encoding rounds that fp32 number;
* slots outside the cache (slot >= num_blocks * block_tokens) are skipped
  like negative ones;
* scales are one float per tensor or one per kv head, as in the decode; K
  scales may come in k_groups groups along head_dim, as the decode reads them.
"""

from __future__ import annotations

import numpy as np

__all__ = ["E4M3_MAX", "e4m3_encode", "cache_write"]

E4M3_MAX = 448.0


def _encode_one(x: float) -> int:
    """E4M3FN code of one float64 number: nearest value, ties to even,
    saturating at +-448, NaN -> 0x7F.  The sign of zero is kept."""
    if x != x:
        return 0x7F
    sign = 0x80 if np.signbit(x) else 0x00
    a = abs(x)
    if a >= E4M3_MAX:
        return sign | 0x7E
    if a < 2.0 ** -6:
        # subnormal range: multiples of 2^-9; a count of 8 is the smallest
        # normal number, whose code is 8 as well (exponent field 1, mantissa 0)
        q = int(np.round(a * 2.0 ** 9))  # numpy rounds halves to even
        return sign | q
    m, e = np.frexp(a)  # a = m * 2^e, m in [0.5, 1)
    e -= 1              # a = (2m) * 2^e, 2m in [1, 2)
    q = int(np.round((2.0 * m - 1.0) * 8.0))
    if q == 8:
        e += 1
        q = 0
    field = e + 7
    if field > 15 or (field == 15 and q == 7):
        return sign | 0x7E  # rounds past 448
    return sign | (field << 3) | q


def e4m3_encode(x) -> np.ndarray:
    """Element-wise E4M3FN codes (uint8) of an array of float64 numbers."""
    x = np.asarray(x, dtype=np.float64)
    flat = np.fromiter((_encode_one(float(v)) for v in x.ravel()), dtype=np.uint8, count=x.size)
    return flat.reshape(x.shape)


def cache_write(key_bits, value_bits, slot_mapping, k_scale, v_scale, k_cache, v_cache,
                k_groups=1, kv_layout="NHD"):
    """Returns copies of (k_cache, v_cache) [num_blocks, bt, Hkv, D] (uint8)
    with every token t whose slot is valid written: element (h, d) of token t
    becomes e4m3(fp32(x * fp32(1 / scale))), x the bf16 value of
    key_bits[t, h, d] (uint16 bit patterns, [T, Hkv, D]) and scale the one
    the decode reads for that element (K: per head_dim group when
    k_groups > 1, laid out as in the decode oracle's k_scale_of_head).  With
    kv_layout="HND" the pools are head-major, [num_blocks, Hkv, bt, D]."""
    k_out = np.array(k_cache, dtype=np.uint8, copy=True)
    v_out = np.array(v_cache, dtype=np.uint8, copy=True)
    assert kv_layout in ("NHD", "HND")
    hnd = kv_layout == "HND"
    if hnd:
        nb, hkv, bt, d = k_out.shape
    else:
        nb, bt, hkv, d = k_out.shape
    ks = np.asarray(k_scale, dtype=np.float32).reshape(-1)
    vs = np.asarray(v_scale, dtype=np.float32).reshape(-1)
    kg = max(1, int(k_groups))

    def scales_of(arr, groups, h):  # float32 [D]: the scale of each element of head h
        base = h * groups if arr.size > groups else 0
        return arr[base + np.arange(d) // (d // groups)]

    for src_bits, scales, groups, dst in ((key_bits, ks, kg, k_out), (value_bits, vs, 1, v_out)):
        src = np.asarray(src_bits, dtype=np.uint16)
        vals = (src.astype(np.uint32) << 16).view(np.float32)  # exact bf16 values
        for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64).reshape(-1)):
            if slot < 0 or slot >= nb * bt:
                continue
            page, off = int(slot) // bt, int(slot) % bt
            for h in range(hkv):
                inv = (np.float32(1.0) / scales_of(scales, groups, h)).astype(np.float32)
                prod = (vals[t, h, :] * inv).astype(np.float32)
                codes = e4m3_encode(prod.astype(np.float64))
                if hnd:
                    dst[page, h, off, :] = codes
                else:
                    dst[page, off, h, :] = codes
    return k_out, v_out
