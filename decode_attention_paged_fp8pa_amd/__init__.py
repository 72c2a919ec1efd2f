"""Paged flash-decode attention over an FP8 (E4M3) KV cache for MI355X.

The work is done by libfp8pa.so (hand-written gfx950 HIP kernels behind a
C ABI, include/fp8pa.h).  This package is a thin binding: `_lib` mirrors the
C entry points one to one (fp8pa_decode, fp8pa_workspace_bytes,
fp8pa_merge, fp8pa_plan, fp8pa_cache_write), `decode` below fills the shape
descriptor from torch tensors and allocates the outputs, and `cache_write`
does the same for the KV-cache writer.  PyTorch provides device
memory and streams only.
"""

from __future__ import annotations

import math

from ._lib import (  # noqa: F401
    FP8PA_FLAG_FORCE_DOT,
    FP8PA_FLAG_FORCE_MFMA,
    FP8PA_FLAG_PARTIAL_ONLY,
    FP8PA_KV_E4M3,
    FP8PA_KV_NVFP4,
    FP8PA_KV_MXFP8,
    FP8PA_LAYOUT_HND,
    FP8PA_LAYOUT_NHD,
    FP8PA_SPLIT_BALANCED,
    FP8PA_SPLIT_DIRECT,
    FP8PA_SPLIT_FIXED,
    Fp8paError,
    LIB_PATH,
    PlanInfo,
    Shape,
    WriteShape,
    fp8pa_cache_write,
    fp8pa_debug_e4m3_to_f32,
    fp8pa_debug_lds_tr8,
    fp8pa_debug_mxfp8,
    fp8pa_debug_mfma_fp8,
    fp8pa_debug_nvfp4,
    fp8pa_debug_wave_ops,
    fp8pa_decode,
    fp8pa_merge,
    fp8pa_plan,
    fp8pa_workspace_bytes,
    lib,
    make_shape,
    status_string,
    version,
)

__all__ = [
    "cache_write",
    "fp8pa_cache_write",
    "decode",
    "shape_for",
    "fp8pa_decode",
    "fp8pa_merge",
    "fp8pa_plan",
    "fp8pa_workspace_bytes",
    "Fp8paError",
    "FP8PA_FLAG_FORCE_DOT",
    "FP8PA_FLAG_FORCE_MFMA",
    "FP8PA_FLAG_PARTIAL_ONLY",
    "FP8PA_KV_E4M3",
    "FP8PA_KV_NVFP4",
    "FP8PA_KV_MXFP8",
    "FP8PA_LAYOUT_HND",
    "FP8PA_LAYOUT_NHD",
    "FP8PA_SPLIT_BALANCED",
    "FP8PA_SPLIT_DIRECT",
    "FP8PA_SPLIT_FIXED",
]


def _layout_code(kv_layout):
    if kv_layout in ("NHD", FP8PA_LAYOUT_NHD):
        return FP8PA_LAYOUT_NHD
    if kv_layout in ("HND", FP8PA_LAYOUT_HND):
        return FP8PA_LAYOUT_HND
    raise ValueError(f"kv_layout must be 'NHD' or 'HND', not {kv_layout!r}")


def _pool_dims(cache, layout):
    """(num_blocks, bt, Hkv, D) of a pool in the given layout code."""
    if layout == FP8PA_LAYOUT_HND:
        nb, Hkv, bt, D = cache.shape
    else:
        nb, bt, Hkv, D = cache.shape
    return nb, bt, Hkv, D


def _format_code(kv_format):
    if kv_format in ("e4m3", FP8PA_KV_E4M3):
        return FP8PA_KV_E4M3
    if kv_format in ("nvfp4", FP8PA_KV_NVFP4):
        return FP8PA_KV_NVFP4
    if kv_format in ("mxfp8", FP8PA_KV_MXFP8):
        return FP8PA_KV_MXFP8
    raise ValueError(f"kv_format must be 'e4m3', 'nvfp4' or 'mxfp8', not {kv_format!r}")


def shape_for(q, k_cache, block_table, k_scale, v_scale, *, window=0, sm_scale=None,
              max_seq_len, num_splits=0, flags=0, k_groups=1, kv_layout="NHD", kv_format="e4m3",
              num_kv_heads=None, block_tokens=None) -> Shape:
    """fp8pa_shape for tensors q [B, q_len, Hq, D] and k_cache [blocks, bt, Hkv, D]
    (kv_layout "NHD") or [blocks, Hkv, bt, D] ("HND"); with kv_format
    "nvfp4" or "mxfp8", k_cache is uint8 [blocks, page_bytes] (any row
    stride) and num_kv_heads / block_tokens give the page geometry."""
    B, q_len, Hq, D = q.shape
    layout = _layout_code(kv_layout)
    fmt = _format_code(kv_format)
    if fmt != FP8PA_KV_E4M3:
        if num_kv_heads is None or block_tokens is None or k_cache.dim() != 2:
            raise ValueError("block-scaled pools are [num_blocks, page_bytes]; pass num_kv_heads and "
                             "block_tokens")
        nb, bt, Hkv, Dk = k_cache.shape[0], int(block_tokens), int(num_kv_heads), D
        page_stride = k_cache.stride(0)
    else:
        nb, bt, Hkv, Dk = _pool_dims(k_cache, layout)
        page_stride = 0
    if Dk != D:
        raise ValueError(f"head_dim mismatch: q has {D}, cache has {Dk}")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    return make_shape(batch=B, q_len=q_len, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                      block_tokens=bt, num_blocks=nb, block_table_stride=block_table.stride(0),
                      max_seq_len=int(max_seq_len), k_scale_count=k_scale.numel(),
                      v_scale_count=v_scale.numel(), k_groups=int(k_groups), kv_layout=layout,
                      kv_format=fmt, kv_page_stride=page_stride, window=int(window),
                      sm_scale=sm_scale,
                      num_splits=int(num_splits), flags=int(flags))


def decode(q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, sinks=None, *,
           window=0, sm_scale=None, max_seq_len=None, num_splits=0, flags=0, out=None, lse=None,
           workspace=None, stream=None, k_groups=1, kv_layout="NHD", kv_format="e4m3",
           num_kv_heads=None, block_tokens=None):
    """Runs fp8pa_decode on torch device tensors; returns (out bf16, lse fp32).

    q bf16 [B, q_len, Hq, D]; k_cache, v_cache uint8 or float8_e4m3fn
    [num_blocks, bt, Hkv, D] (kv_layout "NHD", token-major pages) or
    [num_blocks, Hkv, bt, D] ("HND", head-major pages); block_table int32 [B, stride] (unit column
    stride); seq_lens int32 [B]; k_scale, v_scale float32 [1] or [Hkv] (with
    k_groups > 1, k_scale is [k_groups] or [Hkv, k_groups]: one scale per
    head_dim group);
    sinks float32 [Hq] or None.  max_seq_len should be given by callers that
    must not synchronise (it is read from seq_lens otherwise).  kv_format
    "nvfp4" or "mxfp8": k_cache / v_cache are uint8 [num_blocks, page_bytes]
    NVFP4 / MXFP8 pools (rows may be strided, e.g. views into interleaved
    [K page | V page] blocks) and num_kv_heads / block_tokens are required.
    """
    import torch

    if q.dtype != torch.bfloat16:
        raise ValueError("q must be bfloat16")
    nvfp4 = _format_code(kv_format) != FP8PA_KV_E4M3   # a block-scaled (paged-region) format
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise ValueError(f"{name} must hold E4M3 codes (uint8 or float8_e4m3fn)")
    if nvfp4 and (k_cache.dim() != 2 or k_cache.stride(1) != 1 or v_cache.stride() != k_cache.stride()
                  or v_cache.shape != k_cache.shape):
        raise ValueError("block-scaled pools must be equal uint8 [num_blocks, page_bytes] with unit "
                         "column stride")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be 2-D with unit column stride")
    dense = (("q", q), ("seq_lens", seq_lens), ("k_scale", k_scale), ("v_scale", v_scale))
    if not nvfp4:
        dense += (("k_cache", k_cache), ("v_cache", v_cache))
    for name, t in dense:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if max_seq_len is None:
        max_seq_len = max(1, int(seq_lens.max().item()))   # a batch of empty slots still plans
    shape = shape_for(q, k_cache, block_table, k_scale, v_scale, window=window, sm_scale=sm_scale,
                      max_seq_len=max_seq_len, num_splits=num_splits, flags=flags,
                      k_groups=k_groups, kv_layout=kv_layout, kv_format=kv_format,
                      num_kv_heads=num_kv_heads, block_tokens=block_tokens)
    B, q_len, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, q_len, Hq, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, q_len, Hq), dtype=torch.float32, device=q.device)
    nbytes = fp8pa_workspace_bytes(shape, q.device.index if q.device.index is not None else 0)
    if nbytes > 0 and (workspace is None or workspace.numel() * workspace.element_size() < nbytes):
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fp8pa_decode(shape, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, sinks, out,
                 lse, workspace if nbytes > 0 else None, ws_bytes if nbytes > 0 else 0, stream)
    return out, lse


def cache_write(key, value, slot_mapping, k_scale, v_scale, k_cache, v_cache, *, stream=None,
                k_groups=1, kv_layout="NHD", kv_format="e4m3", block_tokens=None):
    """Runs fp8pa_cache_write on torch device tensors (in place on the caches).

    key, value bf16 [T, Hkv, D] with unit stride inside a token row;
    slot_mapping int64 [T] (negative: skip); k_scale, v_scale float32 [1] or
    [Hkv] (k_scale [k_groups] or [Hkv, k_groups] with k_groups > 1);
    k_cache, v_cache uint8 or float8_e4m3fn [num_blocks, bt, Hkv, D]
    (kv_layout "NHD") or [num_blocks, Hkv, bt, D] ("HND"), contiguous; with
    kv_format "nvfp4" or "mxfp8", uint8 [num_blocks, page_bytes] NVFP4 / MXFP8
    pools (rows may be strided) and block_tokens required.
    """
    import torch

    for name, t in (("key", key), ("value", value)):
        if t.dtype != torch.bfloat16 or t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise ValueError(f"{name} must be bfloat16 [T, Hkv, D] with contiguous token rows")
    fmt = _format_code(kv_format)
    nvfp4 = fmt != FP8PA_KV_E4M3   # a block-scaled (paged-region) format
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise ValueError(f"{name} must be a uint8 or float8_e4m3fn pool")
        if nvfp4 and (t.dim() != 2 or t.stride(1) != 1):
            raise ValueError(f"{name}: block-scaled pools are uint8 [num_blocks, page_bytes]")
        if not nvfp4 and not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous E4M3 pool")
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous int64")
    T, Hkv, D = key.shape
    if tuple(value.shape) != (T, Hkv, D) or slot_mapping.numel() != T:
        raise ValueError("key, value and slot_mapping disagree on the token count or shape")
    layout = _layout_code(kv_layout)
    if nvfp4:
        if block_tokens is None or v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride():
            raise ValueError("block-scaled pools must match each other; pass block_tokens")
        nb, bt, page_stride = k_cache.shape[0], int(block_tokens), k_cache.stride(0)
    else:
        nb, bt, Hkv_c, D_c = _pool_dims(k_cache, layout)
        if (Hkv_c, D_c) != (Hkv, D) or tuple(v_cache.shape) != tuple(k_cache.shape):
            raise ValueError("cache shape does not match key / value")
        page_stride = 0
    shape = WriteShape(T, key.stride(0), value.stride(0), Hkv, D, bt, nb, k_scale.numel(),
                       v_scale.numel(), int(k_groups), layout, fmt, page_stride)
    fp8pa_cache_write(shape, key, value, slot_mapping, k_scale, v_scale, k_cache, v_cache, stream)
    return k_cache, v_cache
