"""ctypes binding of libfp8pa.so: argument marshalling only.

Every computation runs in the library's HIP kernels.  If the library has not
been built (python -m decode_attention_paged_fp8pa_amd.build), loading it
raises; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8pa.so")

FP8PA_OK = 0
FP8PA_ERR_INVALID_ARG = 1
FP8PA_ERR_UNSUPPORTED = 2
FP8PA_ERR_WORKSPACE_TOO_SMALL = 3
FP8PA_ERR_MISALIGNED = 4
FP8PA_ERR_HIP = 5

FP8PA_FLAG_FORCE_DOT = 1
FP8PA_FLAG_FORCE_MFMA = 2
FP8PA_FLAG_PARTIAL_ONLY = 4
FP8PA_SPLIT_DIRECT = 0
FP8PA_SPLIT_FIXED = 1
FP8PA_SPLIT_BALANCED = 2
FP8PA_LAYOUT_NHD = 0
FP8PA_LAYOUT_HND = 1
FP8PA_KV_E4M3 = 0
FP8PA_KV_NVFP4 = 1
FP8PA_KV_MXFP8 = 2


class Fp8paError(RuntimeError):
    """A non-OK status returned by libfp8pa."""

    def __init__(self, status, where):
        self.status = int(status)
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class Shape(ctypes.Structure):
    """Mirror of fp8pa_shape (include/fp8pa.h)."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_tokens", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("block_table_stride", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("k_scale_count", ctypes.c_int32),
        ("v_scale_count", ctypes.c_int32),
        ("k_groups", ctypes.c_int32),
        ("kv_layout", ctypes.c_int32),
        ("kv_format", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("num_splits", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("kv_page_stride", ctypes.c_int64),
    ]


class WriteShape(ctypes.Structure):
    """Mirror of fp8pa_write_shape (include/fp8pa.h)."""

    _fields_ = [
        ("num_tokens", ctypes.c_int64),
        ("key_stride", ctypes.c_int64),
        ("value_stride", ctypes.c_int64),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_tokens", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("k_scale_count", ctypes.c_int32),
        ("v_scale_count", ctypes.c_int32),
        ("k_groups", ctypes.c_int32),
        ("kv_layout", ctypes.c_int32),
        ("kv_format", ctypes.c_int32),
        ("kv_page_stride", ctypes.c_int64),
    ]


class PlanInfo(ctypes.Structure):
    """Mirror of fp8pa_plan_info (include/fp8pa.h)."""

    _fields_ = [
        ("variant", ctypes.c_int32),
        ("split_mode", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("tiles_per_split", ctypes.c_int32),
        ("max_tiles_per_split", ctypes.c_int32),
        ("target_items", ctypes.c_int32),
        ("tile_tokens", ctypes.c_int32),
        ("heads_per_wg", ctypes.c_int32),
        ("waves_per_head", ctypes.c_int32),
        ("rows_per_group", ctypes.c_int32),
        ("row_groups", ctypes.c_int32),
        ("grid_wgs", ctypes.c_int32),
        ("merge_launched", ctypes.c_int32),
        ("heads_per_wave", ctypes.c_int32),
        ("row_blocks", ctypes.c_int32),
        ("nontemporal_kv", ctypes.c_int32),
        ("row_groups_per_wg", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_uint64),
        ("workspace_lse_offset", ctypes.c_uint64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None

_VP = ctypes.c_void_p
_SIGS = {
    "fp8pa_plan": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.POINTER(PlanInfo)]),
    "fp8pa_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_int,
                                             ctypes.POINTER(ctypes.c_size_t)]),
    "fp8pa_decode": (ctypes.c_int, [ctypes.POINTER(Shape), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                    _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    "fp8pa_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(Shape), _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                            _VP, _VP, _VP, _VP]),
    "fp8pa_merge": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   _VP, _VP, _VP, _VP, _VP, _VP]),
    "fp8pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fp8pa_version": (ctypes.c_char_p, []),
    "fp8pa_cache_write": (ctypes.c_int, [ctypes.POINTER(WriteShape), _VP, _VP, _VP, _VP, _VP, _VP,
                                         _VP, _VP]),
    "fp8pa_debug_e4m3_to_f32": (ctypes.c_int, [_VP, _VP, ctypes.c_int32, _VP]),
    "fp8pa_debug_stream_read": (ctypes.c_int, [_VP, ctypes.c_uint64, ctypes.c_int32, _VP, _VP]),
    "fp8pa_debug_lds_tr16": (ctypes.c_int, [_VP, _VP, _VP, _VP]),
    "fp8pa_debug_mfma_fp8": (ctypes.c_int, [_VP, _VP, _VP, _VP]),
    "fp8pa_debug_mfma_scale_fp8": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP]),
    "fp8pa_debug_wave_ops": (ctypes.c_int, [_VP, ctypes.c_int32, _VP, _VP]),
    "fp8pa_debug_fast_div": (ctypes.c_int, [ctypes.c_int64, ctypes.POINTER(ctypes.c_uint32),
                                            ctypes.POINTER(ctypes.c_uint32)]),
    "fp8pa_debug_nvfp4": (ctypes.c_int, [_VP, _VP, _VP, ctypes.c_int32, _VP]),
    "fp8pa_debug_lds_tr8": (ctypes.c_int, [_VP, _VP, _VP, _VP]),
    "fp8pa_debug_mxfp8": (ctypes.c_int, [_VP, _VP, _VP, ctypes.c_int32, _VP]),
}


def lib():
    """The loaded library (loaded once); raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m decode_attention_paged_fp8pa_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status):
    return lib().fp8pa_status_string(int(status)).decode()


def version():
    return lib().fp8pa_version().decode()


def _ptr(x):
    """Device address of a tensor (or an int address, or None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_shape(*, batch, q_len, num_q_heads, num_kv_heads, head_dim, block_tokens, num_blocks,
               block_table_stride, max_seq_len, k_scale_count=1, v_scale_count=1, k_groups=1,
               kv_layout=FP8PA_LAYOUT_NHD, kv_format=FP8PA_KV_E4M3, kv_page_stride=0, window=0,
               sm_scale, num_splits=0, flags=0) -> Shape:
    return Shape(batch=batch, q_len=q_len, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                 head_dim=head_dim, block_tokens=block_tokens, num_blocks=num_blocks,
                 block_table_stride=block_table_stride, max_seq_len=max_seq_len,
                 k_scale_count=k_scale_count, v_scale_count=v_scale_count, k_groups=k_groups,
                 kv_layout=kv_layout, kv_format=kv_format, kv_page_stride=int(kv_page_stride),
                 window=window, sm_scale=float(sm_scale), num_splits=num_splits, flags=flags)


def fp8pa_plan(shape: Shape, cu_count: int) -> dict:
    info = PlanInfo()
    st = lib().fp8pa_plan(ctypes.byref(shape), int(cu_count), ctypes.byref(info))
    if st != FP8PA_OK:
        raise Fp8paError(st, "fp8pa_plan")
    return info.as_dict()


def fp8pa_workspace_bytes(shape: Shape, device: int | None = None) -> int:
    if device is None:
        import torch

        device = torch.cuda.current_device()
    n = ctypes.c_size_t(0)
    st = lib().fp8pa_workspace_bytes(ctypes.byref(shape), int(device), ctypes.byref(n))
    if st != FP8PA_OK:
        raise Fp8paError(st, "fp8pa_workspace_bytes")
    return int(n.value)


def fp8pa_decode(shape: Shape, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale,
                 sinks, out, lse, workspace, workspace_bytes: int, stream=None) -> None:
    st = lib().fp8pa_decode(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                            _ptr(block_table), _ptr(seq_lens), _ptr(k_scale), _ptr(v_scale),
                            _ptr(sinks), _ptr(out), _ptr(lse), _ptr(workspace),
                            int(workspace_bytes), _stream(stream))
    if st != FP8PA_OK:
        raise Fp8paError(st, "fp8pa_decode")


def fp8pa_decode_noalloc(shape: Shape, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale,
                         sinks, out, lse, stream=None) -> None:
    st = lib().fp8pa_decode_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(block_table), _ptr(seq_lens), _ptr(k_scale), _ptr(v_scale),
                                    _ptr(sinks), _ptr(out), _ptr(lse), _stream(stream))
    if st != FP8PA_OK:
        raise Fp8paError(st, "fp8pa_decode_noalloc")


def fp8pa_merge(num_splits, num_rows, num_q_heads, head_dim, partial_o, partial_lse, sinks, out,
                lse, stream=None) -> None:
    st = lib().fp8pa_merge(int(num_splits), int(num_rows), int(num_q_heads), int(head_dim),
                           _ptr(partial_o), _ptr(partial_lse), _ptr(sinks), _ptr(out), _ptr(lse),
                           _stream(stream))
    if st != FP8PA_OK:
        raise Fp8paError(st, "fp8pa_merge")


def fp8pa_cache_write(shape: WriteShape, key, value, slot_mapping, k_scale, v_scale, k_cache,
                      v_cache, stream=None) -> None:
    st = lib().fp8pa_cache_write(ctypes.byref(shape), _ptr(key), _ptr(value), _ptr(slot_mapping),
                                 _ptr(k_scale), _ptr(v_scale), _ptr(k_cache), _ptr(v_cache),
                                 _stream(stream))
    if st != FP8PA_OK:
        raise Fp8paError(st, "fp8pa_cache_write")


def fp8pa_debug_e4m3_to_f32(codes, out, n, stream=None) -> None:
    st = lib().fp8pa_debug_e4m3_to_f32(_ptr(codes), _ptr(out), int(n), _stream(stream))
    if st != FP8PA_OK:
        raise Fp8paError(st, "fp8pa_debug_e4m3_to_f32")


def fp8pa_debug_stream_read(buf, nbytes, sink, stream=None, load_bytes=16) -> None:
    st = lib().fp8pa_debug_stream_read(_ptr(buf), int(nbytes), int(load_bytes), _ptr(sink), _stream(stream))
    if st != FP8PA_OK:
        raise Fp8paError(st, "fp8pa_debug_stream_read")


def fp8pa_debug_fast_div(d: int) -> tuple[int, int]:
    """(multiplier, shift) the kernels divide by d with (host only)."""
    m, sh = ctypes.c_uint32(), ctypes.c_uint32()
    st = lib().fp8pa_debug_fast_div(int(d), ctypes.byref(m), ctypes.byref(sh))
    if st != FP8PA_OK:
        raise Fp8paError(st, "fp8pa_debug_fast_div")
    return m.value, sh.value


def fp8pa_debug_wave_ops(inp, vmax, out, stream=None) -> None:
    st = lib().fp8pa_debug_wave_ops(_ptr(inp), int(vmax), _ptr(out), _stream(stream))
    if st != FP8PA_OK:
        raise Fp8paError(st, "fp8pa_debug_wave_ops")


def fp8pa_debug_nvfp4(data, scales, out, n, stream=None) -> None:
    st = lib().fp8pa_debug_nvfp4(_ptr(data), _ptr(scales), _ptr(out), int(n), _stream(stream))
    if st != FP8PA_OK:
        raise Fp8paError(st, "fp8pa_debug_nvfp4")


def fp8pa_debug_mxfp8(data, scales, out, n, stream=None) -> None:
    st = lib().fp8pa_debug_mxfp8(_ptr(data), _ptr(scales), _ptr(out), int(n), _stream(stream))
    if st != FP8PA_OK:
        raise Fp8paError(st, "fp8pa_debug_mxfp8")


def fp8pa_debug_lds_tr8(lds_bytes, row_addr, out, stream=None) -> None:
    st = lib().fp8pa_debug_lds_tr8(_ptr(lds_bytes), _ptr(row_addr), _ptr(out), _stream(stream))
    if st != FP8PA_OK:
        raise Fp8paError(st, "fp8pa_debug_lds_tr8")


def fp8pa_debug_lds_tr16(lds_bytes, row_addr, out, stream=None) -> None:
    st = lib().fp8pa_debug_lds_tr16(_ptr(lds_bytes), _ptr(row_addr), _ptr(out), _stream(stream))
    if st != FP8PA_OK:
        raise Fp8paError(st, "fp8pa_debug_lds_tr16")


def fp8pa_debug_mfma_scale_fp8(a, a_scale, b, c, stream=None) -> None:
    st = lib().fp8pa_debug_mfma_scale_fp8(_ptr(a), _ptr(a_scale), _ptr(b), _ptr(c), _stream(stream))
    if st != FP8PA_OK:
        raise Fp8paError(st, "fp8pa_debug_mfma_scale_fp8")


def fp8pa_debug_mfma_fp8(a, b, c, stream=None) -> None:
    st = lib().fp8pa_debug_mfma_fp8(_ptr(a), _ptr(b), _ptr(c), _stream(stream))
    if st != FP8PA_OK:
        raise Fp8paError(st, "fp8pa_debug_mfma_fp8")
