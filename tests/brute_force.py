"""Brute-force twin of the oracle for tiny inputs (pure Python loops).

Written independently of oracle/: it decodes E4M3 through torch's
float8_e4m3fn dtype (a library routine), copies the pages into a contiguous
[seq, Hkv, D] layout first, and evaluates each attention row with scalar
loops and the math module.  Used only to pin the oracle on tiny shapes.
"""

from __future__ import annotations

import math

import numpy as np
import torch


def _codes_to_float(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _bf16_to_float(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def depage(cache: np.ndarray, table_row: np.ndarray, seq_len: int) -> np.ndarray:
    """Contiguous [seq_len, Hkv, D] codes of one sequence, page by page."""
    bt = cache.shape[1]
    rows = []
    for t in range(seq_len):
        rows.append(cache[int(table_row[t // bt]), t % bt])
    if not rows:
        return np.zeros((0,) + cache.shape[2:], dtype=cache.dtype)
    return np.stack(rows)


_FP4_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)   # OCP E2M1, codes 0..7


def depage_nvfp4(pool, table_row, seq_len, Hkv, bt, D, layout):
    """Contiguous float64 [seq_len, Hkv, D] (code value x block scale) of one
    sequence of an NVFP4 pool, one element at a time."""
    out = np.zeros((seq_len, Hkv, D))
    data_row, sc_row = D // 2, D // 16
    data_bytes = Hkv * bt * data_row
    for t in range(seq_len):
        page = int(table_row[t // bt])
        slot = t % bt
        for h in range(Hkv):
            row = h * bt + slot if layout == "HND" else slot * Hkv + h
            for d in range(D):
                byte = int(pool[page, row * data_row + d // 2])
                nib = (byte >> 4) if (d & 1) else (byte & 0xF)
                val = _FP4_MAGNITUDES[nib & 7] * (-1.0 if nib & 8 else 1.0)
                sbyte = np.array([pool[page, data_bytes + row * sc_row + d // 16]], dtype=np.uint8)
                out[t, h, d] = val * _codes_to_float(sbyte)[0]
    return out


def depage_mxfp8(pool, table_row, seq_len, Hkv, bt, D, layout):
    """Contiguous float64 [seq_len, Hkv, D] (E4M3 code value x 2^(scale - 127))
    of one sequence of an MXFP8 pool, one element at a time."""
    out = np.zeros((seq_len, Hkv, D))
    sc_row = D // 32
    data_bytes = Hkv * bt * D
    for t in range(seq_len):
        page = int(table_row[t // bt])
        slot = t % bt
        for h in range(Hkv):
            row = h * bt + slot if layout == "HND" else slot * Hkv + h
            for d in range(D):
                code = np.array([pool[page, row * D + d]], dtype=np.uint8)
                s = int(pool[page, data_bytes + row * sc_row + d // 32])
                out[t, h, d] = _codes_to_float(code)[0] * (math.nan if s == 255 else 2.0 ** (s - 127))
    return out


def brute_decode(wl, key_range=None, sinks="from_workload"):
    """Attention of every (b, i, h) row by plain loops; returns (out, lse)."""
    B, q_len, Hq, D = wl.q_bits.shape
    Hkv = wl.Hkv
    G = Hq // Hkv
    sk = wl.sinks if isinstance(sinks, str) else sinks
    q = _bf16_to_float(wl.q_bits)
    out = np.zeros((B, q_len, Hq, D))
    lse = np.zeros((B, q_len, Hq))
    kg = getattr(wl, "k_groups", 1)
    # K scale as a [heads or 1, k_groups] grid; dim d falls in column d * kg // D
    ks_grid = np.asarray(wl.k_scale, dtype=np.float64).reshape(-1, kg)
    vs_all = np.asarray(wl.v_scale, dtype=np.float64).reshape(-1)
    for b in range(B):
        L = int(wl.seq_lens[b])
        if getattr(wl, "kv_format", "e4m3") == "nvfp4":
            K = depage_nvfp4(wl.k_cache, wl.block_table[b], L, Hkv, wl.bt, D, wl.kv_layout)
            V = depage_nvfp4(wl.v_cache, wl.block_table[b], L, Hkv, wl.bt, D, wl.kv_layout)
        elif getattr(wl, "kv_format", "e4m3") == "mxfp8":
            K = depage_mxfp8(wl.k_cache, wl.block_table[b], L, Hkv, wl.bt, D, wl.kv_layout)
            V = depage_mxfp8(wl.v_cache, wl.block_table[b], L, Hkv, wl.bt, D, wl.kv_layout)
        else:
            K = _codes_to_float(depage(wl.k_cache, wl.block_table[b], L))
            V = _codes_to_float(depage(wl.v_cache, wl.block_table[b], L))
        for i in range(q_len):
            pos = L - q_len + i
            for h in range(Hq):
                g = h // G
                ks_row = ks_grid[g] if ks_grid.shape[0] > 1 else ks_grid[0]
                vs = vs_all[g] if vs_all.size > 1 else vs_all[0]
                keys = []
                for t in range(L):
                    if t > pos:
                        continue
                    if wl.window > 0 and t < pos - wl.window + 1:
                        continue
                    if key_range is not None and not (key_range[0] <= t < key_range[1]):
                        continue
                    keys.append(t)
                scores = []
                for t in keys:
                    acc = 0.0
                    for d in range(D):
                        acc += q[b, i, h, d] * (K[t, g, d] * ks_row[d * kg // D])
                    scores.append(wl.sm_scale * acc)
                terms = list(scores)
                if sk is not None:
                    terms.append(float(sk[h]))
                m = max(terms) if terms else -math.inf
                if m == -math.inf:
                    lse[b, i, h] = -math.inf
                    continue
                denom = sum(math.exp(x - m) for x in terms)
                for d in range(D):
                    acc = 0.0
                    for t, s in zip(keys, scores):
                        acc += math.exp(s - m) * (V[t, g, d] * vs)
                    out[b, i, h, d] = acc / denom
                lse[b, i, h] = m + math.log(denom)
    return out, lse
