"""Plain float64 definition of paged decode attention over an E4M3 KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Reference passages:

* [P1] "How do I run paged decode attention over an FP8 KV cache for a
  quantized MoE serving path, with sliding windows, attention sinks and a
  custom scale?" (cerinamroth.com solution record), fields `title` and
  `summary`: paged flash-decode over an E4M3 KV cache with sliding windows,
  attention sinks and a caller-supplied scale; field
  `install.environment.special_requirements`: grouped KV heads
  (`n_kv_heads`), queries in bf16/fp16.
* [P2] FlashInfer API page `flashinfer.gemm.fp8_qkv_qknorm_rope`,
  Parameters: the FP8 dtype is `torch.float8_e4m3fn` (OCP E4M3, "FN").
* [P4] Gist "Qwen3.8-27B ... 451K tokens of KV on a single RTX 5090",
  kernel `reshape_and_cache_nvfp4_kernel`: the cache writer multiplies by
  `1 / k_scale` before encoding, so a reader multiplies decoded codes by
  `k_scale`; a token slot splits into `slot / block_size` (page) and
  `slot % block_size` (offset inside the page).
* [P5] FlashInfer PR #5591 (Cake sparse-MLA hardening), Summary and the
  workspace commit: split-KV producers write partial O and partial LSE that
  one reducer merges.

Readings of points the pages leave open, each the plainest one the rest supports:
positions with q_len > 1 put query i at `seq_len - q_len + i`; a window W > 0
keeps the last W positions including the query's own; a sink is a per-head
logit in the units of `sm_scale * q.k` that joins the softmax denominator
with a zero value; the returned LSE is a natural log and includes the sink;
an empty attended set gives out = 0 and lse = -inf (no sink) or the sink.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "E4M3_TABLE",
    "e4m3_decode_code",
    "bf16_bits_to_f64",
    "k_scale_of_head",
    "attended_range",
    "decode",
    "merge",
]


def e4m3_decode_code(c: int) -> float:
    """Value of one OCP E4M3 ("e4m3fn") code, decoded from its bits [P2].

    Sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.  Exponent 0
    is subnormal (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN; the format
    has no infinities, so every other code is a finite normal number.
    """
    c = int(c) & 0xFF
    sign = -1.0 if (c >> 7) & 1 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (-6)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


#: float64 value of every E4M3 code, indexed by the code byte.
E4M3_TABLE = np.array([e4m3_decode_code(c) for c in range(256)], dtype=np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def attended_range(seq_len: int, q_len: int, i: int, window: int) -> tuple[int, int]:
    """Half-open key range [lo, hi) that query row i of a sequence attends.

    Query i sits at position pos = seq_len - q_len + i and sees keys
    t <= pos (causal among the draft rows); with a window W > 0 it also needs
    t >= pos - W + 1 (the last W positions, its own included) [P1 title].
    Positions below zero do not exist.
    """
    pos = int(seq_len) - int(q_len) + int(i)
    hi = min(pos + 1, int(seq_len))
    lo = 0
    if window > 0:
        lo = max(0, pos - int(window) + 1)
    hi = max(hi, 0)
    lo = min(lo, hi)
    return lo, hi


def _gather(cache: np.ndarray, block_table_row: np.ndarray, g: int, ts: np.ndarray,
            scale, kv_layout: str = "NHD") -> np.ndarray:
    """Dequantised rows [len(ts), D] of kv head g at logical positions ts.

    Token t of the sequence lives in page block_table_row[t // bt] at slot
    t % bt [P4 writer index arithmetic]; the value is decode(code) * scale [P4],
    `scale` one number or one per head_dim element.  A page is token-major
    ("NHD": [bt, Hkv, D]) or head-major ("HND": [Hkv, bt, D], [P4] gist,
    NVFP4 KV writer: head stride block_size * dim, token stride dim).  Only
    the table entries of the positions asked for are read.
    """
    hnd = kv_layout == "HND"
    bt = cache.shape[2] if hnd else cache.shape[1]
    pages = block_table_row[ts // bt].astype(np.int64)
    slots = ts % bt
    codes = cache[pages, g, slots, :] if hnd else cache[pages, slots, g, :]
    return E4M3_TABLE[codes] * np.asarray(scale, dtype=np.float64)


def k_scale_of_head(k_scale, g: int, D: int, k_groups: int = 1) -> np.ndarray:
    """The K scale of every head_dim element of kv head g, float64 [D].

    [P1 `special_requirements`]: K scales may come in k_groups in
    (1, 2, 4, 8, 16) groups along head_dim, head_dim / k_groups >= 32 (V
    keeps one).  Reading: group j covers dims [j D/k_groups, (j+1) D/k_groups);
    k_scale holds k_groups numbers (one set for all kv heads) or Hkv * k_groups
    numbers, kv head major ([Hkv][k_groups]).
    """
    ks = np.asarray(k_scale, dtype=np.float64).reshape(-1)
    kg = max(1, int(k_groups))
    per_head = ks.size > kg
    base = g * kg if per_head else 0
    return ks[base + np.arange(D) // (D // kg)]


def _softmax_rows(scores: np.ndarray, sink: float | None):
    """Exact softmax pieces of a score vector with an optional sink logit.

    Returns (weights for the scores, lse) where weights = e^(s - lse) and
    lse = ln(sum e^s + e^sink).  With no finite term, weights are 0 and
    lse = -inf (no sink) or the sink itself.
    """
    terms = list(scores.tolist())
    if sink is not None:
        terms_max = max(terms + [sink]) if terms else sink
    else:
        terms_max = max(terms) if terms else -math.inf
    if terms_max == -math.inf:
        return np.zeros_like(scores), (-math.inf if sink is None else float(sink))
    e = np.exp(scores - terms_max)
    denom = float(e.sum())
    if sink is not None:
        denom += math.exp(float(sink) - terms_max)
    return e / denom, terms_max + math.log(denom)


def decode(q_bits, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale,
           sinks=None, window=0, sm_scale=None, rows=None, key_range=None,
           key_chunk=16384, k_groups=1, kv_layout="NHD", kv_format="e4m3", num_kv_heads=None,
           block_tokens=None):
    """Reference paged decode attention [P1 title/summary], float64.

    Arguments (numpy arrays, as the library receives them):
      q_bits      uint16 [B, q_len, Hq, D]  bf16 bit patterns of the queries
      k_cache     uint8  [num_blocks, bt, Hkv, D]  E4M3 codes (token-major pages),
                  or [num_blocks, Hkv, bt, D] with kv_layout="HND" (head-major)
      v_cache     uint8  the same shape and layout as k_cache
                  (kv_format="nvfp4" / "mxfp8": uint8 [num_blocks,
                  page_stride] NVFP4 / MXFP8 pools, read by
                  nvfp4_ref.nvfp4_gather / mxfp8_ref.mxfp8_gather; num_kv_heads
                  and block_tokens then give the page geometry)
      block_table int32  [B, max_blocks]  page of each logical page index
      seq_lens    int32  [B]  tokens in each sequence, the q_len new ones included
      k_scale, v_scale  float32 [1] (per tensor) or [Hkv] (per kv head); with
                  k_groups > 1, k_scale is [k_groups] or [Hkv, k_groups]
                  (see k_scale_of_head)
      sinks       float32 [Hq] or None  per-head sink logits
      window      int, <= 0 for none
      sm_scale    float, the softmax scale (default 1/sqrt(D))
      rows        optional list of (b, i, h): compute only these rows
      key_range   optional (lo, hi): restrict every row to keys in [lo, hi)
                  (a split-KV partial; used with sinks=None)

    For every row: g = h // (Hq / Hkv); s_t = sm_scale * sum_d q[d] * K[t, d]
    over the attended keys t; out = sum_t softmax(s, sink)_t * V[t];
    lse = ln(sum_t e^{s_t} + e^{sink}).

    Returns (out float64 [B, q_len, Hq, D], lse float64 [B, q_len, Hq]), or
    with `rows`, (out [len(rows), D], lse [len(rows)]).
    """
    q_bits = np.asarray(q_bits)
    B, q_len, Hq, D = q_bits.shape
    assert kv_layout in ("NHD", "HND") and kv_format in ("e4m3", "nvfp4", "mxfp8")
    if kv_format in ("nvfp4", "mxfp8"):
        from .mxfp8_ref import mxfp8_gather
        from .nvfp4_ref import nvfp4_gather
        Hkv = int(num_kv_heads)
        blocked = nvfp4_gather if kv_format == "nvfp4" else mxfp8_gather

        def gather(cache, row, g, ts, scale, layout):
            return blocked(cache, row, g, ts, scale, Hkv, int(block_tokens), D, layout)
    else:
        Hkv = k_cache.shape[1] if kv_layout == "HND" else k_cache.shape[2]
        gather = _gather
    assert Hq % Hkv == 0, "Hq must be a multiple of Hkv"
    G = Hq // Hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    k_scale = np.asarray(k_scale, dtype=np.float64).reshape(-1)
    v_scale = np.asarray(v_scale, dtype=np.float64).reshape(-1)
    seq_lens = np.asarray(seq_lens).reshape(-1)
    block_table = np.asarray(block_table)

    if rows is None:
        want = [(b, i, h) for b in range(B) for i in range(q_len) for h in range(Hq)]
    else:
        want = [tuple(int(x) for x in r) for r in rows]

    # Group the requested rows by (b, g) so each kv head's keys are gathered once.
    groups: dict[tuple[int, int], list[int]] = {}
    for n, (b, i, h) in enumerate(want):
        groups.setdefault((b, h // G), []).append(n)

    out = np.zeros((len(want), D), dtype=np.float64)
    lse = np.full((len(want),), -math.inf, dtype=np.float64)

    for (b, g), members in groups.items():
        L = int(seq_lens[b])
        ks = k_scale_of_head(k_scale, g, D, k_groups)
        vs = float(v_scale[g if v_scale.size > 1 else 0])
        ranges = []
        for n in members:
            _, i, _ = want[n]
            lo, hi = attended_range(L, q_len, i, window)
            if key_range is not None:
                lo, hi = max(lo, key_range[0]), min(hi, key_range[1])
                hi = max(hi, lo)
            ranges.append((lo, hi))
        u_lo = min(r[0] for r in ranges)
        u_hi = max(r[1] for r in ranges)
        qmat = np.stack([bf16_bits_to_f64(q_bits[want[n][0], want[n][1], want[n][2]])
                         for n in members])  # [R, D]
        # Pass 1: every score of the union range (keys of a chunk at a time).
        n_keys = max(u_hi - u_lo, 0)
        scores = np.empty((len(members), n_keys), dtype=np.float64)
        for c0 in range(u_lo, u_hi, key_chunk):
            ts = np.arange(c0, min(c0 + key_chunk, u_hi))
            kf = gather(k_cache, block_table[b], g, ts, ks, kv_layout)
            scores[:, c0 - u_lo:c0 - u_lo + len(ts)] = sm_scale * (qmat @ kf.T)
        # Pass 2: exact softmax weights of each row over its own key range.
        weights = np.zeros_like(scores)
        for j, n in enumerate(members):
            lo, hi = ranges[j]
            h = want[n][2]
            sink = None if sinks is None else float(np.asarray(sinks).reshape(-1)[h])
            w, row_lse = _softmax_rows(scores[j, lo - u_lo:hi - u_lo], sink)
            weights[j, lo - u_lo:hi - u_lo] = w
            lse[n] = row_lse
        # Pass 3: weighted sum of V, a chunk of keys at a time.
        acc = np.zeros((len(members), D), dtype=np.float64)
        for c0 in range(u_lo, u_hi, key_chunk):
            ts = np.arange(c0, min(c0 + key_chunk, u_hi))
            wchunk = weights[:, c0 - u_lo:c0 - u_lo + len(ts)]
            # Rows whose weights are all zero on this chunk need no V rows.
            live = np.flatnonzero(wchunk.any(axis=0))
            if live.size == 0:
                continue
            vf = gather(v_cache, block_table[b], g, ts[live], vs, kv_layout)
            acc += wchunk[:, live] @ vf
        for j, n in enumerate(members):
            out[n] = acc[j]

    if rows is not None:
        return out, lse
    return out.reshape(B, q_len, Hq, D), lse.reshape(B, q_len, Hq)


def merge(partial_o, partial_lse, sinks=None):
    """Merge split-KV partials with the log-sum-exp rule [P5 Summary].

    partial_o [R, S, D] holds each split's normalised output over a disjoint
    key range, partial_lse [R, S] its natural-log LSE (-inf for an empty
    split), sinks [R] an optional per-row sink logit added once.  With
    M = max(lse_s, sink): w_s = e^(lse_s - M), L = sum w_s + e^(sink - M),
    out = sum w_s o_s / L, lse = M + ln L; when every term is -inf the
    result is out = 0, lse = -inf.
    """
    po = np.asarray(partial_o, dtype=np.float64)
    pl = np.asarray(partial_lse, dtype=np.float64)
    R, S, D = po.shape
    out = np.zeros((R, D), dtype=np.float64)
    lse = np.full((R,), -math.inf, dtype=np.float64)
    for r in range(R):
        terms = [float(x) for x in pl[r]]
        sink = None if sinks is None else float(np.asarray(sinks).reshape(-1)[r])
        M = max(terms + ([sink] if sink is not None else []))
        if M == -math.inf:
            continue
        w = np.array([math.exp(t - M) if t != -math.inf else 0.0 for t in terms])
        L = float(w.sum()) + (math.exp(sink - M) if sink is not None else 0.0)
        acc = np.zeros(D, dtype=np.float64)
        for s in range(S):
            if w[s] != 0.0:
                acc += w[s] * po[r, s]
        out[r] = acc / L
        lse[r] = M + math.log(L)
    return out, lse
