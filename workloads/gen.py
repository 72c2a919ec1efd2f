"""Seeded input generator: five named workloads plus arbitrary small shapes.

Recipe (the same for every workload, drawn in this order from
numpy.random.default_rng(seed)):

1. seq_lens (fixed, a list, or uniform integers in [lo, hi]);
2. the block table: a random permutation of the page pool handed out to the
   sequences in order (or the identity);
3. scales: one float32 per tensor, or one per kv head drawn U[lo, hi]
   (k_scale first, then v_scale); with k_groups > 1 the K scale has one
   number per head_dim group as well ([k_groups] drawn U[s/2, 2s] for a
   per-tensor scale s, or [Hkv, k_groups] drawn U[lo, hi]);
4. q ~ N(0, 1), rounded to bf16 (round to nearest even);
5. K then V: for every position that some query row attends,
   N(0, 1) / scale (the scale of that element's head and group), clamped to
   +-448 and rounded to E4M3 (nearest even);
6. sinks ~ N(0, 1) float32 [Hq] when the workload has sinks.

Every other byte of the pools (positions no row attends, pages no sequence
uses) is the E4M3 NaN code 0x7F when `poison` is on (default), so a kernel
that reads them or lets them leak produces NaN.  Unused block-table entries
are -1.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

POISON_CODE = 0x7F

# The five named workloads.  seq: ("fixed", n) | ("list", [..]) | ("uniform", lo, hi)
CONFIGS = {
    1: dict(name="tiny", B=1, q_len=1, Hq=8, Hkv=1, D=128, bt=16, seq=("fixed", 512),
            table="identity", pool=None, scale=("tensor", 0.05), window=0, sinks=False,
            sm_scale=1.0 / math.sqrt(128)),
    2: dict(name="ragged_gqa", B=16, q_len=1, Hq=32, Hkv=8, D=128, bt=16,
            seq=("uniform", 1024, 8192), table="perm", pool=8192,
            scale=("per_head", 0.02, 0.1), window=0, sinks=False,
            sm_scale=1.0 / math.sqrt(128)),
    3: dict(name="window_sinks", B=32, q_len=1, Hq=64, Hkv=8, D=64, bt=16,
            seq=("fixed", 32768), table="perm", pool=None, scale=("tensor", 0.05),
            window=4096, sinks=True, sm_scale=0.125),
    4: dict(name="long_splitkv", B=4, q_len=1, Hq=24, Hkv=4, D=256, bt=64,
            seq=("list", [196608, 131072, 65536, 8192]), table="perm", pool=None,
            scale=("per_head", 0.02, 0.1), window=0, sinks=False, sm_scale=0.08),
    5: dict(name="mtp_q4", B=256, q_len=4, Hq=32, Hkv=8, D=128, bt=16,
            seq=("uniform", 1024, 4096), table="perm", pool=None, scale=("tensor", 0.05),
            window=2048, sinks=True, sm_scale=1.0 / math.sqrt(128)),
    # Not one of the five named workloads: the ragged GQA batch with one query
    # head per kv head (MHA decode), the shape the VALU dot-product kernel serves.
    6: dict(name="mha_decode", B=16, q_len=1, Hq=8, Hkv=8, D=128, bt=16,
            seq=("uniform", 1024, 8192), table="perm", pool=8192,
            scale=("per_head", 0.02, 0.1), window=0, sinks=False,
            sm_scale=1.0 / math.sqrt(128)),
}


@dataclass
class Workload:
    """Host copies of every input of one decode call (numpy arrays)."""

    name: str
    q_bits: np.ndarray        # uint16 [B, q_len, Hq, D], bf16 bit patterns
    k_cache: np.ndarray       # uint8 [num_blocks, bt, Hkv, D], E4M3 codes
    v_cache: np.ndarray       # uint8 [num_blocks, bt, Hkv, D]
    block_table: np.ndarray   # int32 [B, max_blocks]
    seq_lens: np.ndarray      # int32 [B]
    k_scale: np.ndarray       # float32 [1] or [Hkv]; [k_groups] or [Hkv * k_groups]
    v_scale: np.ndarray       # float32 [1] or [Hkv]
    sinks: np.ndarray | None  # float32 [Hq] or None
    window: int
    sm_scale: float
    meta: dict = field(default_factory=dict)
    k_groups: int = 1
    kv_format: str = "e4m3"   # "nvfp4" / "mxfp8": k_cache / v_cache are uint8 [num_blocks, page_stride]
    kv_layout: str = "NHD"    # page layout of those pools ("NHD" or "HND")

    @property
    def B(self):
        return self.q_bits.shape[0]

    @property
    def q_len(self):
        return self.q_bits.shape[1]

    @property
    def Hq(self):
        return self.q_bits.shape[2]

    @property
    def D(self):
        return self.q_bits.shape[3]

    @property
    def Hkv(self):
        return self.meta["Hkv"] if self.kv_format != "e4m3" else self.k_cache.shape[2]

    @property
    def bt(self):
        return self.meta["bt"] if self.kv_format != "e4m3" else self.k_cache.shape[1]

    @property
    def num_blocks(self):
        return self.k_cache.shape[0]

    def oracle_kwargs(self):
        kw = dict(q_bits=self.q_bits, k_cache=self.k_cache, v_cache=self.v_cache,
                  block_table=self.block_table, seq_lens=self.seq_lens,
                  k_scale=self.k_scale, v_scale=self.v_scale, sinks=self.sinks,
                  window=self.window, sm_scale=self.sm_scale, k_groups=self.k_groups)
        if self.kv_format != "e4m3":
            kw.update(kv_format=self.kv_format, kv_layout=self.kv_layout, num_kv_heads=self.Hkv,
                      block_tokens=self.bt)
        return kw

    def key_union(self, b):
        """[lo, hi) of positions some query row of sequence b attends."""
        L = int(self.seq_lens[b])
        hi = L
        lo = 0
        if self.window > 0:
            lo = max(0, L - self.q_len - self.window + 1)
        return lo, hi

    def attended_positions(self):
        """Sum over sequences of attended positions (the union over rows)."""
        return int(sum(self.key_union(b)[1] - self.key_union(b)[0] for b in range(self.B)))


def _e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float -> E4M3 codes, clamped to +-448, round to nearest even (torch cast)."""
    import torch

    t = torch.from_numpy(np.clip(x, -448.0, 448.0).astype(np.float32, copy=False))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(x.astype(np.float32, copy=False)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def make_workload(*, B, q_len, Hq, Hkv, D, bt, seq_lens, seed, table="perm", pool=None,
                  scale=("tensor", 0.05), window=0, sinks=False, sm_scale=None,
                  poison=True, name="custom", q_zero=False, extra_table_cols=0,
                  key_chunk=8192, k_groups=1):
    """Build one seeded workload.

    seq_lens: an int, a list, or ("uniform", lo, hi).  scale: ("tensor", s) or
    ("per_head", lo, hi).  table: "perm" or "identity".  pool: minimum pool
    size in pages.  extra_table_cols adds -1 columns to every table row.
    k_groups > 1 gives the K scale one number per head_dim group.
    """
    rng = np.random.default_rng(seed)
    # 1. sequence lengths
    if isinstance(seq_lens, tuple) and seq_lens and seq_lens[0] == "uniform":
        sl = rng.integers(seq_lens[1], seq_lens[2] + 1, size=B).astype(np.int32)
    elif np.isscalar(seq_lens):
        sl = np.full((B,), int(seq_lens), dtype=np.int32)
    else:
        sl = np.asarray(seq_lens, dtype=np.int32).reshape(B)
    pages_needed = [(int(n) + bt - 1) // bt for n in sl]
    n_need = int(sum(pages_needed))
    num_blocks = max(n_need, int(pool or 0), 1)
    max_blocks = max(max(pages_needed) if pages_needed else 1, 1) + int(extra_table_cols)
    # 2. block table
    if table == "identity":
        order = np.arange(num_blocks, dtype=np.int64)
    else:
        order = rng.permutation(num_blocks)
    bt_arr = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = pages_needed[b]
        bt_arr[b, :n] = order[off:off + n]
        off += n
    # 3. scales
    kg = max(1, int(k_groups))
    if scale[0] == "tensor":
        if kg > 1:
            k_scale = rng.uniform(scale[1] / 2, scale[1] * 2, size=kg).astype(np.float32)
        else:
            k_scale = np.array([scale[1]], dtype=np.float32)
        v_scale = np.array([scale[1]], dtype=np.float32)
    else:
        k_scale = rng.uniform(scale[1], scale[2], size=Hkv * kg).astype(np.float32)
        v_scale = rng.uniform(scale[1], scale[2], size=Hkv).astype(np.float32)
    # 4. queries
    qf = rng.standard_normal((B, q_len, Hq, D), dtype=np.float32)
    if q_zero:
        qf[:] = 0.0
    q_bits = _bf16_bits(qf)
    # 5. caches
    fill = POISON_CODE if poison else 0
    caches = []
    wl_tmp = Workload(name, q_bits, np.empty((0, bt, Hkv, D), np.uint8), None, bt_arr, sl,
                      k_scale, v_scale, None, int(window), 0.0)
    for which, sc, groups in (("k", k_scale, kg), ("v", v_scale, 1)):
        # the scale of every (head, dim) element, [Hkv, D]
        per_head = sc.reshape(-1, groups) if sc.size > groups else np.tile(sc.reshape(1, groups), (Hkv, 1))
        el_scale = np.repeat(per_head, D // groups, axis=1)
        cache = np.full((num_blocks, bt, Hkv, D), fill, dtype=np.uint8)
        flat = cache.reshape(num_blocks * bt, Hkv, D)
        for b in range(B):
            lo, hi = wl_tmp.key_union(b)
            if not poison:
                lo = 0
                hi = pages_needed[b] * bt
            for c0 in range(lo, hi, key_chunk):
                c1 = min(c0 + key_chunk, hi)
                x = rng.standard_normal((c1 - c0, Hkv, D), dtype=np.float32)
                x /= el_scale[None]
                ts = np.arange(c0, c1)
                phys = bt_arr[b, ts // bt].astype(np.int64) * bt + ts % bt
                flat[phys] = _e4m3_encode(x)
        caches.append(cache)
    # 6. sinks
    sk = rng.standard_normal((Hq,), dtype=np.float32) if sinks else None
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    return Workload(name=name, q_bits=q_bits, k_cache=caches[0], v_cache=caches[1],
                    block_table=bt_arr, seq_lens=sl, k_scale=k_scale, v_scale=v_scale,
                    sinks=sk, window=int(window), sm_scale=float(sm_scale),
                    meta=dict(seed=seed, poison=poison), k_groups=kg)


def make_config(k: int, seed: int | None = None, poison: bool = True, k_groups: int = 1) -> Workload:
    """One of the five named workloads, seeded with 1000 + k by default
    (k_groups > 1: the same workload with K scales in head_dim groups)."""
    c = CONFIGS[k]
    seq = c["seq"]
    if seq[0] == "fixed":
        seq_lens = seq[1]
    elif seq[0] == "list":
        seq_lens = list(seq[1])
    else:
        seq_lens = ("uniform", seq[1], seq[2])
    return make_workload(B=c["B"], q_len=c["q_len"], Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"],
                         bt=c["bt"], seq_lens=seq_lens, seed=1000 + k if seed is None else seed,
                         table=c["table"], pool=c["pool"], scale=c["scale"],
                         window=c["window"], sinks=c["sinks"], sm_scale=c["sm_scale"],
                         poison=poison, k_groups=k_groups,
                         name=f"cfg{k}_{c['name']}" + (f"_kg{k_groups}" if k_groups > 1 else ""))


NVFP4_POISON_SCALE = 0x7F   # E4M3 NaN: a block read where nothing is attended yields NaN
NVFP4_POISON_DATA = 0x77


def make_nvfp4_workload(**kw):
    """A workload whose K/V pools are NVFP4 pages: uint8 [num_blocks,
    page_stride], each page one side's data region ([bt][Hkv] or [Hkv][bt]
    rows of D/2 bytes, two 4-bit codes per byte) followed by its scale region
    (rows of D/16 E4M3 bytes).  Same draw order as make_workload, with step 5
    drawing, for every attended position and kv head, D/2 uniform data bytes
    and D/16 scale bytes uniform over the E4M3 codes 0x48..0x57 (4 to 15).
    Every other byte is NVFP4_POISON_DATA / NVFP4_POISON_SCALE when `poison`.
    """
    return _make_blockscaled_workload(fmt="nvfp4", **kw)


def make_mxfp8_workload(**kw):
    """A workload whose K/V pools are MXFP8 pages: each page one side's data
    region (rows of D E4M3 bytes) followed by its scale region (rows of D/32
    E8M0 bytes), in the same row orders as the NVFP4 pages.  Step 5 draws, for
    every attended position and kv head, D data bytes uniform over the
    non-NaN E4M3 codes and D/32 scale bytes uniform over 119..124 (2^-8 to
    2^-3).  Every other byte is the NaN data code 0x7F or the NaN scale 0xFF
    when `poison`."""
    return _make_blockscaled_workload(fmt="mxfp8", **kw)


def _make_blockscaled_workload(*, fmt, B, q_len, Hq, Hkv, D, bt, seq_lens, seed, table="perm",
                               pool=None, scale=("tensor", 0.05), window=0, sinks=False,
                               sm_scale=None, poison=True, name=None, kv_layout="NHD",
                               page_stride=None, e8m0_centers=None):
    """e8m0_centers (MXFP8 only): per sequence b a pair (k, v) of scale-byte
    centres; that sequence's K (V) scale bytes are then the usual draw moved
    to centre + (draw - 121), i.e. centre - 2 .. centre + 3, so the same
    random stream spreads whole sequences across the E8M0 range."""
    rng = np.random.default_rng(seed)
    if isinstance(seq_lens, tuple) and seq_lens and seq_lens[0] == "uniform":
        sl = rng.integers(seq_lens[1], seq_lens[2] + 1, size=B).astype(np.int32)
    elif np.isscalar(seq_lens):
        sl = np.full((B,), int(seq_lens), dtype=np.int32)
    else:
        sl = np.asarray(seq_lens, dtype=np.int32).reshape(B)
    pages_needed = [(int(n) + bt - 1) // bt for n in sl]
    num_blocks = max(int(sum(pages_needed)), int(pool or 0), 1)
    max_blocks = max(max(pages_needed) if pages_needed else 1, 1)
    order = np.arange(num_blocks, dtype=np.int64) if table == "identity" else rng.permutation(num_blocks)
    bt_arr = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = pages_needed[b]
        bt_arr[b, :n] = order[off:off + n]
        off += n
    if scale[0] == "tensor":
        k_scale = np.array([scale[1]], dtype=np.float32)
        v_scale = np.array([scale[1]], dtype=np.float32)
    else:
        k_scale = rng.uniform(scale[1], scale[2], size=Hkv).astype(np.float32)
        v_scale = rng.uniform(scale[1], scale[2], size=Hkv).astype(np.float32)
    qf = rng.standard_normal((B, q_len, Hq, D), dtype=np.float32)
    q_bits = _bf16_bits(qf)
    data_row, sc_row = (D // 2, D // 16) if fmt == "nvfp4" else (D, D // 32)
    poison_data, poison_scale = ((NVFP4_POISON_DATA, NVFP4_POISON_SCALE) if fmt == "nvfp4"
                                 else (0x7F, 0xFF))
    data_bytes = Hkv * bt * data_row
    side = Hkv * bt * (data_row + sc_row)
    stride = int(page_stride or side)
    name = name or fmt
    wl_tmp = Workload(name, q_bits, np.empty((0, bt, Hkv, D), np.uint8), None, bt_arr, sl,
                      k_scale, v_scale, None, int(window), 0.0)
    pools = []
    for _ in ("k", "v"):
        pool_arr = np.zeros((num_blocks, stride), dtype=np.uint8)
        if poison:
            pool_arr[:, :data_bytes] = poison_data
            pool_arr[:, data_bytes:side] = poison_scale
            pool_arr[:, side:] = poison_scale
        for b in range(B):
            lo, hi = wl_tmp.key_union(b)
            if not poison:
                lo, hi = 0, pages_needed[b] * bt
            if hi <= lo:
                continue
            ts = np.arange(lo, hi)
            pages = bt_arr[b, ts // bt].astype(np.int64)
            slots = ts % bt
            data = rng.integers(0, 256, size=(hi - lo, Hkv, data_row), dtype=np.uint8)
            if fmt == "nvfp4":
                scl = rng.integers(0x48, 0x58, size=(hi - lo, Hkv, sc_row), dtype=np.uint8)
            else:
                data[(data & 0x7F) == 0x7F] -= 1          # no NaN codes in attended data
                scl = rng.integers(119, 125, size=(hi - lo, Hkv, sc_row), dtype=np.uint8)
                if e8m0_centers is not None:
                    centre = int(e8m0_centers[b][len(pools)])
                    scl = (scl.astype(np.int64) - 121 + centre).astype(np.uint8)
            for h in range(Hkv):
                r = h * bt + slots if kv_layout == "HND" else slots * Hkv + h
                d_off = r * data_row
                s_off = data_bytes + r * sc_row
                pool_arr[pages[:, None], d_off[:, None] + np.arange(data_row)] = data[:, h]
                pool_arr[pages[:, None], s_off[:, None] + np.arange(sc_row)] = scl[:, h]
        pools.append(pool_arr)
    sk = rng.standard_normal((Hq,), dtype=np.float32) if sinks else None
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    return Workload(name=name, q_bits=q_bits, k_cache=pools[0], v_cache=pools[1],
                    block_table=bt_arr, seq_lens=sl, k_scale=k_scale, v_scale=v_scale,
                    sinks=sk, window=int(window), sm_scale=float(sm_scale),
                    meta=dict(seed=seed, poison=poison, Hkv=Hkv, bt=bt, page_stride=stride),
                    kv_format=fmt, kv_layout=kv_layout)
