"""C-ABI checks that need no GPU: exported symbols, the planner, validation.

fp8pa_plan is pure host arithmetic, and fp8pa_decode / fp8pa_merge check
every host-known argument before their first HIP call, so these error paths
run on any host.
"""

import ctypes
import math
import os
import re

import numpy as np
import pytest

import decode_attention_paged_fp8pa_amd as fp
from decode_attention_paged_fp8pa_amd import _lib
from workloads import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(inc, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(fp8pa_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert "fp8pa_decode" in names and "fp8pa_merge" in names and "fp8pa_workspace_bytes" in names
    handle = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), f"{n} declared in include/ but not exported"


# The HIP runtime entry points the library may import: kernel registration
# and launch, device queries, the error state and the no-allocation entry
# point's symbol lookup.  No allocation, free, memset, copy, stream or event
# creation, or synchronisation: no call path can allocate or block, under
# graph capture or not, whatever torch's allocator reports.
ALLOWED_HIP_IMPORTS = {
    "__hipPopCallConfiguration", "__hipPushCallConfiguration", "__hipRegisterFatBinary",
    "__hipRegisterFunction", "__hipRegisterVar", "__hipUnregisterFatBinary",
    "hipDeviceGetAttribute", "hipGetDevice", "hipGetLastError", "hipGetSymbolAddress", "hipLaunchKernel",
}


def test_library_imports_no_allocation_or_synchronisation():
    import shutil
    import subprocess

    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    r = subprocess.run([nm, "-D", "--undefined-only", _lib.LIB_PATH], capture_output=True, text=True, check=True)
    imported = {line.split()[-1].split("@")[0] for line in r.stdout.splitlines() if line.strip()}
    hip = {name for name in imported if "hip" in name.lower()}
    assert hip, "no HIP imports found: not the built library?"
    assert hip <= ALLOWED_HIP_IMPORTS, f"unexpected HIP runtime imports: {sorted(hip - ALLOWED_HIP_IMPORTS)}"


def test_status_strings_and_version():
    assert fp.status_string(0) == "ok"
    for s in range(1, 6):
        assert fp.status_string(s) not in ("ok", "unknown status")
    assert "gfx950" in fp.version()


def cfg_shape(k, **over):
    c = CONFIGS[k]
    seq = c["seq"]
    max_seq = {"fixed": lambda: seq[1], "list": lambda: max(seq[1]), "uniform": lambda: seq[2]}[seq[0]]()
    bt = c["bt"]
    kw = dict(batch=c["B"], q_len=c["q_len"], num_q_heads=c["Hq"], num_kv_heads=c["Hkv"],
              head_dim=c["D"], block_tokens=bt, num_blocks=max(c["pool"] or 0, 1 << 16),
              block_table_stride=(max_seq + bt - 1) // bt, max_seq_len=max_seq,
              k_scale_count=c["Hkv"] if c["scale"][0] == "per_head" else 1,
              v_scale_count=c["Hkv"] if c["scale"][0] == "per_head" else 1, window=c["window"],
              sm_scale=c["sm_scale"], num_splits=0, flags=0)
    kw.update(over)
    return fp.make_shape(**kw)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_plan_of_each_workload(k):
    s = cfg_shape(k)
    p = fp.fp8pa_plan(s, 256)
    c = CONFIGS[k]
    rows = c["Hq"] // c["Hkv"] * c["q_len"]
    assert p["variant"] == 1  # every named workload has >= 3 rows per kv head and bt >= 16
    assert p["rows_per_group"] == 16 and p["row_groups"] == math.ceil(rows / 16)
    assert c["Hkv"] % p["heads_per_wg"] == 0
    # head_dim 256 is split over two wavefronts per kv head
    assert p["waves_per_head"] == (2 if c["D"] == 256 else 1)
    # head_dim 64 with <= 8 rows per kv head pairs two kv heads per wavefront
    assert p["heads_per_wave"] == (2 if c["D"] == 64 and rows <= 8 and c["Hkv"] % 2 == 0 else 1)
    assert p["heads_per_wg"] // p["heads_per_wave"] * p["waves_per_head"] <= 8
    upi = (c["Hkv"] // p["heads_per_wg"]) * p["row_groups"]
    assert p["grid_wgs"] % upi == 0
    items = p["grid_wgs"] // upi
    max_keys = s.max_seq_len if c["window"] <= 0 else min(s.max_seq_len, c["window"] + c["q_len"] - 1)
    n_tiles = math.ceil(max_keys / 32) + (1 if c["window"] > 0 else 0)
    if p["split_mode"] == fp.FP8PA_SPLIT_BALANCED:
        # the kernel sizes the chunk in [tiles_per_split, max_tiles_per_split];
        # the slots must hold the longest sequence even at the largest chunk
        assert p["tiles_per_split"] == math.ceil(min(rows, 16) * 64 / 32)
        assert p["num_splits"] * p["max_tiles_per_split"] >= n_tiles
        assert p["num_splits"] == max(min(p["target_items"], n_tiles),
                                      math.ceil(n_tiles / p["max_tiles_per_split"]))
        # enough items for sum_b max(1, ceil(n_b / c)) at any chunk the kernel picks
        assert items == min(c["B"] * p["num_splits"], max(p["target_items"],
                            math.ceil(c["B"] * n_tiles / p["max_tiles_per_split"])) + c["B"])
    else:
        assert items == c["B"] * p["num_splits"]
        # the splits cover every tile a sequence can span
        assert p["num_splits"] * p["tiles_per_split"] >= n_tiles
        assert (p["num_splits"] - 1) * p["tiles_per_split"] < n_tiles
        assert (p["split_mode"] == fp.FP8PA_SPLIT_DIRECT) == (p["num_splits"] == 1)
    rows_total = c["B"] * c["q_len"] * c["Hq"]
    if p["num_splits"] == 1:
        assert p["merge_launched"] == 0 and p["workspace_bytes"] == 0
    else:
        po = rows_total * p["num_splits"] * c["D"] * 4
        pl = rows_total * p["num_splits"] * 4
        want = math.ceil(po / 256) * 256 + math.ceil(pl / 256) * 256 + 256
        assert p["merge_launched"] == 1 and p["workspace_bytes"] == want


def test_plan_is_deterministic_and_forced_splits():
    s = cfg_shape(4)
    assert fp.fp8pa_plan(s, 256) == fp.fp8pa_plan(s, 256)
    # a split of the MFMA kernel spans at most 128 tiles: 196608 tokens need
    # at least ceil(6144 tiles / 128) = 48 splits
    max_tps = 128
    min_splits = math.ceil(6144 / max_tps)
    for n in (1, 2, 7, 64):
        p = fp.fp8pa_plan(cfg_shape(4, num_splits=n), 256)
        assert 1 <= p["num_splits"] <= max(n, min_splits)
        assert p["tiles_per_split"] <= max_tps
    # with a shorter sequence bound one split is possible: no workspace then
    s1 = cfg_shape(5, num_splits=1)
    assert fp.fp8pa_plan(s1, 256)["num_splits"] == 1
    assert fp.fp8pa_plan(s1, 256)["workspace_bytes"] == 0


def test_variant_selection():
    # one query row per kv head (MHA decode): the VALU dot kernel
    s = fp.make_shape(batch=2, q_len=1, num_q_heads=8, num_kv_heads=8, head_dim=128,
                      block_tokens=16, num_blocks=64, block_table_stride=32, max_seq_len=512,
                      sm_scale=0.1)
    assert fp.fp8pa_plan(s, 256)["variant"] == 0
    # pages of 8 tokens: only the dot kernel handles them
    s.block_tokens = 8
    s.block_table_stride = 64
    s.num_q_heads = 32
    assert fp.fp8pa_plan(s, 256)["variant"] == 0
    s.flags = fp.FP8PA_FLAG_FORCE_MFMA
    with pytest.raises(fp.Fp8paError) as e:
        fp.fp8pa_plan(s, 256)
    assert e.value.status == _lib.FP8PA_ERR_UNSUPPORTED
    s.block_tokens = 16
    s.block_table_stride = 32
    assert fp.fp8pa_plan(s, 256)["variant"] == 1
    s.flags = fp.FP8PA_FLAG_FORCE_DOT
    p = fp.fp8pa_plan(s, 256)
    assert p["variant"] == 0 and p["rows_per_group"] == 4 and p["row_groups"] == 1


BAD = [
    (dict(batch=0), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(q_len=0), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(num_q_heads=30), _lib.FP8PA_ERR_INVALID_ARG),      # not a multiple of Hkv = 8
    (dict(head_dim=96), _lib.FP8PA_ERR_UNSUPPORTED),
    (dict(head_dim=512), _lib.FP8PA_ERR_UNSUPPORTED),
    (dict(block_tokens=24), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(block_tokens=2048), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(num_blocks=0), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(block_table_stride=10), _lib.FP8PA_ERR_INVALID_ARG),  # too short for max_seq_len
    (dict(max_seq_len=0), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(k_scale_count=3), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(v_scale_count=0), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(k_groups=-1), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(k_groups=3, k_scale_count=24), _lib.FP8PA_ERR_INVALID_ARG),   # not a power of two
    (dict(k_groups=32, k_scale_count=256), _lib.FP8PA_ERR_INVALID_ARG),  # above 16
    (dict(k_groups=8, k_scale_count=64), _lib.FP8PA_ERR_INVALID_ARG),   # 16 dims per group at D = 128
    (dict(k_groups=4), _lib.FP8PA_ERR_INVALID_ARG),                     # Hkv scales, not Hkv * 4
    (dict(kv_layout=2), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(kv_format=3), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(kv_format=1, k_groups=2, k_scale_count=16), _lib.FP8PA_ERR_INVALID_ARG),  # no groups with NVFP4
    (dict(kv_format=2, k_groups=2, k_scale_count=16), _lib.FP8PA_ERR_INVALID_ARG),  # nor with MXFP8
    # block-scaled pages must be 16-byte multiples (head_dim 64, one token and
    # head per page: 66 MXFP8 / 36 NVFP4 bytes) unless a padded stride is given
    (dict(kv_format=2, head_dim=64, block_tokens=1, num_kv_heads=1, num_q_heads=1, k_scale_count=1,
          v_scale_count=1, block_table_stride=8192), _lib.FP8PA_ERR_MISALIGNED),
    (dict(kv_format=1, head_dim=64, block_tokens=1, num_kv_heads=1, num_q_heads=1, k_scale_count=1,
          v_scale_count=1, block_table_stride=8192), _lib.FP8PA_ERR_MISALIGNED),
    (dict(kv_format=1, flags=2, block_tokens=8, block_table_stride=1024), _lib.FP8PA_ERR_UNSUPPORTED),  # MFMA needs bt >= 16
    (dict(kv_page_stride=-16), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(kv_page_stride=16 * 8 * 128 - 16), _lib.FP8PA_ERR_INVALID_ARG),  # shorter than a page
    (dict(kv_page_stride=16 * 8 * 128 + 8), _lib.FP8PA_ERR_INVALID_ARG),   # not a multiple of 16
    (dict(kv_layout=-1), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(sm_scale=float("nan")), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(sm_scale=float("inf")), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(num_splits=-1), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(flags=8), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(flags=3), _lib.FP8PA_ERR_INVALID_ARG),
]


def test_head_pairing_in_both_page_layouts():
    # cfg3 (D = 64, 8 rows per kv head) pairs kv heads per wavefront, with
    # token-major and head-major pages alike
    assert CONFIGS[3]["D"] == 64
    for layout in (fp.FP8PA_LAYOUT_NHD, fp.FP8PA_LAYOUT_HND):
        p = fp.fp8pa_plan(cfg_shape(3, kv_layout=layout), 256)
        assert p["heads_per_wave"] == 2 and p["variant"] == 1


def test_nvfp4_plans():
    # head_dim 64 and 128: the bf16-MFMA kernel, one head and 16 rows per
    # wavefront; head_dim 256: the VALU kernel
    for k in (2, 3):
        p = fp.fp8pa_plan(cfg_shape(k, kv_format=fp.FP8PA_KV_NVFP4), 256)
        assert (p["variant"], p["rows_per_group"], p["heads_per_wave"], p["waves_per_head"]) == (1, 16, 1, 1)
    p = fp.fp8pa_plan(cfg_shape(4, kv_format=fp.FP8PA_KV_NVFP4), 256)
    assert p["variant"] == 0 and p["rows_per_group"] == 4
    with pytest.raises(fp.Fp8paError) as e:
        fp.fp8pa_plan(cfg_shape(4, kv_format=fp.FP8PA_KV_NVFP4, flags=fp.FP8PA_FLAG_FORCE_MFMA), 256)
    assert e.value.status == _lib.FP8PA_ERR_UNSUPPORTED
    # a page stride that interleaves K and V pages (2 x the NVFP4 page of cfg2:
    # 16 tokens x 8 heads x (64 + 8) bytes)
    fp.fp8pa_plan(cfg_shape(2, kv_format=fp.FP8PA_KV_NVFP4, kv_page_stride=2 * 16 * 8 * 72), 256)


def test_mxfp8_plans():
    # the same kernels as NVFP4: the bf16-MFMA kernel at head_dim 64 and 128,
    # the VALU kernel at 256; a padded stride makes an odd page size legal
    for k in (2, 3):
        p = fp.fp8pa_plan(cfg_shape(k, kv_format=fp.FP8PA_KV_MXFP8), 256)
        assert (p["variant"], p["rows_per_group"], p["heads_per_wave"], p["waves_per_head"]) == (1, 16, 1, 1)
    p = fp.fp8pa_plan(cfg_shape(4, kv_format=fp.FP8PA_KV_MXFP8), 256)
    assert p["variant"] == 0 and p["rows_per_group"] == 4
    fp.fp8pa_plan(cfg_shape(2, kv_format=fp.FP8PA_KV_MXFP8, kv_page_stride=2 * 16 * 8 * 132), 256)
    fp.fp8pa_plan(cfg_shape(3, kv_format=fp.FP8PA_KV_MXFP8, block_tokens=1, block_table_stride=32768,
                            kv_page_stride=8 * 66 + 16 - (8 * 66) % 16), 256)


def test_row_blocks_for_many_rows():
    base = dict(batch=2, num_q_heads=32, num_kv_heads=8, head_dim=128, block_tokens=16,
                num_blocks=1024, block_table_stride=64, max_seq_len=1024, sm_scale=0.1)
    # head_dim 128: one block of 16 rows per wavefront; 2, 4 or 8 row groups
    # of one kv head share each K/V tile through LDS when the row groups
    # divide so (the largest such count)
    for q_len, rg, lw in ((1, 1, 1), (4, 1, 1), (5, 2, 2), (8, 2, 2), (9, 3, 1), (16, 4, 4),
                          (24, 6, 2), (28, 7, 1), (32, 8, 8), (48, 12, 4), (128, 32, 8)):
        p = fp.fp8pa_plan(fp.make_shape(q_len=q_len, **base), 256)
        assert (p["row_blocks"], p["row_groups"], p["rows_per_group"]) == (1, rg, 16), q_len
        assert p["row_groups_per_wg"] == lw, q_len
        if lw > 1:
            assert p["heads_per_wg"] == 1
            assert p["grid_wgs"] % (8 // 1 * (rg // lw)) == 0   # Hkv * row_groups / lw units per item
        # non-temporal loads only where one wavefront reads each K/V byte
        assert p["nontemporal_kv"] == (1 if rg == 1 else 0)
    # head_dim 64: two blocks once a kv head has more than 16 rows, unless 4
    # or 8 row groups share tiles through LDS; non-temporal loads only with paired
    # heads (at most 8 rows), whose wavefront reads whole 128-byte lines
    for q_len, nb, rg, lw in ((2, 1, 1, 1), (4, 1, 1, 1), (5, 2, 1, 1), (8, 2, 1, 1), (9, 2, 2, 1),
                              (16, 1, 4, 4), (24, 2, 3, 1), (128, 1, 32, 8)):
        p = fp.fp8pa_plan(fp.make_shape(q_len=q_len, **dict(base, head_dim=64)), 256)
        assert (p["row_blocks"], p["row_groups"], p["rows_per_group"]) == (nb, rg, 16 * nb), q_len
        assert p["row_groups_per_wg"] == lw, q_len
        paired = 4 * q_len <= 8
        assert p["heads_per_wave"] == (2 if paired else 1)
        assert p["nontemporal_kv"] == (1 if paired else 0)
    # head_dim scale groups keep their third query part: no LDS-shared tiles
    for q_len in (16, 32, 128):
        p = fp.fp8pa_plan(fp.make_shape(q_len=q_len, k_groups=4, k_scale_count=8 * 4, **base), 256)
        assert p["row_groups_per_wg"] == 1, q_len
    # head_dim 256 splits head_dim over two wavefronts and keeps one row block
    p = fp.fp8pa_plan(fp.make_shape(q_len=64, **dict(base, head_dim=256)), 256)
    assert p["row_blocks"] == 1 and p["waves_per_head"] == 2


def test_long_chunk_splits_span_several_table_windows():
    """The LDS-shared kernels reload their 128-tile window of block-table
    entries as they go, so a long chunk's fixed splits span up to 1,024
    tiles (2 splits of a 32,768-token context, one round of workgroups,
    instead of 8); the other kernels keep 128."""
    s = fp.make_shape(batch=2, q_len=512, num_q_heads=32, num_kv_heads=8, head_dim=128, block_tokens=16,
                      num_blocks=4096, block_table_stride=2048, max_seq_len=32768, sm_scale=0.1)
    p = fp.fp8pa_plan(s, 256)
    assert p["row_groups_per_wg"] == 8
    assert p["split_mode"] == fp.FP8PA_SPLIT_FIXED and p["tiles_per_split"] == 512 and p["num_splits"] == 2
    assert p["max_tiles_per_split"] == 1024 and p["grid_wgs"] == 512
    # one query row per kv head: no LDS sharing, 128-tile splits
    s1 = fp.make_shape(batch=2, q_len=1, num_q_heads=8, num_kv_heads=8, head_dim=128, block_tokens=16,
                       num_blocks=4096, block_table_stride=2048, max_seq_len=32768, sm_scale=0.1)
    p1 = fp.fp8pa_plan(s1, 256)
    assert p1["row_groups_per_wg"] <= 1 and p1["max_tiles_per_split"] <= 128
    # a caller's split count is honoured up to the cap
    for ns, tps in ((1, 1024), (2, 512), (3, 342)):
        s2 = fp.make_shape(batch=2, q_len=512, num_q_heads=32, num_kv_heads=8, head_dim=128, block_tokens=16,
                           num_blocks=4096, block_table_stride=2048, max_seq_len=32768, sm_scale=0.1,
                           num_splits=ns)
        p2 = fp.fp8pa_plan(s2, 256)
        assert p2["tiles_per_split"] == tps and p2["num_splits"] == ns


def test_plan_accepts_k_groups():
    c = CONFIGS[2]
    assert c["D"] == 128 and c["scale"][0] == "per_head"
    for kg, count in ((0, c["Hkv"]), (1, 1), (2, 2), (4, 4), (4, 4 * c["Hkv"]), (2, 2 * c["Hkv"])):
        fp.fp8pa_plan(cfg_shape(2, k_groups=kg, k_scale_count=count), 256)
    s = cfg_shape(4, k_groups=8, k_scale_count=8)   # head_dim 256: 32 dims per group
    assert CONFIGS[4]["D"] == 256
    fp.fp8pa_plan(s, 256)


@pytest.mark.parametrize("over,status", BAD)
def test_plan_rejects_bad_shapes(over, status):
    with pytest.raises(fp.Fp8paError) as e:
        fp.fp8pa_plan(cfg_shape(2, **over), 256)
    assert e.value.status == status


def test_plan_rejects_bad_cu_count():
    with pytest.raises(fp.Fp8paError):
        fp.fp8pa_plan(cfg_shape(2), 0)


def test_plan_accepts_sequences_shorter_than_q_len():
    # every sequence shorter than q_len (batches padded with empty slots):
    # the rows at negative positions attend nothing
    p = fp.fp8pa_plan(cfg_shape(5, max_seq_len=3, block_table_stride=1), 256)
    assert p["num_splits"] == 1 and p["grid_wgs"] >= 1


def _call_decode(shape, **ptrs):
    base = dict(q=0x10000, k=0x20000, v=0x30000, bt=0x40000, sl=0x50000, ks=0x60000, vs=0x70000,
                sinks=None, out=0x80000, lse=None, ws=None, ws_bytes=0)
    base.update(ptrs)
    L = _lib.lib()
    return L.fp8pa_decode(ctypes.byref(shape), base["q"], base["k"], base["v"], base["bt"],
                          base["sl"], base["ks"], base["vs"], base["sinks"], base["out"],
                          base["lse"], base["ws"], base["ws_bytes"], None)


def test_decode_checks_pointers_before_the_gpu():
    s = cfg_shape(3)
    for name in ("q", "k", "v", "bt", "sl", "ks", "vs", "out"):
        assert _call_decode(s, **{name: None}) == _lib.FP8PA_ERR_INVALID_ARG, name
    for name, addr in (("q", 0x10008), ("k", 0x20004), ("v", 0x30001), ("out", 0x80002),
                       ("bt", 0x40002), ("lse", 0x90001), ("sinks", 0xa0003), ("ws", 0xb0010)):
        assert _call_decode(s, **{name: addr}) == _lib.FP8PA_ERR_MISALIGNED, name
    bad = cfg_shape(3, head_dim=80)
    assert _call_decode(bad) == _lib.FP8PA_ERR_UNSUPPORTED
    assert _lib.lib().fp8pa_decode(None, 1, 1, 1, 1, 1, 1, 1, None, 1, None, None, 0, None) \
        == _lib.FP8PA_ERR_INVALID_ARG


def test_merge_checks_arguments_before_the_gpu():
    L = _lib.lib()
    assert L.fp8pa_merge(0, 4, 8, 128, 0x1000, 0x2000, None, 0x3000, None, None) == _lib.FP8PA_ERR_INVALID_ARG
    assert L.fp8pa_merge(2, -1, 8, 128, 0x1000, 0x2000, None, 0x3000, None, None) == _lib.FP8PA_ERR_INVALID_ARG
    assert L.fp8pa_merge(2, 4, 0, 128, 0x1000, 0x2000, None, 0x3000, None, None) == _lib.FP8PA_ERR_INVALID_ARG
    assert L.fp8pa_merge(2, 4, 8, 100, 0x1000, 0x2000, None, 0x3000, None, None) == _lib.FP8PA_ERR_UNSUPPORTED
    assert L.fp8pa_merge(2, 4, 8, 128, None, 0x2000, None, 0x3000, None, None) == _lib.FP8PA_ERR_INVALID_ARG
    assert L.fp8pa_merge(2, 4, 8, 128, 0x1000, 0x2000, None, None, None, None) == _lib.FP8PA_ERR_INVALID_ARG
    assert L.fp8pa_merge(2, 4, 8, 128, 0x1004, 0x2000, None, 0x3000, None, None) == _lib.FP8PA_ERR_MISALIGNED
    assert L.fp8pa_merge(2, 4, 8, 128, 0x1000, 0x2002, None, 0x3000, None, None) == _lib.FP8PA_ERR_MISALIGNED


def test_debug_entry_points_check_arguments():
    L = _lib.lib()
    assert L.fp8pa_debug_e4m3_to_f32(None, None, -1, None) == _lib.FP8PA_ERR_INVALID_ARG
    assert L.fp8pa_debug_e4m3_to_f32(None, None, 0, None) == _lib.FP8PA_OK
    assert L.fp8pa_debug_mfma_fp8(None, 0x1000, 0x2000, None) == _lib.FP8PA_ERR_INVALID_ARG
    assert L.fp8pa_debug_wave_ops(None, 5, 0x2000, None) == _lib.FP8PA_ERR_INVALID_ARG
    assert L.fp8pa_debug_lds_tr8(0x1000, None, 0x2000, None) == _lib.FP8PA_ERR_INVALID_ARG
    assert L.fp8pa_debug_lds_tr8(0x1008, 0x3000, 0x2000, None) == _lib.FP8PA_ERR_MISALIGNED
    assert L.fp8pa_debug_wave_ops(0x1000, -1, 0x2000, None) == _lib.FP8PA_ERR_INVALID_ARG
    assert L.fp8pa_debug_nvfp4(None, None, None, -1, None) == _lib.FP8PA_ERR_INVALID_ARG
    assert L.fp8pa_debug_nvfp4(None, None, None, 0, None) == _lib.FP8PA_OK
    assert L.fp8pa_debug_nvfp4(0x1004, 0x2000, 0x3000, 1, None) == _lib.FP8PA_ERR_MISALIGNED
    assert L.fp8pa_debug_mxfp8(None, None, None, -1, None) == _lib.FP8PA_ERR_INVALID_ARG
    assert L.fp8pa_debug_mxfp8(0x1000, None, 0x3000, 1, None) == _lib.FP8PA_ERR_INVALID_ARG
    assert L.fp8pa_debug_mxfp8(None, None, None, 0, None) == _lib.FP8PA_OK
    assert L.fp8pa_debug_mxfp8(0x1002, 0x2000, 0x3000, 1, None) == _lib.FP8PA_ERR_MISALIGNED


def _balanced_items(plan, seq_lens, q_len, window):
    """The balanced split rule the kernels apply, written out for checking the
    planner's bounds: returns {b: [(ts, te), ...]} and the chunk size."""
    def span(L):
        ulo = max(0, L - q_len - window + 1) if window > 0 else 0
        t0 = ulo // 32
        t1 = (L - 1) // 32 + 1 if L > ulo else t0
        return t0, t1
    n = [span(L)[1] - span(L)[0] for L in seq_lens]
    T, M = sum(n), max(n)
    tgt = plan["target_items"]
    ns_max = plan["num_splits"]

    def splits(x, c):
        return min(-(-x // c), ns_max) if x > 0 else 1

    floor_c = max(min(plan["tiles_per_split"], max(1, 2 * T // tgt)), -(-M // ns_max))
    c = min(max(-(-T // tgt), floor_c), plan["max_tiles_per_split"])
    # the tighter chunk T / (target + B), where its items fit the target + B slots
    slots = tgt + len(seq_lens)
    ct = min(max(-(-T // slots), floor_c), plan["max_tiles_per_split"])
    if ct < c and sum(splits(x, ct) for x in n) <= slots:
        c = ct
    out = {}
    for b, L in enumerate(seq_lens):
        t0, t1 = span(L)
        ns = splits(n[b], c)
        out[b] = [(t0 + s * c, min(t0 + s * c + c, t1)) for s in range(ns)]
    return out, c


@pytest.mark.parametrize("seed", range(40))
def test_balanced_plan_covers_every_tile(seed):
    import numpy as np
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 257))
    q_len = int(rng.integers(1, 5))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 3, 4, 8]))
    D = int(rng.choice([64, 128, 256]))
    bt = int(rng.choice([16, 32, 64]))
    window = int(rng.choice([0, 0, 7, 1000]))
    max_seq = int(rng.integers(q_len, 300000 if B < 8 else 20000))
    seq = rng.integers(q_len, max_seq + 1, size=B).tolist()
    seq[0] = max_seq
    s = fp.make_shape(batch=B, q_len=q_len, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D,
                      block_tokens=bt, num_blocks=1 << 16, block_table_stride=-(-max_seq // bt),
                      max_seq_len=max_seq, window=window, sm_scale=0.1)
    for cu in (8, 80, 256):
        p = fp.fp8pa_plan(s, cu)
        if p["split_mode"] != fp.FP8PA_SPLIT_BALANCED:
            continue
        items, c = _balanced_items(p, seq, q_len, window)
        upi = (Hkv // p["heads_per_wg"]) * (p["row_groups"] // p["row_groups_per_wg"])
        # every (sequence, split) item has a workgroup slot and a partial slot
        assert sum(len(v) for v in items.values()) <= p["grid_wgs"] // upi
        assert max(len(v) for v in items.values()) <= p["num_splits"]
        # the splits of a sequence tile its key span exactly, each within the
        # block-table registers (<= 128 tiles; the LDS-shared kernels reload
        # them every 128 tiles, up to 1,024)
        for b, L in enumerate(seq):
            spans = items[b]
            lo = (max(0, L - q_len - window + 1) if window > 0 else 0) // 32
            assert spans[0][0] == lo and spans[-1][1] == max(lo, (L - 1) // 32 + 1)
            for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
                assert a1 == b0 and a0 < a1
            for a0, a1 in spans:
                if p["variant"] == 1:
                    assert a1 - a0 <= (1024 if p["row_groups_per_wg"] > 1 else 128)



@pytest.mark.parametrize("B,q_len,Hq,Hkv,L,want_c", [
    (16, 16, 32, 8, 8192, 32),   # LDS-shared, 4 row groups: 8 splits x 16 = all 128 slots
    (16, 1, 32, 8, 4096, 8),     # MFMA decode: 16 splits x 16 = 256 slots
    (16, 1, 8, 8, 2000, 4),      # VALU decode (MHA): 16 splits x 16 = 256 slots
])
def test_balanced_chunk_fills_the_slots_for_equal_lengths(B, q_len, Hq, Hkv, L, want_c):
    """Equal lengths reach the items bound exactly, so the chunk T / (target
    + B) fits: one round of workgroups, each with the least work (the looser
    T / target would leave slots idle and give every workgroup more)."""
    s = fp.make_shape(batch=B, q_len=q_len, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128, block_tokens=16,
                      num_blocks=1 << 16, block_table_stride=-(-L // 16), max_seq_len=L, sm_scale=0.1)
    p = fp.fp8pa_plan(s, 256)
    assert p["split_mode"] == fp.FP8PA_SPLIT_BALANCED
    items, c = _balanced_items(p, [L] * B, q_len, 0)
    slots = p["target_items"] + B
    assert c == want_c
    assert sum(len(v) for v in items.values()) == slots
    upi = (Hkv // p["heads_per_wg"]) * (p["row_groups"] // p["row_groups_per_wg"])
    assert p["grid_wgs"] == slots * upi
    # the looser chunk would have left slots idle
    T = B * -(-L // 32)
    assert -(-T // p["target_items"]) > c


@pytest.mark.parametrize("q_len,Hq,Hkv,lens,want_c", [
    (2, 8, 8, [5085, 2774, 2270, 5884, 5711, 4095, 2456, 1340, 5625, 1685, 3381, 4080, 1516, 1959, 4474, 1264,
               4078, 5673, 4136, 3912, 2836, 5810], 11),
    (1, 32, 8, [4161, 3420, 5205, 2506, 2790, 2814, 2231, 169, 4104, 3136, 1265, 4340, 1425, 2623, 2371, 2469,
                3072, 2976, 3474, 868, 5734, 624, 1445], 9),
])
def test_balanced_chunk_keeps_the_bound_when_the_tight_one_overflows(q_len, Hq, Hkv, lens, want_c):
    """Ragged lengths where T / slots would give more items than slots: the
    looser chunk T / target stays (one chunk smaller would overflow)."""
    B = len(lens)
    s = fp.make_shape(batch=B, q_len=q_len, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=128, block_tokens=16,
                      num_blocks=1 << 16, block_table_stride=-(-max(lens) // 16), max_seq_len=max(lens),
                      sm_scale=0.1)
    p = fp.fp8pa_plan(s, 256)
    assert p["split_mode"] == fp.FP8PA_SPLIT_BALANCED
    items, c = _balanced_items(p, lens, q_len, 0)
    assert c == want_c
    slots = p["target_items"] + B
    n = [-(-L // 32) for L in lens]
    assert sum(-(-x // (c - 1)) for x in n) > slots
    assert sum(len(v) for v in items.values()) <= slots

def _write_shape(**over):
    kw = dict(num_tokens=4, key_stride=1024, value_stride=1024, num_kv_heads=8, head_dim=128,
              block_tokens=16, num_blocks=8, k_scale_count=8, v_scale_count=1, k_groups=1)
    kw.update(over)
    return _lib.WriteShape(**kw)


def _call_write(shape, **ptrs):
    base = dict(key=0x10000, value=0x20000, slots=0x30000, ks=0x40000, vs=0x50000, kc=0x60000,
                vc=0x70000)
    base.update(ptrs)
    return _lib.lib().fp8pa_cache_write(ctypes.byref(shape), base["key"], base["value"], base["slots"],
                                        base["ks"], base["vs"], base["kc"], base["vc"], None)


WRITE_BAD = [
    (dict(num_tokens=-1), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(num_kv_heads=0), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(head_dim=96), _lib.FP8PA_ERR_UNSUPPORTED),
    (dict(block_tokens=24), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(block_tokens=2048), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(num_blocks=0), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(key_stride=1000), _lib.FP8PA_ERR_INVALID_ARG),       # shorter than a token row
    (dict(value_stride=1028), _lib.FP8PA_ERR_MISALIGNED),       # not a multiple of 8 elements
    (dict(k_scale_count=3), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(v_scale_count=0), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(k_groups=4), _lib.FP8PA_ERR_INVALID_ARG),                      # Hkv scales, not Hkv * 4
    (dict(k_groups=8, k_scale_count=64), _lib.FP8PA_ERR_INVALID_ARG),    # 16 dims per group
    (dict(k_groups=6, k_scale_count=48), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(k_groups=4, v_scale_count=32), _lib.FP8PA_ERR_INVALID_ARG),    # V keeps one per head
    (dict(kv_layout=3), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(kv_format=5), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(kv_format=1, k_groups=2, k_scale_count=16), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(kv_format=2, k_groups=2, k_scale_count=16), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(kv_format=2, kv_page_stride=16 * 8 * 132 - 16), _lib.FP8PA_ERR_INVALID_ARG),
    (dict(kv_format=2, head_dim=64, block_tokens=1, num_kv_heads=1, k_scale_count=1, v_scale_count=1,
          key_stride=64, value_stride=64), _lib.FP8PA_ERR_MISALIGNED),
    (dict(kv_format=1, kv_page_stride=16 * 8 * 72 - 16), _lib.FP8PA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("over,status", WRITE_BAD)
def test_cache_write_rejects_bad_shapes(over, status):
    assert _call_write(_write_shape(**over)) == status


def test_cache_write_checks_pointers_before_the_gpu():
    L = _lib.lib()
    assert L.fp8pa_cache_write(None, 1, 1, 1, 1, 1, 1, 1, None) == _lib.FP8PA_ERR_INVALID_ARG
    s = _write_shape()
    for name in ("key", "value", "slots", "ks", "vs", "kc", "vc"):
        assert _call_write(s, **{name: None}) == _lib.FP8PA_ERR_INVALID_ARG, name
    for name, addr in (("key", 0x10008), ("value", 0x20004), ("kc", 0x60004), ("vc", 0x70002),
                       ("slots", 0x30004), ("ks", 0x40002)):
        assert _call_write(s, **{name: addr}) == _lib.FP8PA_ERR_MISALIGNED, name
    # nothing to write: no pointer is needed and nothing is queued
    assert _call_write(_write_shape(num_tokens=0), key=None, value=None, slots=None) == _lib.FP8PA_OK


def test_stream_read_diagnostic_argument_checks():
    """fp8pa_debug_stream_read rejects its bad arguments before any GPU call."""
    lib = _lib.lib()
    sink = ctypes.c_uint32(0)
    s = ctypes.addressof(sink)
    assert lib.fp8pa_debug_stream_read(16, 64, 16, None, None) == _lib.FP8PA_ERR_INVALID_ARG
    assert lib.fp8pa_debug_stream_read(None, 64, 16, s, None) == _lib.FP8PA_ERR_INVALID_ARG
    assert lib.fp8pa_debug_stream_read(16, 65, 16, s, None) == _lib.FP8PA_ERR_INVALID_ARG
    for w in (0, 2, 12, 32, -16):
        assert lib.fp8pa_debug_stream_read(16, 64, w, s, None) == _lib.FP8PA_ERR_INVALID_ARG
    assert lib.fp8pa_debug_stream_read(24, 64, 16, s, None) == _lib.FP8PA_ERR_MISALIGNED


def test_fast_division_multipliers_match_integer_division():
    """The multiply-and-shift the kernels divide by host-known divisors with
    (workgroups per item, row groups, query heads per kv head, split slots,
    rows per sequence) equals integer division for every numerator below
    2^31: checked here against Python's // on divisors 1..4096, every power
    of two and its neighbours, and random ones, at the numerators where an
    off-by-one would show (multiples of d and their neighbours, the top of
    the range) plus random ones."""
    rng = np.random.default_rng(31)
    divisors = list(range(1, 4097)) + [2 ** k + e for k in range(1, 31) for e in (-1, 0, 1)]
    divisors += [int(x) for x in rng.integers(1, 2 ** 31 - 1, size=500)]
    top = 2 ** 31 - 1
    for d in divisors:
        m, sh = fp.fp8pa_debug_fast_div(d)
        assert 0 < m < 2 ** 32 and 31 <= sh <= 62
        ks = [1, 2, 3, 1000, top // d]
        ns = [0, 1, d - 1, d, d + 1, top, top - 1]
        ns += [k * d + r for k in ks for r in (-1, 0, 1, d - 1)]
        ns += [int(x) for x in rng.integers(0, top, size=16)]
        for n in ns:
            if 0 <= n <= top:
                assert (n * m) >> sh == n // d, (n, d, m, sh)
    # divisors below 1 are taken as 1; null outputs are refused
    assert fp.fp8pa_debug_fast_div(0) == fp.fp8pa_debug_fast_div(1)
    L = _lib.lib()
    assert L.fp8pa_debug_fast_div(7, None, None) == _lib.FP8PA_ERR_INVALID_ARG
