"""A sweep of the shape space against the oracle: GQA ratios from 1 (MHA) to
64 (one kv head for 64 query heads), 1, 2 and 5 query tokens, head_dim 64,
128 and 256, so every planner branch is taken (VALU kernel, paired heads,
two row blocks, head_dim split, LDS-shared row groups of 2, 4 and 8); a
batch past the balanced planner's limit (fixed splits); a sequence of 2^20
tokens; and a max_seq_len bound far above the real lengths."""

import pytest

import oracle
from tests.gpu_harness import compare, run, to_host, upload
from workloads import make_workload

torch = pytest.importorskip("torch")
fp = pytest.importorskip("decode_attention_paged_fp8pa_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp.lib()


RATIOS = [(4, 4), (8, 4), (12, 4), (20, 4), (28, 4), (32, 4), (64, 4), (64, 1)]   # (Hq, Hkv)
CASES = [(hq, hkv, ql, d) for hq, hkv in RATIOS for ql in (1, 2, 5) for d in (64, 128, 256)]


@pytest.mark.parametrize("hq,hkv,ql,d", CASES)
def test_shape_sweep(hq, hkv, ql, d):
    wl = make_workload(seed=900 + CASES.index((hq, hkv, ql, d)), B=2, q_len=ql, Hq=hq, Hkv=hkv, D=d, bt=16,
                       seq_lens=[333, 70], window=250 if ql != 2 else 0, sinks=ql != 1)
    ro, rl = oracle.decode(**wl.oracle_kwargs())
    out, lse = to_host(*run(wl, upload(wl)))
    compare(out, lse, ro, rl, label=f"Hq={hq} Hkv={hkv} q_len={ql} D={d}")


@pytest.mark.parametrize("flags", [0, fp.FP8PA_FLAG_FORCE_DOT])
def test_batch_past_the_balanced_limit(flags):
    """300 sequences (the balanced plan reads all seq_lens for up to 256):
    fixed-size splits from max_seq_len, ragged lengths, empty slots."""
    seq = [0 if i % 17 == 0 else 1 + (53 * i * i + 7 * i) % 900 for i in range(300)]
    wl = make_workload(seed=990, B=300, q_len=1, Hq=8, Hkv=2, D=128, bt=16, seq_lens=seq, sinks=True)
    ro, rl = oracle.decode(**wl.oracle_kwargs())
    out, lse = to_host(*run(wl, upload(wl), flags=flags))
    compare(out, lse, ro, rl, label=f"B=300 flags={flags}")


@pytest.mark.parametrize("window", [0, 700000])
def test_million_token_sequence(window):
    """A sequence of 2^20 tokens beside a shorter one (the longest named
    workload has 196,608): 256 splits of 128 tiles for the long one, a pool
    of ~335 MB, every output row against the oracle, on the planned kernel
    and the VALU kernel."""
    wl = make_workload(seed=951, B=2, q_len=2, Hq=8, Hkv=2, D=64, bt=256, seq_lens=[1 << 20, 300001],
                       window=window, sinks=True)
    ro, rl = oracle.decode(**wl.oracle_kwargs())
    t = upload(wl)
    for flags in (0, fp.FP8PA_FLAG_FORCE_DOT):
        out, lse = to_host(*run(wl, t, flags=flags))
        compare(out, lse, ro, rl, label=f"2^20 tokens window={window} flags={flags}")


@pytest.mark.parametrize("flags", [0, fp.FP8PA_FLAG_FORCE_DOT])
def test_max_seq_len_far_above_the_lengths(flags):
    """max_seq_len is only a bound: a caller that passes 2^20 for sequences of
    5 to 2,000 tokens (the table as wide as the bound asks) gets the same
    results; the plan and workspace follow the bound, the kernels the real
    lengths."""
    bound = 1 << 20
    wl = make_workload(seed=952, B=3, q_len=1, Hq=16, Hkv=4, D=128, bt=16, seq_lens=[100, 5, 2000],
                       extra_table_cols=bound // 16 - 125, sinks=True)
    assert wl.block_table.shape[1] >= bound // 16
    ro, rl = oracle.decode(**wl.oracle_kwargs())
    t = upload(wl)
    out, lse = fp.decode(t["q"], t["k"], t["v"], t["bt"], t["sl"], t["ks"], t["vs"], t["sinks"],
                         window=wl.window, sm_scale=wl.sm_scale, max_seq_len=bound, flags=flags)
    compare(*to_host(out, lse), ro, rl, label=f"max_seq_len 2^20, flags={flags}")


@pytest.mark.parametrize("ns", [0, 3])
def test_prefill_rows_past_one_merge_round(ns):
    """A 256-token chunk of 16 query heads over two sequences: 8,192 rows, so
    the splits merge through the many-rows merge; every row against the
    oracle."""
    wl = make_workload(seed=953, B=2, q_len=256, Hq=16, Hkv=4, D=128, bt=16, seq_lens=[2600, 900], window=1500,
                       sinks=True)
    ro, rl = oracle.decode(**wl.oracle_kwargs())
    out, lse = to_host(*run(wl, upload(wl), num_splits=ns))
    compare(out, lse, ro, rl, label=f"prefill 8192 rows, splits={ns}")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("window", [0, 9000])
@pytest.mark.parametrize("ns,ctx", [(0, 12000), (1, 12000), (2, 12000), (1, 40000)])
def test_prefill_splits_past_one_table_window(d, window, ns, ctx):
    """Row groups sharing tiles through LDS take splits of up to 1,024
    tiles, reloading their 128-tile register window of block-table entries
    as they go: a 64-token chunk over 12,000 tokens (375 tiles) in one
    (3 windows, the output written directly), two or the planner's number
    of parts, and over 40,000 tokens (1,250 tiles: a 1,024-tile split, 8
    windows), every row against the oracle."""
    wl = make_workload(seed=954, B=1, q_len=64, Hq=16, Hkv=4, D=d, bt=16, seq_lens=[ctx], window=window,
                       sinks=True)
    ro, rl = oracle.decode(**wl.oracle_kwargs())
    t = upload(wl)
    shape = fp.shape_for(t["q"], t["k"], t["bt"], t["ks"], t["vs"], window=window, max_seq_len=ctx,
                         num_splits=ns)
    plan = fp.fp8pa_plan(shape, torch.cuda.get_device_properties(0).multi_processor_count)
    assert plan["row_groups_per_wg"] > 1
    if ns:
        assert plan["tiles_per_split"] > 128
    out, lse = to_host(*run(wl, t, num_splits=ns))
    compare(out, lse, ro, rl, label=f"LDS-shared splits past 128 tiles D={d} window={window} splits={ns}")


EQUAL_LENGTHS = [
    # (B, q_len, Hq, Hkv, D, length): the MFMA kernel, the VALU kernel (MHA)
    # and the LDS-shared kernel of four row groups (a 16-token prefill chunk)
    (16, 1, 32, 8, 128, 4096),
    (16, 1, 8, 8, 128, 2000),
    (16, 16, 32, 8, 128, 8192),
]


@pytest.mark.parametrize("B,ql,hq,hkv,d,L", EQUAL_LENGTHS)
def test_balanced_equal_lengths_fill_every_slot(B, ql, hq, hkv, d, L):
    """Sequences of one length: the balanced chunk is T / slots (every
    workgroup slot of the grid gets an item) rather than the looser
    T / (slots - B); every output row against the oracle."""
    from tests.test_abi import _balanced_items

    wl = make_workload(seed=995 + L, B=B, q_len=ql, Hq=hq, Hkv=hkv, D=d, bt=16, seq_lens=[L] * B,
                       poison=False)
    t = upload(wl)
    shape = fp.shape_for(t["q"], t["k"], t["bt"], t["ks"], t["vs"], sm_scale=wl.sm_scale, max_seq_len=L)
    plan = fp.fp8pa_plan(shape, torch.cuda.get_device_properties(0).multi_processor_count)
    assert plan["split_mode"] == fp.FP8PA_SPLIT_BALANCED
    items, c = _balanced_items(plan, [L] * B, ql, 0)
    n = -(-L // 32)
    assert sum(len(v) for v in items.values()) == B * -(-n // c)
    ro, rl = oracle.decode(**wl.oracle_kwargs())
    out, lse = to_host(*run(wl, t))
    compare(out, lse, ro, rl, label=f"B={B} q_len={ql} Hq={hq} Hkv={hkv} L={L} chunk {c}")


# Ragged batches whose tighter chunk would give more items than slots (the
# kernel counts them and keeps the looser chunk): the VALU kernel (MHA,
# 2 query tokens) and the MFMA kernel.
FALLBACK = [
    (2, 8, 8, [5085, 2774, 2270, 5884, 5711, 4095, 2456, 1340, 5625, 1685, 3381, 4080, 1516, 1959, 4474, 1264,
               4078, 5673, 4136, 3912, 2836, 5810]),
    (1, 32, 8, [4161, 3420, 5205, 2506, 2790, 2814, 2231, 169, 4104, 3136, 1265, 4340, 1425, 2623, 2371, 2469,
                3072, 2976, 3474, 868, 5734, 624, 1445]),
]


@pytest.mark.parametrize("ql,hq,hkv,lens", FALLBACK)
def test_balanced_tight_chunk_that_overflows_is_not_taken(ql, hq, hkv, lens):
    from tests.test_abi import _balanced_items

    wl = make_workload(seed=997 + hq, B=len(lens), q_len=ql, Hq=hq, Hkv=hkv, D=128, bt=16, seq_lens=lens)
    t = upload(wl)
    shape = fp.shape_for(t["q"], t["k"], t["bt"], t["ks"], t["vs"], sm_scale=wl.sm_scale, max_seq_len=max(lens))
    plan = fp.fp8pa_plan(shape, torch.cuda.get_device_properties(0).multi_processor_count)
    assert plan["split_mode"] == fp.FP8PA_SPLIT_BALANCED
    items, c = _balanced_items(plan, lens, ql, 0)
    assert sum(len(v) for v in items.values()) <= plan["target_items"] + len(lens)
    ro, rl = oracle.decode(**wl.oracle_kwargs())
    out, lse = to_host(*run(wl, t))
    compare(out, lse, ro, rl, label=f"ragged B={len(lens)} q_len={ql} Hq={hq} chunk {c}")
