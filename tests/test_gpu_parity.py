"""GPU parity of libfp8pa against the float64 oracle, through the C ABI.

Small cases compare every output element; the five named workloads run at
full size in the launch configuration the benchmark times and compare
every output row (the forced VALU kernel: sampled rows).  Invariance tests
compare GPU runs with each other bit for bit.
"""

import math

import time

import numpy as np
import pytest

import oracle
from tests.gpu_harness import compare, run, to_host, upload
from workloads import make_config, make_workload

torch = pytest.importorskip("torch")
fp = pytest.importorskip("decode_attention_paged_fp8pa_amd")

pytestmark = pytest.mark.gpu

DOT = fp.FP8PA_FLAG_FORCE_DOT
MFMA = fp.FP8PA_FLAG_FORCE_MFMA


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp.lib()  # fails loudly when the library is not built


# ------------------------------------------------------------- hardware pins

def test_hw_e4m3_decode_matches_oracle_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).cuda()
    out = torch.empty(256, dtype=torch.float32, device="cuda")
    fp.fp8pa_debug_e4m3_to_f32(codes, out, 256)
    got = out.cpu().numpy().astype(np.float64)
    want = oracle.E4M3_TABLE
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def _mfma(a, b):
    c = torch.empty((16, 16), dtype=torch.float32, device="cuda")
    fp.fp8pa_debug_mfma_fp8(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), c)
    return c.cpu().numpy().astype(np.float64)


def test_hw_mfma_fp8_layout_exact():
    # codes of 0, +-0.5, +-1, +-2: every product and partial sum is exact, so any
    # mistake in the assumed lane layout shows as a mismatch.
    rng = np.random.default_rng(0)
    vals = np.array([0x00, 0x30, 0x38, 0x40, 0xB0, 0xB8, 0xC0], dtype=np.uint8)
    a = vals[rng.integers(0, len(vals), size=(16, 32))]
    b = vals[rng.integers(0, len(vals), size=(32, 16))]
    want = oracle.E4M3_TABLE[a] @ oracle.E4M3_TABLE[b]
    assert np.array_equal(_mfma(a, b), want)


def test_hw_mfma_fp8_accumulation_precision():
    # Random finite codes: the MFMA sums 32 products with less than fp32
    # precision; the error stays below 2^-10 of the sum of |products|.
    rng = np.random.default_rng(1)
    a = rng.integers(0, 0x78, size=(16, 32)).astype(np.uint8)
    b = rng.integers(0, 0x78, size=(32, 16)).astype(np.uint8)
    a |= (rng.integers(0, 2, size=a.shape) << 7).astype(np.uint8)
    A, Bm = oracle.E4M3_TABLE[a], oracle.E4M3_TABLE[b]
    want = A @ Bm
    scale = np.abs(A) @ np.abs(Bm)
    assert np.all(np.abs(_mfma(a, b) - want) <= scale * 2.0 ** -10)


def _scaled_mfma_ref(a, sa, b):
    """The block-scaled 16x16x128 FP8 MFMA as the kernels use it: lane group
    g's bytes 0-15 (a[m][32 g + j]) are k = 16 g + j and its bytes 16-31 are
    k = 64 + 16 g + (j - 16), for A and B alike, and the 32 k of block c
    (k // 32 = c) take row m's scale byte from lane group c, sa[m][c]."""
    k = np.arange(128)
    g = np.where(k < 64, k // 16, (k - 64) // 16)
    j = np.where(k < 64, k % 16, 16 + (k - 64) % 16)
    A = oracle.E4M3_TABLE[a[:, 32 * g + j]] * np.exp2(sa[:, k // 32].astype(np.float64) - 127)
    B = oracle.E4M3_TABLE[b[32 * g + j, :]]
    return A @ B, np.abs(A) @ np.abs(B)


@pytest.mark.parametrize("seed", [0, 1])
def test_hw_mfma_block_scale_layout(seed):
    """The lane layout and scale assignment of v_mfma_scale_f32_16x16x128_f8f6f4
    that the MXFP8 kernel relies on (each lane's A scale multiplies one
    32-element block of its row, laid out as above): random codes, E8M0
    scales 120..134 per row and block, against the exact sum within the
    MFMA's accumulation precision."""
    rng = np.random.default_rng(50 + seed)
    a = rng.integers(0, 0x78, size=(16, 128)).astype(np.uint8)
    a |= (rng.integers(0, 2, size=a.shape) << 7).astype(np.uint8)
    b = rng.integers(0, 0x78, size=(128, 16)).astype(np.uint8)
    b |= (rng.integers(0, 2, size=b.shape) << 7).astype(np.uint8)
    sa = rng.integers(120, 135, size=(16, 4)).astype(np.uint8)
    c = torch.empty(256, dtype=torch.float32, device="cuda")
    fp.fp8pa_debug_mfma_scale_fp8(torch.from_numpy(a).cuda(), torch.from_numpy(sa).cuda(),
                                  torch.from_numpy(b).cuda(), c)
    got = c.cpu().numpy().reshape(16, 16).astype(np.float64)
    want, mag = _scaled_mfma_ref(a, sa, b)
    assert np.all(np.abs(got - want) <= mag * 2.0 ** -10)


@pytest.mark.parametrize("vmax", [0, 1, 7, 300, 65535])
def test_hw_wave_reductions_and_prefix(vmax):
    rng = np.random.default_rng(vmax)
    x = rng.integers(0, vmax + 1, size=64).astype(np.int32)
    if vmax:
        x[rng.integers(0, 64)] = vmax
    out = torch.empty(256, dtype=torch.int32, device="cuda")
    fp.fp8pa_debug_wave_ops(torch.from_numpy(x).cuda(), vmax, out)
    got = out.cpu().numpy().astype(np.int64)
    x64 = x.astype(np.int64)
    assert np.array_equal(got[:64], np.concatenate([[0], np.cumsum(x64)[:-1]]))
    assert np.all(got[64:128] == x64.sum())
    assert np.all(got[128:192] == x64.max())
    assert np.all(got[192:] == x64.sum())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_hw_lds_transposing_read(seed):
    """The lane mapping of ds_read_b64_tr_b8 that the LDS-shared prefill path
    builds PV's V^T operands with: lane 16 g + 8 h + c gets byte c of the rows
    named by lanes 16 g + h, 16 g + h + 2, ..., 16 g + h + 14."""
    rng = np.random.default_rng(seed)
    src = rng.integers(0, 256, size=4096, dtype=np.uint8)
    addr = (rng.integers(0, 4096 // 8, size=64) * 8).astype(np.int32)
    out = torch.empty(512, dtype=torch.uint8, device="cuda")
    fp.fp8pa_debug_lds_tr8(torch.from_numpy(src).cuda(), torch.from_numpy(addr).cuda(), out)
    got = out.cpu().numpy().reshape(64, 8)
    want = np.empty((64, 8), dtype=np.uint8)
    for lane in range(64):
        g, h, c = lane // 16, (lane % 16) // 8, lane % 8
        for t in range(8):
            want[lane, t] = src[addr[16 * g + 2 * t + h] + c]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("seed", [0, 1])
def test_hw_lds_transposing_read_16bit(seed):
    """The lane mapping of ds_read_b64_tr_b16 that the LDS-shared kernels
    build PV's bf16 V^T operands with: lane 16 g + 4 h + c gets, as its
    element t, 16-bit element c of the 8-byte row named by lane
    16 g + 4 t + h."""
    rng = np.random.default_rng(100 + seed)
    src = rng.integers(0, 256, size=4096, dtype=np.uint8)
    addr = (rng.integers(0, 4096 // 8, size=64) * 8).astype(np.int32)
    out = torch.empty(512, dtype=torch.uint8, device="cuda")
    fp.fp8pa_debug_lds_tr16(torch.from_numpy(src).cuda(), torch.from_numpy(addr).cuda(), out)
    got = out.cpu().numpy().view(np.uint16).reshape(64, 4)
    src16 = src.view(np.uint16)
    want = np.empty((64, 4), dtype=np.uint16)
    for lane in range(64):
        g, h, c = lane // 16, (lane % 16) // 4, lane % 4
        for t in range(4):
            want[lane, t] = src16[addr[16 * g + 4 * t + h] // 2 + c]
    assert np.array_equal(got, want), (got[:8], want[:8])


# ------------------------------------------------------- small, every element

SMALL = {
    "cfg1_twin": dict(B=1, q_len=1, Hq=8, Hkv=1, D=128, bt=16, seq_lens=[512]),
    "gqa4_ragged": dict(B=4, q_len=1, Hq=32, Hkv=8, D=128, bt=16, seq_lens=[33, 700, 129, 1000],
                        scale=("per_head", 0.02, 0.1)),
    "d64_window_sinks": dict(B=2, q_len=1, Hq=64, Hkv=8, D=64, bt=16, seq_lens=[300, 517],
                             window=100, sinks=True),
    "d256_bt64": dict(B=3, q_len=1, Hq=24, Hkv=4, D=256, bt=64, seq_lens=[1000, 65, 200],
                      scale=("per_head", 0.02, 0.1), sm_scale=0.08),
    "mtp4_window_sinks": dict(B=4, q_len=4, Hq=32, Hkv=8, D=128, bt=16, seq_lens=[20, 300, 4, 155],
                              window=40, sinks=True),
    "rows32_two_groups": dict(B=2, q_len=2, Hq=16, Hkv=1, D=128, bt=32, seq_lens=[100, 250]),
    "g3_q3_window1": dict(B=2, q_len=3, Hq=6, Hkv=2, D=64, bt=16, seq_lens=[50, 3], window=1,
                          sinks=True),
    "d256_bt128_long": dict(B=1, q_len=1, Hq=16, Hkv=2, D=256, bt=128, seq_lens=[2000]),
    "q4_window5": dict(B=2, q_len=4, Hq=8, Hkv=2, D=128, bt=16, seq_lens=[64, 97], window=5),
    "seq_eq_qlen": dict(B=2, q_len=4, Hq=8, Hkv=2, D=64, bt=16, seq_lens=[4, 4], sinks=True),
    "tiny_seqs": dict(B=4, q_len=1, Hq=8, Hkv=2, D=128, bt=16, seq_lens=[1, 17, 32, 33]),
    # a batch padded with empty slots (0 tokens), and sequences shorter than
    # q_len: rows at negative positions attend nothing
    "padded_zero_lengths": dict(B=4, q_len=1, Hq=8, Hkv=2, D=128, bt=16, seq_lens=[0, 300, 0, 17],
                                sinks=True),
    "short_seqs_q4": dict(B=3, q_len=4, Hq=8, Hkv=2, D=64, bt=16, seq_lens=[2, 0, 90]),
    "all_slots_empty": dict(B=2, q_len=2, Hq=8, Hkv=2, D=128, bt=16, seq_lens=[0, 0], sinks=True),
    "short_seqs_prefill_lw4": dict(B=3, q_len=16, Hq=16, Hkv=4, D=128, bt=16, seq_lens=[5, 0, 200],
                                   sinks=True),
    "mha_rows1": dict(B=2, q_len=1, Hq=8, Hkv=8, D=128, bt=16, seq_lens=[100, 513]),
    "bt1_pages": dict(B=2, q_len=2, Hq=4, Hkv=2, D=64, bt=1, seq_lens=[37, 90], window=10, sinks=True),
    "bt8_d256": dict(B=1, q_len=1, Hq=8, Hkv=4, D=256, bt=8, seq_lens=[300]),
    "window_ge_seq": dict(B=2, q_len=1, Hq=8, Hkv=2, D=128, bt=16, seq_lens=[40, 70], window=5000,
                          sinks=True),
    "big_negative_sinks": dict(B=2, q_len=1, Hq=8, Hkv=2, D=64, bt=32, seq_lens=[77, 130], sinks=True),
    # head_dim 64 with 8 rows per kv head: two kv heads per wavefront
    "pair_q2_perhead": dict(B=3, q_len=2, Hq=16, Hkv=4, D=64, bt=16, seq_lens=[50, 300, 130],
                            window=77, sinks=True, scale=("per_head", 0.02, 0.1)),
    # batches that span several 64-sequence groups of the balanced split plan
    # (130 and 256 sequences) and one just past it (257: fixed-size splits)
    "batch130_mqa": dict(B=130, q_len=1, Hq=8, Hkv=1, D=128, bt=16,
                         seq_lens=[1 + (37 * i * i + 11 * i) % 600 for i in range(130)]),
    "batch256_d64": dict(B=256, q_len=1, Hq=4, Hkv=1, D=64, bt=16,
                         seq_lens=[1 + (13 * i * i + 5 * i) % 300 for i in range(256)]),
    "batch257_d64": dict(B=257, q_len=1, Hq=4, Hkv=1, D=64, bt=16,
                         seq_lens=[1 + (13 * i * i + 5 * i) % 300 for i in range(257)]),
    # K scales in groups along head_dim: [Hkv, k_groups] or [k_groups]
    "kg4_gqa_ragged": dict(B=3, q_len=1, Hq=32, Hkv=8, D=128, bt=16, seq_lens=[45, 800, 260],
                           scale=("per_head", 0.005, 0.2), sinks=True, k_groups=4),
    "kg2_d64_pair": dict(B=2, q_len=2, Hq=8, Hkv=4, D=64, bt=16, seq_lens=[90, 333], window=60,
                         scale=("per_head", 0.02, 0.1), k_groups=2),
    "kg2_d64_rows16": dict(B=2, q_len=1, Hq=32, Hkv=2, D=64, bt=32, seq_lens=[200, 71],
                           scale=("tensor", 0.05), sinks=True, k_groups=2),
    "kg8_d256_window": dict(B=2, q_len=1, Hq=16, Hkv=2, D=256, bt=16, seq_lens=[700, 150], window=300,
                            scale=("tensor", 0.05), k_groups=8),
    "kg4_mha": dict(B=2, q_len=1, Hq=4, Hkv=4, D=128, bt=16, seq_lens=[150, 61],
                    scale=("per_head", 0.01, 0.1), k_groups=4),
    # many query rows per sequence (chunked prefill, causal over the new
    # tokens): a row group's tiles end where its last row's keys end
    "prefill_q64": dict(B=2, q_len=64, Hq=8, Hkv=2, D=128, bt=16, seq_lens=[64, 300], sinks=True),
    "prefill_q128_window": dict(B=1, q_len=128, Hq=16, Hkv=4, D=64, bt=16, seq_lens=[500],
                                window=100, scale=("per_head", 0.02, 0.1)),
    "prefill_q16_d256": dict(B=2, q_len=16, Hq=8, Hkv=2, D=256, bt=64, seq_lens=[16, 1000],
                             scale=("per_head", 0.02, 0.1), sinks=True),
    "prefill_q512": dict(B=1, q_len=512, Hq=4, Hkv=1, D=128, bt=16, seq_lens=[1500]),
    # 64 rows per kv head: four row groups share each K/V tile through LDS
    "prefill_q16_lw4": dict(B=2, q_len=16, Hq=16, Hkv=4, D=128, bt=16, seq_lens=[16, 700], window=300,
                            sinks=True, scale=("per_head", 0.02, 0.1)),
    "prefill_q16_lw4_d64": dict(B=3, q_len=16, Hq=8, Hkv=2, D=64, bt=32, seq_lens=[40, 333, 1000],
                                k_groups=2, scale=("per_head", 0.02, 0.1)),
    "prefill_q32_lw8_hnd_pages": dict(B=2, q_len=32, Hq=16, Hkv=4, D=128, bt=16, seq_lens=[32, 450]),
    "prefill_q32_mha_kg": dict(B=2, q_len=32, Hq=4, Hkv=4, D=128, bt=32, seq_lens=[40, 233],
                               window=64, k_groups=2, scale=("per_head", 0.02, 0.1)),
    "kg4_q4_mtp": dict(B=2, q_len=4, Hq=16, Hkv=4, D=128, bt=16, seq_lens=[130, 44], window=50,
                       scale=("per_head", 0.02, 0.1), sinks=True, k_groups=4),
    # 32 or 96 rows per kv head at head_dim 128: two row groups share each tile
    "mtp_q4_g8_lw2": dict(B=3, q_len=4, Hq=64, Hkv=8, D=128, bt=16, seq_lens=[100, 700, 33],
                          window=50, sinks=True),
    "prefill_q24_lw2": dict(B=2, q_len=24, Hq=16, Hkv=4, D=128, bt=32, seq_lens=[24, 610],
                            scale=("per_head", 0.02, 0.1), sinks=True),
    # group K scales folded into the query with few keys per row: the LSE of
    # the first rows rests on a handful of scores, so the folded query must be
    # held to well beyond E4M3's 4 bits
    "kg4_q8_few_keys_lw2": dict(B=2, q_len=8, Hq=32, Hkv=8, D=128, bt=32, seq_lens=[8, 520],
                                k_groups=4, scale=("per_head", 0.02, 0.1)),
    # Softmax weights far below the row's maximum must still reach the output
    # (their mass is in the denominator either way).  Values have mean 2, so
    # a kernel that drops small weights from P.V misses ~0.1 * 2 of the output.
    # One key per (sequence, kv head) scores ~11 nats above ~4000 others:
    "peaked_row_mean_v": dict(B=2, q_len=1, Hq=16, Hkv=4, D=128, bt=16, seq_lens=[4000, 2500]),
    # the same with head_dim 64 (two kv heads per wavefront) and a window
    "peaked_row_mean_v_d64": dict(B=2, q_len=1, Hq=16, Hkv=4, D=64, bt=16, seq_lens=[3000, 1800],
                                  window=2500),
    # sinks of +8 and +12 dominate every row: with one split they enter the
    # partial kernel's running maximum, so every key's weight is ~e^-12
    "big_positive_sinks_mean_v": dict(B=2, q_len=1, Hq=16, Hkv=4, D=128, bt=16, seq_lens=[3000, 700],
                                      sinks=True),
    "big_positive_sinks_mtp": dict(B=2, q_len=4, Hq=16, Hkv=4, D=128, bt=16, seq_lens=[2000, 300],
                                   sinks=True, window=1000),
}


def _shift_values(wl, mean):
    """Adds `mean` to every attended value (the E4M3 codes of x / v_scale are
    re-encoded from x + mean); NaN poison bytes stay as they are."""
    from workloads.gen import _e4m3_encode

    v = wl.v_cache
    vs = wl.v_scale.reshape(-1)
    scale = vs[None, None, :, None] if vs.size > 1 else vs.reshape(1, 1, 1, 1)
    x = oracle.E4M3_TABLE[v] * scale
    live = ~np.isnan(x)
    y = np.where(live, (x + mean) / scale, 0.0)
    wl.v_cache[...] = np.where(live, _e4m3_encode(y.astype(np.float32)), v)


def _peak_one_key(wl, rng, nats=11.0):
    """Gives every query head of a kv group the same query and, in each
    sequence, sets one attended key of that group to a multiple of it, so its
    score stands ~`nats` above the N(0, 1) scores of the others."""
    from workloads.gen import _bf16_bits, _e4m3_encode

    G = wl.Hq // wl.Hkv
    q = (wl.q_bits.astype(np.uint32) << 16).view(np.float32).copy()
    ks = wl.k_scale.reshape(-1)
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        lo = max(0, L - wl.window) if wl.window > 0 else 0
        for g in range(wl.Hkv):
            qg = q[b, :, g * G, :].copy()
            q[b, :, g * G:(g + 1) * G, :] = qg[:, None, :]
            qv = qg[-1].astype(np.float64)
            beta = nats / (wl.sm_scale * float(qv @ qv))
            t = int(rng.integers(lo, L))
            page, slot = int(wl.block_table[b, t // wl.bt]), t % wl.bt
            kscale = ks[g] if ks.size > 1 else ks[0]
            wl.k_cache[page, slot, g, :] = _e4m3_encode((beta * qv / kscale).astype(np.float32))
    wl.q_bits[...] = _bf16_bits(q)

# (case, flags, num_splits)
SMALL_RUNS = []
for name in SMALL:
    for flags in (0, DOT):
        for ns in (0, 1, 3):
            SMALL_RUNS.append((name, flags, ns))
    if SMALL[name]["bt"] >= 16:
        SMALL_RUNS.append((name, MFMA, 0))

_small_cache = {}


def _small(name):
    if name not in _small_cache:
        kw = dict(SMALL[name])
        wl = make_workload(seed=100 + list(SMALL).index(name), **kw)
        if name == "big_negative_sinks":
            wl.sinks[:] = -30.0
        if name.startswith("peaked_row") or name.startswith("big_positive_sinks"):
            _shift_values(wl, 2.0)
        if name.startswith("peaked_row"):
            _peak_one_key(wl, np.random.default_rng(7))
        if name.startswith("big_positive_sinks"):
            wl.sinks[:] = 12.0
            wl.sinks[::3] = 8.0
        ref = oracle.decode(**wl.oracle_kwargs())
        _small_cache[name] = (wl, upload(wl), ref)
    return _small_cache[name]


@pytest.mark.parametrize("name,flags,ns", SMALL_RUNS)
def test_parity_small(name, flags, ns):
    wl, t, (ro, rl) = _small(name)
    out, lse = to_host(*run(wl, t, num_splits=ns, flags=flags))
    compare(out, lse, ro, rl, label=f"{name} flags={flags} splits={ns}")


HND_CASES = ["gqa4_ragged", "d64_window_sinks", "d256_bt64", "mtp4_window_sinks", "bt1_pages",
             "pair_q2_perhead", "kg4_gqa_ragged", "prefill_q64", "mha_rows1", "batch130_mqa",
             "prefill_q32_lw8_hnd_pages", "prefill_q16_lw4_d64", "prefill_q24_lw2", "padded_zero_lengths"]


@pytest.mark.parametrize("name", HND_CASES)
@pytest.mark.parametrize("flags,ns", [(0, 0), (0, 3), (DOT, 0)])
def test_parity_head_major_pages(name, flags, ns):
    """The same pages stored head-major ([blocks, Hkv, bt, D]); the oracle's
    result does not depend on the layout (pinned on the CPU)."""
    wl, _, (ro, rl) = _small(name)
    t = upload(wl, kv_layout="HND")
    out, lse = to_host(*run(wl, t, num_splits=ns, flags=flags))
    compare(out, lse, ro, rl, label=f"{name} HND flags={flags} splits={ns}")


@pytest.mark.parametrize("name", ["gqa4_ragged", "prefill_q64", "d256_bt64"])
@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("flags,ns", [(0, 0), (0, 3), (DOT, 0)])
def test_parity_interleaved_e4m3_pages(name, layout, flags, ns):
    """K and V pages interleaved in one buffer ([blocks, 2, page]): the pools
    are strided views whose page stride is two pages, and the result is the
    dense pools' (the oracle's)."""
    wl, _, (ro, rl) = _small(name)
    t = upload(wl, kv_layout=layout)
    buf = torch.stack([t["k"], t["v"]], dim=1)
    t["k"], t["v"] = buf[:, 0], buf[:, 1]
    assert t["k"].stride(0) == 2 * t["k"][0].numel()
    out, lse = to_host(*run(wl, t, num_splits=ns, flags=flags))
    compare(out, lse, ro, rl, label=f"{name} interleaved {layout} flags={flags} splits={ns}")


def test_parity_output_without_lse_pointer():
    wl, t, (ro, rl) = _small("mtp4_window_sinks")
    out = torch.empty(tuple(wl.q_bits.shape), dtype=torch.bfloat16, device="cuda")
    shape = fp.shape_for(t["q"], t["k"], t["bt"], t["ks"], t["vs"], window=wl.window,
                         sm_scale=wl.sm_scale, max_seq_len=int(wl.seq_lens.max()))
    n = fp.fp8pa_workspace_bytes(shape)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    fp.fp8pa_decode(shape, t["q"], t["k"], t["v"], t["bt"], t["sl"], t["ks"], t["vs"], t["sinks"],
                    out, None, ws if n else None, n)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    compare(o, rl, ro, rl, label="lse=NULL")


def test_partial_only_flag_skips_the_merge():
    # a merge plan: the partial pass alone leaves out / lse untouched
    wl, t, (ro, rl) = _small("gqa4_ragged")
    shape = fp.shape_for(t["q"], t["k"], t["bt"], t["ks"], t["vs"], window=wl.window,
                         sm_scale=wl.sm_scale, max_seq_len=int(wl.seq_lens.max()),
                         flags=fp.FP8PA_FLAG_PARTIAL_ONLY)
    assert fp.fp8pa_plan(shape, 256)["merge_launched"] == 1
    n = fp.fp8pa_workspace_bytes(shape)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    out = torch.full(tuple(wl.q_bits.shape), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full(tuple(wl.q_bits.shape[:3]), 7.0, dtype=torch.float32, device="cuda")
    fp.fp8pa_decode(shape, t["q"], t["k"], t["v"], t["bt"], t["sl"], t["ks"], t["vs"], t["sinks"],
                    out, lse, ws, n)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())
    # a one-split plan has no merge to skip: the flag changes nothing
    shape1 = fp.shape_for(t["q"], t["k"], t["bt"], t["ks"], t["vs"], window=wl.window,
                          sm_scale=wl.sm_scale, max_seq_len=int(wl.seq_lens.max()), num_splits=1,
                          flags=fp.FP8PA_FLAG_PARTIAL_ONLY)
    assert fp.fp8pa_plan(shape1, 256)["merge_launched"] == 0
    fp.fp8pa_decode(shape1, t["q"], t["k"], t["v"], t["bt"], t["sl"], t["ks"], t["vs"], t["sinks"],
                    out, lse, None, 0)
    o, l = to_host(out, lse)
    compare(o, l, ro, rl, label="partial-only, one split")


def test_workspace_too_small_is_reported():
    wl, t, _ = _small("gqa4_ragged")
    shape = fp.shape_for(t["q"], t["k"], t["bt"], t["ks"], t["vs"], window=wl.window,
                         sm_scale=wl.sm_scale, max_seq_len=int(wl.seq_lens.max()), num_splits=3)
    n = fp.fp8pa_workspace_bytes(shape)
    assert n > 0
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    out = torch.empty(tuple(wl.q_bits.shape), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fp.Fp8paError) as e:
        fp.fp8pa_decode(shape, t["q"], t["k"], t["v"], t["bt"], t["sl"], t["ks"], t["vs"], None,
                        out, None, ws, n - 1)
    assert e.value.status == 3


# ------------------------------------------------------------------ merge

@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("R,S", [(40, 5), (10, 100), (3, 300)])
def test_merge_matches_oracle(D, R, S):
    """Few splits (one wavefront per row and 64 dims, or four), and many
    (sixteen wavefronts per row and 64 dims, each a share of the splits)."""
    rng = np.random.default_rng(D + 7 * S)
    Hq = 8
    po = rng.standard_normal((R, S, D)).astype(np.float32)
    pl = (rng.standard_normal((R, S)) * 3).astype(np.float32)
    pl[rng.random((R, S)) < 0.25] = -np.inf
    pl[min(3, R - 1), :] = -np.inf
    po[np.isneginf(pl)] = np.nan            # never read for an empty split
    sinks = rng.standard_normal(Hq).astype(np.float32)
    for use_sinks in (False, True):
        out = torch.empty((R, D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((R,), dtype=torch.float32, device="cuda")
        sk = torch.from_numpy(sinks).cuda() if use_sinks else None
        fp.fp8pa_merge(S, R, Hq, D, torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(), sk,
                       out, lse)
        torch.cuda.synchronize()
        ro, rl = oracle.merge(po.astype(np.float64), pl.astype(np.float64),
                              np.tile(sinks, R // Hq + 1)[:R] if use_sinks else None)
        compare(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, label=f"merge D={D} R={R} S={S}")


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("S", [1, 2, 8, 9, 20])
def test_merge_many_rows_matches_oracle(D, S):
    """More rows than one round of (row, 64 dims) workgroups holds (chunked
    prefill): the many-rows merge, 4 rows per wavefront, splits in batches,
    a row count that is not a multiple of 4, empty splits with NaN payloads."""
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    R, Hq = (32 * cu) // (D // 64) + 7, 8
    rng = np.random.default_rng(1000 * D + S)
    po = rng.standard_normal((R, S, D)).astype(np.float32)
    pl = (rng.standard_normal((R, S)) * 3).astype(np.float32)
    pl[rng.random((R, S)) < 0.25] = -np.inf
    pl[5, :] = -np.inf
    po[np.isneginf(pl)] = np.nan
    sinks = rng.standard_normal(Hq).astype(np.float32)
    for use_sinks in (False, True):
        out = torch.empty((R, D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((R,), dtype=torch.float32, device="cuda")
        sk = torch.from_numpy(sinks).cuda() if use_sinks else None
        fp.fp8pa_merge(S, R, Hq, D, torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(), sk, out, lse)
        torch.cuda.synchronize()
        ro, rl = oracle.merge(po.astype(np.float64), pl.astype(np.float64),
                              np.tile(sinks, R // Hq + 1)[:R] if use_sinks else None)
        compare(out.float().cpu().numpy(), lse.cpu().numpy(), ro, rl, label=f"many-rows merge D={D} S={S}")


# --------------------------------------------------- full-size named workloads

_cfg_cache = {}


def _cfg(k):
    if k not in _cfg_cache:
        _cfg_cache.clear()
        torch.cuda.empty_cache()
        wl = make_config(k)
        _cfg_cache[k] = (wl, upload(wl))
    return _cfg_cache[k]


_ref_cache = {}


def _cfg_ref(k):
    """The oracle's output for every row of workload k (and its time)."""
    if k not in _ref_cache:
        _ref_cache.clear()
        wl, _ = _cfg(k)
        t0 = time.perf_counter()
        ro, rl = oracle.decode(**wl.oracle_kwargs())
        _ref_cache[k] = (ro, rl, time.perf_counter() - t0)
    return _ref_cache[k]


FULL_RUNS = [(k, v) for k in (1, 2, 3, 4, 5) for v in ("planned", "dot")]


@pytest.mark.parametrize("k,variant", FULL_RUNS)
def test_parity_full_workload(k, variant):
    """Every output row of each named workload, at full size, against the
    oracle (which takes seconds per workload on the host): in the launch
    configuration the benchmark times ("planned"), and with the VALU
    kernel forced ("dot"), the path of kv heads with one or two query rows."""
    wl, t = _cfg(k)
    out, lse = run(wl, t, flags=DOT if variant == "dot" else 0)
    o, l = to_host(out, lse)
    ro, rl, secs = _cfg_ref(k)
    err, ratio, lerr = compare(o, l, ro, rl, label=f"cfg{k} {variant}")
    rel = float(np.max(np.abs(o - ro) / np.maximum(np.abs(ro), 1e-3)))
    print(f"\n[full parity] cfg{k} {variant}: {o.size} outputs, max |dout| {err:.3e}, max err/tol "
          f"{ratio:.3f}, max |dout|/max(|ref|, 1e-3) {rel:.3e}, max |dlse| {lerr:.3e}; oracle {secs:.1f} s "
          f"({wl.B * wl.q_len / secs:.1f} tokens/s)", flush=True)


def test_determinism_and_split_invariance_cfg2():
    wl, t = _cfg(2)
    a = to_host(*run(wl, t))
    b = to_host(*run(wl, t))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), "run-to-run bits differ"
    for ns in (1, 7):
        c = to_host(*run(wl, t, num_splits=ns))
        # different split counts change only rounding
        assert np.max(np.abs(c[0] - a[0])) < 2e-2
        assert np.max(np.abs(c[1] - a[1])) < 1e-3


def _repeat_bitwise(wl, t, label):
    """Eight eager calls and three graph replays of one call give the same
    bits: the kernels have no race and no timing-dependent read (a VALU read
    of an MFMA result too early, say, shows up here as run-to-run noise)."""
    ns = 0
    ref = tuple(x.clone() for x in run(wl, t, num_splits=ns))
    for i in range(8):
        got = run(wl, t, num_splits=ns)
        assert all(torch.equal(g, r) for g, r in zip(got, ref)), f"{label}: eager call {i} differs"
    out, lse = torch.empty_like(ref[0]), torch.empty_like(ref[1])
    ws = _ws_for(wl, t, ns)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(wl, t, num_splits=ns, out=out, lse=lse, workspace=ws)
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), f"{label}: replay {i} differs"


@pytest.mark.parametrize("k,kg", [(2, 1), (2, 4), (3, 1), (5, 1)])
def test_bitwise_repeatable_full_workloads(k, kg):
    if kg == 1:
        wl, t = _cfg(k)
    else:
        _cfg_cache.clear()
        torch.cuda.empty_cache()
        wl = make_config(k, k_groups=kg)
        t = upload(wl)
    _repeat_bitwise(wl, t, f"cfg{k} k_groups={kg}")


@pytest.mark.parametrize("name", ["prefill_q64", "prefill_q16_lw4_d64", "mtp_q4_g8_lw2", "kg4_q8_few_keys_lw2"])
def test_bitwise_repeatable_shared_tiles(name):
    wl, t, _ = _small(name)
    _repeat_bitwise(wl, t, name)


def test_block_permutation_invariance_cfg2():
    wl, t = _cfg(2)
    a = to_host(*run(wl, t))
    g = torch.Generator().manual_seed(5)
    perm = torch.randperm(wl.num_blocks, generator=g)          # page j moves to perm[j]
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(wl.num_blocks)
    t2 = dict(t)
    t2["k"] = t["k"][inv.cuda()].contiguous()
    t2["v"] = t["v"][inv.cuda()].contiguous()
    btab = t["bt"].long()
    t2["bt"] = torch.where(btab >= 0, perm.cuda()[btab.clamp(min=0)], btab).int().contiguous()
    b = to_host(*run(wl, t2))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_graph_capture_replay_cfg5():
    wl, t = _cfg(5)
    shape = fp.shape_for(t["q"], t["k"], t["bt"], t["ks"], t["vs"], window=wl.window,
                         sm_scale=wl.sm_scale, max_seq_len=int(wl.seq_lens.max()), num_splits=3)
    n = fp.fp8pa_workspace_bytes(shape)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty(tuple(wl.q_bits.shape), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(tuple(wl.q_bits.shape[:3]), dtype=torch.float32, device="cuda")

    def call():
        fp.fp8pa_decode(shape, t["q"], t["k"], t["v"], t["bt"], t["sl"], t["ks"], t["vs"],
                        t["sinks"], out, lse, ws, n)

    call()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone())
    out.zero_()
    lse.zero_()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        before = torch.cuda.memory_allocated()
        call()
        after = torch.cuda.memory_allocated()
    # (torch's allocator sees only torch's own allocations; that the library
    # cannot allocate at all is pinned on the CPU by
    # test_library_imports_no_allocation_or_synchronisation)
    assert after == before
    for it in range(3):
        out.fill_(float(it))
        lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), f"replay {it} differs"


@pytest.mark.parametrize("name", ["prefill_q64", "prefill_q16_lw4_d64", "mtp_q4_g8_lw2"])
@pytest.mark.parametrize("ns", [0, 3])
def test_graph_capture_replay_shared_tiles(name, ns):
    """The kernels whose row groups share K/V tiles through LDS (8, 4 and 2
    groups), captured once and replayed: every replay equals the eager call
    bit for bit."""
    wl, t, _ = _small(name)
    out, lse = run(wl, t, num_splits=ns)
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(wl, t, num_splits=ns, out=out, lse=lse, workspace=_ws_for(wl, t, ns))
    for it in range(3):
        out.fill_(float(it))
        lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), f"{name}: replay {it} differs"


def _ws_for(wl, t, ns):
    """A workspace allocated before capture (the library allocates nothing)."""
    shape = fp.shape_for(t["q"], t["k"], t["bt"], t["ks"], t["vs"], window=wl.window,
                         sm_scale=wl.sm_scale, max_seq_len=max(1, int(wl.seq_lens.max())),
                         num_splits=ns, k_groups=wl.k_groups)
    return torch.empty(max(fp.fp8pa_workspace_bytes(shape), 256), dtype=torch.uint8, device="cuda")


# ------------------------------------------- sharded KV (context parallel)

def test_context_parallel_shards_merge():
    # The way the path shards a long sequence over devices, on one GPU: each
    # shard holds a page range of every sequence and runs fp8pa_decode over
    # it with no sink; fp8pa_merge then combines the shards' (out, lse) pairs
    # and adds the sink once.  q_len 1 and no window, so a shard's query
    # attends all its keys.
    wl = make_workload(seed=77, B=2, q_len=1, Hq=24, Hkv=4, D=256, bt=64, seq_lens=[3000, 1300],
                       scale=("per_head", 0.02, 0.1), sinks=True, sm_scale=0.08)
    ro, rl = oracle.decode(**wl.oracle_kwargs())
    t = upload(wl)
    split_pages = 12  # shard 0: tokens [0, 768) of each sequence; shard 1: the rest
    cut = split_pages * wl.bt
    assert all(L > cut for L in wl.seq_lens)
    rows = wl.B * wl.q_len * wl.Hq
    po = torch.empty((rows, 2, wl.D), dtype=torch.float32, device="cuda")
    pl = torch.empty((rows, 2), dtype=torch.float32, device="cuda")
    tables = [t["bt"][:, :split_pages].contiguous(), t["bt"][:, split_pages:].contiguous()]
    lens = [torch.full_like(t["sl"], cut), t["sl"] - cut]
    for s in range(2):
        shape = fp.shape_for(t["q"], t["k"], tables[s], t["ks"], t["vs"], window=0, sm_scale=wl.sm_scale,
                             max_seq_len=int(lens[s].max()))
        n = fp.fp8pa_workspace_bytes(shape)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
        out = torch.empty(tuple(wl.q_bits.shape), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(tuple(wl.q_bits.shape[:3]), dtype=torch.float32, device="cuda")
        fp.fp8pa_decode(shape, t["q"], t["k"], t["v"], tables[s], lens[s], t["ks"], t["vs"], None,
                        out, lse, ws if n else None, n)
        po[:, s, :] = out.reshape(rows, wl.D).float()
        pl[:, s] = lse.reshape(rows)
    out = torch.empty(tuple(wl.q_bits.shape), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(tuple(wl.q_bits.shape[:3]), dtype=torch.float32, device="cuda")
    fp.fp8pa_merge(2, rows, wl.Hq, wl.D, po, pl, t["sinks"], out, lse)
    o, l = to_host(out, lse)
    compare(o, l, ro, rl, label="two KV shards + merge")


# ------------------------------------------------------------- size limits

@pytest.mark.parametrize("flags", [0, DOT])
def test_pool_beyond_4_gib(flags):
    """A 4.9 GiB pool per side (300,000 pages of 16 KiB) whose attended pages
    sit at its top: page offsets need more than 32 bits.  The oracle reads
    the same pages renumbered into a small pool (page permutation is pinned
    to be exact)."""
    wl = make_workload(B=2, q_len=1, Hq=32, Hkv=8, D=128, bt=16, seq_lens=[700, 1500],
                       scale=("per_head", 0.02, 0.1), sinks=True, seed=77, table="identity")
    ro, rl = oracle.decode(**wl.oracle_kwargs())
    nbig = 300_000
    top = nbig - wl.num_blocks                       # small page j lives at big page top + j
    page = wl.bt * wl.Hkv * wl.D
    assert top * page > (1 << 32)
    kbig = torch.full((nbig, wl.bt, wl.Hkv, wl.D), oracle_poison(), dtype=torch.uint8, device="cuda")
    vbig = torch.full_like(kbig, oracle_poison())
    kbig[top:] = torch.from_numpy(wl.k_cache).cuda()
    vbig[top:] = torch.from_numpy(wl.v_cache).cuda()
    t = upload(wl)
    t["k"], t["v"] = kbig, vbig
    t["bt"] = torch.from_numpy(np.where(wl.block_table >= 0, wl.block_table + top, -1).astype(np.int32)).cuda()
    out, lse = to_host(*run(wl, t, flags=flags))
    compare(out, lse, ro, rl, label=f"4.9 GiB pool flags={flags}")
    del kbig, vbig, t
    torch.cuda.empty_cache()


def oracle_poison():
    from workloads import POISON_CODE
    return POISON_CODE


@pytest.mark.parametrize("D,flags,ns", [(128, 0, 0), (128, DOT, 0), (256, 0, 3), (64, 0, 0), (64, DOT, 2)])
def test_largest_pages(D, flags, ns):
    """1024-token pages (the largest the ABI takes), with windows that start
    and end inside pages."""
    wl = make_workload(B=2, q_len=2, Hq=8, Hkv=2, D=D, bt=1024, seq_lens=[2500, 700], window=900,
                       sinks=True, seed=88 + D, scale=("per_head", 0.02, 0.1))
    ro, rl = oracle.decode(**wl.oracle_kwargs())
    out, lse = to_host(*run(wl, upload(wl), num_splits=ns, flags=flags))
    compare(out, lse, ro, rl, label=f"bt 1024 D {D} flags={flags} splits={ns}")
