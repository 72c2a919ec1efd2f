"""GPU parity of the NVFP4 KV path (VALU kernel and writer) against the oracle.

Decode outputs are compared element by element with the float64 oracle at
small sizes (token- and head-major pages, padded and interleaved page
strides, windows, sinks, several splits) and on every row of a
full-size ragged GQA batch; the writer's bytes are compared bit for bit.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_harness import compare, run, to_host, upload
from workloads import CONFIGS, make_nvfp4_workload

torch = pytest.importorskip("torch")
fp = pytest.importorskip("decode_attention_paged_fp8pa_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp.lib()


def test_hw_nvfp4_block_decode_matches_oracle():
    """Every data byte value, with scale codes across E4M3's range: the
    kernel's element order (low nibble first) and values, times the block
    scale, equal the oracle's E2M1 x E4M3 (exact in fp32)."""
    rng = np.random.default_rng(2)
    data = np.arange(256, dtype=np.uint8).repeat(2)            # 64 blocks of 8 bytes
    rng.shuffle(data)
    n = data.size // 8
    scales = rng.choice(np.r_[np.arange(0x00, 0x7F), np.arange(0x80, 0xFF)], size=n).astype(np.uint8)
    out = torch.empty(16 * n, dtype=torch.float32, device="cuda")
    fp.fp8pa_debug_nvfp4(torch.from_numpy(data).cuda(), torch.from_numpy(scales).cuda(), out, n)
    torch.cuda.synchronize()
    d = data.reshape(n, 8)
    codes = np.stack([d & 0xF, d >> 4], axis=-1).reshape(n, 16)
    want = oracle.E2M1_TABLE[codes] * oracle.E4M3_TABLE[scales][:, None]
    got = out.cpu().numpy().reshape(n, 16).astype(np.float64)
    assert np.array_equal(got, want)


NV_SMALL = {
    "gqa_nhd": dict(B=4, q_len=1, Hq=32, Hkv=8, D=128, bt=16, seq_lens=[33, 700, 129, 1000],
                    scale=("per_head", 0.02, 0.1)),
    "gqa_hnd_window_sinks": dict(B=3, q_len=1, Hq=16, Hkv=4, D=128, bt=16, seq_lens=[300, 45, 517],
                                 window=100, sinks=True, kv_layout="HND"),
    "d64_mtp": dict(B=2, q_len=4, Hq=16, Hkv=2, D=64, bt=32, seq_lens=[90, 251], window=40, sinks=True),
    "d256_bt64_hnd": dict(B=2, q_len=1, Hq=8, Hkv=2, D=256, bt=64, seq_lens=[1000, 65], kv_layout="HND",
                          scale=("per_head", 0.02, 0.1)),
    "mha_bt1": dict(B=2, q_len=1, Hq=4, Hkv=4, D=128, bt=1, seq_lens=[37, 90]),
    "padded_stride": dict(B=2, q_len=2, Hq=8, Hkv=2, D=128, bt=16, seq_lens=[200, 77], page_stride=4864,
                          sinks=True),
    "tiny_seqs": dict(B=4, q_len=1, Hq=8, Hkv=2, D=64, bt=16, seq_lens=[1, 17, 32, 33]),
    # empty batch slots and a sequence shorter than q_len
    "padded_short_q4": dict(B=3, q_len=4, Hq=8, Hkv=2, D=128, bt=16, seq_lens=[0, 150, 2], sinks=True),
    "d64_hnd_window_per_head": dict(B=3, q_len=1, Hq=32, Hkv=4, D=64, bt=32, seq_lens=[500, 96, 1200],
                                    window=200, sinks=True, kv_layout="HND", scale=("per_head", 0.02, 0.1)),
    "prefill_q40": dict(B=2, q_len=40, Hq=8, Hkv=2, D=128, bt=16, seq_lens=[40, 333], sinks=True),
    "batch130": dict(B=130, q_len=1, Hq=8, Hkv=1, D=128, bt=16,
                     seq_lens=[1 + (37 * i * i + 11 * i) % 600 for i in range(130)]),
}
_cache = {}


def _nv(name):
    if name not in _cache:
        wl = make_nvfp4_workload(seed=300 + list(NV_SMALL).index(name), **NV_SMALL[name])
        _cache[name] = (wl, upload(wl), oracle.decode(**wl.oracle_kwargs()))
    return _cache[name]


@pytest.mark.parametrize("name", list(NV_SMALL))
@pytest.mark.parametrize("flags,ns", [(0, 0), (0, 1), (0, 3), (fp.FP8PA_FLAG_FORCE_DOT, 0),
                                      (fp.FP8PA_FLAG_FORCE_DOT, 3)])
def test_nvfp4_parity_small(name, flags, ns):
    """The planner's kernel (f16 MFMA at head_dim 64/128 with bt >= 16 and
    >= 3 rows per kv head, else the VALU kernel) and the forced VALU kernel."""
    wl, t, (ro, rl) = _nv(name)
    out, lse = to_host(*run(wl, t, num_splits=ns, flags=flags))
    compare(out, lse, ro, rl, label=f"nvfp4 {name} flags={flags} splits={ns}")


# Large positive sinks dominate every row; with one split they enter the
# partial kernel's running maximum, so every key's weight is e^-8 .. e^-14 of
# it.  V codes are made non-negative (mean > 0), so a kernel that loses small
# weights from P.V (its P is f16, shifted by 2^7) misses a visible share of
# the output while the denominator keeps their mass.
NV_SINKS = {
    "big_sinks_mean_v": dict(B=2, q_len=1, Hq=16, Hkv=4, D=128, bt=16, seq_lens=[3000, 700], sinks=True),
    "big_sinks_mtp_d64_hnd": dict(B=2, q_len=4, Hq=16, Hkv=4, D=64, bt=16, seq_lens=[2000, 300], sinks=True,
                                  window=1000, kv_layout="HND"),
}
_sinks_cache = {}


def _nv_sinks(name):
    if name not in _sinks_cache:
        kw = NV_SINKS[name]
        wl = make_nvfp4_workload(seed=400 + list(NV_SINKS).index(name), **kw)
        data_bytes = kw["Hkv"] * kw["bt"] * kw["D"] // 2
        wl.v_cache[:, :data_bytes] &= 0x77          # clear each E2M1 code's sign bit
        wl.sinks[:] = 12.0
        wl.sinks[::3] = 8.0
        wl.sinks[1::4] = 14.0
        _sinks_cache[name] = (wl, upload(wl), oracle.decode(**wl.oracle_kwargs()))
    return _sinks_cache[name]


@pytest.mark.parametrize("name", list(NV_SINKS))
@pytest.mark.parametrize("flags,ns", [(0, 0), (0, 1), (0, 3), (fp.FP8PA_FLAG_FORCE_DOT, 1)])
def test_nvfp4_parity_big_positive_sinks(name, flags, ns):
    wl, t, (ro, rl) = _nv_sinks(name)
    out, lse = to_host(*run(wl, t, num_splits=ns, flags=flags))
    compare(out, lse, ro, rl, label=f"nvfp4 {name} flags={flags} splits={ns}")


def test_nvfp4_interleaved_k_and_v_pages():
    """The gist's page order: [K side | V side] per block; the pools passed are
    views of one buffer, each with a page stride of two sides."""
    wl, _, (ro, rl) = _nv("gqa_hnd_window_sinks")
    side = oracle.nvfp4_side_bytes(wl.Hkv, wl.bt, wl.D)
    both = np.concatenate([wl.k_cache[:, :side], wl.v_cache[:, :side]], axis=1)
    buf = torch.from_numpy(both).cuda()
    t = upload(wl)
    t["k"], t["v"] = buf[:, :side], buf[:, side:]
    out, lse = to_host(*run(wl, t))
    compare(out, lse, ro, rl, label="nvfp4 interleaved pages")


def test_nvfp4_parity_full_size_ragged_gqa():
    """The ragged GQA batch (16 sequences of 1024-8192 tokens, Hq 32, Hkv 8,
    D 128) with NVFP4 pages, in the launch configuration the bench times;
    every row against the oracle."""
    c = CONFIGS[2]
    wl = make_nvfp4_workload(B=c["B"], q_len=c["q_len"], Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"], bt=c["bt"],
                             seq_lens=("uniform", c["seq"][1], c["seq"][2]), seed=1002, pool=c["pool"],
                             scale=c["scale"], sm_scale=c["sm_scale"], kv_layout="HND")
    t = upload(wl)
    out, lse = to_host(*run(wl, t))
    ro, rl = oracle.decode(**wl.oracle_kwargs())   # every row: seconds on the host
    compare(out, lse, ro, rl, label="nvfp4 full-size ragged GQA")
    # the same bits on every call (no race, no timing-dependent read)
    ref = tuple(x.clone() for x in run(wl, t))
    for i in range(6):
        got = run(wl, t)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), f"nvfp4 call {i} differs"


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("layout,stride,per_head", [("NHD", 0, True), ("HND", 0, False), ("HND", 4864, True)])
def test_nvfp4_writer_matches_oracle(layout, stride, per_head):
    rng = np.random.default_rng(17)
    T, Hkv, D, bt, nb = 70, 4, 128, 16, 6
    side = oracle.nvfp4_side_bytes(Hkv, bt, D)
    page = stride or side
    mag = np.exp2(rng.uniform(-12, 10, size=(T, Hkv, D)))
    x = (rng.standard_normal((T, Hkv, D)) * mag).astype(np.float32)
    x[0, 0, :16] = 0.0                                       # an all-zero block
    x[1, 1, 16:32] = -0.0
    key = torch.from_numpy(x).to(torch.bfloat16).cuda()
    value = torch.from_numpy(x[::-1].copy()).to(torch.bfloat16).cuda()
    slots = rng.permutation(nb * bt)[:T].astype(np.int64)
    slots[5] = -1
    slots[9] = nb * bt + 2
    nsc = Hkv if per_head else 1
    ks = rng.uniform(0.01, 0.2, size=nsc).astype(np.float32)
    vs = rng.uniform(0.01, 0.2, size=nsc).astype(np.float32)
    k0 = rng.integers(0, 256, size=(nb, page)).astype(np.uint8)
    v0 = rng.integers(0, 256, size=(nb, page)).astype(np.uint8)
    kc, vc = torch.from_numpy(k0).cuda(), torch.from_numpy(v0).cuda()
    fp.cache_write(key, value, torch.from_numpy(slots).cuda(), torch.from_numpy(ks).cuda(),
                   torch.from_numpy(vs).cuda(), kc, vc, kv_layout=layout, kv_format="nvfp4", block_tokens=bt)
    torch.cuda.synchronize()
    wk, wv = oracle.nvfp4_cache_write(_bits(key), _bits(value), slots, ks, vs, k0, v0, Hkv, bt, D, layout)
    for got, want, name in ((kc.cpu().numpy(), wk, "k"), (vc.cpu().numpy(), wv, "v")):
        diff = got != want
        assert not diff.any(), (name, np.argwhere(diff)[:5], got[diff][:5], want[diff][:5])


def test_nvfp4_write_then_decode():
    rng = np.random.default_rng(23)
    B, Hq, Hkv, D, bt = 2, 16, 4, 128, 16
    lens = [300, 77]
    nb = sum((L + bt - 1) // bt for L in lens) + 2
    perm = rng.permutation(nb)
    table = np.full((B, max((L + bt - 1) // bt for L in lens)), -1, np.int32)
    slots, off = [], 0
    for b, L in enumerate(lens):
        pages = perm[off: off + (L + bt - 1) // bt]
        off += len(pages)
        table[b, : len(pages)] = pages
        slots.extend(int(pages[t // bt]) * bt + t % bt for t in range(L))
    T = len(slots)
    key = torch.from_numpy(rng.standard_normal((T, Hkv, D)).astype(np.float32)).to(torch.bfloat16).cuda()
    value = torch.from_numpy(rng.standard_normal((T, Hkv, D)).astype(np.float32)).to(torch.bfloat16).cuda()
    ks = rng.uniform(0.02, 0.1, size=Hkv).astype(np.float32)
    vs = rng.uniform(0.02, 0.1, size=Hkv).astype(np.float32)
    side = oracle.nvfp4_side_bytes(Hkv, bt, D)
    zero = np.zeros((nb, side), np.uint8)
    kc, vc = torch.from_numpy(zero).cuda(), torch.from_numpy(zero).cuda()
    ks_t, vs_t = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
    slot_t = torch.tensor(slots, dtype=torch.int64).cuda()
    fp.cache_write(key, value, slot_t, ks_t, vs_t, kc, vc, kv_format="nvfp4", block_tokens=bt)
    wk, wv = oracle.nvfp4_cache_write(_bits(key), _bits(value), np.array(slots), ks, vs, zero, zero,
                                      Hkv, bt, D)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), wk) and np.array_equal(vc.cpu().numpy(), wv)
    q = torch.from_numpy(rng.standard_normal((B, 1, Hq, D)).astype(np.float32)).to(torch.bfloat16).cuda()
    out, lse = fp.decode(q, kc, vc, torch.from_numpy(table).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(),
                         ks_t, vs_t, None, sm_scale=1 / np.sqrt(D), kv_format="nvfp4", num_kv_heads=Hkv,
                         block_tokens=bt)
    ro, rl = oracle.decode(q_bits=_bits(q), k_cache=wk, v_cache=wv, block_table=table,
                           seq_lens=np.array(lens, np.int32), k_scale=ks, v_scale=vs,
                           sm_scale=1 / np.sqrt(D), kv_format="nvfp4", num_kv_heads=Hkv, block_tokens=bt)
    o, l = to_host(out, lse)
    compare(o, l, ro, rl, label="nvfp4 cache_write -> decode")


def test_nvfp4_writer_golden_midpoint_block():
    """The hand-worked block of tests/golden/nvfp4_writer_midpoint.json
    through the GPU writer: scale byte 0x44 (the even code at the midpoint
    2.875) and the stated E2M1 codes, in every block of the row."""
    import json
    import os

    with open(os.path.join(os.path.dirname(__file__), "golden", "nvfp4_writer_midpoint.json")) as f:
        gd = json.load(f)
    Hkv, D, bt = 1, 64, 16
    blk = np.array([int(h, 16) for h in gd["x_bf16_bits"]], dtype=np.uint16)
    bits = np.tile(blk, D // 16).reshape(1, Hkv, D)
    key = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    ks = torch.from_numpy(np.array([int(gd["k_scale_f32_bits"], 16)], dtype=np.uint32).view(np.float32)).cuda()
    side = oracle.nvfp4_side_bytes(Hkv, bt, D)
    kc = torch.zeros((1, side), dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    fp.cache_write(key, key, torch.tensor([3], dtype=torch.int64).cuda(), ks, ks, kc, vc,
                   kv_format="nvfp4", block_tokens=bt)
    torch.cuda.synchronize()
    data = [int(h, 16) for h in gd["expected_data_bytes"]] * (D // 16)
    sbyte = int(gd["expected_scale_byte"], 16)
    for got in (kc.cpu().numpy()[0], vc.cpu().numpy()[0]):
        assert got[3 * (D // 2): 4 * (D // 2)].tolist() == data
        sc0 = bt * (D // 2)
        assert got[sc0 + 3 * (D // 16): sc0 + 4 * (D // 16)].tolist() == [sbyte] * (D // 16)
