"""GPU parity of the MXFP8 KV path (bf16-MFMA and VALU kernels, writer)
against the oracle.

Decode outputs are compared element by element with the float64 oracle at
small sizes (token- and head-major pages, padded and interleaved page
strides, windows, sinks, several splits) and on every row of a
full-size ragged GQA batch; the writer's bytes are compared bit for bit.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_harness import compare, run, to_host, upload
from workloads import CONFIGS, make_mxfp8_workload

torch = pytest.importorskip("torch")
fp = pytest.importorskip("decode_attention_paged_fp8pa_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp.lib()


def test_hw_mxfp8_block_decode_matches_oracle():
    """Every E4M3 code, with E8M0 scales whose products stay inside bf16's
    exact range (2^-133 .. 2^127 for three mantissa bits): the kernel's
    element order and values equal the oracle's E4M3 x 2^(s - 127)."""
    rng = np.random.default_rng(3)
    data = np.arange(256, dtype=np.uint8).repeat(4)            # 32 blocks of 32 bytes
    rng.shuffle(data)
    n = data.size // 32
    scales = np.r_[3, 127, 246, rng.integers(3, 247, size=n - 3)].astype(np.uint8)
    out = torch.empty(32 * n, dtype=torch.float32, device="cuda")
    fp.fp8pa_debug_mxfp8(torch.from_numpy(data).cuda(), torch.from_numpy(scales).cuda(), out, n)
    torch.cuda.synchronize()
    want = oracle.E4M3_TABLE[data.reshape(n, 32)] * oracle.e8m0_decode(scales)[:, None]
    got = out.cpu().numpy().reshape(n, 32).astype(np.float64)
    assert np.array_equal(got, want, equal_nan=True)


MX_SMALL = {
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


def _mx(name):
    if name not in _cache:
        wl = make_mxfp8_workload(seed=400 + list(MX_SMALL).index(name), **MX_SMALL[name])
        _cache[name] = (wl, upload(wl), oracle.decode(**wl.oracle_kwargs()))
    return _cache[name]


@pytest.mark.parametrize("name", list(MX_SMALL))
@pytest.mark.parametrize("flags,ns", [(0, 0), (0, 1), (0, 3), (fp.FP8PA_FLAG_FORCE_DOT, 0),
                                      (fp.FP8PA_FLAG_FORCE_DOT, 3)])
def test_mxfp8_parity_small(name, flags, ns):
    """The planner's kernel (bf16 MFMA at head_dim 64/128 with bt >= 16 and
    >= 3 rows per kv head, else the VALU kernel) and the forced VALU kernel."""
    wl, t, (ro, rl) = _mx(name)
    out, lse = to_host(*run(wl, t, num_splits=ns, flags=flags))
    compare(out, lse, ro, rl, label=f"mxfp8 {name} flags={flags} splits={ns}")


def test_mxfp8_interleaved_k_and_v_pages():
    """The gist's page order: [K side | V side] per block; the pools passed are
    views of one buffer, each with a page stride of two sides."""
    wl, _, (ro, rl) = _mx("gqa_hnd_window_sinks")
    side = oracle.mxfp8_side_bytes(wl.Hkv, wl.bt, wl.D)
    both = np.concatenate([wl.k_cache[:, :side], wl.v_cache[:, :side]], axis=1)
    buf = torch.from_numpy(both).cuda()
    t = upload(wl)
    t["k"], t["v"] = buf[:, :side], buf[:, side:]
    out, lse = to_host(*run(wl, t))
    compare(out, lse, ro, rl, label="mxfp8 interleaved pages")


def test_mxfp8_parity_full_size_ragged_gqa():
    """The ragged GQA batch (16 sequences of 1024-8192 tokens, Hq 32, Hkv 8,
    D 128) with MXFP8 pages, in the launch configuration the bench times;
    every row against the oracle."""
    c = CONFIGS[2]
    wl = make_mxfp8_workload(B=c["B"], q_len=c["q_len"], Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"], bt=c["bt"],
                             seq_lens=("uniform", c["seq"][1], c["seq"][2]), seed=1003, pool=c["pool"],
                             scale=c["scale"], sm_scale=c["sm_scale"], kv_layout="HND")
    t = upload(wl)
    out, lse = to_host(*run(wl, t))
    ro, rl = oracle.decode(**wl.oracle_kwargs())   # every row: seconds on the host
    compare(out, lse, ro, rl, label="mxfp8 full-size ragged GQA")
    # the same bits on every call (no race, no timing-dependent read)
    ref = tuple(x.clone() for x in run(wl, t))
    for i in range(6):
        got = run(wl, t)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), f"mxfp8 call {i} differs"


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("layout,stride,per_head", [("NHD", 0, True), ("HND", 0, False), ("HND", 8704, True)])
def test_mxfp8_writer_matches_oracle(layout, stride, per_head):
    rng = np.random.default_rng(17)
    T, Hkv, D, bt, nb = 70, 4, 128, 16, 6
    side = oracle.mxfp8_side_bytes(Hkv, bt, D)
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
                   torch.from_numpy(vs).cuda(), kc, vc, kv_layout=layout, kv_format="mxfp8", block_tokens=bt)
    torch.cuda.synchronize()
    wk, wv = oracle.mxfp8_cache_write(_bits(key), _bits(value), slots, ks, vs, k0, v0, Hkv, bt, D, layout)
    for got, want, name in ((kc.cpu().numpy(), wk, "k"), (vc.cpu().numpy(), wv, "v")):
        diff = got != want
        assert not diff.any(), (name, np.argwhere(diff)[:5], got[diff][:5], want[diff][:5])


def test_mxfp8_write_then_decode():
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
    side = oracle.mxfp8_side_bytes(Hkv, bt, D)
    zero = np.zeros((nb, side), np.uint8)
    kc, vc = torch.from_numpy(zero).cuda(), torch.from_numpy(zero).cuda()
    ks_t, vs_t = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
    slot_t = torch.tensor(slots, dtype=torch.int64).cuda()
    fp.cache_write(key, value, slot_t, ks_t, vs_t, kc, vc, kv_format="mxfp8", block_tokens=bt)
    wk, wv = oracle.mxfp8_cache_write(_bits(key), _bits(value), np.array(slots), ks, vs, zero, zero,
                                      Hkv, bt, D)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), wk) and np.array_equal(vc.cpu().numpy(), wv)
    q = torch.from_numpy(rng.standard_normal((B, 1, Hq, D)).astype(np.float32)).to(torch.bfloat16).cuda()
    out, lse = fp.decode(q, kc, vc, torch.from_numpy(table).cuda(), torch.tensor(lens, dtype=torch.int32).cuda(),
                         ks_t, vs_t, None, sm_scale=1 / np.sqrt(D), kv_format="mxfp8", num_kv_heads=Hkv,
                         block_tokens=bt)
    ro, rl = oracle.decode(q_bits=_bits(q), k_cache=wk, v_cache=wv, block_table=table,
                           seq_lens=np.array(lens, np.int32), k_scale=ks, v_scale=vs,
                           sm_scale=1 / np.sqrt(D), kv_format="mxfp8", num_kv_heads=Hkv, block_tokens=bt)
    o, l = to_host(out, lse)
    compare(o, l, ro, rl, label="mxfp8 cache_write -> decode")


# Scale-byte centres (K, V) per sequence: with the draw's spread of -2..+3
# the bytes cover 10..200, the range fp8pa.h supports.
E8M0_CENTRES = [(12, 197), (40, 12), (70, 150), (100, 70), (121, 121), (150, 40), (180, 180), (197, 100)]


@pytest.mark.parametrize("flags", [0, fp.FP8PA_FLAG_FORCE_DOT])
def test_mxfp8_scale_bytes_across_the_supported_range(flags):
    """MXFP8 pages whose E8M0 bytes cover 10..200 (elements from 2^-126 to
    about 2^82).  Sequence b's queries are scaled by 2^(121 - k centre) so that
    its scores keep the magnitude of the other MXFP8 cases (the LSE bar is
    absolute), and its outputs, which scale with 2^(v centre - 127), are
    compared after dividing both sides by 2^(v centre - 121), an exact power
    of two, so the bar keeps its meaning at every magnitude."""
    B = len(E8M0_CENTRES)
    wl = make_mxfp8_workload(B=B, q_len=2, Hq=16, Hkv=4, D=128, bt=16,
                             seq_lens=[70, 300, 33, 200, 513, 96, 17, 260], seed=61, sinks=True,
                             scale=("per_head", 0.02, 0.1), e8m0_centers=E8M0_CENTRES)
    q = (wl.q_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for b, (ck, _) in enumerate(E8M0_CENTRES):
        q[b] *= 2.0 ** (121 - ck)          # exact: a power of two on bf16 values
    from workloads.gen import _bf16_bits
    wl.q_bits[...] = _bf16_bits(q.astype(np.float32))
    ro, rl = oracle.decode(**wl.oracle_kwargs())
    o, l = to_host(*run(wl, upload(wl), flags=flags))
    norm = np.array([2.0 ** (cv - 121) for _, cv in E8M0_CENTRES]).reshape(B, 1, 1, 1)
    assert np.isfinite(ro).all() and np.isfinite(o).all()
    compare(o / norm, l, ro / norm, rl, label=f"mxfp8 e8m0 10..200 flags={flags}")
