"""Calls on several streams.  fp8pa_decode keeps no state between calls (the
caller owns the workspace), so decodes of different batches issued on two
side streams, interleaved and overlapping, must give bit for bit what the
same calls give one after the other on the default stream; the stream
argument must be the one the work goes on; and a cache write followed by a
decode on one side stream must see the written pages.  Also: pools typed
torch.float8_e4m3fn behave exactly as the same bytes typed uint8, and sinks
at -inf add nothing."""

import numpy as np
import pytest

import oracle
from tests.gpu_harness import compare, run, to_host, upload
from workloads import make_nvfp4_workload, make_workload

torch = pytest.importorskip("torch")
fp = pytest.importorskip("decode_attention_paged_fp8pa_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp.lib()


def _cases():
    a = make_workload(B=6, q_len=1, Hq=32, Hkv=8, D=128, bt=16, seq_lens=("uniform", 300, 3000), seed=901)
    b = make_workload(B=3, q_len=4, Hq=16, Hkv=2, D=64, bt=32, seq_lens=[900, 40, 2500], window=700,
                      sinks=True, seed=902)
    c = make_nvfp4_workload(B=4, q_len=2, Hq=8, Hkv=2, D=128, bt=16, seq_lens=[100, 1200, 5, 800],
                            sinks=True, seed=903, kv_layout="HND")
    return [(w, upload(w, kv_layout=getattr(w, "kv_layout", "NHD"))) for w in (a, b, c)]


def test_concurrent_streams_match_one_stream():
    cases = _cases()
    refs = []
    for wl, t in cases:
        o, l = run(wl, t)
        refs.append((o.clone(), l.clone()))
    torch.cuda.synchronize()
    for (wl, _), (o, l) in zip(cases, refs):
        ro, rl = oracle.decode(**wl.oracle_kwargs())
        compare(*to_host(o, l), ro, rl, label=f"{wl.name} default stream")

    side = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    for s in side:
        s.wait_stream(torch.cuda.current_stream())
    got = []
    for rep in range(4):
        for i, (wl, t) in enumerate(cases):
            s = side[(i + rep) % 2]
            with torch.cuda.stream(s):
                o, l = run(wl, t, num_splits=0)
            got.append((i, rep, o, l))
    torch.cuda.synchronize()
    for i, rep, o, l in got:
        ro, rl = refs[i]
        assert torch.equal(o, ro), f"case {i} rep {rep}: output differs from the default-stream call"
        assert torch.equal(l, rl), f"case {i} rep {rep}: lse differs from the default-stream call"


def test_stream_argument_is_the_launch_stream():
    """With a side stream passed explicitly, the work goes there: after the
    side stream alone is synchronised, the result is complete."""
    (wl, t), = _cases()[:1]
    ro, rl = run(wl, t)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    out = torch.full_like(ro, float("nan"))
    lse = torch.full_like(rl, float("nan"))
    torch.cuda.synchronize()
    fp.decode(t["q"], t["k"], t["v"], t["bt"], t["sl"], t["ks"], t["vs"], t["sinks"], window=wl.window,
              sm_scale=wl.sm_scale, max_seq_len=int(wl.seq_lens.max()), out=out, lse=lse, stream=s)
    s.synchronize()
    assert torch.equal(out, ro) and torch.equal(lse, rl)


def test_write_then_decode_on_a_side_stream():
    """New tokens written into the pages and then attended, both on one side
    stream: the decode sees the written bytes (stream order)."""
    wl = make_workload(B=2, q_len=1, Hq=8, Hkv=2, D=128, bt=16, seq_lens=[200, 77], seed=904, poison=False)
    t = upload(wl)
    rng = np.random.default_rng(905)
    # overwrite the last 5 tokens of each sequence through the writer
    slots = []
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        for pos in range(L - 5, L):
            page = int(wl.block_table[b, pos // wl.bt])
            slots.append(page * wl.bt + pos % wl.bt)
    T = len(slots)
    key = torch.from_numpy(rng.standard_normal((T, wl.Hkv, wl.D)).astype(np.float32)).to("cuda").bfloat16()
    val = torch.from_numpy(rng.standard_normal((T, wl.Hkv, wl.D)).astype(np.float32)).to("cuda").bfloat16()
    slot_t = torch.tensor(slots, dtype=torch.int64, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fp.cache_write(key, val, slot_t, t["ks"], t["vs"], t["k"], t["v"])
        out, lse = run(wl, t)
    s.synchronize()
    # the oracle on the pages as the writer left them (read back after the stream is done)
    kw = wl.oracle_kwargs()
    kw["k_cache"] = t["k"].cpu().numpy().view(np.uint8)
    kw["v_cache"] = t["v"].cpu().numpy().view(np.uint8)
    ro, rl = oracle.decode(**kw)
    compare(*to_host(out, lse), ro, rl, label="write then decode on one side stream")
    # and the written bytes are the writer oracle's
    def bits(x):
        return x.view(torch.int16).cpu().numpy().view(np.uint16)

    want_k, want_v = oracle.cache_write(bits(key), bits(val), np.array(slots, dtype=np.int64), wl.k_scale,
                                        wl.v_scale, wl.k_cache, wl.v_cache)
    assert np.array_equal(kw["k_cache"], want_k) and np.array_equal(kw["v_cache"], want_v)


def test_float8_typed_pools_equal_byte_pools():
    """Pools may be torch.float8_e4m3fn as well as uint8 (the same bytes):
    decode and the cache writer give the same results bit for bit."""
    wl = make_workload(B=3, q_len=2, Hq=16, Hkv=4, D=128, bt=16, seq_lens=[300, 1000, 17], window=500,
                       sinks=True, seed=906)
    t = upload(wl)
    t8 = dict(t)
    t8["k"] = t["k"].clone().view(torch.float8_e4m3fn)
    t8["v"] = t["v"].clone().view(torch.float8_e4m3fn)
    o1, l1 = run(wl, t)
    o2, l2 = run(wl, t8)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ro, rl = oracle.decode(**wl.oracle_kwargs())
    compare(*to_host(o2, l2), ro, rl, label="float8_e4m3fn pools")
    # the writer into both forms of the same pages
    rng = np.random.default_rng(907)
    T = 40
    key = torch.from_numpy(rng.standard_normal((T, wl.Hkv, wl.D)).astype(np.float32)).to("cuda").bfloat16()
    val = torch.from_numpy(rng.standard_normal((T, wl.Hkv, wl.D)).astype(np.float32)).to("cuda").bfloat16()
    slots = torch.from_numpy(rng.permutation(t["k"].shape[0] * wl.bt)[:T].astype(np.int64)).to("cuda")
    fp.cache_write(key, val, slots, t["ks"], t["vs"], t["k"], t["v"])
    fp.cache_write(key, val, slots, t8["ks"], t8["vs"], t8["k"], t8["v"])
    torch.cuda.synchronize()
    assert torch.equal(t["k"], t8["k"].view(torch.uint8)) and torch.equal(t["v"], t8["v"].view(torch.uint8))


@pytest.mark.parametrize("fmt", ["e4m3", "nvfp4"])
@pytest.mark.parametrize("flags,ns", [(0, 0), (0, 1), (fp.FP8PA_FLAG_FORCE_DOT, 0)])
def test_sinks_at_minus_infinity(fmt, flags, ns):
    """A sink of -inf adds nothing: every sink at -inf gives the no-sink
    result bit for bit (one split, where the partial kernel folds the sink,
    and several, where the merge does), and a mix of -inf and finite sinks
    matches the oracle."""
    make = make_workload if fmt == "e4m3" else make_nvfp4_workload
    kw = dict(B=3, q_len=2, Hq=16, Hkv=4, D=128, bt=16, seq_lens=[500, 3, 1400], window=600, sinks=True, seed=960)
    if fmt != "e4m3":
        kw["kv_layout"] = "HND"
    wl = make(**kw)
    t = upload(wl)
    ref_o, ref_l = fp.decode(t["q"], t["k"], t["v"], t["bt"], t["sl"], t["ks"], t["vs"], None,
                             window=wl.window, sm_scale=wl.sm_scale, max_seq_len=int(wl.seq_lens.max()),
                             num_splits=ns, flags=flags, kv_layout=t["layout"], kv_format=fmt,
                             num_kv_heads=wl.Hkv, block_tokens=wl.bt)
    t["sinks"] = torch.full_like(t["sinks"], float("-inf"))
    o, l = run(wl, t, num_splits=ns, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)
    mixed = wl.sinks.copy()
    mixed[::2] = -np.inf
    wl.sinks[:] = mixed
    t["sinks"] = torch.from_numpy(mixed).cuda()
    ro, rl = oracle.decode(**wl.oracle_kwargs())
    compare(*to_host(*run(wl, t, num_splits=ns, flags=flags)), ro, rl, label=f"{fmt} mixed -inf sinks")
