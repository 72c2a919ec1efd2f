"""GPU parity of the KV-cache writer (fp8pa_cache_write) against the oracle.

Codes are compared bit for bit (a NaN input only has to give a NaN code);
a round trip writes a sequence's keys and values with the library and reads
them with fp8pa_decode.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_harness import compare, to_host
from workloads import make_workload

torch = pytest.importorskip("torch")
fp = pytest.importorskip("decode_attention_paged_fp8pa_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp.lib()


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _inputs(rng, T, Hkv, D, pad, specials):
    """bf16 [T, Hkv, D] views with `pad` extra elements per token row, values
    spread from the E4M3 subnormal range to past saturation."""
    mag = np.exp2(rng.uniform(-14, 11, size=(T, Hkv, D)))
    x = (rng.standard_normal((T, Hkv, D)) * mag).astype(np.float32)
    if specials:
        x[0, 0, :4] = [np.nan, np.inf, -np.inf, -0.0]
        x[min(1, T - 1), -1, -3:] = [448.0, 464.0, -1e6]
    full = torch.zeros((T, Hkv * D + pad), dtype=torch.bfloat16)
    full[:, : Hkv * D] = torch.from_numpy(x.reshape(T, Hkv * D)).to(torch.bfloat16)
    return full.cuda()[:, : Hkv * D].view(T, Hkv, D) if pad == 0 else \
        full.cuda().as_strided((T, Hkv, D), (Hkv * D + pad, D, 1))


CASES = [
    # T, Hkv, D, bt, num_blocks, pad, per_head, k_groups
    (37, 8, 128, 16, 5, 0, True, 1),
    (64, 4, 256, 64, 2, 24, False, 1),
    (100, 8, 64, 16, 10, 8, True, 1),
    (9, 2, 128, 1, 16, 0, True, 1),
    (1, 1, 64, 32, 1, 0, False, 1),
    # K scales in groups along head_dim
    (37, 8, 128, 16, 5, 0, True, 4),
    # head-major pages (k_groups negative here: the same case with HND pools)
    (37, 8, 128, 16, 5, 0, True, -4),
    (100, 8, 64, 16, 10, 8, True, -1),
    (64, 4, 256, 64, 2, 24, False, -8),
    (64, 4, 256, 64, 2, 24, False, 8),
    (100, 8, 64, 16, 10, 8, True, 2),
    (20, 2, 256, 16, 3, 0, True, 8),
]


@pytest.mark.parametrize("T,Hkv,D,bt,nb,pad,per_head,kg", CASES)
def test_writer_codes_match_oracle(T, Hkv, D, bt, nb, pad, per_head, kg):
    layout = "HND" if kg < 0 else "NHD"
    kg = abs(kg)
    rng = np.random.default_rng(T * 7 + D)
    key = _inputs(rng, T, Hkv, D, pad, True)
    value = _inputs(rng, T, Hkv, D, pad, False)
    nslots = nb * bt
    slots = rng.permutation(nslots)[:T] if T <= nslots else rng.integers(0, nslots, size=T)
    slots = slots.astype(np.int64)
    slots[rng.random(T) < 0.15] = -1          # skipped tokens
    if T > 2:
        slots[2] = nslots + 3                  # past the cache: skipped as well
    if T > nslots:                             # keep written slots distinct (no races)
        seen = set()
        for i, sl in enumerate(slots):
            if sl in seen:
                slots[i] = -1
            seen.add(sl)
    nsc = Hkv if per_head else 1
    ks = rng.uniform(0.01, 0.2, size=nsc * kg).astype(np.float32)
    vs = rng.uniform(0.01, 0.2, size=nsc).astype(np.float32)
    pool_shape = (nb, Hkv, bt, D) if layout == "HND" else (nb, bt, Hkv, D)
    k0 = rng.integers(0, 256, size=pool_shape).astype(np.uint8)
    v0 = rng.integers(0, 256, size=pool_shape).astype(np.uint8)
    kc, vc = torch.from_numpy(k0).cuda(), torch.from_numpy(v0).cuda()
    fp.cache_write(key, value, torch.from_numpy(slots).cuda(), torch.from_numpy(ks).cuda(),
                   torch.from_numpy(vs).cuda(), kc, vc, k_groups=kg, kv_layout=layout)
    torch.cuda.synchronize()
    want_k, want_v = oracle.cache_write(_bits(key), _bits(value), slots, ks, vs, k0, v0, k_groups=kg,
                                        kv_layout=layout)
    for got, want, name in ((kc.cpu().numpy(), want_k, "k"), (vc.cpu().numpy(), want_v, "v")):
        nan_w = np.isnan(oracle.E4M3_TABLE[want])
        assert np.array_equal(np.isnan(oracle.E4M3_TABLE[got]), nan_w), name
        diff = (got != want) & ~nan_w
        assert not diff.any(), (name, np.argwhere(diff)[:5], got[diff][:5], want[diff][:5])


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_writer_into_interleaved_pages(layout):
    """K and V pages interleaved in one buffer ([blocks, 2, page]): the pools
    are strided views, each written exactly where the dense pools would be,
    and the other half of every page keeps its bytes."""
    T, Hkv, D, bt, nb = 40, 4, 128, 16, 6
    rng = np.random.default_rng(31)
    key = _inputs(rng, T, Hkv, D, 0, True)
    value = _inputs(rng, T, Hkv, D, 0, False)
    slots = rng.permutation(nb * bt)[:T].astype(np.int64)
    slots[::7] = -1
    ks = rng.uniform(0.01, 0.2, size=Hkv).astype(np.float32)
    vs = rng.uniform(0.01, 0.2, size=Hkv).astype(np.float32)
    page = (Hkv, bt, D) if layout == "HND" else (bt, Hkv, D)
    buf0 = rng.integers(0, 256, size=(nb, 2) + page).astype(np.uint8)
    buf = torch.from_numpy(buf0).cuda()
    kc, vc = buf[:, 0], buf[:, 1]
    fp.cache_write(key, value, torch.from_numpy(slots).cuda(), torch.from_numpy(ks).cuda(),
                   torch.from_numpy(vs).cuda(), kc, vc, kv_layout=layout)
    torch.cuda.synchronize()
    want_k, want_v = oracle.cache_write(_bits(key), _bits(value), slots, ks, vs, buf0[:, 0].copy(),
                                        buf0[:, 1].copy(), kv_layout=layout)
    got = buf.cpu().numpy()
    for half, want, name in ((0, want_k, "k"), (1, want_v, "v")):
        g = got[:, half]
        nan_w = np.isnan(oracle.E4M3_TABLE[want])
        assert np.array_equal(np.isnan(oracle.E4M3_TABLE[g]), nan_w), name
        assert not ((g != want) & ~nan_w).any(), name


@pytest.mark.parametrize("kg", [1, 4])
def test_writer_then_decode_round_trip(kg):
    # keys and values of two sequences written by the library, then read back
    rng = np.random.default_rng(11 + kg)
    B, Hq, Hkv, D, bt = 2, 16, 4, 128, 16
    lens = [300, 77]
    nb = sum((L + bt - 1) // bt for L in lens) + 3
    perm = rng.permutation(nb)
    table = np.full((B, max((L + bt - 1) // bt for L in lens)), -1, np.int32)
    slots, k_rows, v_rows, off = [], [], [], 0
    for b, L in enumerate(lens):
        pages = perm[off: off + (L + bt - 1) // bt]
        off += len(pages)
        table[b, : len(pages)] = pages
        slots.extend(int(pages[t // bt]) * bt + t % bt for t in range(L))
    T = len(slots)
    key = torch.from_numpy(rng.standard_normal((T, Hkv, D)).astype(np.float32)).to(torch.bfloat16).cuda()
    value = torch.from_numpy(rng.standard_normal((T, Hkv, D)).astype(np.float32)).to(torch.bfloat16).cuda()
    ks = rng.uniform(0.02, 0.1, size=Hkv * kg).astype(np.float32)
    vs = rng.uniform(0.02, 0.1, size=Hkv).astype(np.float32)
    zeros = np.zeros((nb, bt, Hkv, D), np.uint8)
    kc, vc = torch.from_numpy(zeros).cuda(), torch.from_numpy(zeros).cuda()
    slot_t = torch.tensor(slots, dtype=torch.int64).cuda()
    ks_t, vs_t = torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda()
    fp.cache_write(key, value, slot_t, ks_t, vs_t, kc, vc, k_groups=kg)
    k_or, v_or = oracle.cache_write(_bits(key), _bits(value), np.array(slots), ks, vs, zeros, zeros,
                                    k_groups=kg)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), k_or) and np.array_equal(vc.cpu().numpy(), v_or)
    q = torch.from_numpy(rng.standard_normal((B, 1, Hq, D)).astype(np.float32)).to(torch.bfloat16).cuda()
    sl = torch.tensor(lens, dtype=torch.int32).cuda()
    bt_t = torch.from_numpy(table).cuda()
    out, lse = fp.decode(q, kc, vc, bt_t, sl, ks_t, vs_t, None, sm_scale=1 / np.sqrt(D), k_groups=kg)
    ro, rl = oracle.decode(q_bits=_bits(q), k_cache=k_or, v_cache=v_or, block_table=table,
                           seq_lens=np.array(lens, np.int32), k_scale=ks, v_scale=vs,
                           sm_scale=1 / np.sqrt(D), k_groups=kg)
    o, l = to_host(out, lse)
    compare(o, l, ro, rl, label="cache_write -> decode")


def test_writer_slots_beyond_4_gib():
    """Slots in the top pages of a 4.9 GiB pool (byte offsets past 2^32)."""
    rng = np.random.default_rng(31)
    T, Hkv, D, bt, nb = 40, 8, 128, 16, 300_000
    key = torch.from_numpy(rng.standard_normal((T, Hkv, D)).astype(np.float32)).to(torch.bfloat16).cuda()
    value = -key
    slots = (nb * bt - 1 - rng.permutation(4 * bt)[:T]).astype(np.int64)
    assert int(slots.min()) // bt * bt * Hkv * D > (1 << 32)
    ks = np.full((Hkv,), 0.05, np.float32)
    kc = torch.zeros((nb, bt, Hkv, D), dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    fp.cache_write(key, value, torch.from_numpy(slots).cuda(), torch.from_numpy(ks).cuda(),
                   torch.from_numpy(ks).cuda(), kc, vc)
    torch.cuda.synchronize()
    top = nb - 4
    small = np.zeros((4, bt, Hkv, D), np.uint8)
    wk, wv = oracle.cache_write(_bits(key), _bits(value), slots - top * bt, ks, ks, small, small)
    assert np.array_equal(kc[top:].cpu().numpy(), wk) and np.array_equal(vc[top:].cpu().numpy(), wv)
    assert int(kc[:top].sum().item()) == 0
    del kc, vc
    torch.cuda.empty_cache()


def test_writer_golden_reciprocal_order():
    """The hand-worked cases of tests/golden/writer_reciprocal_order.json on
    the GPU writer: each element of head h is the golden x under the golden
    scale of head h, so every code must be the golden one."""
    import json
    import os

    with open(os.path.join(os.path.dirname(__file__), "golden", "writer_reciprocal_order.json")) as f:
        cases = json.load(f)["cases"]
    Hkv, D, bt = len(cases), 64, 16
    bits = np.array([int(c["x_bf16_bits"], 16) for c in cases], dtype=np.uint16)
    scales = np.array([int(c["scale_f32_bits"], 16) for c in cases], dtype=np.uint32).view(np.float32)
    want = np.array([int(c["expected_code"], 16) for c in cases], dtype=np.uint8)
    key_bits = np.repeat(bits[None, :, None], D, axis=2)  # [1, Hkv, D]
    key = torch.from_numpy(key_bits.view(np.int16)).cuda().view(torch.bfloat16)
    kc = torch.zeros((1, bt, Hkv, D), dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    sc = torch.from_numpy(scales.copy()).cuda()
    fp.cache_write(key, key, torch.tensor([5], dtype=torch.int64).cuda(), sc, sc, kc, vc)
    torch.cuda.synchronize()
    for got in (kc.cpu().numpy(), vc.cpu().numpy()):
        assert np.array_equal(got[0, 5], np.repeat(want[:, None], D, axis=1))
