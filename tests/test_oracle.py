"""Pins of the float64 oracle against things other than itself.

Each test ties one part of the oracle to a library routine, a closed form,
an invariant, a hand-worked example or a brute-force twin, so that a dropped
term, a wrong sign or index, or a transposed operand fails at least one.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests.brute_force import brute_decode
from workloads import make_workload, POISON_CODE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- E4M3 decode

def test_e4m3_table_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = oracle.E4M3_TABLE
    assert np.array_equal(np.isnan(ref), np.isnan(tab))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], tab[ok])
    # sign of zero as well
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(tab[ok]))


def test_e4m3_spec_values():
    n = 0
    with open(os.path.join(GOLDEN, "e4m3_spec_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            got = oracle.e4m3_decode_code(int(code, 16))
            want = float(val)
            if math.isnan(want):
                assert math.isnan(got)
            else:
                assert got == want and math.copysign(1, got) == math.copysign(1, want), code
            n += 1
    assert n >= 10


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    x = torch.from_numpy(rng.standard_normal(1000).astype(np.float32)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), x.to(torch.float64).numpy())


# ------------------------------------------------------------ worked example

def _golden_case(case):
    with open(os.path.join(GOLDEN, "handworked_tiny.json")) as f:
        g = json.load(f)
    return g


def test_handworked_tiny_example():
    g = _golden_case(None)
    for case in g["cases"]:
        out, lse = oracle.decode(
            np.array(g["q_bits"], dtype=np.uint16), np.array(g["k_codes"], dtype=np.uint8),
            np.array(g["v_codes"], dtype=np.uint8), np.array(g["block_table"], dtype=np.int32),
            np.array(g["seq_lens"], dtype=np.int32), np.array([1.0], np.float32),
            np.array([1.0], np.float32),
            sinks=None if case["sinks"] is None else np.array(case["sinks"], np.float32),
            window=case["window"], sm_scale=1.0)
        np.testing.assert_allclose(out.reshape(-1), case["out"], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(lse.reshape(-1), [case["lse"]], rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- brute force

TINY = [
    dict(B=2, q_len=1, Hq=4, Hkv=2, D=8, bt=4, seq_lens=[9, 17], window=0, sinks=False),
    dict(B=2, q_len=1, Hq=2, Hkv=1, D=16, bt=8, seq_lens=[40, 3], window=5, sinks=True),
    dict(B=1, q_len=4, Hq=4, Hkv=2, D=8, bt=4, seq_lens=[13], window=6, sinks=True),
    dict(B=2, q_len=3, Hq=3, Hkv=3, D=4, bt=2, seq_lens=[7, 3], window=0, sinks=False),
]


@pytest.mark.parametrize("k", range(len(TINY)))
def test_oracle_matches_brute_force(k):
    c = TINY[k]
    wl = make_workload(seed=10 + k, scale=("per_head", 0.02, 0.1), **c)
    out, lse = oracle.decode(**wl.oracle_kwargs())
    bo, bl = brute_decode(wl)
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-13)


def test_brute_force_partial_key_range():
    wl = make_workload(B=1, q_len=2, Hq=2, Hkv=1, D=8, bt=4, seq_lens=[21], seed=3, window=0)
    out, lse = oracle.decode(**wl.oracle_kwargs(), key_range=(4, 11))
    bo, bl = brute_decode(wl, key_range=(4, 11), sinks=None)
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- invariants

def _wl(**kw):
    base = dict(B=2, q_len=1, Hq=8, Hkv=2, D=32, bt=16, seq_lens=[100, 37], seed=7)
    base.update(kw)
    return make_workload(**base)


def test_block_permutation_invariance_is_bitwise():
    wl = _wl(window=20, sinks=True)
    out, lse = oracle.decode(**wl.oracle_kwargs())
    rng = np.random.default_rng(99)
    perm = rng.permutation(wl.num_blocks)          # new position of each old page
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    kc = np.empty_like(wl.k_cache)
    vc = np.empty_like(wl.v_cache)
    kc[perm] = wl.k_cache
    vc[perm] = wl.v_cache
    tab = np.where(wl.block_table >= 0, perm[np.maximum(wl.block_table, 0)], -1).astype(np.int32)
    kw = wl.oracle_kwargs()
    kw.update(k_cache=kc, v_cache=vc, block_table=tab)
    out2, lse2 = oracle.decode(**kw)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_zero_query_gives_mean_of_values():
    wl = _wl(q_zero=True, window=30)
    out, lse = oracle.decode(**wl.oracle_kwargs())
    from tests.brute_force import depage, _codes_to_float
    G = wl.Hq // wl.Hkv
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        lo = max(0, L - wl.window)
        V = _codes_to_float(depage(wl.v_cache, wl.block_table[b], L))[lo:L]
        for h in range(wl.Hq):
            vs = wl.v_scale[0]
            np.testing.assert_allclose(out[b, 0, h], V[:, h // G].mean(axis=0) * vs, rtol=1e-12, atol=1e-14)
            assert abs(lse[b, 0, h] - math.log(L - lo)) < 1e-12


def test_scale_folding_invariance():
    wl = _wl(sinks=True)
    out, lse = oracle.decode(**wl.oracle_kwargs())
    kw = wl.oracle_kwargs()
    c = 3.0
    kw.update(k_scale=wl.k_scale.astype(np.float64) * c, sm_scale=wl.sm_scale / c)
    out2, lse2 = oracle.decode(**kw)
    np.testing.assert_allclose(out, out2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-13)


# ------------------------------------------------ K scale groups along head_dim

KG_TINY = [
    dict(B=2, q_len=1, Hq=4, Hkv=2, D=8, bt=4, seq_lens=[9, 17], window=0, sinks=True,
         scale=("per_head", 0.02, 0.1), k_groups=2),
    dict(B=1, q_len=2, Hq=2, Hkv=1, D=16, bt=8, seq_lens=[23], window=7, sinks=False,
         scale=("tensor", 0.05), k_groups=4),
    dict(B=2, q_len=1, Hq=6, Hkv=3, D=16, bt=4, seq_lens=[5, 14], window=0, sinks=True,
         scale=("per_head", 0.01, 0.2), k_groups=8),
]


@pytest.mark.parametrize("k", range(len(KG_TINY)))
def test_k_groups_oracle_matches_brute_force(k):
    wl = make_workload(seed=40 + k, **KG_TINY[k])
    assert wl.k_scale.size in (wl.k_groups, wl.Hkv * wl.k_groups)
    out, lse = oracle.decode(**wl.oracle_kwargs())
    bo, bl = brute_decode(wl)
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-13)


def test_k_groups_with_equal_scales_is_one_scale():
    wl = _wl(scale=("per_head", 0.02, 0.1), sinks=True, window=40)
    out, lse = oracle.decode(**wl.oracle_kwargs())
    kw = wl.oracle_kwargs()
    kw.update(k_scale=np.repeat(wl.k_scale, 4), k_groups=4)   # [Hkv, 4], equal within a head
    out2, lse2 = oracle.decode(**kw)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_k_groups_scale_moves_into_the_query():
    """Multiplying group j's K scale by a power of two and the query's dims of
    that group by its inverse changes no score, so no output (bf16 queries
    stay exact under power-of-two scaling)."""
    import torch
    wl = make_workload(B=2, q_len=1, Hq=8, Hkv=2, D=32, bt=16, seq_lens=[70, 33], seed=8,
                       scale=("per_head", 0.02, 0.1), sinks=True, k_groups=4)
    out, lse = oracle.decode(**wl.oracle_kwargs())
    f = np.array([2.0, 0.5, 4.0, 0.25])
    ks2 = (wl.k_scale.reshape(wl.Hkv, 4) * f).astype(np.float32).reshape(-1)
    q = torch.from_numpy(wl.q_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    q = q / torch.from_numpy(np.repeat(f, 8))
    q_bits = q.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    kw = wl.oracle_kwargs()
    kw.update(q_bits=q_bits, k_scale=ks2)
    out2, lse2 = oracle.decode(**kw)
    np.testing.assert_allclose(out, out2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lse2, rtol=1e-12, atol=1e-13)


def test_k_groups_per_tensor_scale_layout():
    """A [k_groups] scale serves every kv head: it equals the [Hkv, k_groups]
    scale that repeats it per head."""
    wl = make_workload(B=1, q_len=1, Hq=4, Hkv=2, D=32, bt=8, seq_lens=[30], seed=9,
                       scale=("tensor", 0.05), k_groups=2)
    assert wl.k_scale.size == 2
    out, lse = oracle.decode(**wl.oracle_kwargs())
    kw = wl.oracle_kwargs()
    kw.update(k_scale=np.tile(wl.k_scale, 2))
    out2, lse2 = oracle.decode(**kw)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    d = oracle.k_scale_of_head(np.arange(6, dtype=np.float32), 1, 12, 3)
    assert list(d) == [3] * 4 + [4] * 4 + [5] * 4


# ------------------------------------------------------ head-major (HND) pages

def test_hnd_pages_equal_token_major_pages():
    """The same pages stored head-major ([blocks, Hkv, bt, D]) decode to
    exactly the token-major result; poison bytes (NaN codes) in unattended
    slots catch a read at a wrong place."""
    for kw in (dict(window=20, sinks=True), dict(scale=("per_head", 0.02, 0.1), k_groups=2)):
        wl = _wl(**kw)
        out, lse = oracle.decode(**wl.oracle_kwargs())
        k2 = np.ascontiguousarray(wl.k_cache.transpose(0, 2, 1, 3))
        v2 = np.ascontiguousarray(wl.v_cache.transpose(0, 2, 1, 3))
        kw2 = wl.oracle_kwargs()
        kw2.update(k_cache=k2, v_cache=v2, kv_layout="HND")
        out2, lse2 = oracle.decode(**kw2)
        assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
        assert not np.isnan(out).any()


def test_hnd_gather_reads_head_major_offsets():
    """One hand-placed code: head 1, token 5 of a 4-token page layout lives at
    [page 1, head 1, slot 1] head-major and at [page 1, slot 1, head 1] token-major."""
    cache = np.zeros((2, 2, 4, 3), np.uint8)      # [blocks, Hkv, bt, D]
    cache[1, 1, 1, :] = [0x38, 0x40, 0xB8]         # 1.0, 2.0, -1.0
    got = oracle.fp8pa_ref._gather(cache, np.array([0, 1]), 1, np.array([5]), 1.0, "HND")
    assert got.tolist() == [[1.0, 2.0, -1.0]]
    nhd = np.ascontiguousarray(cache.transpose(0, 2, 1, 3))
    assert oracle.fp8pa_ref._gather(nhd, np.array([0, 1]), 1, np.array([5]), 1.0).tolist() == [[1.0, 2.0, -1.0]]


def _scores_row(wl, b, h, ts, i=0):
    """Scores of row (b, i, h) at positions ts computed with torch's E4M3 decode."""
    from tests.brute_force import depage, _codes_to_float, _bf16_to_float
    L = int(wl.seq_lens[b])
    G = wl.Hq // wl.Hkv
    K = _codes_to_float(depage(wl.k_cache, wl.block_table[b], L))[:, h // G] * wl.k_scale[0]
    q = _bf16_to_float(wl.q_bits[b, i, h])
    return wl.sm_scale * (K[ts] @ q)


def test_window_one_returns_own_value():
    for sinks in (False, True):
        wl = _wl(window=1, sinks=sinks)
        out, lse = oracle.decode(**wl.oracle_kwargs())
        from tests.brute_force import depage, _codes_to_float
        G = wl.Hq // wl.Hkv
        for b in range(wl.B):
            L = int(wl.seq_lens[b])
            V = _codes_to_float(depage(wl.v_cache, wl.block_table[b], L))
            for h in range(wl.Hq):
                s = _scores_row(wl, b, h, [L - 1])[0]
                v = V[L - 1, h // G] * wl.v_scale[0]
                if sinks:
                    sk = float(wl.sinks[h])
                    np.testing.assert_allclose(out[b, 0, h], v * math.exp(s) / (math.exp(s) + math.exp(sk)),
                                               rtol=1e-12, atol=1e-14)
                    assert abs(lse[b, 0, h] - math.log(math.exp(s) + math.exp(sk))) < 1e-12
                else:
                    np.testing.assert_allclose(out[b, 0, h], v, rtol=1e-15, atol=0)
                    assert abs(lse[b, 0, h] - s) < 1e-12


def test_window_at_least_seq_len_equals_no_window():
    wl = _wl(sinks=True)
    out0, lse0 = oracle.decode(**wl.oracle_kwargs())
    kw = wl.oracle_kwargs()
    kw["window"] = int(wl.seq_lens.max())
    out1, lse1 = oracle.decode(**kw)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def test_multi_token_rows_equal_single_token_calls():
    wl = make_workload(B=2, q_len=4, Hq=4, Hkv=2, D=16, bt=16, seq_lens=[50, 9], seed=5,
                       window=7, sinks=True)
    out, lse = oracle.decode(**wl.oracle_kwargs())
    for i in range(4):
        kw = wl.oracle_kwargs()
        kw["q_bits"] = wl.q_bits[:, i:i + 1]
        kw["seq_lens"] = wl.seq_lens - (4 - 1 - i)
        o1, l1 = oracle.decode(**kw)
        np.testing.assert_allclose(out[:, i], o1[:, 0], rtol=1e-14, atol=0)
        np.testing.assert_allclose(lse[:, i], l1[:, 0], rtol=1e-14, atol=0)


@pytest.mark.parametrize("sinks", [True, False])
def test_padded_and_short_sequences(sinks):
    """Sequences shorter than q_len, down to 0 tokens (a batch padded with
    empty slots): a query whose position L - q_len + i is negative attends
    nothing, so its output is 0 and its LSE the sink logit (or -inf); the
    other rows follow the plain definition (pure-Python brute force)."""
    from tests.brute_force import brute_decode
    wl = make_workload(B=3, q_len=4, Hq=4, Hkv=2, D=16, bt=16, seq_lens=[0, 23, 2], seed=11,
                       sinks=sinks)
    out, lse = oracle.decode(**wl.oracle_kwargs())
    empty_lse = np.broadcast_to(wl.sinks.astype(np.float64), (4, 4)) if sinks else np.full((4, 4), -np.inf)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    np.testing.assert_array_equal(lse[0], empty_lse)
    assert np.array_equal(out[2, :2], np.zeros_like(out[2, :2]))
    np.testing.assert_array_equal(lse[2, :2], empty_lse[:2])
    assert np.isfinite(lse[1]).all() and np.isfinite(lse[2, 2:]).all()
    bo, bl = brute_decode(wl)
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-14)


def test_constant_keys_closed_form_with_sink():
    wl = _wl(sinks=True, window=0)
    wl.k_cache[:] = 0x38   # every key element decodes to 1.0
    out, lse = oracle.decode(**wl.oracle_kwargs())
    from tests.brute_force import depage, _codes_to_float, _bf16_to_float
    G = wl.Hq // wl.Hkv
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        V = _codes_to_float(depage(wl.v_cache, wl.block_table[b], L)) * wl.v_scale[0]
        for h in range(wl.Hq):
            s = wl.sm_scale * float(wl.k_scale[0]) * _bf16_to_float(wl.q_bits[b, 0, h]).sum()
            sk = float(wl.sinks[h])
            n = L
            mean_v = V[:, h // G].mean(axis=0)
            np.testing.assert_allclose(out[b, 0, h], mean_v * n / (n + math.exp(sk - s)),
                                       rtol=1e-11, atol=1e-14)
            assert abs(lse[b, 0, h] - math.log(n * math.exp(s) + math.exp(sk))) < 1e-11


def test_sink_at_minus_infinity_equals_no_sink():
    wl = _wl(sinks=True, window=10)
    kw = wl.oracle_kwargs()
    kw["sinks"] = np.full_like(wl.sinks, -np.inf)
    o1, l1 = oracle.decode(**kw)
    kw["sinks"] = None
    o0, l0 = oracle.decode(**kw)
    np.testing.assert_allclose(o1, o0, rtol=1e-15, atol=0)
    np.testing.assert_allclose(l1, l0, rtol=1e-15, atol=0)


def test_unit_values_close_the_softmax_with_sink():
    # V == 1 everywhere: out_d = sum_t p_t = 1 - e^(sink - lse), a check of out and lse together.
    wl = _wl(sinks=True, window=9)
    wl.v_cache[:] = 0x38
    kw = wl.oracle_kwargs()
    kw["v_scale"] = np.array([1.0], np.float32)
    out, lse = oracle.decode(**kw)
    want = 1.0 - np.exp(wl.sinks.astype(np.float64)[None, None, :] - lse)
    np.testing.assert_allclose(out, np.broadcast_to(want[..., None], out.shape), rtol=1e-12, atol=1e-14)


def test_torch_softmax_with_sink_column():
    wl = _wl(sinks=True, window=25, seed=11)
    out, lse = oracle.decode(**wl.oracle_kwargs())
    from tests.brute_force import depage, _codes_to_float
    G = wl.Hq // wl.Hkv
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        lo = max(0, L - wl.window)
        K = _codes_to_float(depage(wl.k_cache, wl.block_table[b], L))[lo:L] * wl.k_scale[0]
        V = _codes_to_float(depage(wl.v_cache, wl.block_table[b], L))[lo:L] * wl.v_scale[0]
        for h in range(wl.Hq):
            s = torch.from_numpy(_scores_row(wl, b, h, np.arange(lo, L)))
            logits = torch.cat([s, torch.tensor([float(wl.sinks[h])], dtype=torch.float64)])
            p = torch.softmax(logits, dim=0)
            o = (p[:-1, None] * torch.from_numpy(V[:, h // G])).sum(0)
            np.testing.assert_allclose(out[b, 0, h], o.numpy(), rtol=1e-12, atol=1e-14)
            assert abs(lse[b, 0, h] - torch.logsumexp(logits, 0).item()) < 1e-12


def test_torch_sdpa_float64():
    wl = make_workload(B=2, q_len=4, Hq=8, Hkv=2, D=32, bt=16, seq_lens=[70, 33], seed=21,
                       window=12, scale=("per_head", 0.02, 0.1))
    out, lse = oracle.decode(**wl.oracle_kwargs())
    from tests.brute_force import depage, _codes_to_float, _bf16_to_float
    G = wl.Hq // wl.Hkv
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        K = _codes_to_float(depage(wl.k_cache, wl.block_table[b], L)) * wl.k_scale[None, :, None]
        V = _codes_to_float(depage(wl.v_cache, wl.block_table[b], L)) * wl.v_scale[None, :, None]
        # positions no row attends hold NaN poison; SDPA's masked matmul would still touch them
        K = np.nan_to_num(K)
        V = np.nan_to_num(V)
        Kh = torch.from_numpy(np.repeat(K, G, axis=1)).permute(1, 0, 2).contiguous()  # [Hq, L, D]
        Vh = torch.from_numpy(np.repeat(V, G, axis=1)).permute(1, 0, 2).contiguous()
        q = torch.from_numpy(_bf16_to_float(wl.q_bits[b])).permute(1, 0, 2).contiguous()  # [Hq, q_len, D]
        pos = torch.arange(L - 4, L)[:, None]
        t = torch.arange(L)[None, :]
        mask = (t <= pos) & (t > pos - wl.window)
        o = torch.nn.functional.scaled_dot_product_attention(q, Kh, Vh, attn_mask=mask, scale=wl.sm_scale)
        np.testing.assert_allclose(out[b], o.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-14)
        logits = wl.sm_scale * (q @ Kh.transpose(1, 2).contiguous())
        logits = logits.masked_fill(~mask, -math.inf)
        np.testing.assert_allclose(lse[b], torch.logsumexp(logits, -1).permute(1, 0).numpy(), rtol=1e-12)


def test_gqa_equals_expanded_mha():
    wl = _wl(sinks=True, window=40, scale=("per_head", 0.02, 0.1))
    out, lse = oracle.decode(**wl.oracle_kwargs())
    G = wl.Hq // wl.Hkv
    kw = wl.oracle_kwargs()
    kw.update(k_cache=np.repeat(wl.k_cache, G, axis=2), v_cache=np.repeat(wl.v_cache, G, axis=2),
              k_scale=np.repeat(wl.k_scale, G), v_scale=np.repeat(wl.v_scale, G))
    out2, lse2 = oracle.decode(**kw)
    # BLAS may order a one-row product differently from a G-row one: rounding only
    np.testing.assert_allclose(out, out2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, lse2, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("cuts", [[0, 37, 100], [0, 5, 6, 64, 100], [0, 100]])
def test_split_partials_merge_to_direct(cuts):
    wl = make_workload(B=1, q_len=2, Hq=4, Hkv=2, D=16, bt=16, seq_lens=[100], seed=2,
                       window=0, sinks=True)
    out, lse = oracle.decode(**wl.oracle_kwargs())
    parts_o, parts_l = [], []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        kw = wl.oracle_kwargs()
        kw["sinks"] = None
        o, l = oracle.decode(**kw, key_range=(lo, hi))
        parts_o.append(o.reshape(-1, wl.D))
        parts_l.append(l.reshape(-1))
    po = np.stack(parts_o, axis=1)
    pl = np.stack(parts_l, axis=1)
    sink_rows = np.tile(wl.sinks, wl.B * wl.q_len)
    mo, ml = oracle.merge(po, pl, sink_rows)
    np.testing.assert_allclose(mo, out.reshape(-1, wl.D), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ml, lse.reshape(-1), rtol=1e-12, atol=1e-13)


def test_merge_closed_forms():
    # Two splits with lse ln 1 and ln 3: weights 1/4 and 3/4.
    po = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    pl = np.array([[0.0, math.log(3.0)]])
    o, l = oracle.merge(po, pl)
    np.testing.assert_allclose(o, [[0.25, 0.75]], rtol=1e-15)
    assert abs(l[0] - math.log(4.0)) < 1e-15
    # a sink of ln 4 halves both and doubles the partition function
    o, l = oracle.merge(po, pl, np.array([math.log(4.0)]))
    np.testing.assert_allclose(o, [[0.125, 0.375]], rtol=1e-15)
    assert abs(l[0] - math.log(8.0)) < 1e-15
    # an empty split (-inf) contributes nothing, even with NaN output bytes
    po2 = np.array([[[2.0, 3.0], [np.nan, np.nan]]])
    o, l = oracle.merge(po2, np.array([[0.5, -np.inf]]))
    np.testing.assert_allclose(o, [[2.0, 3.0]])
    assert l[0] == 0.5
    # every split empty, no sink: zeros and -inf, never NaN
    o, l = oracle.merge(np.zeros((1, 3, 2)), np.full((1, 3), -np.inf))
    assert np.array_equal(o, np.zeros((1, 2))) and l[0] == -np.inf
    # a single split is the identity
    o, l = oracle.merge(np.array([[[0.3, -0.7]]]), np.array([[1.25]]))
    np.testing.assert_allclose(o, [[0.3, -0.7]], rtol=0)
    assert l[0] == 1.25


def test_merge_is_associative():
    rng = np.random.default_rng(4)
    po = rng.standard_normal((5, 4, 8))
    pl = rng.standard_normal((5, 4))
    o_all, l_all = oracle.merge(po, pl)
    o_a, l_a = oracle.merge(po[:, :2], pl[:, :2])
    o_b, l_b = oracle.merge(po[:, 2:], pl[:, 2:])
    o2, l2 = oracle.merge(np.stack([o_a, o_b], 1), np.stack([l_a, l_b], 1))
    np.testing.assert_allclose(o2, o_all, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l2, l_all, rtol=1e-13)


def test_empty_attended_set():
    wl = _wl(sinks=True)
    kw = wl.oracle_kwargs()
    o, l = oracle.decode(**kw, key_range=(1000, 2000))
    assert np.array_equal(o, np.zeros_like(o))
    np.testing.assert_array_equal(l, np.broadcast_to(wl.sinks.astype(np.float64), l.shape))
    kw["sinks"] = None
    o, l = oracle.decode(**kw, key_range=(1000, 2000))
    assert np.array_equal(o, np.zeros_like(o)) and np.all(l == -np.inf)


def test_poison_bytes_never_read():
    wl = _wl(window=21, sinks=True)
    out, lse = oracle.decode(**wl.oracle_kwargs())
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert (wl.k_cache == POISON_CODE).any()
    rng = np.random.default_rng(1)
    kc = wl.k_cache.copy()
    vc = wl.v_cache.copy()
    pk = kc == POISON_CODE
    kc[pk] = rng.integers(0, 0x7E, size=int(pk.sum()))
    pv = vc == POISON_CODE
    vc[pv] = rng.integers(0, 0x7E, size=int(pv.sum()))
    kw = wl.oracle_kwargs()
    kw.update(k_cache=kc, v_cache=vc)
    out2, lse2 = oracle.decode(**kw)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_sampled_rows_equal_full_decode():
    wl = _wl(window=33, sinks=True)
    out, lse = oracle.decode(**wl.oracle_kwargs())
    rows = [(1, 0, 7), (0, 0, 0), (0, 0, 5)]
    o, l = oracle.decode(**wl.oracle_kwargs(), rows=rows)
    for n, (b, i, h) in enumerate(rows):
        np.testing.assert_allclose(o[n], out[b, i, h], rtol=1e-13, atol=1e-15)
        assert abs(l[n] - lse[b, i, h]) < 1e-13
