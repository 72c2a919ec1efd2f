"""Pins of the NVFP4 oracle (oracle/nvfp4_ref.py) against things other than
itself: the OCP E2M1 value table, explicit rounding midpoints, a brute-force
twin that decodes pools element by element, and a writer round trip on
values the format holds exactly."""

import math
import os

import numpy as np
import pytest

import oracle
from tests.brute_force import brute_decode
from workloads import make_nvfp4_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m1_table_matches_spec_values():
    n = 0
    with open(os.path.join(GOLDEN, "e2m1_spec_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            got = oracle.e2m1_decode_code(int(code, 16))
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), code
            n += 1
    assert n == 16


def test_e2m1_encode_midpoints_ties_and_saturation():
    # (input, code): midpoints go to the even code, beyond 6 saturates
    cases = [(0.0, 0), (0.25, 0), (0.2500001, 1), (0.75, 2), (0.7499999, 1), (1.25, 2),
             (1.75, 4), (2.5, 4), (2.5000001, 5), (3.5, 6), (5.0, 6), (5.0000001, 7), (6.0, 7),
             (1e9, 7), (-0.0, 8), (-0.1, 8), (-0.3, 9), (-3.5, 14), (-100.0, 15)]
    got = oracle.e2m1_encode([c[0] for c in cases])
    assert got.tolist() == [c[1] for c in cases]
    # every code round-trips
    assert oracle.e2m1_encode(oracle.E2M1_TABLE).tolist() == list(range(16))


NV_TINY = [
    dict(B=2, q_len=1, Hq=4, Hkv=2, D=16, bt=4, seq_lens=[9, 17], window=0, sinks=True, kv_layout="NHD"),
    dict(B=1, q_len=3, Hq=4, Hkv=2, D=32, bt=8, seq_lens=[21], window=6, sinks=False, kv_layout="HND"),
    dict(B=2, q_len=1, Hq=3, Hkv=1, D=16, bt=2, seq_lens=[5, 1], window=0, sinks=True, kv_layout="HND",
         scale=("per_head", 0.02, 0.1)),
]


@pytest.mark.parametrize("k", range(len(NV_TINY)))
def test_nvfp4_decode_matches_brute_force(k):
    wl = make_nvfp4_workload(seed=60 + k, **NV_TINY[k])
    out, lse = oracle.decode(**wl.oracle_kwargs())
    assert not np.isnan(out).any()           # no poison byte was read
    bo, bl = brute_decode(wl)
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-13)


def test_nvfp4_padded_page_stride_and_layouts_agree():
    """The same draws in token-major and head-major pools, and with pages
    padded to a larger stride, decode to the same result."""
    base = dict(B=2, q_len=2, Hq=8, Hkv=2, D=32, bt=4, seq_lens=[13, 30], seed=9, window=10,
                sinks=True)
    ref = None
    for layout, stride in (("NHD", None), ("HND", None), ("NHD", 400), ("HND", 512)):
        wl = make_nvfp4_workload(kv_layout=layout, page_stride=stride, **base)
        out, lse = oracle.decode(**wl.oracle_kwargs())
        if ref is None:
            ref = (out, lse)
        else:
            assert np.array_equal(out, ref[0]) and np.array_equal(lse, ref[1]), (layout, stride)


def _bf16_bits(x):
    b = np.asarray(x, np.float32).view(np.uint32)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_nvfp4_writer_round_trip_exact(layout):
    """Keys built from codes and scale bytes the format holds exactly (each
    16-element block has one element of magnitude 6, so its scale is
    max / 6 exactly): the writer must reproduce those bytes, placed where the
    format puts them, and the gather must return the keys."""
    rng = np.random.default_rng(4)
    Hkv, bt, D, nb, T = 2, 4, 32, 3, 5
    scale_codes = np.array([0x30, 0x38, 0x3C, 0x44, 0x4B, 0x52], np.uint8)   # 0.5 .. 10
    ks = np.array([0.5, 2.0], np.float32)                                     # powers of two
    codes = rng.integers(0, 16, size=(T, Hkv, D)).astype(np.uint8)
    codes[:, :, ::16] = 7                                                     # a 6 per block
    sbytes = rng.choice(scale_codes, size=(T, Hkv, D // 16)).astype(np.uint8)
    vals = oracle.E2M1_TABLE[codes] * oracle.E4M3_TABLE[np.repeat(sbytes, 16, axis=2)] * ks[None, :, None]
    bits = _bf16_bits(vals)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), vals.astype(np.float32))
    slots = np.array([0, 7, 5, 11, 2])
    side = oracle.nvfp4_side_bytes(Hkv, bt, D)
    zero = np.zeros((nb, side), np.uint8)
    kp, vp = oracle.nvfp4_cache_write(bits, bits, slots, ks, ks, zero, zero, Hkv, bt, D, layout)
    # the bytes, placed by hand from the format's description
    want = np.zeros((nb, side), np.uint8)
    data_bytes = Hkv * bt * D // 2
    for t, sl in enumerate(slots):
        page, off = sl // bt, sl % bt
        for h in range(Hkv):
            row = h * bt + off if layout == "HND" else off * Hkv + h
            c = codes[t, h]
            want[page, row * D // 2: row * D // 2 + D // 2] = c[0::2] | (c[1::2] << 4)
            want[page, data_bytes + row * D // 16: data_bytes + (row + 1) * D // 16] = sbytes[t, h]
    assert np.array_equal(kp, want) and np.array_equal(vp, want)
    for t, sl in enumerate(slots):
        for h in range(Hkv):
            table = np.arange(nb)
            got = oracle.nvfp4_gather(kp, table, h, np.array([sl]), ks[h], Hkv, bt, D, layout)
            assert np.array_equal(got[0], vals[t, h])


def test_nvfp4_writer_rounds_and_skips():
    """Random keys: every written element is the E2M1 code nearest to
    x / (key scale * block scale) and every block's max magnitude decodes
    to within one E4M3 step of max / 6; negative and past-the-end slots are
    skipped."""
    rng = np.random.default_rng(6)
    Hkv, bt, D, nb = 1, 4, 32, 2
    x = rng.standard_normal((3, Hkv, D)).astype(np.float32) * 3
    bits = _bf16_bits(x)
    xb = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    side = oracle.nvfp4_side_bytes(Hkv, bt, D)
    pool0 = np.full((nb, side), 0xAB, np.uint8)
    ks = np.array([0.25], np.float32)
    kp, _ = oracle.nvfp4_cache_write(bits, bits, np.array([1, -1, nb * bt]), ks, ks, pool0, pool0,
                                     Hkv, bt, D)
    touched = np.zeros_like(kp, bool)
    touched[0, 1 * D // 2: 2 * D // 2] = True
    touched[0, bt * D // 2 + 1 * D // 16: bt * D // 2 + 2 * D // 16] = True
    assert np.all(kp[~touched] == 0xAB)
    got = oracle.nvfp4_gather(kp, np.arange(nb), 0, np.array([1]), 1.0, Hkv, bt, D)[0]
    y = xb[0, 0] / 0.25
    for blk in range(D // 16):
        sv = oracle.E4M3_TABLE[kp[0, bt * D // 2 + D // 16 + blk]]
        amax = np.abs(y[16 * blk: 16 * blk + 16]).max()
        assert abs(sv - amax / 6) <= 2.0 ** -3 * amax / 6          # E4M3 keeps 3 mantissa bits
        codes_val = got[16 * blk: 16 * blk + 16] / sv
        t = y[16 * blk: 16 * blk + 16] / sv
        mags = oracle.E2M1_TABLE[:8]
        for a, c in zip(t, codes_val):
            a_sat = min(abs(a), 6.0)
            # the chosen magnitude is a nearest one (ties either way here; ties
            # to even are pinned above) and keeps the sign
            assert abs(abs(c) - a_sat) <= np.abs(mags - a_sat).min() + 1e-9
            assert c == 0 or np.sign(c) == np.sign(a)


def _nvfp4_golden():
    import json
    import os

    with open(os.path.join(os.path.dirname(__file__), "golden", "nvfp4_writer_midpoint.json")) as f:
        return json.load(f)


def test_nvfp4_golden_derivation_is_consistent():
    """The golden block's numbers in exact rational arithmetic: fp32(1/6),
    the global scale, the block scale that rounds onto the E4M3 midpoint
    2.875, and the other order's scale that stays below it."""
    from fractions import Fraction

    gd = _nvfp4_golden()

    def f32(h):
        return Fraction(float(np.array([int(h, 16)], dtype=np.uint32).view(np.float32)[0]))

    def rne32(x):
        e = x.numerator.bit_length() - x.denominator.bit_length()
        e = e if Fraction(2) ** e <= x else e - 1
        ulp = Fraction(2) ** (e - 23)
        q = x / ulp
        n = q.numerator // q.denominator
        rem = q - n
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2):
            n += 1
        return n * ulp

    ks, g, sixth = f32(gd["k_scale_f32_bits"]), f32(gd["g_f32_bits"]), f32(gd["sixth_f32_bits"])
    assert g == rne32(1 / ks) and sixth == rne32(Fraction(1, 6))
    a = Fraction(1421875, 1000000)
    s = rne32(g * rne32(a * sixth))
    assert s == Fraction(23, 8)                                # 2.875, the midpoint of 2.75 and 3
    assert rne32(rne32(a * g) / 6) < Fraction(23, 8)          # the other order stays below


def test_nvfp4_writer_golden_block():
    """oracle.nvfp4_cache_write on the golden block: the scale byte is the
    even code at the midpoint and the element codes are the hand-worked ones."""
    gd = _nvfp4_golden()
    Hkv, D, bt = 1, 16, 1
    bits = np.array([int(h, 16) for h in gd["x_bf16_bits"]], dtype=np.uint16).reshape(1, 1, D)
    ks = np.array([int(gd["k_scale_f32_bits"], 16)], dtype=np.uint32).view(np.float32)
    side = oracle.nvfp4_side_bytes(Hkv, bt, D)
    pool = np.zeros((1, side), np.uint8)
    k_out, v_out = oracle.nvfp4_cache_write(bits, bits, np.array([0]), ks, ks, pool, pool.copy(), Hkv, bt, D)
    want_data = [int(h, 16) for h in gd["expected_data_bytes"]]
    for out in (k_out, v_out):
        assert out[0, :8].tolist() == want_data
        assert int(out[0, 8]) == int(gd["expected_scale_byte"], 16)
