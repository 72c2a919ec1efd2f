"""Pins of the KV-cache writer oracle (oracle/fp8pa_write_ref.py), no GPU.

The E4M3 encoder is checked against the decode table (every code round
trips), against the definition of ties-to-even at every midpoint between
neighbouring values, at the saturation and subnormal edges, and against
torch's float8_e4m3fn cast; the cache writer against hand-placed slots and
the decode of what it wrote.
"""

import numpy as np
import pytest

import oracle

T = oracle.E4M3_TABLE
FINITE = [c for c in range(256) if not np.isnan(T[c])]


def test_every_code_round_trips():
    got = oracle.e4m3_encode(T[FINITE])
    assert got.tolist() == FINITE  # includes 0x80 for -0.0


def test_midpoints_round_to_the_even_code():
    pos = sorted((T[c], c) for c in range(0x00, 0x7F))  # +0 .. 448
    for (a, ca), (b, cb) in zip(pos, pos[1:]):
        mid = (a + b) / 2
        even = ca if ca % 2 == 0 else cb
        assert oracle.e4m3_encode(mid) == even, (a, b)
        assert oracle.e4m3_encode(-mid) == even | 0x80
        assert oracle.e4m3_encode(np.nextafter(mid, a)) == ca
        assert oracle.e4m3_encode(np.nextafter(mid, b)) == cb


def test_saturation_and_special_values():
    assert oracle.e4m3_encode(448.0) == 0x7E
    for x in (449.0, 463.99, 464.0, 480.0, 1e30, np.inf):
        assert oracle.e4m3_encode(x) == 0x7E
        assert oracle.e4m3_encode(-x) == 0xFE
    assert oracle.e4m3_encode(0.0) == 0x00 and oracle.e4m3_encode(-0.0) == 0x80
    assert np.isnan(T[oracle.e4m3_encode(np.nan)])
    # the subnormal grid is 2^-9; half of it rounds to the even neighbour 0
    assert oracle.e4m3_encode(2.0 ** -9) == 0x01
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02
    assert oracle.e4m3_encode(-2.0 ** -11) == 0x80
    assert oracle.e4m3_encode(2.0 ** -6) == 0x08  # smallest normal
    assert oracle.e4m3_encode(7.5 * 2.0 ** -9) == 0x08  # 7.5 -> 8 (even)


def test_encoder_matches_torch_cast_in_range():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-12, 9, size=20000))).astype(np.float32)
    x = np.clip(x, -448.0, 448.0)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x.astype(np.float64)), want)


def _bf16_bits(x):
    b = np.asarray(x, np.float32).view(np.uint32)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def test_cache_write_places_and_skips():
    nb, bt, hkv, d = 3, 4, 2, 8
    k0 = np.full((nb, bt, hkv, d), 0x11, np.uint8)
    v0 = np.full((nb, bt, hkv, d), 0x22, np.uint8)
    key = np.arange(3 * hkv * d, dtype=np.float32).reshape(3, hkv, d) / 16
    val = -key
    slots = np.array([5, -1, 11])  # page 1 offset 1, skipped, page 2 offset 3
    ks = np.array([0.5, 2.0], np.float32)
    vs = np.array([1.0], np.float32)
    k1, v1 = oracle.cache_write(_bf16_bits(key), _bf16_bits(val), slots, ks, vs, k0, v0)
    touched = np.zeros((nb, bt), bool)
    touched[1, 1] = touched[2, 3] = True
    assert np.all(k1[~touched] == 0x11) and np.all(v1[~touched] == 0x22)
    for t, (pg, off) in ((0, (1, 1)), (2, (2, 3))):
        for h in range(hkv):
            assert np.array_equal(k1[pg, off, h], oracle.e4m3_encode(key[t, h] / ks[h]))
            assert np.array_equal(v1[pg, off, h], oracle.e4m3_encode(val[t, h] / vs[0]))
    # a slot past the cache is skipped too
    k2, _ = oracle.cache_write(_bf16_bits(key[:1]), _bf16_bits(val[:1]), [nb * bt], ks, vs, k0, v0)
    assert np.array_equal(k2, k0)


def test_cache_write_then_decode_is_close():
    rng = np.random.default_rng(5)
    nb, bt, hkv, d = 6, 16, 2, 64
    key = rng.standard_normal((40, hkv, d)).astype(np.float32)
    ks = np.array([0.03, 0.07], np.float32)
    slots = rng.permutation(nb * bt)[:40]
    zeros = np.zeros((nb, bt, hkv, d), np.uint8)
    k1, _ = oracle.cache_write(_bf16_bits(key), _bf16_bits(key), slots, ks, ks, zeros, zeros)
    xb = (_bf16_bits(key).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for t, s in enumerate(slots):
        back = T[k1[s // bt, s % bt]] * ks[:, None]
        # E4M3 keeps 3 mantissa bits: relative error <= 2^-4 for normal values
        assert np.all(np.abs(back - xb[t]) <= 2.0 ** -4 * np.abs(xb[t]) + 2.0 ** -10 * ks[:, None])


def test_cache_write_k_groups():
    """With k_groups, each head_dim group of the key is encoded against its own
    scale ([Hkv, k_groups] or [k_groups] for all heads); values keep one."""
    nb, bt, hkv, d = 2, 4, 2, 16
    rng = np.random.default_rng(3)
    key = rng.standard_normal((3, hkv, d)).astype(np.float32)
    slots = np.array([1, 6, -3])
    zeros = np.zeros((nb, bt, hkv, d), np.uint8)
    xb = (_bf16_bits(key).astype(np.uint32) << 16).view(np.float32)
    for ks in (np.array([0.5, 0.25, 2.0, 1.0, 0.125, 4.0, 8.0, 0.5], np.float32),
               np.array([0.5, 0.25, 2.0, 1.0], np.float32)):
        k1, v1 = oracle.cache_write(_bf16_bits(key), _bf16_bits(key), slots, ks, np.array([1.0], np.float32),
                                    zeros, zeros, k_groups=4)
        grid = ks.reshape(-1, 4)
        for t, s in ((0, 1), (1, 6)):
            for h in range(hkv):
                row = grid[h] if grid.shape[0] > 1 else grid[0]
                # power-of-two scales: x * (1/s) is exact, so encode(x / s) is the answer
                want = oracle.e4m3_encode(xb[t, h].astype(np.float64) / np.repeat(row, d // 4))
                assert np.array_equal(k1[s // bt, s % bt, h], want)
                assert np.array_equal(v1[s // bt, s % bt, h], oracle.e4m3_encode(xb[t, h].astype(np.float64)))


def test_cache_write_hnd_is_the_transposed_nhd_write():
    nb, bt, hkv, d = 3, 4, 2, 32
    rng = np.random.default_rng(8)
    key = rng.standard_normal((7, hkv, d)).astype(np.float32)
    val = rng.standard_normal((7, hkv, d)).astype(np.float32)
    slots = np.array([0, 5, -1, 11, 3, 6, 12])
    ks = np.array([0.5, 0.25, 2.0, 1.0], np.float32)
    vs = np.array([0.125], np.float32)
    k0 = rng.integers(0, 256, size=(nb, bt, hkv, d)).astype(np.uint8)
    v0 = rng.integers(0, 256, size=(nb, bt, hkv, d)).astype(np.uint8)
    k1, v1 = oracle.cache_write(_bits16(key), _bits16(val), slots, ks, vs, k0, v0, k_groups=2)
    k2, v2 = oracle.cache_write(_bits16(key), _bits16(val), slots, ks, vs, k0.transpose(0, 2, 1, 3),
                                v0.transpose(0, 2, 1, 3), k_groups=2, kv_layout="HND")
    assert np.array_equal(k2, k1.transpose(0, 2, 1, 3)) and np.array_equal(v2, v1.transpose(0, 2, 1, 3))


def _bits16(x):
    return _bf16_bits(x)


def _golden_reciprocal_cases():
    import json
    import os

    path = os.path.join(os.path.dirname(__file__), "golden", "writer_reciprocal_order.json")
    with open(path) as f:
        return json.load(f)["cases"]


def _f32(bits_hex):
    return np.array([int(bits_hex, 16)], dtype=np.uint32).view(np.float32)[0]


def test_golden_reciprocal_derivation_is_consistent():
    """The hand-worked numbers of the golden cases check out in exact
    rational arithmetic: the stored reciprocal is the fp32 number nearest
    1/s, and the product rounds to the stated fp32 midpoint."""
    from fractions import Fraction

    for c in _golden_reciprocal_cases():
        s = Fraction(float(_f32(c["scale_f32_bits"])))
        r = Fraction(float(_f32(c["reciprocal_f32_bits"])))
        e = r.numerator.bit_length() - r.denominator.bit_length()
        e = e if Fraction(2) ** e <= r else e - 1
        ulp = Fraction(2) ** (e - 23)
        assert abs(1 / s - r) <= ulp / 2
        x = Fraction(float(np.array([int(c["x_bf16_bits"], 16) << 16], dtype=np.uint32).view(np.float32)[0]))
        prod = x * r
        p32 = Fraction(float(c["product_f32"].split()[0]))
        pe = p32.numerator.bit_length() - p32.denominator.bit_length()
        pe = pe if Fraction(2) ** pe <= p32 else pe - 1
        assert abs(prod - p32) < Fraction(2) ** (pe - 23) / 2  # strictly nearer than the next fp32
        # the quotient itself lies strictly above the midpoint: the other code
        assert x / s > p32


def test_cache_write_uses_the_fp32_reciprocal_then_an_fp32_product():
    """Pinned to the golden cases: a plausible variant of the writer (exact
    division, a float64 reciprocal, an fp32 division, or encoding the
    unrounded product) writes the neighbouring code instead."""
    cases = _golden_reciprocal_cases()
    hkv = len(cases)
    key = np.zeros((1, hkv, 1), dtype=np.uint16)
    ks = np.zeros(hkv, dtype=np.float32)
    want = []
    for h, c in enumerate(cases):
        key[0, h, 0] = int(c["x_bf16_bits"], 16)
        ks[h] = _f32(c["scale_f32_bits"])
        want.append(int(c["expected_code"], 16))
    kc = np.zeros((1, 1, hkv, 1), dtype=np.uint8)
    k_out, v_out = oracle.cache_write(key, key, np.array([0]), ks, ks, kc, kc.copy())
    assert k_out[0, 0, :, 0].tolist() == want
    assert v_out[0, 0, :, 0].tolist() == want
