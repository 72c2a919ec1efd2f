"""Pins of the MXFP8 oracle (oracle/mxfp8_ref.py) against things other than
itself: the OCP E8M0 scale values, the shared-exponent rule at powers of two
and at the E4M3 saturation point, torch's float8_e4m3fn cast, a brute-force
twin that decodes pools element by element, and a writer round trip on
values the format holds exactly."""

import math
import os

import numpy as np
import pytest

import oracle
from oracle.mxfp8_ref import shared_exponent
from tests.brute_force import brute_decode
from workloads import make_mxfp8_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e8m0_matches_spec_values():
    n = 0
    with open(os.path.join(GOLDEN, "e8m0_spec_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            got = float(oracle.e8m0_decode(int(code, 16)))
            if val == "nan":
                assert math.isnan(got), code
            else:
                assert got == float(val), code
            n += 1
    assert n == 9


def test_shared_exponent_rule():
    # floor(log2(max|y|)) - 8: a block whose maximum is 2^k scales it into [256, 512)
    for k in range(-100, 120):
        assert shared_exponent(2.0 ** k) == max(k - 8, -127)
        assert shared_exponent(np.nextafter(2.0 ** k, 0.0)) == max(k - 9, -127)
    assert shared_exponent(0.0) == -127
    assert shared_exponent(float(np.finfo(np.float32).max)) == 119


def test_writer_codes_equal_torch_cast_of_the_scaled_block():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    T, Hkv, D, bt = 5, 2, 64, 32
    side = oracle.mxfp8_side_bytes(Hkv, bt, D)
    x = (rng.standard_normal((T, Hkv, D)) * np.exp(rng.uniform(-6, 6, (T, Hkv, 1)))).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    pool = np.zeros((1, side), np.uint8)
    kp, _ = oracle.mxfp8_cache_write(bits, bits, np.arange(T), np.float32([0.25]), np.float32([1.0]),
                                     pool, pool, Hkv, bt, D)
    y = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(4.0)       # x / 0.25
    for t in range(T):
        for h in range(Hkv):
            r = t * Hkv + h
            for blk in range(D // 32):
                yb = y[t, h, 32 * blk:32 * blk + 32].astype(np.float64)
                s = int(kp[0, Hkv * bt * D + r * 2 + blk])
                X = s - 127
                assert 2.0 ** (X + 8) <= np.abs(yb).max() < 2.0 ** (X + 9)
                want = torch.from_numpy(np.clip(yb * 2.0 ** -X, -448, 448).astype(np.float32)) \
                    .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                assert np.array_equal(kp[0, r * D + 32 * blk: r * D + 32 * blk + 32], want)


MX_TINY = [
    dict(B=2, q_len=1, Hq=4, Hkv=2, D=32, bt=32, seq_lens=[9, 40], window=0, sinks=True, kv_layout="NHD"),
    dict(B=1, q_len=3, Hq=4, Hkv=2, D=64, bt=32, seq_lens=[45], window=6, sinks=False, kv_layout="HND"),
    dict(B=2, q_len=1, Hq=3, Hkv=1, D=32, bt=32, seq_lens=[5, 1], window=0, sinks=True, kv_layout="HND",
         scale=("per_head", 0.02, 0.1)),
]


@pytest.mark.parametrize("k", range(len(MX_TINY)))
def test_mxfp8_decode_matches_brute_force(k):
    wl = make_mxfp8_workload(seed=70 + k, **MX_TINY[k])
    out, lse = oracle.decode(**wl.oracle_kwargs())
    assert not np.isnan(out).any()           # no poison byte was read
    bo, bl = brute_decode(wl)
    np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-13)


def test_mxfp8_layouts_and_padded_stride_agree():
    kw = dict(B=2, q_len=2, Hq=4, Hkv=2, D=64, bt=32, seq_lens=[33, 70], window=0, sinks=True, seed=81)
    ref = oracle.decode(**make_mxfp8_workload(kv_layout="NHD", **kw).oracle_kwargs())
    for layout, stride in (("HND", None), ("NHD", 4608), ("HND", 4352)):
        wl = make_mxfp8_workload(kv_layout=layout, page_stride=stride, **kw)
        o, l = oracle.decode(**wl.oracle_kwargs())
        assert np.array_equal(o, ref[0]) and np.array_equal(l, ref[1]), (layout, stride)


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_mxfp8_writer_round_trip_exact(layout):
    """Values the format holds exactly (E4M3 values times a block's power of
    two, with the block maximum in [256, 448]) are written bit for bit and
    decode back to themselves; bytes are checked at hand-computed offsets."""
    rng = np.random.default_rng(5)
    T, Hkv, D, bt, nb = 3, 2, 64, 32, 2
    side = oracle.mxfp8_side_bytes(Hkv, bt, D)
    codes = rng.integers(0, 0x70, size=(T, Hkv, D)).astype(np.uint8)     # magnitudes <= 240 ...
    codes[..., 0] = 0x7C                                                  # ... and one 384 per block
    codes[..., 32] = 0xFC                                                 # -384
    X = rng.integers(-12, -4, size=(T, Hkv, D // 32))
    vals = oracle.E4M3_TABLE[codes] * np.repeat(2.0 ** X, 32, axis=-1)
    import torch
    bits = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), vals.astype(np.float32))
    slots = np.array([0, 33, 62])
    pool = np.zeros((nb, side), np.uint8)
    kp, vp = oracle.mxfp8_cache_write(bits, bits, slots, np.float32([1.0]), np.float32([1.0]), pool, pool,
                                      Hkv, bt, D, kv_layout=layout)
    for t, slot in enumerate(slots):
        page, off = slot // bt, slot % bt
        for h in range(Hkv):
            r = h * bt + off if layout == "HND" else off * Hkv + h
            assert np.array_equal(kp[page, r * D:(r + 1) * D], codes[t, h])
            assert np.array_equal(kp[page, Hkv * bt * D + 2 * r:Hkv * bt * D + 2 * r + 2], X[t, h] + 127)
    back = oracle.mxfp8_gather(kp, [0, 1], 1, slots, 1.0, Hkv, bt, D, layout)
    assert np.array_equal(back, vals[:, 1])


def test_mxfp8_writer_saturates_and_skips():
    # a block whose maximum lies in [448, 512) after scaling saturates to +-448
    import torch
    D, Hkv, bt = 32, 1, 32
    y = np.zeros((1, 1, D), np.float32)
    y[0, 0, 0] = 500.0
    y[0, 0, 1] = -480.0
    y[0, 0, 2] = 1.0
    bits = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    pool = np.full((2, oracle.mxfp8_side_bytes(Hkv, bt, D)), 0xAB, np.uint8)
    kp, _ = oracle.mxfp8_cache_write(bits, bits, np.array([3]), np.float32([1.0]), np.float32([1.0]),
                                     pool, pool, Hkv, bt, D)
    assert kp[0, 32 * bt + 3] == 127                  # X = floor(log2 500) - 8 = 0
    assert kp[0, 3 * D + 0] == 0x7E and kp[0, 3 * D + 1] == 0xFE and kp[0, 3 * D + 2] == 0x38
    # negative and out-of-range slots leave the pool as it was
    kp2, _ = oracle.mxfp8_cache_write(bits, bits, np.array([-1]), np.float32([1.0]), np.float32([1.0]),
                                      pool, pool, Hkv, bt, D)
    assert np.array_equal(kp2, pool)
    kp3, _ = oracle.mxfp8_cache_write(bits, bits, np.array([64]), np.float32([1.0]), np.float32([1.0]),
                                      pool, pool, Hkv, bt, D)
    assert np.array_equal(kp3, pool)
