"""Query magnitude: scaling every query by 2^k and sm_scale by 2^-k leaves
every score, and so the whole result, unchanged in exact arithmetic; the
kernels stage the query under a per-row power of two (E4M3 hi + lo parts,
f16 for NVFP4 pages, bf16 for MXFP8 at head_dim 64), so each must give the
unscaled oracle's result at any k whose query stays a normal bf16 number.
Planner and forced VALU kernels, E4M3 / NVFP4 / MXFP8 pages."""

import dataclasses

import numpy as np
import pytest

import oracle
from tests.gpu_harness import compare, run, to_host, upload
from workloads import make_mxfp8_workload, make_nvfp4_workload, make_workload
from workloads.gen import _bf16_bits

torch = pytest.importorskip("torch")
fp = pytest.importorskip("decode_attention_paged_fp8pa_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp.lib()


SHAPE = dict(B=3, q_len=2, Hq=16, Hkv=4, bt=16, seq_lens=[300, 45, 517], window=200, sinks=True)
MAKERS = {
    "e4m3_d128": lambda: make_workload(seed=700, D=128, **SHAPE),
    "e4m3_d64": lambda: make_workload(seed=701, D=64, **SHAPE),
    "nvfp4_d128": lambda: make_nvfp4_workload(seed=702, D=128, kv_layout="HND", **SHAPE),
    "mxfp8_d128": lambda: make_mxfp8_workload(seed=703, D=128, **SHAPE),
    "mxfp8_d64": lambda: make_mxfp8_workload(seed=704, D=64, kv_layout="HND", **SHAPE),
    # 128 and 64 query rows per kv head: the LDS-shared kernels (8 and 4 row groups)
    "e4m3_prefill_lw8": lambda: make_workload(seed=705, D=128, B=2, q_len=32, Hq=16, Hkv=4, bt=16,
                                              seq_lens=[300, 517], sinks=True),
    "e4m3_prefill_lw4_d64": lambda: make_workload(seed=706, D=64, B=2, q_len=16, Hq=16, Hkv=4, bt=16,
                                                  seq_lens=[200, 90], window=60, sinks=True),
}
_cache = {}


def _case(name):
    if name not in _cache:
        wl = MAKERS[name]()
        _cache[name] = (wl, oracle.decode(**wl.oracle_kwargs()))
    return _cache[name]


@pytest.mark.parametrize("name", list(MAKERS))
@pytest.mark.parametrize("k", [-100, -40, 0, 40, 100])
@pytest.mark.parametrize("flags", [0, fp.FP8PA_FLAG_FORCE_DOT])
def test_query_scale_invariance(name, k, flags):
    wl, (ro, rl) = _case(name)
    q = (wl.q_bits.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** k)
    scaled = dataclasses.replace(wl, q_bits=_bf16_bits(q), sm_scale=float(wl.sm_scale * 2.0 ** -k))
    assert np.array_equal(scaled.q_bits, _bf16_bits(q))  # (exact: a power-of-two scale)
    out, lse = to_host(*run(scaled, upload(scaled), flags=flags))
    compare(out, lse, ro, rl, label=f"{name} q x 2^{k} flags={flags}")


# Signs and zeros the ABI allows: any finite sm_scale (negative flips every
# score, zero makes every attended key equal), and per-head K / V scales of
# either sign (a negative K scale flips that head's scores, a negative V
# scale its outputs).
SIGN_CASES = {
    "sm_neg": dict(sm=-0.09),
    "sm_zero": dict(sm=0.0),
    "kv_scale_signs": dict(k_neg=True, v_neg=True),
}


@pytest.mark.parametrize("name", list(MAKERS))
@pytest.mark.parametrize("case", list(SIGN_CASES))
@pytest.mark.parametrize("flags", [0, fp.FP8PA_FLAG_FORCE_DOT])
def test_scale_signs_and_zero(name, case, flags):
    wl, _ = _case(name)
    c = SIGN_CASES[case]
    ks, vs = wl.k_scale.copy(), wl.v_scale.copy()
    if c.get("k_neg"):
        ks = np.resize(ks, wl.Hkv) * np.where(np.arange(wl.Hkv) % 2 == 1, -1, 1).astype(np.float32)
    if c.get("v_neg"):
        vs = np.resize(vs, wl.Hkv) * np.where(np.arange(wl.Hkv) % 3 == 0, -1, 1).astype(np.float32)
    w2 = dataclasses.replace(wl, k_scale=ks.astype(np.float32), v_scale=vs.astype(np.float32),
                             sm_scale=float(c.get("sm", wl.sm_scale)))
    ro, rl = oracle.decode(**w2.oracle_kwargs())
    out, lse = to_host(*run(w2, upload(w2), flags=flags))
    compare(out, lse, ro, rl, label=f"{name} {case} flags={flags}")
