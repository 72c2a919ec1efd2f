"""Every page size the ABI allows (a power of two in [1, 1024] tokens), on
E4M3, NVFP4 and MXFP8 pages, the planner's kernel and the forced VALU
kernel, against the oracle: sequences span several pages, the window and
the causal drafts cut pages in the middle, and unattended table entries and
bytes are poison."""

import numpy as np
import pytest

import oracle
from tests.gpu_harness import compare, run, to_host, upload
from workloads import make_mxfp8_workload, make_nvfp4_workload, make_workload

torch = pytest.importorskip("torch")
fp = pytest.importorskip("decode_attention_paged_fp8pa_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp.lib()


PAGE_SIZES = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024]
MAKE = {"e4m3": make_workload, "nvfp4": make_nvfp4_workload, "mxfp8": make_mxfp8_workload}
_cache = {}


def _case(fmt, bt):
    key = (fmt, bt)
    if key not in _cache:
        kw = dict(B=2, q_len=3, Hq=16, Hkv=4, D=128, bt=bt, seq_lens=[700, 1500], window=900, sinks=True)
        if fmt != "e4m3":
            kw["kv_layout"] = "HND" if bt % 2 == 0 else "NHD"
        wl = MAKE[fmt](seed=800 + PAGE_SIZES.index(bt), **kw)
        _cache[key] = (wl, upload(wl), oracle.decode(**wl.oracle_kwargs()))
    return _cache[key]


@pytest.mark.parametrize("bt", PAGE_SIZES)
@pytest.mark.parametrize("fmt", list(MAKE))
@pytest.mark.parametrize("flags,ns", [(0, 0), (0, 3), (fp.FP8PA_FLAG_FORCE_DOT, 0)])
def test_page_sizes(fmt, bt, flags, ns):
    wl, t, (ro, rl) = _case(fmt, bt)
    out, lse = to_host(*run(wl, t, num_splits=ns, flags=flags))
    compare(out, lse, ro, rl, label=f"{fmt} bt={bt} flags={flags} splits={ns}")


@pytest.mark.parametrize("fmt", list(MAKE))
@pytest.mark.parametrize("ns", [2, 7, 64, 500])
def test_forced_split_counts(fmt, ns):
    """A caller's split count, from a few to far more splits than a sequence
    has tiles (the extra splits hold no keys and must merge as nothing)."""
    wl, t, (ro, rl) = _case(fmt, 16)
    out, lse = to_host(*run(wl, t, num_splits=ns))
    compare(out, lse, ro, rl, label=f"{fmt} splits={ns}")
