"""fp8pa_decode_noalloc, the entry point whose split workspace is the
library's static per-device scratch array, against fp8pa_decode with a
caller workspace: two calls in a row (the second smaller, so stale partials
of the first lie in the array), each checked against fp8pa_decode's output
on the same inputs, to the parity bar and bit for bit (same plan, same
kernels), and against the float64 oracle.
"""

import numpy as np
import pytest

import oracle
from tests.gpu_harness import compare, to_host, upload
from workloads import make_workload

torch = pytest.importorskip("torch")
fp = pytest.importorskip("decode_attention_paged_fp8pa_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fp.lib()


def _shape(wl, t, num_splits=0):
    return fp.shape_for(t["q"], t["k"], t["bt"], t["ks"], t["vs"], window=wl.window,
                        sm_scale=wl.sm_scale, max_seq_len=int(wl.seq_lens.max()),
                        num_splits=num_splits, k_groups=wl.k_groups)


def _with_workspace(wl, t, shape):
    out = torch.empty(tuple(wl.q_bits.shape), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(tuple(wl.q_bits.shape[:3]), dtype=torch.float32, device="cuda")
    n = fp.fp8pa_workspace_bytes(shape)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    fp.fp8pa_decode(shape, t["q"], t["k"], t["v"], t["bt"], t["sl"], t["ks"], t["vs"], t["sinks"],
                    out, lse, ws if n else None, n)
    return out, lse, n


def _noalloc(wl, t, shape):
    out = torch.full(tuple(wl.q_bits.shape), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(tuple(wl.q_bits.shape[:3]), float("nan"), dtype=torch.float32, device="cuda")
    fp.fp8pa_decode_noalloc(shape, t["q"], t["k"], t["v"], t["bt"], t["sl"], t["ks"], t["vs"],
                            t["sinks"], out, lse)
    return out, lse


CALLS = [
    # the ragged GQA decode batch at a quarter of its lengths (balanced splits)
    ("gqa_ragged", dict(B=16, q_len=1, Hq=32, Hkv=8, D=128, bt=16, seq_lens=("uniform", 256, 2048),
                        scale=("per_head", 0.02, 0.1)), 0),
    # smaller, and different in every dimension: head_dim 64, windows, sinks, MTP rows, fixed splits
    ("mtp_window_sinks", dict(B=3, q_len=2, Hq=16, Hkv=4, D=64, bt=16, seq_lens=[300, 47, 1000],
                              window=200, sinks=True), 3),
]


def test_two_calls_in_a_row_match_the_workspace_entry_point():
    results = []
    for i, (name, kw, ns) in enumerate(CALLS):
        wl = make_workload(seed=900 + i, **kw)
        t = upload(wl)
        shape = _shape(wl, t, ns)
        ref_out, ref_lse, n = _with_workspace(wl, t, shape)
        assert 0 < n <= (64 << 20), (name, n)   # a split plan that fits the scratch array
        out, lse = _noalloc(wl, t, shape)
        results.append((name, wl, ref_out, ref_lse, out, lse))
    # both calls' outputs after both ran: the second call must not have
    # disturbed the first's results, and stale partials must not leak
    for name, wl, ref_out, ref_lse, out, lse in results:
        o, l = to_host(out, lse)
        ro, rl = to_host(ref_out, ref_lse)
        compare(o, l, ro, rl, label=f"noalloc vs workspace entry point: {name}")
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), name
        want_o, want_l = oracle.decode(**wl.oracle_kwargs())
        compare(o, l, want_o, want_l, label=f"noalloc vs oracle: {name}")


def test_one_split_plan_needs_no_scratch():
    wl = make_workload(seed=950, B=2, q_len=4, Hq=8, Hkv=2, D=128, bt=16, seq_lens=[90, 33],
                       window=40, sinks=True)
    t = upload(wl)
    shape = _shape(wl, t, 1)
    ref_out, ref_lse, n = _with_workspace(wl, t, shape)
    assert n == 0
    out, lse = _noalloc(wl, t, shape)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


def test_plan_beyond_the_scratch_array_is_rejected():
    wl = make_workload(seed=951, B=2, q_len=1, Hq=8, Hkv=2, D=128, bt=16, seq_lens=[64, 64])
    t = upload(wl)
    # a shape whose planned workspace exceeds 64 MiB (many rows, many
    # splits); the call is rejected before anything is read or launched
    big = fp.make_shape(batch=64, q_len=8, num_q_heads=64, num_kv_heads=8, head_dim=256,
                        block_tokens=16, num_blocks=wl.num_blocks, block_table_stride=4096,
                        max_seq_len=65536, sm_scale=0.06, num_splits=64)
    assert fp.fp8pa_workspace_bytes(big) > (64 << 20)
    out = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fp.Fp8paError) as e:
        fp.fp8pa_decode_noalloc(big, t["q"], t["k"], t["v"], t["bt"], t["sl"], t["ks"], t["vs"],
                                None, out, None)
    assert e.value.status == fp._lib.FP8PA_ERR_WORKSPACE_TOO_SMALL
