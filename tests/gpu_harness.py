"""Helpers of the GPU tests: upload a workload, run the C ABI, compare.

The comparison bar (per output element and per row):
  |out_gpu - out_oracle| <= 2e-2 + 1e-2 * |out_oracle|     (bf16 outputs)
  |lse_gpu - lse_oracle| <= 1e-3                           (fp32 LSE, natural log)
and both must be finite wherever the oracle is finite; an oracle LSE of
-inf must come back as -inf.
"""

from __future__ import annotations

import numpy as np

ATOL_OUT = 2e-2
RTOL_OUT = 1e-2
ATOL_LSE = 1e-3


def upload(wl, device="cuda", kv_layout="NHD"):
    """Device tensors of a workload; kv_layout "HND" stores the pools head-major."""
    import torch

    def pool(c):
        if getattr(wl, "kv_format", "e4m3") != "e4m3":
            return c  # block-scaled pools: the layout is in the pool's bytes
        return np.ascontiguousarray(c.transpose(0, 2, 1, 3)) if kv_layout == "HND" else c

    t = {
        "layout": wl.kv_layout if getattr(wl, "kv_format", "e4m3") != "e4m3" else kv_layout,
        "q": torch.from_numpy(wl.q_bits.view(np.int16)).to(device).view(torch.bfloat16),
        "k": torch.from_numpy(pool(wl.k_cache)).to(device),
        "v": torch.from_numpy(pool(wl.v_cache)).to(device),
        "bt": torch.from_numpy(wl.block_table).to(device),
        "sl": torch.from_numpy(wl.seq_lens).to(device),
        "ks": torch.from_numpy(wl.k_scale).to(device),
        "vs": torch.from_numpy(wl.v_scale).to(device),
        "sinks": None if wl.sinks is None else torch.from_numpy(wl.sinks).to(device),
    }
    return t


def run(wl, t, num_splits=0, flags=0, out=None, lse=None, workspace=None):
    """fp8pa_decode through the binding; returns (out, lse) device tensors."""
    import decode_attention_paged_fp8pa_amd as fp

    return fp.decode(t["q"], t["k"], t["v"], t["bt"], t["sl"], t["ks"], t["vs"], t["sinks"],
                     window=wl.window, sm_scale=wl.sm_scale,
                     max_seq_len=max(1, int(wl.seq_lens.max())), num_splits=num_splits, flags=flags,
                     out=out, lse=lse, workspace=workspace, k_groups=wl.k_groups,
                     kv_layout=t.get("layout", "NHD"), kv_format=getattr(wl, "kv_format", "e4m3"),
                     num_kv_heads=wl.Hkv, block_tokens=wl.bt)


def to_host(out, lse):
    import torch

    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def compare(out, lse, ref_out, ref_lse, label=""):
    """Asserts the bar; returns (max abs err out, max err/tol out, max abs err lse)."""
    out = np.asarray(out, np.float64)
    ref_out = np.asarray(ref_out, np.float64)
    assert out.shape == ref_out.shape, (label, out.shape, ref_out.shape)
    assert np.isfinite(out).all(), f"{label}: non-finite output"
    err = np.abs(out - ref_out)
    tol = ATOL_OUT + RTOL_OUT * np.abs(ref_out)
    ratio = float(np.max(err / tol)) if err.size else 0.0
    if ratio > 1.0:
        idx = np.unravel_index(int(np.argmax(err / tol)), err.shape)
        raise AssertionError(f"{label}: out mismatch at {idx}: gpu {out[idx]} oracle {ref_out[idx]} "
                             f"(max err/tol {ratio:.3f})")
    lse = np.asarray(lse, np.float64)
    ref_lse = np.asarray(ref_lse, np.float64)
    ninf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), ninf), f"{label}: -inf LSE pattern differs"
    fin = ~ninf
    assert np.isfinite(lse[fin]).all(), f"{label}: non-finite LSE"
    lerr = float(np.max(np.abs(lse[fin] - ref_lse[fin]))) if fin.any() else 0.0
    assert lerr <= ATOL_LSE, f"{label}: LSE error {lerr:.3e} > {ATOL_LSE}"
    return float(err.max()) if err.size else 0.0, ratio, lerr


def sample_rows(wl, n, seed=0):
    """n distinct (b, i, h) rows, always including the first and last sequence."""
    rng = np.random.default_rng(seed)
    rows = {(0, 0, 0), (wl.B - 1, wl.q_len - 1, wl.Hq - 1)}
    total = wl.B * wl.q_len * wl.Hq
    n = min(n, total)
    while len(rows) < n:
        rows.add((int(rng.integers(wl.B)), int(rng.integers(wl.q_len)), int(rng.integers(wl.Hq))))
    return sorted(rows)
