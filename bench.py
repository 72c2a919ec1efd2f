#!/usr/bin/env python3
"""Benchmark of paged FP8 decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--configs 1,2,3,4,5]

A step is one fp8pa_decode call (split-KV partial kernel, then the LSE merge
kernel when the plan has more than one split) over one batch of synthetic
input already resident in HBM.  The JSON line's workload is the largest
named one, the speculative decode batch (B=256, q_len=4 causal, Hq=32,
Hkv=8, D=128, bt=16, seq_lens U[1024, 4096], window 2048, sinks); all five
named workloads are measured the same way and reported under
"per_workload", workloads 1-4 with a flag for the 70%-of-peak bar.

Cold-cache discipline: each workload keeps C copies of its K/V page pools
(same block table) and the steps rotate through them, so that between two
reads of the same bytes at least 1 GiB of other KV has streamed through the
256 MB Infinity Cache (a workload too small for that, the tiny one, is
timed cold instead: 1 GiB written before each of 50 single calls, each
bracketed by HIP events).  The K timed steps are captured once in a HIP graph
(after W eager warmup steps and an eager timing pass) and replayed back to
back on torch's current stream, bracketed by torch.cuda.synchronize() and
HIP events; the replayed output is checked bit for bit against the eager
one.  The graph is replayed REPLAYS times: the step time is the median of
the per-replay averages, reported with p10 / p90.  The partial kernel alone
is timed from a second graph of the same steps run with
FP8PA_FLAG_PARTIAL_ONLY (no merge launch).  A 1 GiB device-to-device copy is
timed as the practical HBM ceiling ("copy_ceiling"), and one launch that
only reads each workload's KV byte count, plus an empty launch, as the floor
of its step ("read_ceiling"), and the KV-cache writer
fp8pa_cache_write at a decode step's and a prefill chunk's size ("writer").
Five widenings are timed after the decode: the ragged GQA batch with K
scales in four head_dim groups ("k_groups_variant"), that batch and the
windowed head_dim-64 workloads with head-major pages ("hnd_variant"), the
ragged GQA batch with NVFP4 pages ("nvfp4_variant", bytes = D/2 + D/16 per
token, kv head and side) and with MXFP8 pages ("mxfp8_variant", D + D/32
bytes), and chunked prefill,
q_len 16 to 512 new tokens over a paged context ("prefill", in algorithmic
TFLOP/s against the dense FP8 peak).

HBM traffic (roofline.traffic): four rocprofv3 --pmc passes, FETCH_SIZE and
WRITE_SIZE over this workload and over `--calibrate-copy` (device copies of
a known size), turned into bytes per launch by `--write-traffic`; see the
profiles/ summary for the commands.  The figure is dropped (null) when the
kernel sources have changed since the counters were taken.

Prints ONE JSON line (rank 0, N=1):
  value = attended KV bytes read per step / step time, in GB/s;
  roofline = the partial kernel's KV bytes / its average duration (the
    partial-only graph above), against 8 TB/s;
  cpu_baseline = the float64 CPU oracle on a time-bounded sample of the
    headline workload, in the same unit.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV-read HBM GB/s (% of MI355X peak) and decode tokens/s, FP8 paged attn"
PEAK_GBPS = 8000.0
# The JSON line's workload: the largest of the named workloads (the metric
# names none), the MTP batch.  The widenings are timed on the ragged GQA batch.
HEADLINE = 5
WIDEN = 2
BAR_PCT = 70.0             # KV-read bandwidth asked of workloads 1-4, % of peak
BAR_WORKLOADS = (1, 2, 3, 4)
MALL_FLUSH_BYTES = 1 << 30
REPLAYS = 5                # timed replays of the captured K steps
COPY_BYTES = 1 << 30       # device-copy ceiling measurement
COLD_CALLS = 50            # flushed single calls of a workload the rotation cannot keep cold


def kv_bytes(wl):
    """Algorithmic KV bytes of one call: each attended K and V byte once.

    Per attended token per kv head the method must read D bytes of K and D
    of V; tokens outside every row's window are not counted.
    """
    per_row = {"nvfp4": wl.D // 2 + wl.D // 16, "mxfp8": wl.D + wl.D // 32}.get(wl.kv_format, wl.D)
    return wl.attended_positions() * wl.Hkv * per_row * 2


def other_bytes(wl):
    """q, out, lse, the table entries of touched pages and seq_lens."""
    rows = wl.B * wl.q_len * wl.Hq
    pages = 0
    for b in range(wl.B):
        lo, hi = wl.key_union(b)
        if hi > lo:
            pages += (hi - 1) // wl.bt - lo // wl.bt + 1
    return rows * wl.D * 2 * 2 + rows * 4 + pages * 4 + wl.B * 4


def describe(wl):
    seq = wl.seq_lens
    return (f"{wl.name}: B={wl.B} q_len={wl.q_len} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} bt={wl.bt} "
            f"seq_lens[min={int(seq.min())},max={int(seq.max())},sum={int(seq.sum())}] "
            f"window={wl.window} sinks={'yes' if wl.sinks is not None else 'no'} "
            f"sm_scale={wl.sm_scale:.6g} k_scale={'per-kv-head' if wl.k_scale.size > wl.k_groups else 'per-tensor'}"
            + (f" x {wl.k_groups} head_dim groups" if wl.k_groups > 1 else ""))


def partial_kernel_name(plan, D):
    """The partial kernel a plan launches, as rocprofv3 names it."""
    if plan["variant"] == 1:
        pr = plan["heads_per_wave"]
        lw = plan["row_groups_per_wg"] if plan["row_groups_per_wg"] > 1 else 0
        return (f"partial_mfma_kernel<{D * pr}, {plan['waves_per_head']}, {pr}, "
                f"{plan['row_blocks']}, {plan['nontemporal_kv']}, {lw}>")
    return (f"partial_dot_kernel<{D}, 0, {plan['rows_per_group']}"
            + (", 1>" if plan["nontemporal_kv"] else ">"))


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("kernels.hip", "host.cpp", "plan.h"):
        with open(os.path.join(ROOT, "decode_attention_paged_fp8pa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload_name):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, if current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    h = t.get("hbm_bytes_per_launch")
    return None if not h else int(h["read"] + h["write"])


def sample_gpu_state(busy, seconds_cap=20.0):
    """GPU clocks and socket power read by `amd-smi metric` (a child process)
    while `busy()` keeps the GPU running the timed work; None where the tool
    is missing or its output is not understood.  Taken outside every timed
    region."""
    import shutil
    import subprocess

    exe = shutil.which("amd-smi")
    if exe is None:
        return None
    # Under a profiler, whose preloaded library starts the GPU runtime in
    # every child, the tool's own exec would be refused: no sample then.
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ):
        return None
    try:
        proc = subprocess.Popen([exe, "metric", "--clock", "--power", "--json"],
                                stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    except OSError:
        return None
    t_end = time.time() + seconds_cap
    while proc.poll() is None and time.time() < t_end:
        busy()
    try:
        text, _ = proc.communicate(timeout=max(1.0, t_end - time.time()))
    except subprocess.TimeoutExpired:
        proc.kill()
        proc.communicate()
        return None
    try:
        data = json.loads(text)
        g = data["gpu_data"][0] if isinstance(data, dict) else data[0]
        clock = g["clock"]

        def mhz(entry, key="clk"):
            v = entry.get(key) if isinstance(entry, dict) else None
            return v.get("value") if isinstance(v, dict) else None

        gfx = [mhz(v) for k_, v in sorted(clock.items()) if k_.startswith("gfx_")]
        gfx = [x for x in gfx if isinstance(x, (int, float))]
        gfx_max = [mhz(v, "max_clk") for k_, v in clock.items() if k_.startswith("gfx_")]
        gfx_max = [x for x in gfx_max if isinstance(x, (int, float))]
        power = g.get("power", {}).get("socket_power")
        return {
            "tool": "amd-smi metric --clock --power",
            "sampled": "while the headline step's graph replays",
            "gfx_clk_mhz_per_xcd": gfx,
            "gfx_max_clk_mhz": max(gfx_max) if gfx_max else None,
            "mem_clk_mhz": mhz(clock.get("mem_0", {})),
            "socket_power_w": power.get("value") if isinstance(power, dict) else None,
        }
    except (ValueError, KeyError, IndexError, TypeError, AttributeError):
        return None


def measure(k, steps, warmup, log, use_graph=True, k_groups=1, kv_layout="NHD", kv_format="e4m3",
            sample_clocks=False):
    import torch

    import decode_attention_paged_fp8pa_amd as fp
    from workloads import CONFIGS, make_config, make_mxfp8_workload, make_nvfp4_workload

    t_gen = time.time()
    blockscaled = kv_format != "e4m3"
    if blockscaled:  # the same batch shape with block-scaled pages (random codes and block scales)
        c = CONFIGS[k]
        seq = c["seq"]
        sls = seq[1] if seq[0] == "fixed" else (list(seq[1]) if seq[0] == "list" else ("uniform", seq[1], seq[2]))
        make = make_nvfp4_workload if kv_format == "nvfp4" else make_mxfp8_workload
        wl = make(B=c["B"], q_len=c["q_len"], Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"], bt=c["bt"],
                                 seq_lens=sls, seed=1000 + k, pool=c["pool"], scale=c["scale"],
                                 window=c["window"], sinks=c["sinks"], sm_scale=c["sm_scale"],
                                 kv_layout=kv_layout, name=f"cfg{k}_{c['name']}_{kv_format}")
    else:
        wl = make_config(k, k_groups=k_groups)
    label = (f"cfg{k}" + (f"_kg{k_groups}" if k_groups > 1 else "") + (f"_{kv_format}" if blockscaled else "")
             + ("_hnd" if kv_layout == "HND" else ""))
    log(f"[bench] {label}: generated in {time.time() - t_gen:.1f}s; {describe(wl)}")
    dev = torch.device("cuda")
    kvb = kv_bytes(wl)
    copies = int(min(16, max(2, math.ceil(MALL_FLUSH_BYTES / max(kvb, 1)))))
    q = torch.from_numpy(wl.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    if kv_layout == "HND" and not blockscaled:  # the same pages stored head-major
        kc0 = torch.from_numpy(np.ascontiguousarray(wl.k_cache.transpose(0, 2, 1, 3))).to(dev)
        vc0 = torch.from_numpy(np.ascontiguousarray(wl.v_cache.transpose(0, 2, 1, 3))).to(dev)
    else:
        kc0 = torch.from_numpy(wl.k_cache).to(dev)
        vc0 = torch.from_numpy(wl.v_cache).to(dev)
    pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(copies - 1)]
    btab = torch.from_numpy(wl.block_table).to(dev)
    sl = torch.from_numpy(wl.seq_lens).to(dev)
    ks = torch.from_numpy(wl.k_scale).to(dev)
    vs = torch.from_numpy(wl.v_scale).to(dev)
    sinks = None if wl.sinks is None else torch.from_numpy(wl.sinks).to(dev)
    shape = fp.shape_for(q, kc0, btab, ks, vs, window=wl.window, sm_scale=wl.sm_scale,
                         max_seq_len=int(wl.seq_lens.max()), k_groups=wl.k_groups, kv_layout=kv_layout,
                         kv_format=wl.kv_format, num_kv_heads=wl.Hkv, block_tokens=wl.bt)
    plan = fp.fp8pa_plan(shape, torch.cuda.get_device_properties(0).multi_processor_count)
    nws = fp.fp8pa_workspace_bytes(shape)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    out = torch.empty(tuple(wl.q_bits.shape), dtype=torch.bfloat16, device=dev)
    lse = torch.empty(tuple(wl.q_bits.shape[:3]), dtype=torch.float32, device=dev)

    def step(i):
        kc, vc = pools[i % copies]
        fp.fp8pa_decode(shape, q, kc, vc, btab, sl, ks, vs, sinks, out, lse,
                        ws if nws else None, nws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # eager: one library call per step from Python (CPU launch cost included)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    eager_ms = e0.elapsed_time(e1) / steps
    eager_out = out.clone()

    # timed: the same K steps captured once in a HIP graph and replayed, so
    # the GPU runs them back to back without Python launch gaps
    if not use_graph:
        return _result(wl, label, kvb, copies, plan, eager_ms, eager_ms, wall_ms, wall_ms, False,
                       eager_ms, 0.0, log), wl
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    graph_ok = bool(torch.equal(out, eager_out))
    if not graph_ok:
        log(f"[bench] {label}: graph replay output differs from eager; reporting eager timing")
    torch.cuda.synchronize()
    # REPLAYS timed replays of the K steps: the step time is their median,
    # reported with the spread over replays
    per_replay = []
    t0 = time.perf_counter()
    for _ in range(REPLAYS):
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        per_replay.append(e0.elapsed_time(e1) / steps)
    graph_wall_ms = (time.perf_counter() - t0) * 1e3 / (steps * REPLAYS)
    per_replay.sort()
    step_ms = per_replay[len(per_replay) // 2] if graph_ok else eager_ms
    spread = {"p10_us": round(float(np.percentile(per_replay, 10)) * 1e3, 2),
              "median_us": round(step_ms * 1e3, 2),
              "p90_us": round(float(np.percentile(per_replay, 90)) * 1e3, 2),
              "replays": REPLAYS}
    gpu_state = None
    if sample_clocks:
        gpu_state = sample_gpu_state(lambda: (graph.replay(), torch.cuda.synchronize()))
        if gpu_state:
            log(f"[bench] {label}: under load gfx clock {gpu_state['gfx_clk_mhz_per_xcd']} MHz, memory "
                f"{gpu_state['mem_clk_mhz']} MHz, socket power {gpu_state['socket_power_w']} W")
    del graph

    # the partial kernel alone: the same K steps with the merge launch left
    # out (FP8PA_FLAG_PARTIAL_ONLY), also captured and replayed, on the
    # stream the kernel is launched on
    partial_ms = step_ms
    if plan["merge_launched"]:
        pshape = fp.shape_for(q, kc0, btab, ks, vs, window=wl.window, sm_scale=wl.sm_scale,
                              max_seq_len=int(wl.seq_lens.max()), flags=fp.FP8PA_FLAG_PARTIAL_ONLY,
                              k_groups=wl.k_groups, kv_layout=kv_layout, kv_format=wl.kv_format,
                              num_kv_heads=wl.Hkv, block_tokens=wl.bt)

        def partial_only(i):
            kc, vc = pools[i % copies]
            fp.fp8pa_decode(pshape, q, kc, vc, btab, sl, ks, vs, sinks, out, lse, ws, nws)

        for i in range(3):
            partial_only(i)
        torch.cuda.synchronize()
        pgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(pgraph):
            for i in range(steps):
                partial_only(i)
        pgraph.replay()
        torch.cuda.synchronize()
        e0.record()
        pgraph.replay()
        e1.record()
        torch.cuda.synchronize()
        partial_ms = e0.elapsed_time(e1) / steps
        del pgraph
        step(0)  # leave the outputs as one full step writes them
        torch.cuda.synchronize()
    merge_ms = max(step_ms - partial_ms, 0.0)
    # A workload too small for the pool rotation to push its bytes out of the
    # 256 MB Infinity Cache (C copies of under 1 GiB in all) is timed cold
    # instead: 1 GiB is written before each of COLD_CALLS eager calls, each
    # bracketed by HIP events on this stream; the graph figure stays as the
    # warm one.
    warm_step_ms = None
    timing = None
    if copies * kvb < MALL_FLUSH_BYTES:
        flush = torch.empty(MALL_FLUSH_BYTES, dtype=torch.uint8, device=dev)
        cold = []
        for i in range(COLD_CALLS):
            flush.fill_(i & 0xFF)
            e0.record()
            step(i)
            e1.record()
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        del flush
        cold.sort()
        warm_step_ms = step_ms
        step_ms = cold[len(cold) // 2]
        spread = {"p10_us": round(float(np.percentile(cold, 10)) * 1e3, 2),
                  "median_us": round(step_ms * 1e3, 2),
                  "p90_us": round(float(np.percentile(cold, 90)) * 1e3, 2), "calls": COLD_CALLS}
        timing = f"cold: 1 GiB written before each of {COLD_CALLS} eager calls, HIP events per call"
        log(f"[bench] {label}: cold step {step_ms * 1e3:.1f} us (warm graph replay {warm_step_ms * 1e3:.1f} us)")
    res = _result(wl, label, kvb, copies, plan, step_ms, eager_ms, wall_ms, graph_wall_ms, graph_ok,
                  partial_ms, merge_ms, log)
    res["spread"] = spread
    res["gpu_state"] = gpu_state
    res["timing"] = timing
    res["warm_graph_step_us"] = None if warm_step_ms is None else round(warm_step_ms * 1e3, 2)
    del pools, kc0, vc0
    torch.cuda.empty_cache()
    return res, wl


def _result(wl, label, kvb, copies, plan, step_ms, eager_ms, wall_ms, graph_wall_ms, graph_ok,
            partial_ms, merge_ms, log):
    res = dict(
        workload=wl.name,
        describe=describe(wl),
        D=wl.D,
        kv_bytes=kvb,
        other_bytes=other_bytes(wl),
        copies=copies,
        plan=plan,
        step_ms=step_ms,
        eager_ms=eager_ms,
        wall_ms_per_step=wall_ms,
        graph_wall_ms_per_step=graph_wall_ms,
        graph_ok=graph_ok,
        partial_ms=partial_ms,
        merge_ms=merge_ms,
        kv_gbps=kvb / (step_ms * 1e-3) / 1e9,
        partial_kv_gbps=kvb / (partial_ms * 1e-3) / 1e9,
        tokens_per_s=wl.B * wl.q_len / (step_ms * 1e-3),
    )
    res["pct_peak"] = 100.0 * res["kv_gbps"] / PEAK_GBPS
    log(f"[bench] {label}: step {step_ms * 1e3:.1f} us (partial {partial_ms * 1e3:.1f} us, merge "
        f"{merge_ms * 1e3:.1f} us), KV {res['kv_gbps']:.0f} GB/s = {res['pct_peak']:.1f}% of peak, "
        f"{res['tokens_per_s']:.3g} tok/s, splits {plan['num_splits']}, copies {copies}")
    return res


def copy_ceiling(log):
    """A plain 1 GiB device-to-device copy: (read + write bytes) / time, the
    practical HBM ceiling the decode kernels are compared with."""
    import torch

    n = COPY_BYTES
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(5):
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    t = sorted(times)[len(times) // 2]
    gbps = 2 * n / t / 1e9
    log(f"[bench] device copy of {n >> 20} MiB: {t * 1e6:.1f} us, {gbps:.0f} GB/s read+write "
        f"({gbps / PEAK_GBPS * 100:.1f}% of {PEAK_GBPS:.0f} GB/s)")
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_read_plus_written": 2 * n, "median_us": round(t * 1e6, 1), "gbps": round(gbps, 1),
            "pct_of_peak": round(gbps / PEAK_GBPS * 100, 2)}


def read_ceiling(results, log, launches=50):
    """The practical floor of each workload's step: one launch that reads
    only the workload's KV byte count (fp8pa_debug_stream_read: contiguous
    chunks, 16-byte loads; and at the ragged GQA batch's byte count with 4-
    and 8-byte loads too), cold (buffers rotated through >= 1 GiB), timed
    from graph replays like the decode; and one empty launch, which the merge
    kernel adds on top of any partial pass."""
    import torch

    import decode_attention_paged_fp8pa_amd as fp

    sink = torch.zeros(64, dtype=torch.int32, device="cuda")

    def timed(nbytes, bufs, load_bytes=16):
        for i in range(3):
            fp.fp8pa_debug_stream_read(bufs[i % len(bufs)], nbytes, sink, load_bytes=load_bytes)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(launches):
                fp.fp8pa_debug_stream_read(bufs[i % len(bufs)], nbytes, sink, load_bytes=load_bytes)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        per = []
        for _ in range(REPLAYS):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / launches * 1e3)
        del g
        return sorted(per)[len(per) // 2]

    out = {"empty_launch_us": round(timed(0, [sink]), 2)}
    # The same read with 4-, 8- and 16-byte loads (1x, 2x, 4x the load
    # instructions for the same bytes), at the ragged GQA batch's byte count.
    if 2 in results:
        nbytes = (int(results[2]["kv_bytes"]) + 15) // 16 * 16
        copies = int(min(16, max(2, math.ceil(MALL_FLUSH_BYTES / nbytes))))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
        widths = {}
        for w in (16, 8, 4):
            widths[w] = round(timed(nbytes, bufs, w), 2)
        out["load_width_us"] = {"kv_bytes": nbytes, **{f"{w}B": us for w, us in widths.items()}}
        log(f"[bench] read ceiling by load width, {nbytes / 1e6:.1f} MB: " +
            ", ".join(f"{w}-byte loads {us:.1f} us" for w, us in widths.items()))
        del bufs
        torch.cuda.empty_cache()
    for k, r in results.items():
        nbytes = (int(r["kv_bytes"]) + 15) // 16 * 16
        if nbytes < (64 << 20):
            continue  # launch-bound: nothing to stream
        copies = int(min(16, max(2, math.ceil(MALL_FLUSH_BYTES / nbytes))))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
        us = timed(nbytes, bufs)
        floor_step = us + (out["empty_launch_us"] if r["merge_ms"] > 0 else 0.0)
        out[f"cfg{k}"] = {"kv_bytes": nbytes, "read_us": round(us, 2),
                          "read_gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
                          "floor_step_us": round(floor_step, 2),
                          "floor_pct_of_peak": round(nbytes / (floor_step * 1e-6) / 1e9 / PEAK_GBPS * 100, 1)}
        log(f"[bench] read ceiling cfg{k}: {nbytes / 1e6:.1f} MB in one launch {us:.1f} us "
            f"({nbytes / (us * 1e-6) / 1e9:.0f} GB/s); with an empty merge launch {floor_step:.1f} us")
        del bufs
        torch.cuda.empty_cache()
    log(f"[bench] empty launch {out['empty_launch_us']:.2f} us")
    return out


def measure_writer(steps, log):
    """fp8pa_cache_write: new tokens' bf16 keys and values into E4M3 pages
    (Hkv = 8, D = 128, 16-token pages, per-kv-head scales), at the size of
    one MTP decode step (256 sequences x 4 tokens) and of a prefill chunk
    (65536 tokens).  Bytes moved per call = T * Hkv * D * (2 + 2 read + 1 + 1
    written) + 8 T of slots; timed from graph replays like the decode."""
    import torch

    import decode_attention_paged_fp8pa_amd as fp

    out = {}
    Hkv, D, bt = 8, 128, 16
    gen = torch.Generator(device="cpu").manual_seed(7)
    for name, T in (("decode_step_1024_tokens", 1024), ("prefill_65536_tokens", 65536)):
        nb = (T + bt - 1) // bt + 64
        key = torch.randn((T, Hkv, D), generator=gen).to(torch.bfloat16).cuda()
        value = torch.randn((T, Hkv, D), generator=gen).to(torch.bfloat16).cuda()
        slots = torch.randperm(nb * bt, generator=gen)[:T].to(torch.int64).cuda()
        ks = torch.full((Hkv,), 0.05).cuda()
        vs = torch.full((Hkv,), 0.05).cuda()
        kc = torch.zeros((nb, bt, Hkv, D), dtype=torch.uint8, device="cuda")
        vc = torch.zeros_like(kc)
        for _ in range(3):
            fp.cache_write(key, value, slots, ks, vs, kc, vc)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                fp.cache_write(key, value, slots, ks, vs, kc, vc)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        per = []
        for _ in range(REPLAYS):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / steps * 1e-3)
        t = sorted(per)[len(per) // 2]
        nbytes = T * Hkv * D * 6 + 8 * T
        out[name] = {"tokens": T, "us": round(t * 1e6, 2), "bytes": nbytes,
                     "gbps": round(nbytes / t / 1e9, 1), "pct_of_peak": round(nbytes / t / 1e9 / PEAK_GBPS * 100, 2)}
        log(f"[bench] writer {name}: {t * 1e6:.1f} us, {nbytes / t / 1e9:.0f} GB/s read+write "
            f"({nbytes / t / 1e9 / PEAK_GBPS * 100:.1f}% of peak)")
        del g, key, value, kc, vc
        torch.cuda.empty_cache()
    return out


PEAK_FP8_TFLOPS = 5000.0    # MI355X dense FP8 MFMA
PREFILL_SHAPES = (
    # name, B, q_len, Hq, Hkv, D, bt, context (seq_len, the chunk included)
    ("chunk512_ctx32k", 2, 512, 32, 8, 128, 16, 32768),
    ("chunk128_ctx8k", 8, 128, 32, 8, 128, 16, 8192),
    ("chunk16_ctx8k", 16, 16, 32, 8, 128, 16, 8192),
)


def measure_prefill(log, steps=5):
    """Chunked prefill through fp8pa_decode: q_len new tokens per sequence,
    causal among themselves, over a paged E4M3 context.  MFMA-bound, so the
    rate is algorithmic FLOP/s, 4 D per (query row, attended key) (q.K and
    P.V, a multiply and an add each), against the dense FP8 peak; the
    matrix cores spend twice the time an FP8-only pass would (the query goes
    in as an E4M3 hi + lo pair, and P.V runs in bf16, at half the FP8 rate).
    A chunk of few rows per kv head reads more KV bytes per FLOP than the
    FP8 ridge (625 FLOP/byte): its bound is HBM, its rate the KV bytes (2 D
    per attended key and kv head) against 8 TB/s; both rates are reported.
    Timed from graph replays like the decode."""
    import torch

    import decode_attention_paged_fp8pa_amd as fp
    from workloads import make_workload

    out = {}
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    for name, B, ql, Hq, Hkv, D, bt, ctx in PREFILL_SHAPES:
        wl = make_workload(B=B, q_len=ql, Hq=Hq, Hkv=Hkv, D=D, bt=bt, seq_lens=[ctx] * B, seed=17,
                           poison=False, scale=("per_head", 0.02, 0.1), name=name)
        flops = sum(4 * D * Hq * (ctx - ql + i + 1) for i in range(ql)) * B
        kv_bytes = B * ctx * Hkv * 2 * D
        bound = "hbm" if kv_bytes / (PEAK_GBPS * 1e9) > flops / (PEAK_FP8_TFLOPS * 1e12) else "mfma"
        dev = "cuda"
        q = torch.from_numpy(wl.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        kc = torch.from_numpy(wl.k_cache).to(dev)
        vc = torch.from_numpy(wl.v_cache).to(dev)
        btab = torch.from_numpy(wl.block_table).to(dev)
        sl = torch.from_numpy(wl.seq_lens).to(dev)
        ks = torch.from_numpy(wl.k_scale).to(dev)
        vs = torch.from_numpy(wl.v_scale).to(dev)
        shape = fp.shape_for(q, kc, btab, ks, vs, sm_scale=wl.sm_scale, max_seq_len=ctx)
        plan = fp.fp8pa_plan(shape, cu)
        nws = fp.fp8pa_workspace_bytes(shape)
        ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
        o = torch.empty(tuple(wl.q_bits.shape), dtype=torch.bfloat16, device=dev)
        lse = torch.empty(tuple(wl.q_bits.shape[:3]), dtype=torch.float32, device=dev)

        def step():
            fp.fp8pa_decode(shape, q, kc, vc, btab, sl, ks, vs, None, o, lse, ws if nws else None, nws)

        for _ in range(3):
            step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                step()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        per = []
        for _ in range(REPLAYS):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / steps * 1e-3)
        t = sorted(per)[len(per) // 2]
        tflops = flops / t / 1e12
        out[name] = {"workload": f"B={B} q_len={ql} Hq={Hq} Hkv={Hkv} D={D} bt={bt} seq_len={ctx}",
                     "us": round(t * 1e6, 1), "algorithmic_flops": flops, "tflops": round(tflops, 1),
                     "pct_of_fp8_peak": round(tflops / PEAK_FP8_TFLOPS * 100, 2),
                     "kv_bytes": kv_bytes, "kv_gbps": round(kv_bytes / t / 1e9, 1),
                     "pct_of_hbm_peak": round(kv_bytes / t / 1e9 / PEAK_GBPS * 100, 2), "bound": bound,
                     "variant": "mfma" if plan["variant"] == 1 else "dot",
                     "num_splits": plan["num_splits"], "grid_wgs": plan["grid_wgs"]}
        log(f"[bench] prefill {name}: {t * 1e6:.1f} us, {tflops:.1f} TFLOP/s "
            f"({tflops / PEAK_FP8_TFLOPS * 100:.2f}% of dense FP8 peak), KV {kv_bytes / t / 1e9:.0f} GB/s "
            f"({kv_bytes / t / 1e9 / PEAK_GBPS * 100:.1f}% of 8 TB/s), {bound}-bound, splits {plan['num_splits']}")
        del g, kc, vc, q, ws
        torch.cuda.empty_cache()
    return out


def cpu_baseline(wl, budget_s, log):
    """The float64 oracle, as it stands, on whole sequences until the budget is used."""
    import oracle

    from threadpoolctl import threadpool_info, threadpool_limits

    ncores = len(os.sched_getaffinity(0))
    limiter = threadpool_limits(limits=ncores)
    t0 = time.perf_counter()
    done_bytes = 0
    done_tokens = 0
    seqs = 0
    passes = 0
    # whole sequences (all heads), in order, repeating the workload until the
    # time budget is used (at least one full pass)
    while True:
        for b in range(wl.B):
            rows = [(b, i, h) for i in range(wl.q_len) for h in range(wl.Hq)]
            oracle.decode(**wl.oracle_kwargs(), rows=rows)
            lo, hi = wl.key_union(b)
            done_bytes += (hi - lo) * wl.Hkv * wl.D * 2
            done_tokens += wl.q_len
            seqs += 1
            if passes > 0 and time.perf_counter() - t0 >= budget_s:
                break
        passes += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = int(infos[0].get("num_threads", ncores)) if infos else 1
    limiter.restore_original_limits()
    log(f"[bench] cpu oracle: {seqs} sequence decodes in {el:.1f}s, {done_bytes / el / 1e9:.3f} GB/s")
    return {"value": done_bytes / el / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{wl.name}: {seqs} sequence decodes (all {wl.Hq} heads each; the {wl.B}-sequence "
                      f"batch repeated, {passes} pass(es)), {done_bytes} KV bytes in {el:.1f}s; "
                      f"{done_tokens / el:.3g} tokens/s",
            "host": {"cpu_model": cpu_model(), "cpus_available": ncores, "blas_threads": threads}}


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


CALIB_BYTES = 256 << 20
CALIB_COPIES = 8


def calibrate_copy():
    """Device-to-device copies of CALIB_BYTES each: the counter scale reference."""
    import torch

    a = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    for _ in range(CALIB_COPIES):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copies": CALIB_COPIES, "bytes_each": CALIB_BYTES}), flush=True)


def _counter_rows(csv_dir, counter):
    import csv
    import glob
    import re

    rows = []
    for f in glob.glob(os.path.join(csv_dir, "*counter_collection.csv")):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                m = re.search(r"(\w+<[\w, ]+>|__amd_\w+)", r["Kernel_Name"])
                rows.append((int(r["Dispatch_Id"]), m.group(1) if m else r["Kernel_Name"][:40],
                             float(r["Counter_Value"])))
    return sorted(rows)


def write_traffic(wl_fetch, wl_write, cal_fetch, cal_write, workload_name):
    """Bytes per launch of each decode kernel from FETCH_SIZE / WRITE_SIZE (KiB),
    each scaled by what the same counter reads for a copy of known size."""
    cf = [v for _, k, v in _counter_rows(cal_fetch, "FETCH_SIZE") if k.startswith("__amd")]
    cw = [v for _, k, v in _counter_rows(cal_write, "WRITE_SIZE") if k.startswith("__amd")]
    cf = [v for v in cf if v > 0][-CALIB_COPIES:]
    cw = [v for v in cw if v > 0][-CALIB_COPIES:]
    fetch_scale = CALIB_BYTES / (sum(cf) / len(cf) * 1024.0)
    write_scale = CALIB_BYTES / (sum(cw) / len(cw) * 1024.0)
    out = {"workload": workload_name, "kernel_source_hash": kernel_source_hash(),
           "calibration": {"copy_bytes": CALIB_BYTES, "fetch_kib_read": sum(cf) / len(cf),
                           "write_kib_read": sum(cw) / len(cw), "fetch_scale": fetch_scale,
                           "write_scale": write_scale}, "kernels": {}}
    for name, rows_f, rows_w in (("fetch", _counter_rows(wl_fetch, "FETCH_SIZE"), None),
                                 ("write", _counter_rows(wl_write, "WRITE_SIZE"), None)):
        per = {}
        for _, k, v in rows_f:
            if k.startswith("__amd"):
                continue
            per.setdefault(k, []).append(v)
        for k, vals in per.items():
            d = out["kernels"].setdefault(k, {})
            scale = fetch_scale if name == "fetch" else write_scale
            d[name + "_bytes_per_launch"] = sum(vals) / len(vals) * 1024.0 * scale
            d[name + "_launches"] = len(vals)
    partial = [k for k in out["kernels"] if k.startswith("partial_")]
    if partial:
        d = out["kernels"][partial[0]]
        out["hbm_bytes_per_launch"] = {"kernel": partial[0],
                                       "read": round(d.get("fetch_bytes_per_launch", 0.0)),
                                       "write": round(d.get("write_bytes_per_launch", 0.0))}
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--configs", default="1,2,3,4,5,6",
                    help="named workloads 1-5, and 6: the ragged GQA batch as MHA decode (VALU kernel)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="time the named decode workloads only (for profiler runs)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches only (for profiler passes that do not follow graphs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the known-size device copies used to scale traffic counters")
    ap.add_argument("--only", choices=ONLY_CHOICES,
                    help="time one workload alone and print its [bench] line, no JSON line "
                         "(for kernel traces that attribute every launch to one workload)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("WL_FETCH", "WL_WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="rocprofv3 --pmc output dirs -> profiles/traffic_<workload>.json (no GPU)")
    ap.add_argument("--traffic-workload", default=str(HEADLINE),
                    help="named workload (1-5) the --write-traffic counters were taken on")
    args = ap.parse_args()
    if args.write_traffic:
        from workloads import CONFIGS

        k = int(args.traffic_workload)
        write_traffic(*args.write_traffic, workload_name=f"cfg{k}_{CONFIGS[k]['name']}")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU form in this library)", file=sys.stderr)
        sys.exit(2)

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    import torch

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy()
        return
    import decode_attention_paged_fp8pa_amd as fp

    fp.lib()
    if args.only:
        run_only(args, log)
        return
    cfgs = [int(x) for x in args.configs.split(",") if x]
    if HEADLINE not in cfgs:
        cfgs.insert(0, HEADLINE)
    results = {}
    head_wl = None
    ceiling = None if args.decode_only else copy_ceiling(log)
    for k in cfgs:
        res, wl = measure(k, args.steps, args.warmup, log, use_graph=not args.no_graph,
                          sample_clocks=(k == HEADLINE and not args.decode_only))
        results[k] = res
        if k == HEADLINE:
            head_wl = wl
        else:
            del wl
    h = results[HEADLINE]
    traffic = load_traffic(h["workload"])
    roof = {
        "bound": "hbm",
        "achieved": round(h["partial_kv_gbps"], 1),
        "peak": PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(h["partial_kv_gbps"] / PEAK_GBPS, 4),
        "traffic": traffic,
        "kernel": partial_kernel_name(h["plan"], head_wl.D),
        "kernel_avg_us": round(h["partial_ms"] * 1e3, 2),
        "algorithmic_bytes_per_launch": h["kv_bytes"],
    }
    writer = kg = hnd = nv = prefill = None
    ceiling_reads = read_ceiling(results, log)
    if not args.decode_only:
        writer, kg, hnd, nv, prefill = widenings(args, log)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(head_wl, args.cpu_budget, log)
    emit(args, results, h, head_wl, roof, cpu, ceiling, writer, kg, hnd, nv, prefill, ceiling_reads)


ONLY_CHOICES = ("cfg1", "cfg2", "cfg3", "cfg4", "cfg5", "cfg6", "writer", "cfg2_kg4", "cfg2_hnd", "cfg3_hnd",
                "cfg2_nvfp4_hnd", "cfg2_mxfp8_hnd", "prefill")


def run_only(args, log):
    """One workload of the bench, alone in the process (profiler runs)."""
    name = args.only
    graph = not args.no_graph
    if name == "writer":
        measure_writer(min(args.steps, 100), log)
    elif name == "prefill":
        measure_prefill(log)
    else:
        k = int(name[3])
        kw = {}
        if name.endswith("_kg4"):
            kw["k_groups"] = 4
        if name.endswith("_hnd"):
            kw["kv_layout"] = "HND"
        for f in ("nvfp4", "mxfp8"):
            if f"_{f}" in name:
                kw["kv_format"] = f
        measure(k, args.steps, args.warmup, log, use_graph=graph, **kw)


def widenings(args, log):
    """The library's widenings, timed after the decode workloads."""
    writer = measure_writer(min(args.steps, 100), log)
    # the headline workload with K scales in 4 head_dim groups per kv head
    kg_res, kg_wl = measure(WIDEN, args.steps, args.warmup, log, use_graph=not args.no_graph,
                            k_groups=4)
    del kg_wl
    kg = {
        "workload": kg_res["describe"], "step_us": round(kg_res["step_ms"] * 1e3, 2),
        "partial_us": round(kg_res["partial_ms"] * 1e3, 2),
        "kv_gbps": round(kg_res["kv_gbps"], 1), "pct_peak": round(kg_res["pct_peak"], 2),
        "partial_kv_gbps": round(kg_res["partial_kv_gbps"], 1),
    }
    # the headline and the windowed head_dim-64 workloads with head-major pages
    hnd = {}
    for k in (WIDEN, 3):
        r, w_ = measure(k, args.steps, args.warmup, log, use_graph=not args.no_graph, kv_layout="HND")
        hnd[f"cfg{k}"] = {"workload": r["describe"] + " kv_layout=HND", "step_us": round(r["step_ms"] * 1e3, 2),
                          "partial_us": round(r["partial_ms"] * 1e3, 2), "kv_gbps": round(r["kv_gbps"], 1),
                          "pct_peak": round(r["pct_peak"], 2)}
        del w_
    # the headline batch with NVFP4 pages (head-major, as the gist runs them)
    # and with MXFP8 pages (the same row orders)
    bs = {}
    for f in ("nvfp4", "mxfp8"):
        r, w_ = measure(WIDEN, args.steps, args.warmup, log, use_graph=not args.no_graph, kv_layout="HND",
                        kv_format=f)
        bs[f] = {"workload": r["describe"] + f" kv_format={f} kv_layout=HND",
                 "step_us": round(r["step_ms"] * 1e3, 2), "partial_us": round(r["partial_ms"] * 1e3, 2),
                 "kv_bytes": r["kv_bytes"], "kv_gbps": round(r["kv_gbps"], 1), "pct_peak": round(r["pct_peak"], 2),
                 "tokens_per_s": round(r["tokens_per_s"], 1),
                 "variant": "dot" if r["plan"]["variant"] == 0 else "mfma"}
        del w_
    prefill = measure_prefill(log)
    return writer, kg, hnd, bs, prefill


def emit(args, results, h, head_wl, roof, cpu, ceiling, writer, kg, hnd, nv, prefill, ceiling_reads=None):
    """Print the one JSON line."""
    line = {
        "metric": METRIC,
        "value": round(h["kv_gbps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3-mfma+f32",
        "data": "synthetic (seeded; E4M3 K/V of N(0,1)/scale, bf16 q ~ N(0,1))",
        "config": {"workload": h["describe"], "parallelism": "none (1 GPU)",
                   "pct_of_peak": round(h["pct_peak"], 2),
                   "tokens_per_s": round(h["tokens_per_s"], 1)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "gpu_state": h.get("gpu_state"),
        "copy_ceiling": ceiling,
        "read_ceiling": ceiling_reads,
        "writer": writer,
        "k_groups_variant": kg,
        "hnd_variant": hnd,
        "nvfp4_variant": (nv or {}).get("nvfp4"),
        "mxfp8_variant": (nv or {}).get("mxfp8"),
        "prefill": prefill,
        "per_workload": {
            f"cfg{k}": {
                "workload": r["describe"], "step_us": round(r["step_ms"] * 1e3, 2),
                "partial_us": round(r["partial_ms"] * 1e3, 2), "merge_us": round(r["merge_ms"] * 1e3, 2),
                "kv_bytes": r["kv_bytes"], "kv_gbps": round(r["kv_gbps"], 1),
                "partial_kv_gbps": round(r["partial_kv_gbps"], 1),
                "pct_peak": round(r["pct_peak"], 2), "tokens_per_s": round(r["tokens_per_s"], 1),
                "num_splits": r["plan"]["num_splits"], "grid_wgs": r["plan"]["grid_wgs"],
                "variant": "mfma" if r["plan"]["variant"] == 1 else "dot",
                "eager_us_per_step": round(r["eager_ms"] * 1e3, 2),
                "timing": r.get("timing") or ("hip graph replay" if r["graph_ok"] else "eager"),
                "step_spread": r.get("spread"),
                "warm_graph_step_us": r.get("warm_graph_step_us"),
                "bar_70pct_of_peak": (bool(r["pct_peak"] >= BAR_PCT) if k in BAR_WORKLOADS
                                      else "not in the bar"),
                "partial_kernel": partial_kernel_name(r["plan"], r["D"]),
            } for k, r in results.items()},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
