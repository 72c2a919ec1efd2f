"""Plausible mistakes planted in a copy of the oracle, on the CPU.

Each entry names one oracle source file, a snippet that occurs exactly once
in it and the mistaken text that replaces it.  `apply(name)` re-executes the
oracle package with that one mistake (the files on disk are not touched),
so that the pin tests, run in a fresh process with FP8PA_ORACLE_MUTATION set
(tests/conftest.py), see the mistaken oracle.  tests/test_oracle_mutations.py
requires every mistake to make some pin fail.
"""

from __future__ import annotations

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name: (file under oracle/, text, mistaken text, pin test files)
DECODE_PINS = ("tests/test_oracle.py",)
WRITER_PINS = ("tests/test_writer_oracle.py",)
NVFP4_PINS = ("tests/test_nvfp4_oracle.py",)
MXFP8_PINS = ("tests/test_mxfp8_oracle.py",)

MUTATIONS = {
    # decode oracle
    "window_off_by_one": ("fp8pa_ref.py", "lo = max(0, pos - int(window) + 1)",
                          "lo = max(0, pos - int(window))", DECODE_PINS),
    "own_token_not_attended": ("fp8pa_ref.py", "hi = min(pos + 1, int(seq_len))",
                               "hi = min(pos, int(seq_len))", DECODE_PINS),
    "query_position_shifted": ("fp8pa_ref.py", "pos = int(seq_len) - int(q_len) + int(i)",
                               "pos = int(seq_len) - int(q_len) + int(i) - 1", DECODE_PINS),
    "sink_dropped": ("fp8pa_ref.py",
                     "sink = None if sinks is None else float(np.asarray(sinks).reshape(-1)[h])",
                     "sink = None", DECODE_PINS),
    "sink_outside_denominator": ("fp8pa_ref.py", "denom += math.exp(float(sink) - terms_max)",
                                 "denom += 0.0", DECODE_PINS),
    "lse_without_its_max": ("fp8pa_ref.py", "return e / denom, terms_max + math.log(denom)",
                            "return e / denom, math.log(denom)", DECODE_PINS),
    "gqa_modulo": ("fp8pa_ref.py", "groups.setdefault((b, h // G), []).append(n)",
                   "groups.setdefault((b, h % Hkv), []).append(n)", DECODE_PINS),
    "page_index_modulo": ("fp8pa_ref.py", "pages = block_table_row[ts // bt].astype(np.int64)",
                          "pages = block_table_row[ts % bt].astype(np.int64)", DECODE_PINS),
    "slot_index_divided": ("fp8pa_ref.py", "    slots = ts % bt\n    codes = cache",
                           "    slots = (ts // bt) % bt\n    codes = cache", DECODE_PINS),
    "head_major_read_token_major": ("fp8pa_ref.py",
                                    "codes = cache[pages, g, slots, :] if hnd else cache[pages, slots, g, :]",
                                    "codes = cache[pages, slots, g, :] if hnd else cache[pages, slots, g, :]",
                                    DECODE_PINS),
    "e4m3_bias_8": ("fp8pa_ref.py", "return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)",
                    "return sign * (1.0 + m / 8.0) * 2.0 ** (e - 8)", DECODE_PINS),
    "e4m3_subnormal_scale": ("fp8pa_ref.py", "return sign * (m / 8.0) * 2.0 ** (-6)",
                             "return sign * (m / 8.0) * 2.0 ** (-7)", DECODE_PINS),
    "e4m3_no_nan": ("fp8pa_ref.py", "if e == 0xF and m == 0x7:\n        return float(\"nan\")",
                    "if False:\n        return float(\"nan\")", DECODE_PINS),
    "scale_dropped": ("fp8pa_ref.py",
                      "return E4M3_TABLE[codes] * np.asarray(scale, dtype=np.float64)",
                      "return E4M3_TABLE[codes] * 1.0", DECODE_PINS),
    "k_and_v_scales_swapped": ("fp8pa_ref.py", "ks = k_scale_of_head(k_scale, g, D, k_groups)",
                               "ks = k_scale_of_head(v_scale, g, D, k_groups)", DECODE_PINS),
    "k_groups_interleaved": ("fp8pa_ref.py", "return ks[base + np.arange(D) // (D // kg)]",
                             "return ks[base + np.arange(D) % kg]", DECODE_PINS),
    "sm_scale_dropped": ("fp8pa_ref.py",
                         "scores[:, c0 - u_lo:c0 - u_lo + len(ts)] = sm_scale * (qmat @ kf.T)",
                         "scores[:, c0 - u_lo:c0 - u_lo + len(ts)] = (qmat @ kf.T)", DECODE_PINS),
    "bf16_as_low_half": ("fp8pa_ref.py", "b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)",
                         "b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)",
                         DECODE_PINS),
    "merge_without_sink": ("fp8pa_ref.py",
                           "L = float(w.sum()) + (math.exp(sink - M) if sink is not None else 0.0)",
                           "L = float(w.sum())", DECODE_PINS),
    "merge_unweighted": ("fp8pa_ref.py", "acc += w[s] * po[r, s]", "acc += po[r, s] * (L / S)",
                         DECODE_PINS),
    # E4M3 writer
    "writer_exact_division": ("fp8pa_write_ref.py", "prod = (vals[t, h, :] * inv).astype(np.float32)",
                              "prod = (vals[t, h, :].astype(np.float64) / scales_of(scales, groups, h))",
                              WRITER_PINS),
    "writer_ties_away": ("fp8pa_write_ref.py", "q = int(np.round((2.0 * m - 1.0) * 8.0))",
                         "q = int(np.floor((2.0 * m - 1.0) * 8.0 + 0.5))", WRITER_PINS),
    "writer_saturates_to_nan": ("fp8pa_write_ref.py", "    if a >= E4M3_MAX:\n        return sign | 0x7E",
                                "    if a >= E4M3_MAX:\n        return sign | 0x7F", WRITER_PINS),
    "writer_page_and_place_swapped": ("fp8pa_write_ref.py", "page, off = int(slot) // bt, int(slot) % bt",
                                      "page, off = int(slot) % nb, int(slot) // nb", WRITER_PINS),
    # NVFP4
    "nvfp4_scale_from_scaled_max": ("nvfp4_ref.py", "s = np.float32(g * np.float32(a * SIXTH))",
                                    "s = np.float32(np.float32(a * g) / np.float32(6.0))", NVFP4_PINS),
    "nvfp4_nibbles_swapped": ("nvfp4_ref.py", "codes = np.where(d % 2 == 0, data & 0xF, data >> 4)",
                              "codes = np.where(d % 2 == 0, data >> 4, data & 0xF)", NVFP4_PINS),
    "e2m1_bias_0": ("nvfp4_ref.py", "return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)",
                    "return sign * (1.0 + m / 2.0) * 2.0 ** e", NVFP4_PINS),
    "nvfp4_block_of_8": ("nvfp4_ref.py", "sc = pool[pages[:, None], soff[:, None] + d // 16]",
                         "sc = pool[pages[:, None], soff[:, None] + d // 8 % (head_dim // 16)]", NVFP4_PINS),
    # MXFP8
    "e8m0_bias_128": ("mxfp8_ref.py", "v = np.ldexp(1.0, s - 127)", "v = np.ldexp(1.0, s - 128)",
                      MXFP8_PINS),
    "mxfp8_exponent_off_by_one": ("mxfp8_ref.py", "return int(min(max(x - E4M3_EMAX, -127), 127))",
                                  "return int(min(max(x - E4M3_EMAX + 1, -127), 127))", MXFP8_PINS),
}

_ORDER = ("fp8pa_ref", "fp8pa_write_ref", "nvfp4_ref", "mxfp8_ref")


def apply(name: str) -> None:
    """Re-executes the oracle package with mutation `name` planted."""
    import importlib

    fname, old, new, _ = MUTATIONS[name]
    pkg = importlib.import_module("oracle")
    for mod_name in _ORDER:
        mod = importlib.import_module(f"oracle.{mod_name}")
        path = os.path.join(ROOT, "oracle", mod_name + ".py")
        with open(path) as f:
            src = f.read()
        if mod_name + ".py" == fname:
            if src.count(old) != 1:
                raise RuntimeError(f"mutation {name}: the snippet occurs {src.count(old)} times in {fname}")
            src = src.replace(old, new)
        exec(compile(src, path, "exec"), mod.__dict__)
    init = os.path.join(ROOT, "oracle", "__init__.py")
    with open(init) as f:
        exec(compile(f.read(), init, "exec"), pkg.__dict__)
    sys.modules["oracle"] = pkg
