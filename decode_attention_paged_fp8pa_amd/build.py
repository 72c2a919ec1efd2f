"""Builds libfp8pa.so in-tree with hipcc for gfx950.

    python -m decode_attention_paged_fp8pa_amd.build      (or build() from Python)

The host TU (validation and planning) and the HIP TUs (decode kernels and
entry points; the KV-cache writer) are compiled separately and linked into
one shared library next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB_NAME = "libfp8pa.so"
ARCH = "gfx950"

# Packed fp32 VALU ops stay off: hipcc would otherwise form v_pk_* fp32 ops
# from plain float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the fp8pa library needs ROCm's hipcc to build")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose: bool = False) -> str:
    """Compiles every source and links libfp8pa.so; returns its path."""
    hipcc = _hipcc()
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    common = ["-O3", "-fPIC", "-std=c++17", "-Wall", f"-I{INCLUDE}"]
    host_o = os.path.join(bdir, "host.o")
    kern_o = os.path.join(bdir, "kernels.o")
    _run([hipcc, *common, "-c", os.path.join(CSRC, "host.cpp"), "-o", host_o])
    _run([hipcc, *common, f"--offload-arch={ARCH}", *DEVICE_FLAGS, "-x", "hip", "-c",
          os.path.join(CSRC, "kernels.hip"), "-o", kern_o])
    write_o = os.path.join(bdir, "cache_write.o")
    _run([hipcc, *common, f"--offload-arch={ARCH}", *DEVICE_FLAGS, "-x", "hip", "-c",
          os.path.join(CSRC, "cache_write.hip"), "-o", write_o])
    out = os.path.join(HERE, LIB_NAME)
    tmp = out + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", host_o, kern_o, write_o, "-o", tmp])
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
