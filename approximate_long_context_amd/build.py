"""Builds libplsh.so in-tree with hipcc for gfx950.

    python -m approximate_long_context_amd.build

Device code is compiled without fast-math (the block predicate must be
bit-exact with the host table) and without packed-fp32 instructions; the
device sampler (plsh_sample.hip) also without contraction of multiply-adds
(its draws must round exactly as the host sampler's).
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libplsh.so")
ARCH = os.environ.get("PLSH_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-std=c++17", "-O3", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function"]
DEVICE = ["-x", "hip", f"--offload-arch={ARCH}", "-ffp-contract=fast",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "unknown target feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build failed ({' '.join(cmd)}):\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source into libplsh.so (always rebuilds)."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    host_obj = os.path.join(objdir, "plsh_host.o")
    dev_obj = os.path.join(objdir, "plsh_attention.o")
    # host half: plain C++ (no HIP), strict IEEE binary64
    _run(["g++", "-std=c++17", "-O2", "-fPIC", "-fvisibility=hidden", "-ffp-contract=off", "-Wall", "-c",
          os.path.join(CSRC, "plsh_host.cpp"), "-o", host_obj])
    _run([HIPCC, *COMMON, *DEVICE, "-c", os.path.join(CSRC, "plsh_attention.hip"), "-o", dev_obj])
    fwd_obj = os.path.join(objdir, "plsh_fwd.o")
    _run([HIPCC, *COMMON, *DEVICE, "-c", os.path.join(CSRC, "plsh_fwd.hip"), "-o", fwd_obj])
    # the device sampler: no contraction, so its draws round as the host's
    samp_obj = os.path.join(objdir, "plsh_sample.o")
    _run([HIPCC, *COMMON, *DEVICE, "-ffp-contract=off", "-c", os.path.join(CSRC, "plsh_sample.hip"),
          "-o", samp_obj])
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", host_obj, dev_obj, fwd_obj, samp_obj, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
