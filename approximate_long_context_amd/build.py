"""Builds libplsh.so in-tree with hipcc for gfx950.

    python -m approximate_long_context_amd.build

Device code is compiled without fast-math and without packed-fp32
instructions; the pre-pass (plsh_prepass.hip: block intervals that must equal
the host table's bit for bit) and the device sampler (plsh_sample.hip: draws
that must round exactly as the host sampler's) also without contraction of
multiply-adds.
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
    objs = [host_obj, dev_obj]
    # kernel translation units; the pre-pass (block intervals, which must equal
    # the host table's) and the device sampler (draws that round as the
    # host's) without contraction of multiply-adds
    for name, extra in (("plsh_fwd", []), ("plsh_mfma16", []), ("plsh_exact", []),
                        ("plsh_prepass", ["-ffp-contract=off"]), ("plsh_sample", ["-ffp-contract=off"])):
        obj = os.path.join(objdir, name + ".o")
        _run([HIPCC, *COMMON, *DEVICE, *extra, "-c", os.path.join(CSRC, name + ".hip"), "-o", obj])
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
