"""Compile libkda.so in-tree for gfx950 with hipcc (no JIT, no torch extension)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkda.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# every HIP translation unit is built without packed-fp32 VALU instructions
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
INCLUDES = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
# kernel translation units and their extra flags
# (the max-ilp scheduling strategy: prep 1.2 % faster at the long prefill, the
#  segment-parallel scan 4 %; the backward is slower with it)
KERNEL_UNITS = [
    ("kda_prep.hip", ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]),
    ("kda_scan.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form",  # accumulators in VGPRs: no AGPR copies in the chunk loop
                      "-mllvm", "-amdgpu-sched-strategy=max-ilp"]),
    ("kda_scan_pair.hip", []),
    ("kda_decode.hip", []),
    ("kda_bwd.hip", []),
    ("kda_noalloc.hip", []),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "not a recognized feature for this target" not in line)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("command failed: " + " ".join(cmd))
    return out


def build(verbose: bool = False) -> str:
    """Compile the kernels and the C ABI into kimi_delta_attention_fwd_amd/libkda.so."""
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    for name, extra in KERNEL_UNITS:
        obj = os.path.join(bdir, name.replace(".hip", ".o"))
        _run([HIPCC, *DEVICE_FLAGS, *extra, *INCLUDES, "-c", os.path.join(CSRC, name), "-o", obj])
        objs.append(obj)
    a_obj = os.path.join(bdir, "kda_api.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O2", "-fPIC", "-std=c++17", "-Wall", "-fvisibility=hidden", *INCLUDES, "-c",
          os.path.join(CSRC, "kda_api.cpp"), "-o", a_obj])
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, a_obj, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
