"""Guards on the generated gfx950 code that the tests of results cannot see.

The scan kernels issue their LDS-DMA loads (global_load_lds_dword[x4], whose LDS
address is taken from m0) through inline assembly that sets m0 itself. m0 is a
register the compiler reserves, so declaring it clobbered does not oblige the
compiler to preserve a value of its own across the statement. The kernels are
correct only while the compiler keeps nothing in m0: this test compiles each
such source with the build's own flags and requires that every instruction
naming m0 is one of those `s_mov_b32 m0, <sgpr>` immediately followed by its
LDS-DMA load. (CPU only: hipcc cross-compiles.)
"""
import os
import re
import shutil
import subprocess

import pytest

from kimi_delta_attention_fwd_amd import build as kbuild

LDS_DMA = re.compile(r"^global_load_lds_dword(x4)?\b")
SRCS = ("kda_scan.hip", "kda_scan_pair.hip")


def _device_asm(name, tmp_path):
    hipcc = kbuild.HIPCC
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    extra = dict(kbuild.KERNEL_UNITS)[name]
    out = tmp_path / (name + ".s")
    cmd = [hipcc, *kbuild.DEVICE_FLAGS, *extra, *kbuild.INCLUDES, "--cuda-device-only", "-S",
           os.path.join(kbuild.CSRC, name), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    return out.read_text()


def _instructions(asm):
    for line in asm.splitlines():
        t = line.split(";", 1)[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        yield t


@pytest.mark.parametrize("name", SRCS)
def test_m0_only_set_for_lds_dma(name, tmp_path):
    ins = list(_instructions(_device_asm(name, tmp_path)))
    n_dma = 0
    for i, t in enumerate(ins):
        if not re.search(r"\bm0\b", t):
            continue
        # the asm's SGPR operand: any SGPR, vcc_lo / vcc_hi included
        assert re.match(r"^s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)$", t), "compiler-generated use of m0: %r" % t
        assert i + 1 < len(ins) and LDS_DMA.match(ins[i + 1]), "m0 set without its LDS-DMA load: %r" % t
        n_dma += 1
    assert n_dma > 0, "no LDS-DMA sequence found; the guard is checking the wrong file"
