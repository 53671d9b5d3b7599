"""Compile every kernel source for gfx950 on the CPU and check the resource
use the compiler reports: no kernel may use scratch (private) memory.  A
lane-dependent index into a register array, for example, would silently move
the array to scratch and make every access a memory access.  Register spills
that stay in registers are allowed, with the private segment at 0: scalar
registers spilled into lanes of a vector register, and at most a few vector
registers spilled into accumulation registers (the other half of gfx950's
unified register file; a move each way, no memory)."""
import os
import re
import subprocess

import pytest

from fp8_kv_cache_append_amd import build

HIPCC = build.HIPCC
SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


@pytest.mark.parametrize("src", SOURCES)
def test_kernels_use_no_scratch(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, *build.FLAGS, "--cuda-device-only", "-S", os.path.join(build.CSRC, src),
           "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    text = out.read_text()
    names = re.findall(r"^\s+\.name:\s+(_Z\S+)", text, flags=re.M)
    private = [int(x) for x in re.findall(r"^\s+\.private_segment_fixed_size:\s+(\d+)", text,
                                          flags=re.M)]
    spills = [int(x) for x in re.findall(r"^\s+\.vgpr_spill_count:\s+(\d+)", text,
                                         flags=re.M)]
    has_kernels = "__global__" in open(os.path.join(build.CSRC, src)).read()
    assert bool(names) == has_kernels and len(private) == len(names)
    bad = [(n, p) for n, p in zip(names, private) if p != 0]
    assert not bad, f"kernels using scratch memory: {bad}"
    # private segment 0 everywhere (checked above), so any vector spill went
    # to accumulation registers; keep those to a handful
    big = [(n, v) for n, v in zip(names, spills) if v > 4]
    assert not big, f"vector register spills in {src}: {big}"
