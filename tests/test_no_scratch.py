"""Every device kernel of the library fits its registers: no kernel uses
scratch (private) memory or spills (CPU only: compiles each source to gfx950
assembly and reads the kernel descriptors).

A spilled kernel would move its spilled registers through memory on every use
(a large slowdown for these HBM-bound kernels), and builds of the group-scaling
hold kernel forced to spill (register caps for 5 or 6 waves per SIMD) wrote
wrong codes and scales in the row-major tests while the unspilled build stays
exact, so a spilling build must not ship.
"""
import os
import re
import subprocess

import pytest

from float8_quantization_moe_amd import build as B


@pytest.mark.slow
@pytest.mark.parametrize("src", B.SOURCES)
def test_kernels_use_no_scratch(src, tmp_path):
    out = str(tmp_path / (src + ".s"))
    cmd = [B.hipcc(), *B.COMMON_FLAGS, *B.DEVICE_FLAGS, "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = open(out).read()
    sizes = re.findall(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", asm)
    names = re.findall(r"\.amdhsa_kernel\s+(\S+)", asm)      # (none in the host-only sources)
    assert len(names) == len(sizes)
    used = [(n, int(s)) for n, s in zip(names, sizes) if int(s) != 0]
    assert not used, f"{src}: kernels using scratch (bytes per lane): {used}"
    spills = re.findall(r"^\s+(scratch_\w+)", asm, re.M)
    assert not spills, f"{src}: scratch accesses: {spills[:5]}"
