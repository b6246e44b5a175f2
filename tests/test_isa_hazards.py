"""Static checks of the compiled gfx950 code (CPU only: hipcc -S, no GPU).

The stage copies are inline asm (global_load_lds_*) that read an SGPR address
base and M0.  The compiler's hazard recognizer does not look inside inline
asm, so the asm must itself provide the wait states the gfx9 family needs
after a VALU write of an SGPR it reads (five) -- e.g. an SGPR reloaded from a
spill with v_readlane just before the copy.  A copy issued too early reads a
stale base address.  This test builds the kernels to assembly and checks that
every copy is preceded by an s_nop of at least 4 (5 wait states) with no
instruction in between.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp8_fine_grained_e4m3_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def device_asm(src, tmp_path):
    from fp8_fine_grained_e4m3_amd import build as b
    out = tmp_path / (os.path.basename(src) + ".s")
    flags = [f for f in b.FLAGS if f not in ("-shared", "-fPIC", "-Wall")]
    cmd = [HIPCC] + flags + ["--cuda-device-only", "-S", src, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text().split("\n")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["nt_kernel.hip", "tn_kernel.hip"])
def test_every_lds_dma_is_padded(src, tmp_path):
    lines = device_asm(os.path.join(CSRC, src), tmp_path)
    n = 0
    for k, line in enumerate(lines):
        if "global_load_lds" not in line:
            continue
        n += 1
        j = k - 1
        while lines[j].strip().startswith(";") or not lines[j].strip():
            j -= 1
        m = re.match(r"\s*s_nop\s+(\d+)", lines[j])
        assert m and int(m.group(1)) >= 4, f"unpadded LDS DMA at asm line {k}: {line.strip()}"
    assert n > 0
