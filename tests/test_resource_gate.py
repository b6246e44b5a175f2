"""Register gate on the compiled gfx950 kernels (CPU only: hipcc, no GPU).

Every kernel instance of every HIP source must compile with no VGPR spill,
no scratch (per-lane private memory) and no dynamic stack.  A spill turns a
register access in the main loop into a scratch round trip through the
vector memory pipe the tile copies also use; it has cost the dense kernel
several per cent before, so a change that brings one back fails here rather
than in a timing.  SGPR spills are allowed: they go to VGPR lanes
(v_writelane / v_readlane), not to memory.

The report comes from the compiler's kernel-resource-usage remarks, with the
same flags the library is built with.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp8_fine_grained_e4m3_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def kernel_reports(src):
    """{kernel name: {field: value}} from the resource-usage remarks."""
    from fp8_fine_grained_e4m3_amd import build as b
    flags = [f for f in b.FLAGS if f not in ("-shared", "-Wall")] + b.SEPARATE.get(src, [])
    cmd = [HIPCC] + flags + ["--cuda-device-only", "-c", "-Rpass-analysis=kernel-resource-usage",
                             os.path.join(CSRC, src), "-o", os.devnull]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    reports, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = reports.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][^:]*): (\S+) \[-Rpass", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return reports


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["nt_kernel.hip", "tn_kernel.hip", "cast_kernel.hip", "mqa_kernel.hip"])
def test_no_vgpr_spill_no_scratch(src):
    reports = kernel_reports(src)
    assert reports, f"no kernels reported for {src}"
    bad = []
    for name, r in reports.items():
        if (int(r["VGPRs Spill"]) != 0 or int(r["ScratchSize [bytes/lane]"]) != 0
                or r["Dynamic Stack"] != "False"):
            bad.append(f"{name}: VGPR spill {r['VGPRs Spill']}, scratch "
                       f"{r['ScratchSize [bytes/lane]']} B/lane, dynamic stack {r['Dynamic Stack']}")
    assert not bad, "\n".join(bad)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_gate_sees_every_gemm_instance():
    """The gate is only as good as its coverage: the NT source must report
    at least the dense, grouped-contiguous and masked instances of both tile
    families, the TN source its weight-gradient instances."""
    nt = kernel_reports("nt_kernel.hip")
    tn = kernel_reports("tn_kernel.hip")
    assert sum("nt_fp8_kernel" in k for k in nt) >= 12, sorted(nt)
    assert sum("tn_" in k for k in tn) >= 4, sorted(tn)
