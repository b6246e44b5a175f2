"""The rocprofv3 summaries under profiles/ against the code they describe
(CPU only).

* Every command a summary records is one bench.py defines (PROFILE_COMMANDS,
  DETAIL_PROFILE_COMMANDS), so the summary can be regenerated as written.
* Every summary records the hashes of the kernel sources it was taken on, and
  they are the current ones: a kernel change without a new profile fails here
  (bench.py then also reports the dominant kernel's traffic as null).
"""
import glob
import os
import re

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUMMARIES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))


def recorded_commands(text):
    return [ln.strip() for ln in text.splitlines()
            if ln.startswith("    rocprofv3 ") or ln.startswith("    python3 bench.py ")]


def test_there_are_summaries():
    names = [os.path.basename(p) for p in SUMMARIES]
    assert "nt_dense_bf16_256x256__dense_sweep.md" in names
    for fam in bench.DENSE_FAMILIES[1:] + bench.DETAIL_FAMILIES:
        assert fam["file"] in names, fam["file"]


@pytest.mark.parametrize("path", SUMMARIES, ids=os.path.basename)
def test_commands_are_benchs_own(path):
    known = set(bench.PROFILE_COMMANDS) | set(bench.DETAIL_PROFILE_COMMANDS)
    cmds = recorded_commands(open(path).read())
    assert cmds, "no command recorded"
    for c in cmds:
        assert c in known or any(c.startswith(k.split(" profiles/")[0]) for k in known), c


@pytest.mark.parametrize("path", SUMMARIES, ids=os.path.basename)
def test_kernel_sources_unchanged_since_profile(path):
    text = open(path).read()
    line = re.search(r"kernel_source_sha256_16:\s*(.+)", text)
    assert line, "no kernel source hash recorded"
    pairs = re.findall(r"(nt|tn|cast|mqa)\s+([0-9a-f]{16})", line.group(1))
    if not pairs:   # a single-family summary records the bare hash
        fam = os.path.basename(path).split("_")[0]
        pairs = [(fam, line.group(1).strip())]
    for fam, h in pairs:
        assert h == bench.source_hash(fam), f"{fam} kernels changed since this profile"


def test_dominant_kernel_traffic_is_current():
    assert bench.measured_traffic("nt_dense_bf16_256x256") is not None
