"""The direct global->LDS loads (``csrc/lds_pipe.hpp``) set the m0 register in
inline assembly without telling the compiler, which cannot take m0 as a
clobber.  That is safe only while no compiler-generated instruction of those
kernels uses m0.  This test compiles the sources that use the loads to gfx950
assembly and checks that every line naming m0 is one of the loads' own
sequences: m0 set from a scalar register inside an inline-assembly block,
then s_nop 0, then the direct load."""

import os
import re
import shutil
import subprocess

import pytest

from latent_routing_mxfp4_amd import build
from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "latent_routing_mxfp4_amd", "csrc")


def _users():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip") and '"lds_pipe.hpp"' in open(os.path.join(CSRC, f)).read())


@pytest.mark.parametrize("src", _users())
def test_m0_is_written_only_by_the_direct_load_sequences(src, tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    out = tmp_path / (src + ".s")
    cmd = [hipcc, *build.flags(), "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln.strip() for ln in out.read_text().splitlines()]
    seen = 0
    for i, ln in enumerate(lines):
        if not re.search(r"\bm0\b", ln) or ln.startswith(";"):
            continue
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", ln), f"{src}: compiler use of m0: {ln!r}"
        assert lines[i - 1] == ";;#ASMSTART", f"{src}: m0 written outside inline assembly: {ln!r}"
        assert lines[i + 1] == "s_nop 0" and lines[i + 2].startswith("global_load_lds_"), (src, lines[i:i + 3])
        seen += 1
    assert seen > 0
