"""Resource use of every kernel of the library, from the compiler's own
report (device-only compile of kda_kernels.hip for gfx950, CPU only).

No kernel may use scratch memory: a register spill, or a private array the
compiler could not keep in registers (an indexed pick over a per-lane array
once put one in the verify kernel), moves per-lane data through memory on
every access, which the kernels' bounds (HBM for the state, the issue rate
for the verify kernel's arithmetic) leave no room for.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from gated_delta_rule_decode_amd import build as kbuild

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def _report(tmp_path):
    out = tmp_path / "k.o"
    cmd = [kbuild.hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-c", "--cuda-device-only",
           *kbuild.DEVICE_FLAGS, "-I", os.path.join(kbuild.ROOT, "include"), kbuild.SOURCES[0],
           "-o", str(out), "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels = {}
    name = None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[bytes/lane\])?: (\d+)", line)
        if m and name:
            kernels[name][m.group(1).strip()] = int(m.group(2))
    return kernels


def test_no_kernel_uses_scratch(tmp_path):
    kernels = _report(tmp_path)
    assert len(kernels) >= 30, sorted(kernels)  # every family and instantiation was reported
    families = {"kda_recurrent_kernel", "kda_fused_kernel", "kda_packed_fused_kernel", "kda_verify_wy_kernel"}
    assert all(any(f in k for k in kernels) for f in families)
    bad = {k: v for k, v in kernels.items()
           if v.get("ScratchSize", 0) or v.get("VGPRs Spill", 0) or v.get("SGPRs Spill", 0)}
    assert not bad, bad
