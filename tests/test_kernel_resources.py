"""Every gfx950 kernel of the library keeps its working set in registers.

The compiler reports each kernel's resource use (-Rpass-analysis=
kernel-resource-usage).  A kernel with a private segment ("ScratchSize") has
spilled registers or put a local array in per-lane memory - a wavefront then
waits on memory round trips inside its inner loop; both have happened when a
kernel's launch bounds or captures changed.  Compiled here (no GPU needed).
"""
import os
import re
import shutil
import subprocess

import pytest

from token_decode_llama_amd import build as b

pytestmark = pytest.mark.skipif(shutil.which(b.hipcc()) is None and not os.path.exists(b.hipcc()),
                                reason="hipcc not available")


def _resource_remarks(tmp_path):
    flags = [f for f in b.HIPCC_FLAGS if f != "-shared"]
    cmd = [b.hipcc(), *flags, "--cuda-device-only", "-c", "-o", str(tmp_path / "k.o"),
           os.path.join(b.CSRC, "lm_kernels.hip"), "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels = {}
    name = None
    for line in res.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+(ScratchSize \[bytes/lane\]|VGPRs Spill|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and name:
            kernels[name][m.group(1).split(" ")[0]] = int(m.group(2))
    return kernels


def test_no_kernel_uses_scratch(tmp_path):
    kernels = _resource_remarks(tmp_path)
    assert len(kernels) > 50          # every template instance of the GEMV, attention, ... kernels
    assert all("ScratchSize" in v and "Occupancy" in v for v in kernels.values())   # (remarks parsed)
    bad = {k: v for k, v in kernels.items() if v.get("ScratchSize", 0) or v.get("VGPRs", 0)}
    assert not bad, f"kernels with a private segment or spills: {sorted(bad.items())[:8]}"
    assert all(v.get("Occupancy", 0) >= 1 for v in kernels.values())
