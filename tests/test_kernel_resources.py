"""Register use of the decode path's kernels (CPU: compiles the device code
only).  Under its launch bounds no route, gate/up, down+blend or pre-norm
instantiation spills vector registers, and those the bf16-activation
workloads run use no scratch at all (a few f32-activation instantiations
spill scalar registers to scratch).  The grouped path's kernels are left
out: one of them trades a small spill for a second workgroup per CU."""
import glob
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from mixture_experts_decode_amd import build as hip_build

CSRC = hip_build.CSRC


def _remarks(src):
    cmd = [hip_build.HIPCC, *hip_build.CFLAGS, "--cuda-device-only", "-c", src, "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out[name] = {}
        for key in ("ScratchSize \\[bytes/lane\\]", "VGPRs Spill", "SGPRs Spill"):
            m = re.search(key + r": (\d+)", line)
            if m and name:
                out[name][key.split()[0]] = int(m.group(1))
    return os.path.basename(src), out


@pytest.fixture(scope="module")
def usage():
    srcs = sorted(glob.glob(os.path.join(CSRC, "inst_*.hip"))) + [os.path.join(CSRC, "route.hip")]
    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        return dict(ex.map(_remarks, srcs))


def test_decode_path_kernels_do_not_spill(usage):
    checked = 0
    for unit, kernels in usage.items():
        for name, res in kernels.items():
            if "grouped" in name or not re.search(r"(route|gate_up|down_blend|pre_norm)_kernel", name):
                continue
            checked += 1
            assert res.get("VGPRs", 0) == 0, f"{unit}: {name} spills vector registers"
            if unit.startswith("inst_bf16_") or unit == "route.hip":
                assert res.get("ScratchSize", 0) == 0, f"{unit}: {name} uses {res['ScratchSize']} B of scratch"
    assert checked >= 60
