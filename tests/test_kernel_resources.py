"""Every kernel compiles for gfx950 without scratch memory (no register spills to
memory), checked on the host: hipcc's kernel-resource-usage remarks for each
kernel source, compiled for the device only with the library's own flags."""

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from exact_tiled_attention_34_amd import build as B

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")

KERNEL_SOURCES = [s for s in B.SOURCES if s != "fa2_api.hip"]


def resource_report(src):
    cmd = [HIPCC, *B.COMMON_FLAGS, *B.SOURCE_FLAGS.get(src, []), "--cuda-device-only", "-c", os.path.join(B.CSRC, src),
           "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark: ([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and cur is not None:
            kernels[cur][m.group(1).strip()] = int(m.group(2))
    return kernels


@pytest.fixture(scope="module")
def reports():
    with ThreadPoolExecutor(max_workers=len(KERNEL_SOURCES)) as ex:
        return dict(zip(KERNEL_SOURCES, ex.map(resource_report, KERNEL_SOURCES)))


def test_every_kernel_reported(reports):
    names = [k for rep in reports.values() for k in rep]
    for kind in ("fwd_kernel", "bwd_preprocess_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"):
        assert any(kind in n for n in names), kind


def test_head_dim_256_dq_in_its_own_unit(reports):
    # the dQ kernel at head dim 256 is built only by its own unit (other flags)
    assert any("bwd_dq_kernelILi256" in k for k in reports["fa2_bwd_dq256.hip"])
    assert not any("bwd_dq_kernelILi256" in k for k in reports["fa2_bwd.hip"])
    assert not any("dkdv" in k or "fwd_kernel" in k for k in reports["fa2_bwd_dq256.hip"])


def test_no_scratch(reports):
    spilled = {k: v.get("ScratchSize") for rep in reports.values() for k, v in rep.items()
               if v.get("ScratchSize", 0) != 0 or v.get("VGPRs Spill", 0) != 0}
    assert not spilled, f"kernels using scratch memory: {spilled}"
