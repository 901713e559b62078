"""Every HIP kernel of the library compiles for gfx950 without register spills
or scratch memory.

A spill reload is a vector-memory load.  The gfx9 vector-memory counter
completes in issue order, so waiting for a reload also waits for every load
issued before it: a spill inside a streaming loop turns its prefetch into a
full wait.  (The 320-row direct-to-LDS tile once spilled three registers and
its slice loop waited for all DMA at every reload.)  The build flags are the
library's own device flags.
"""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from speculative_decoding_verification_02_amd import build

SOURCES = sorted(f for f in os.listdir(build.CSRC) if f.endswith(".hip"))


def _resource_usage(src):
    cmd = [build.hipcc(), f"--offload-arch={build.ARCH}", "-O3", "-std=c++17", "-fPIC", "-c", "--cuda-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Rpass-analysis=kernel-resource-usage",
           os.path.join(build.CSRC, src), "-o", os.devnull]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    kernels, name = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs Spill|SGPRs Spill|ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and name:
            kernels[name][m.group(1)] = int(m.group(2))
    return kernels


@pytest.fixture(scope="module")
def usage():
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        return dict(zip(SOURCES, ex.map(_resource_usage, SOURCES)))


def test_every_source_reports_its_kernels(usage):
    total = sum(len(k) for k in usage.values())
    assert total >= 30, usage   # the LM-head, statistics, accept, residual and drafter kernels
    for src, kernels in usage.items():
        for name, u in kernels.items():
            assert set(u) == {"VGPRs Spill", "SGPRs Spill", "ScratchSize [bytes/lane]"}, (src, name, u)


@pytest.mark.parametrize("src", SOURCES)
def test_no_vector_spills_or_scratch(usage, src):
    bad = {n: u for n, u in usage[src].items() if u["VGPRs Spill"] or u["ScratchSize [bytes/lane]"]}
    assert not bad, "kernels with vector spills or scratch in %s: %s" % (src, bad)
