"""Host check: the committed rocprofv3 summaries were taken from the kernel sources as they stand.

bench.py reports a launch's profiled HBM traffic only while the summary's recorded source hash
matches the decode kernel's sources; this test fails when a kernel or graph-builder change leaves
the summaries stale, and checks the recorded figures against the summary's own table."""
import os
import re

import pytest

from persistent_megakernel_03_amd import roofline as rf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUMMARIES = ["mk_megakernel_llama8b_b1_decode.md", "mk_megakernel_llama8b_b1_fp8_decode.md",
             "mk_megakernel_llama8b_b16_decode.md"]


@pytest.mark.parametrize("name", SUMMARIES)
def test_summary_matches_the_kernel_sources(name):
    path = os.path.join(ROOT, "profiles", name)
    traffic = rf.profiled_traffic(path)
    assert traffic is not None, "%s was taken from other kernel sources than these" % name
    txt = open(path).read()
    steps = int(re.search(r"steps_per_launch = (\d+)", txt).group(1))
    # the recorded bytes per step are the FETCH and WRITE rows' raw KiB x scale / steps
    total = 0.0
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        m = re.search(r"\| %s \| ([\d.]+) \| x([\d.]+) \|" % counter, txt)
        total += float(m.group(1)) * 1024 * float(m.group(2)) / steps
    assert abs(total - traffic) <= 1e-6 * traffic + 2
    alg = int(re.search(r"per step[^:]*:\n(\d+)\.", txt).group(1))
    assert 1.0 <= traffic / alg < 1.2  # no fewer bytes than the algorithm needs, and little waste
