"""The kernels' reciprocal rcp_rn (one Newton-Raphson step from the hardware approximation) is the IEEE
reciprocal fl32(1/s) for every fp32 s in [2^-100, 2^101), the range in which the quantizers use it: an
exhaustive check on the GPU (tests/division/rcp_check.hip, built by __graft_entry__.build()).  Everything the
quantizers compute from it is then the same as with the IEEE division."""
import os
import re
import subprocess

import pytest

from conftest import ROOT

pytestmark = pytest.mark.gpu

BIN = os.path.join(ROOT, "tests", "division", "rcp_check")


def test_rcp_rn_is_the_ieee_reciprocal_on_its_whole_domain():
    if not os.path.exists(BIN):
        pytest.fail("tests/division/rcp_check is not built (run __graft_entry__.build())")
    print("rcp_check: every fp32 in [2^-100, 2^101)", flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    m = re.search(r"checked (\d+) mismatches (\d+) approximation_mismatches (\d+)", r.stdout)
    assert m, r.stdout
    checked, bad, raw = (int(v) for v in m.groups())
    assert checked == 201 * 2 ** 23
    assert bad == 0, r.stdout
    assert raw > 0  # the approximation alone is not the IEEE reciprocal: the correction step is needed
