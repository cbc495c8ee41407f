"""The kernels' reciprocal rcp_rn (one Newton-Raphson step from the hardware approximation) is the IEEE
reciprocal fl32(1/s) for every fp32 s in [2^-100, 2^101), the range in which the quantizers use it: an
exhaustive check on the GPU (tests/division/rcp_check.hip, built by __graft_entry__.build()).  Everything the
quantizers compute from it is then the same as with the IEEE division.  The same program checks the SSZ search's
fp64 reciprocal rcp64 (within 2^-51 relative of 1/s on every one of those divisors) and its quotient quot64 (the
fp64 product with rcp64(s), rounded to fp32) against the IEEE quotient on the GPU's own conversion: every mantissa
of twelve numerator binades around each of 4096 divisors, and every finite numerator for 8 special divisors."""
import os
import re
import subprocess

import pytest

from conftest import ROOT

pytestmark = pytest.mark.gpu

BIN = os.path.join(ROOT, "tests", "division", "rcp_check")


def test_reciprocals_and_fp64_quotient_on_their_domains():
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
    m = re.search(r"rcp64 checked (\d+) over_bound (\d+) max_residual (\S+)", r.stdout)
    assert m, r.stdout
    assert int(m.group(1)) == 201 * 2 ** 23 and int(m.group(2)) == 0, r.stdout
    assert 0.0 < float(m.group(3)) <= 2.0 ** -51, r.stdout
    print(f"rcp64: largest relative error {float(m.group(3)):.3e}", flush=True)
    m = re.search(r"quot64 checked (\d+) mismatches (\d+) subnormal_within_one_step (\d+) "
                  r"f32_product_mismatches (\d+)", r.stdout)
    assert m, r.stdout
    checked, bad, sub, f32_bad = (int(v) for v in m.groups())
    assert checked == (4096 * 12 + 8 * 255) * 2 ** 23
    assert bad == 0, r.stdout
    print(f"quot64: {checked} quotients, subnormal results one step off: {sub}", flush=True)
    assert f32_bad > checked // 100  # the plain fp32 product is not the quotient: the fp64 product is needed
