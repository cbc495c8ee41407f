"""The corrected quotients of the kernels against IEEE division, on the host.

The quantizers take fl32(x / s) as one residual correction of x * fl32(1/s) (see div_rn in the device helpers:
Markstein's method, Muller et al., Handbook of Floating-Point Arithmetic, division chapter) wherever its result
is the IEEE quotient: for |x| >= 2^-102 and divisors s in [2^-100, 2^100].  This sweep checks that claim bit for
bit in C on this host (IEEE binary32 arithmetic and a correctly rounded fmaf): every fp32 mantissa of x against
hundreds of divisor mantissas, at the exponents the claim spans, and it shows that the bound on x is needed
(the residual underflows below it).  The SSZ search, whose rows sit in registers as fp64, takes the quotient as
the fp64 product with fl64(1/s) rounded once to fp32 (quot64 in the device helpers): the same sweep checks that it
is the IEEE quotient wherever that is a normal number (within one step below), and that the plain fp32 product
with fl32(1/s) is not.  CPU only; compiled with gcc when the test runs.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "division", "sweep.c")


@pytest.fixture(scope="module")
def sweep(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("division") / "sweep")
    subprocess.check_call(["gcc", "-O2", "-march=native", "-fopenmp", "-ffp-contract=off", SRC, "-o", exe, "-lm"])

    def run(n_div, ex, es, method=0):
        out = subprocess.run([exe, str(n_div), str(ex), str(es), str(method)], capture_output=True, text=True,
                             check=True)
        checked, bad = (int(v) for v in out.stdout.split())
        return checked, bad
    return run


def test_one_binade_many_divisors(sweep):
    """Every numerator mantissa against 1024 divisor mantissas (2^33 quotients) in one binade: equal."""
    checked, bad = sweep(1024, 0, 0)
    assert checked == 1024 * 2 ** 23 and bad == 0


@pytest.mark.parametrize("ex,es", [(-102, 0), (-102, -100), (-60, -20), (0, -100), (0, 100), (100, 100),
                                   (127, 0), (127, 100), (-20, 100), (60, -60), (-101, 60)])
def test_exponent_ends(sweep, ex, es):
    """The ends of the proven domain (x down to 2^-102, s from 2^-100 to 2^100, quotients up to overflow)."""
    checked, bad = sweep(64, ex, es)
    assert checked > 0 and bad == 0, (ex, es, bad)


def test_bound_on_x_is_needed(sweep):
    """Below |x| = 2^-102 the residual x - q0 s leaves the normal range and the corrected product can differ
    from the quotient: the kernels keep such x away from any output (or take the IEEE division)."""
    _, bad = sweep(64, -110, 0)
    assert bad > 0


def test_fp64_product_one_binade_many_divisors(sweep):
    """The fp64 product rounded to fp32: every numerator mantissa against 1024 divisor mantissas, equal."""
    checked, bad = sweep(1024, 0, 0, method=1)
    assert checked == 1024 * 2 ** 23 and bad == 0


@pytest.mark.parametrize("ex,es", [(-126, 0), (-126, -100), (-126, 100), (0, -100), (0, 100), (127, 0),
                                   (127, 100), (100, -20), (-60, 66), (7, 0), (-3, -3)])
def test_fp64_product_exponent_ends(sweep, ex, es):
    """Quotients from the subnormal range (within one step there) up to overflow."""
    checked, bad = sweep(64, ex, es, method=1)
    assert checked > 0 and bad == 0, (ex, es, bad)


def test_fp32_product_is_not_the_quotient(sweep):
    """Contrast: the plain product with the fp32 reciprocal misses the IEEE quotient on a large share of values."""
    checked, bad = sweep(16, 0, 0, method=2)
    assert bad > checked // 100
