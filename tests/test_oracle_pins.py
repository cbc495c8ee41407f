"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compares the oracle with a copy of itself: each checks a value
printed or implied by the pages (golden files), a closed form, an exact special
case, a brute-force search, a textbook/library routine, or an invariant that
a dropped term, a wrong sign, a wrong axis or a transposed operand breaks.
CPU only.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden

U = 2.0 ** -24  # unit roundoff of binary32


def f32(x):
    return np.float32(x)


# ---------------------------------------------------------------- rounding (pin 1)

def test_rounding_table_golden():
    """Ties to even and saturation, from the golden table (quantizer at S = 1)."""
    for r, qmax, want in read_golden("rounding_table.txt"):
        got = oracle.quant_row(np.array([float(r)], dtype=np.float32), 1.0, int(qmax))[0]
        assert got == int(want), (r, qmax, got, want)


def test_rounding_power_of_two_scale():
    """S a power of two makes R*(1/S) exact, so the code is the library rint of R/S."""
    rng = np.random.default_rng(1)
    for S in (0.5, 0.125, 2.0 ** -12, 4.0):
        r = (rng.standard_normal(20000) * 60 * S).astype(np.float32)
        ties = (np.arange(-130, 130) + 0.5).astype(np.float32) * np.float32(S)
        r = np.concatenate([r, ties])
        want = np.clip(np.rint(r.astype(np.float64) / S), -127, 127).astype(np.int8)
        np.testing.assert_array_equal(oracle.quant_row(r, S, 127), want)


def _boundary_values(rng, S, reach=4):
    """fp32 values within `reach` ulps of every half-integer multiple (k + 1/2) S, k = -128..127 -- where a
    quotient rounded in another order (for instance through the fp32 reciprocal) lands on the other code --
    plus normal values."""
    mids = ((np.arange(-128, 128) + 0.5) * np.float64(S)).astype(np.float32)
    out, up, down = [mids], mids, mids
    for _ in range(reach):
        up = np.nextafter(up, np.float32(np.inf)).astype(np.float32)
        down = np.nextafter(down, np.float32(-np.inf)).astype(np.float32)
        out += [up, down]
    return np.concatenate(out + [(rng.standard_normal(4000) * 50 * S).astype(np.float32)])


def test_rounding_is_rint_of_fp32_quotient():
    """General S: the code is numpy's rint (ties to even) of numpy's IEEE float32 quotient R / S, clipped
    ([INT8] 2.1 Q = round(R/S)).  The values sit next to every rounding boundary, where the product with the
    rounded reciprocal fl32(R fl32(1/S)) gives another code: the test asserts that such values are present."""
    rng = np.random.default_rng(2)
    differs = 0
    for _ in range(200):
        S = np.float32(rng.uniform(1e-4, 1.0))
        r = _boundary_values(rng, S)
        want = np.clip(np.rint(r / S), -127, 127).astype(np.int8)
        np.testing.assert_array_equal(oracle.quant_row(r, S, 127), want)
        via_recip = np.clip(np.rint(r * (np.float32(1.0) / S)), -127, 127).astype(np.int8)
        differs += int(np.count_nonzero(via_recip != want))
    assert differs > 0, "no value separates the quotient from the reciprocal product"


def test_fold_act_is_fp32_quotient():
    """x_hat = fl32(X / s_j) ([SQ] X diag(s)^-1): numpy's float32 division, column by column, on values that
    include cases where the product with fl32(1/s_j) differs."""
    rng = np.random.default_rng(3)
    T, K = 64, 512
    x = (rng.standard_normal((T, K)) * 3).astype(np.float32)
    s = np.exp(rng.uniform(-4, 4, K)).astype(np.float32)
    want = x / s[None, :]
    got = oracle.fold_act(x, s)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    assert np.count_nonzero(x * (np.float32(1.0) / s)[None, :] != want) > 0


# ---------------------------------------------------------------- smoothing (pins 2, 4)

def test_smoothing_invariance_fp32_bound():
    """(X diag(s)^-1)(diag(s) W^T) = X W^T; on the fp32-folded operands each product carries
    at most three roundings, so |x_hat w_hat - x w| <= 3.01 u |x w| term by term."""
    rng = np.random.default_rng(3)
    T, K, N = 12, 48, 10
    x = rng.standard_normal((T, K)).astype(np.float32)
    x[:, 5] *= 80
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    s = np.exp(rng.uniform(-4, 4, K)).astype(np.float32)
    xh = oracle.fold_act(x, s).astype(np.float64)
    wh = oracle.fold_weight(w, s).astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    got = xh @ wh.T
    bound = 3.01 * U * (np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T)
    assert np.all(np.abs(got - ref) <= bound)
    # dividing both operands by s (a dropped inverse) breaks the identity by far
    bad = (x.astype(np.float64) / s) @ (w.astype(np.float64) / s).T
    assert np.max(np.abs(bad - ref)) > 1e3 * np.max(bound)


def test_fold_none_is_identity():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 32)).astype(np.float32)
    np.testing.assert_array_equal(oracle.fold_act(x, None), x)
    np.testing.assert_array_equal(oracle.fold_weight(x, None), x)


def test_smoothing_closed_forms():
    """alpha = 0 -> s = 1/a_w; alpha = 1 -> s = a_x; alpha = 1/2 -> s = sqrt(a_x/a_w)."""
    rng = np.random.default_rng(5)
    K = 257
    ax = np.exp(rng.uniform(-3, 5, K)).astype(np.float32)
    aw = np.exp(rng.uniform(-7, 0, K)).astype(np.float32)
    s0 = oracle.smooth_factors(ax, aw, 0.0)
    np.testing.assert_array_equal(s0, (1.0 / aw.astype(np.float64)).astype(np.float32))
    s1 = oracle.smooth_factors(ax, aw, 1.0)
    np.testing.assert_array_equal(s1, ax)
    sh = oracle.smooth_factors(ax, aw, 0.5).astype(np.float64)
    ref = np.sqrt(ax.astype(np.float64) / aw.astype(np.float64))
    assert np.max(np.abs(sh - ref) / ref) <= 1.01 * U


@pytest.mark.parametrize("alpha", [0.0, 0.25, 0.5, 0.8, 1.0])
def test_smoothing_migrates_range(alpha):
    """After folding, max|x_hat_j| = (a_x a_w)^(1-alpha) and max|w_hat_j| = (a_x a_w)^alpha."""
    c = synth.cases("tiny")[0]
    x = synth.widen(c.x_batch(0))
    w = synth.widen(c.w())
    ax = oracle.absmax_cols(x)
    aw = oracle.absmax_cols(w)
    s = oracle.smooth_factors(ax, aw, alpha)
    mx = oracle.absmax_cols(oracle.fold_act(x, s)).astype(np.float64)
    mw = oracle.absmax_cols(oracle.fold_weight(w, s)).astype(np.float64)
    p = ax.astype(np.float64) * aw.astype(np.float64)
    assert np.max(np.abs(mx / p ** (1 - alpha) - 1)) < 4 * U
    assert np.max(np.abs(mw / p ** alpha - 1)) < 4 * U


def test_smoothing_zero_channel_gets_one():
    ax = np.array([0.0, 2.0, 3.0], dtype=np.float32)
    aw = np.array([1.0, 0.0, 0.5], dtype=np.float32)
    s = oracle.smooth_factors(ax, aw, 0.5)
    assert s[0] == 1.0 and s[1] == 1.0 and s[2] == np.float32(math.sqrt(6.0))


def test_absmax_running_over_batches():
    """Calibration over batches is the column max of their concatenation; axis is the column."""
    rng = np.random.default_rng(6)
    bs = [rng.standard_normal((7, 33)).astype(np.float32) for _ in range(4)]
    bs[2][3, 9] = -55.0
    a = None
    for b in bs:
        a = oracle.absmax_cols(b, a)
    np.testing.assert_array_equal(a, np.max(np.abs(np.concatenate(bs)), axis=0))
    assert a[9] == 55.0


# ---------------------------------------------------------------- granularity (pin 3)

def test_per_channel_not_worse_than_per_tensor_two_channel_example():
    """The tutorial's example: channels spanning [-1,1] and [-0.1,0.1]."""
    rows = read_golden("two_channel_example.txt")
    K = 64
    rng = np.random.default_rng(7)
    w = []
    for _, lo, hi in rows:
        lo, hi = float(lo), float(hi)
        v = rng.uniform(lo, hi, K)
        v[0], v[1] = lo, hi  # both ends present
        w.append(v)
    w = np.array(w, dtype=np.float32)
    pc = oracle.ssz(w, None, 8, max_iter=0)  # per-channel MinMax
    St, qt = oracle.minmax_per_tensor(w, 8)
    mse_t = [oracle.mse_row(w[i], qt[i], St) for i in range(2)]
    mse_c = pc["mse"]
    assert St == np.float32(np.float32(1.0) / np.float32(127.0))
    assert pc["S"][0] == St  # the wide channel sets the per-tensor scale
    assert mse_c[0] == pytest.approx(mse_t[0], rel=0, abs=0)
    assert mse_c[1] <= mse_t[1]
    # step 10x smaller -> error power ~100x smaller on the narrow channel
    assert 30 < mse_t[1] / mse_c[1] < 300


# ---------------------------------------------------------------- SSZ (pins 5, 6, 7)

def _ssz_rows(seed, N=64, K=256, heavy=True):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K)) * 0.02 * np.exp(rng.uniform(np.log(0.05), 0, (N, 1)))
    if heavy:
        m = rng.random((N, K)) < 0.004
        w[m] *= 20
    return w.astype(np.float32)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("smooth", [False, True])
def test_ssz_monotone_and_not_worse_than_minmax(bits, smooth):
    w = _ssz_rows(10 + bits)
    s = np.exp(np.random.default_rng(9).uniform(-1, 1, w.shape[1])).astype(np.float32) if smooth else None
    r = oracle.ssz(w, s, bits, hist=True)
    mm = oracle.ssz(w, s, bits, max_iter=0)
    h = r["hist"]
    for n in range(w.shape[0]):
        it = r["iters"][n]
        seq = h[n, : it + 1]
        assert np.all(np.diff(seq) <= 0), seq
        assert r["mse"][n] == seq[-1]
        assert r["mse"][n] <= mm["mse"][n]
        assert h[n, 0] == mm["mse"][n]
    # the reported error is the error of the reported scale and codes
    wh = oracle.fold_weight(w, s)
    for n in range(0, w.shape[0], 7):
        assert oracle.mse_row(wh[n], r["q"][n], r["S"][n]) == r["mse"][n]
        np.testing.assert_array_equal(oracle.quant_row(wh[n], r["S"][n], 127 if bits == 8 else 7), r["q"][n])


def test_ssz_improves_somewhere_int4():
    """SSZ exists to beat MinMax; on heavy-tailed int4 rows it must do so on many rows."""
    w = _ssz_rows(21, N=128)
    r = oracle.ssz(w, None, 4)
    mm = oracle.ssz(w, None, 4, max_iter=0)
    assert np.mean(r["mse"] < mm["mse"]) > 0.5
    assert np.all(r["iters"] >= 1)


def test_lsq_step_brute_force():
    """For fixed codes, sum(w - S q)^2 is minimised at S = sum(w q) / sum(q^2): grid search."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        K = int(rng.integers(1, 9))
        w = rng.standard_normal(K).astype(np.float32)
        q = rng.integers(-127, 128, K).astype(np.int8)
        if not np.any(q):
            q[0] = 1
        S_ls = oracle.lsq_scale(w, q)
        grid = np.linspace(S_ls - 0.05, S_ls + 0.05, 20001)
        err = ((w.astype(np.float64)[None, :] - grid[:, None] * q.astype(np.float64)[None, :]) ** 2).sum(1)
        assert abs(grid[np.argmin(err)] - S_ls) <= 1.01 * (grid[1] - grid[0])
    assert oracle.lsq_scale(np.ones(4, np.float32), np.zeros(4, np.int8)) == 0.0


def test_mse_closed_form():
    """w_hat = S q exactly -> 0; one element off by e -> e^2 / K."""
    q = np.array([3, -7, 0, 127, -127, 1, 2, 5], dtype=np.int8)
    S = 2.0 ** -9
    w = (q.astype(np.float64) * S).astype(np.float32)
    assert oracle.mse_row(w, q, S) == 0.0
    w2 = w.copy()
    w2[3] += np.float32(2.0 ** -12)
    assert oracle.mse_row(w2, q, S) == (2.0 ** -12) ** 2 / 8


def _exact_sum(terms):
    """The exact real sum of float terms (each a Fraction-exact product), rounded once to fp64."""
    from fractions import Fraction
    return float(sum((Fraction(t) for t in terms), Fraction(0)))


def test_mse_is_the_exact_sum_rounded_once():
    """mse = fl64(exact sum of (w - S q)^2) / K: python's exact rationals on rows whose terms span many binary
    orders, and a row where the fp64 running sum in index order gives another double (1 + 3 * 2^-54 -> the
    exact sum rounds up; the running sum never moves off 1)."""
    from fractions import Fraction
    w = np.array([1.0, 2.0 ** -27, 2.0 ** -27, 2.0 ** -27], dtype=np.float32)
    q = np.zeros(4, dtype=np.int8)
    want = float(1 + 3 * Fraction(2) ** -54) / 4
    assert want == (1 + 2.0 ** -52) / 4
    assert oracle.mse_row(w, q, 1.0) == want
    run = 0.0
    for v in w.astype(np.float64):
        run += v * v
    assert run / 4 != want
    rng = np.random.default_rng(12)
    for _ in range(300):
        K = int(rng.integers(1, 48))
        S = np.float32(np.exp(rng.uniform(-12, 0)))
        w = (rng.standard_normal(K) * np.exp(rng.uniform(-20, 3, K)) * S * 40).astype(np.float32)
        q = oracle.quant_row(w, S, 127)
        terms = [(Fraction(float(a)) - Fraction(float(S)) * int(b)) ** 2 for a, b in zip(w, q)]
        assert oracle.mse_row(w, q, S) == float(sum(terms, Fraction(0))) / K


def test_lsq_numerator_is_the_exact_sum_rounded_once():
    """S' = fl64(exact sum w q) / sum q^2: exact rationals, and a row where the running fp64 sum cancels to 0."""
    from fractions import Fraction
    w = np.array([1.0, 2.0 ** -60, -1.0], dtype=np.float32)
    q = np.array([1, 1, 1], dtype=np.int8)
    assert oracle.lsq_scale(w, q) == 2.0 ** -60 / 3
    rng = np.random.default_rng(13)
    for _ in range(300):
        K = int(rng.integers(1, 48))
        w = (rng.standard_normal(K) * np.exp(rng.uniform(-30, 3, K))).astype(np.float32)
        q = rng.integers(-127, 128, K).astype(np.int8)
        B = int(np.sum(q.astype(np.int64) ** 2))
        if B == 0:
            continue
        A = float(sum((Fraction(float(a)) * int(b) for a, b in zip(w, q)), Fraction(0)))
        assert oracle.lsq_scale(w, q) == A / B


@pytest.mark.parametrize("bits,qmax", [(8, 127), (4, 7)])
def test_ssz_exact_grid_row(bits, qmax):
    """Row = c * integers with max |k| = qmax, c = 2^-k: lossless, S = c, one step, error 0."""
    rng = np.random.default_rng(12)
    for e in (6, 10, 13):
        c = 2.0 ** -e
        k = rng.integers(-qmax, qmax + 1, (3, 96))
        k[:, 17] = qmax
        k[1, 40] = -qmax
        w = (k * c).astype(np.float32)
        r = oracle.ssz(w, None, bits)
        assert np.all(r["S"] == np.float32(c))
        np.testing.assert_array_equal(r["q"], k.astype(np.int8))
        assert np.all(r["mse"] == 0.0)
        assert np.all(r["iters"] == 1)


def test_ssz_single_nonzero_element():
    K = 64
    for val in (0.37, -1.9, 3e-3):
        w = np.zeros((1, K), dtype=np.float32)
        w[0, 11] = val
        r = oracle.ssz(w, None, 8)
        S = np.float32(abs(np.float32(val))) / np.float32(127)
        assert r["S"][0] == S
        assert r["q"][0, 11] == (127 if val > 0 else -127)
        assert np.count_nonzero(r["q"]) == 1
        assert r["iters"][0] == 1
        assert r["mse"][0] <= (abs(val) * 2 * U) ** 2 / K


def test_ssz_zero_row_and_floor():
    K = 32
    fmin = np.float32(1e-5)
    w = np.zeros((3, K), dtype=np.float32)
    w[1] = np.linspace(-5e-4, 9e-4, K, dtype=np.float32)  # absmax/127 < 1e-5: floor binds the init
    w[2] = 6e-6  # codes round 0.6 up to 1; the refit 6e-6 < 1e-5 must be floored back to 1e-5
    r = oracle.ssz(w, None, 8)
    assert r["S"][0] == fmin and not np.any(r["q"][0]) and r["iters"][0] == 1 and r["mse"][0] == 0.0
    assert r["S"][1] >= fmin
    assert r["S"][2] == fmin and np.all(r["q"][2] == 1) and r["iters"][2] == 1
    mm = oracle.ssz(w, None, 8, max_iter=0)
    assert np.all(mm["iters"] == 0) and mm["S"][1] == fmin and mm["S"][2] == fmin
    assert np.max(np.abs(mm["q"][1])) == 90  # 9e-4 / 1e-5


def test_ssz_converged_is_a_fixed_point():
    """At exit (iters < 20) the next least-squares candidate improves by less than the thresholds."""
    w = _ssz_rows(13, N=48)
    thr = 1e-10
    r = oracle.ssz(w, None, 8)
    fmin = np.float32(1e-5)
    for n in range(w.shape[0]):
        if r["iters"][n] >= 20:
            continue
        S = r["S"][n]
        q = r["q"][n]
        Sn = max(np.float32(oracle.lsq_scale(w[n], q)), fmin)
        cur = oracle.mse_row(w[n], oracle.quant_row(w[n], Sn, 127), Sn)
        best = r["mse"][n]
        d = best - cur
        assert best == 0 or d / best < thr or abs(d) < thr


# ------------------------------------------------------- asymmetric int8 SSZ (NEXT-1)

def test_asym_code_table():
    """Q = clamp(rne(R/S) + Z, -128, 127) at S = 1: ties to even, then the offset, then saturation."""
    cases = [(0.5, 0, 0), (1.5, 0, 2), (2.5, 3, 5), (-2.5, 3, 1), (126.5, 0, 126), (127.5, 0, 127),
             (-128.5, 0, -128), (-127.5, 0, -128), (100.0, 40, 127), (-100.0, -40, -128), (-3.0, -128, -128),
             (0.0, -128, -128), (255.0, -128, 127), (254.5, -128, 126)]
    for r, z, want in cases:
        got = oracle.quant_row_asym(np.array([r], dtype=np.float32), 1.0, z)[0]
        assert got == want, (r, z, got, want)
    # quotients far beyond the int range saturate at their own end
    for r, z, want in ((3e9, 0, 127), (-3e9, 0, -128), (1e36, -128, 127), (-1e36, 127, -128)):
        got = oracle.quant_row_asym(np.array([r], dtype=np.float32), 1.0, z)[0]
        assert got == want, (r, z, got, want)


def test_asym_init_of_a_constant_row_under_a_tiny_floor():
    """A constant positive row: range 0, so S is the floor; with the floor 1e-38 the offset
    -128 - rne(w / S) saturates at -128 and every code at 127 (the value sits far above the grid)."""
    w = np.full((1, 64), 0.01, dtype=np.float32)
    r = oracle.ssz_asym(w, None, min_scale=1e-38)
    assert r["S"][0] == np.float32(1e-38) and r["Z"][0] == -128 and np.all(r["q"][0] == 127)


def test_asym_lsq_brute_force():
    """For fixed codes and offset Z, sum(w - a (q - Z) - b)^2 is minimised at the normal-equation solution:
    grid search."""
    rng = np.random.default_rng(31)
    for _ in range(60):
        K = int(rng.integers(2, 9))
        w = rng.standard_normal(K).astype(np.float32)
        q = rng.integers(-128, 128, K).astype(np.int8)
        Z = int(rng.integers(-128, 128))
        if np.all(q == q[0]):
            q[0] = q[0] ^ 1
        a, b = oracle.lsq_affine(w, q, Z)
        wd, qd = w.astype(np.float64), q.astype(np.float64) - Z
        ga = np.linspace(a - 2e-3, a + 2e-3, 401)
        gb = np.linspace(b - 0.05, b + 0.05, 401)
        err = ((wd[None, None, :] - ga[:, None, None] * qd[None, None, :] - gb[None, :, None]) ** 2).sum(-1)
        i, j = np.unravel_index(np.argmin(err), err.shape)
        assert abs(ga[i] - a) <= 1.01 * (ga[1] - ga[0]) and abs(gb[j] - b) <= 1.01 * (gb[1] - gb[0])
    assert oracle.lsq_affine(np.ones(5, np.float32), np.full(5, 7, np.int8)) is None


def test_asym_lsq_sums_are_exact():
    """The fit's sums (sum w r, sum w) are the exact sums rounded once, then the normal equations in fp64 in
    the written order: python's exact rationals and IEEE doubles reproduce (a, b) bit for bit."""
    from fractions import Fraction
    rng = np.random.default_rng(35)
    for _ in range(200):
        K = int(rng.integers(2, 40))
        w = (rng.standard_normal(K) * np.exp(rng.uniform(-25, 2, K))).astype(np.float32)
        q = rng.integers(-128, 128, K).astype(np.int8)
        Z = int(rng.integers(-128, 128))
        r = [int(v) - Z for v in q]
        sr, srr = sum(r), sum(v * v for v in r)
        det = K * srr - sr * sr
        if det <= 0:
            continue
        swr = float(sum((Fraction(float(a)) * b for a, b in zip(w, r)), Fraction(0)))
        sw = float(sum((Fraction(float(a)) for a in w), Fraction(0)))
        a = (float(K) * swr - sw * float(sr)) / float(det)
        b = (sw - a * float(sr)) / float(K)
        assert oracle.lsq_affine(w, q, Z) == (a, b)


def test_asym_exact_grid_row():
    """w = c (k - z) with k spanning [-128, 127], c = 2^-e: MinMax recovers S = c and Z = z exactly,
    the codes are k, the error is 0 and the first step converges."""
    rng = np.random.default_rng(32)
    for e, z in ((6, 37), (11, -90), (9, 0), (13, 127)):
        c = 2.0 ** -e
        k = rng.integers(-128, 128, (3, 80))
        k[:, 5] = -128
        k[:, 60] = 127
        w = ((k - z) * c).astype(np.float32)
        r = oracle.ssz_asym(w)
        assert np.all(r["S"] == np.float32(c)) and np.all(r["Z"] == z), (r["S"], r["Z"])
        np.testing.assert_array_equal(r["q"], k.astype(np.int8))
        assert np.all(r["mse"] == 0.0) and np.all(r["iters"] == 1)


def test_asym_degenerate_rows():
    """All-zero row: floor scale, Z = -128, codes -128 (dequantized 0), error 0, one step.
    Constant non-zero row: floor scale, Z saturates, all codes equal, nothing to fit (one step)."""
    K = 24
    w = np.zeros((2, K), dtype=np.float32)
    w[1] = 0.5
    r = oracle.ssz_asym(w)
    fmin = np.float32(1e-5)
    assert r["S"][0] == fmin and r["Z"][0] == -128 and np.all(r["q"][0] == -128) and r["mse"][0] == 0.0
    assert r["S"][1] == fmin and r["Z"][1] == -128 and np.all(r["q"][1] == 127)
    assert r["mse"][1] == pytest.approx((0.5 - float(fmin) * 255) ** 2, rel=1e-14)
    assert np.all(r["iters"] == 1)


def test_asym_offset_halves_the_step_on_one_sided_rows():
    """Rows uniform on [0, 1]: the symmetric grid wastes its negative half, so its MinMax step is about
    twice the asymmetric one and its error about four times larger.  A lost or mis-signed offset fails."""
    rng = np.random.default_rng(33)
    w = rng.uniform(0.0, 1.0, (16, 2048)).astype(np.float32)
    w[:, 0], w[:, 1] = 0.0, 1.0
    sym = oracle.ssz(w, None, 8, max_iter=0)
    asym = oracle.ssz_asym(w, max_iter=0)
    assert np.all(asym["Z"] == -128)
    np.testing.assert_allclose(sym["S"] / asym["S"], 255 / 127, rtol=1e-6)
    ratio = sym["mse"] / asym["mse"]
    assert np.all((ratio > 3.3) & (ratio < 4.8)), ratio
    # and shifted to [-1, 0] the offset flips to the top of the range
    asym_n = oracle.ssz_asym(-w, max_iter=0)
    assert np.all(asym_n["Z"] == 127)


def test_asym_monotone_consistent_and_fixed_point():
    w = _ssz_rows(34, N=64)
    w[::3] += np.float32(0.01)  # some rows off-centre
    r = oracle.ssz_asym(w, hist=True)
    mm = oracle.ssz_asym(w, max_iter=0)
    thr = 1e-10
    fmin = np.float32(1e-5)
    for n in range(w.shape[0]):
        it = r["iters"][n]
        seq = r["hist"][n, : it + 1]
        assert np.all(np.diff(seq) <= 0) and r["mse"][n] == seq[-1] and r["mse"][n] <= mm["mse"][n]
        assert -128 <= r["Z"][n] <= 127
        np.testing.assert_array_equal(oracle.quant_row_asym(w[n], r["S"][n], r["Z"][n]), r["q"][n])
        assert oracle.mse_row_asym(w[n], r["q"][n], r["S"][n], r["Z"][n]) == r["mse"][n]
        if 1 <= it < 20 and r["mse"][n] > 0:
            if seq[-1] == seq[-2]:
                # the last candidate was rejected: it is rebuilt from the kept codes and is again no better
                a, b = oracle.lsq_affine(w[n], r["q"][n], int(r["Z"][n]))
                Sn = max(np.float32(a), fmin)
                Zn = int(min(127, max(-128, int(r["Z"][n]) - np.rint(b / a))))
                cur = oracle.mse_row_asym(w[n], oracle.quant_row_asym(w[n], Sn, Zn), Sn, Zn)
                assert cur >= r["mse"][n]
            else:
                # the last candidate was kept with a change under the relative or absolute threshold
                d = seq[-2] - seq[-1]
                assert d / seq[-2] < thr or abs(d) < thr
    assert np.mean(r["mse"] < mm["mse"]) > 0.3


def test_ssz_constants_golden():
    rows = {k: float(v) for k, v in read_golden("ssz_constants.txt")}
    import inspect
    sig = inspect.signature(oracle.ssz).parameters
    assert sig["max_iter"].default == rows["SCALE_SEARCH_ITER_NUM"]
    assert sig["thr"].default == rows["SCALE_SEARCH_CONVERGE_THRESHOLD"]
    assert sig["min_scale"].default == rows["SCALE_SEARCH_MIN_SCALE"]


def test_pack_int4_layout():
    q = np.array([[1, -1, 7, -7, 0, -8 + 1, 3, 4]], dtype=np.int8)
    p = oracle.pack_int4(q)
    assert p.tolist() == [[0xF1, 0x97, 0x90, 0x43]]  # -7 -> 0x9, 1 -> 0x1, -1 -> 0xF


# ---------------------------------------------------------------- per token (pin 8)

def test_per_token_invariants():
    c = synth.cases("tiny")[0]
    x = synth.widen(c.x_batch(0)).copy()
    x[5] = 0.0
    xq, d = oracle.quant_per_token(x, None)
    assert np.all(np.abs(xq.astype(int)) <= 127)
    for t in range(x.shape[0]):
        if t == 5:
            assert d[t] == 1.0 and not np.any(xq[t])
            continue
        a = np.max(np.abs(x[t]))
        assert np.max(np.abs(xq[t].astype(int))) == 127
        assert d[t] == np.float32(a) / np.float32(127)
        # round to nearest: reconstruction error at most half a step (plus fp32 slack)
        err = np.abs(x[t].astype(np.float64) - d[t] * xq[t].astype(np.float64))
        assert np.all(err <= 0.5 * d[t] * (1 + 4e-6) + 4 * U * np.abs(x[t]))


def test_per_token_scale_is_per_row():
    """Scaling one token row leaves every other row's codes and scales untouched."""
    rng = np.random.default_rng(14)
    x = rng.standard_normal((6, 64)).astype(np.float32)
    xq, d = oracle.quant_per_token(x, None)
    x2 = x.copy()
    x2[2] *= 1000
    xq2, d2 = oracle.quant_per_token(x2, None)
    keep = [0, 1, 3, 4, 5]
    np.testing.assert_array_equal(xq[keep], xq2[keep])
    np.testing.assert_array_equal(d[keep], d2[keep])
    np.testing.assert_array_equal(xq[2], xq2[2])  # power-of-ten scaling leaves codes (nearly) alone
    assert d2[2] > 900 * d[2]


# ---------------------------------------------------------------- GEMM (pin 9)

def test_gemm_brute_force():
    rng = np.random.default_rng(15)
    for M, N, K in ((1, 1, 1), (3, 5, 7), (4, 9, 33), (2, 3, 64)):
        a = rng.integers(-127, 128, (M, K)).astype(np.int8)
        b = rng.integers(-127, 128, (N, K)).astype(np.int8)
        got = oracle.gemm_i8(a, b)
        for t in range(M):
            for n in range(N):
                assert got[t, n] == sum(int(a[t, k]) * int(b[n, k]) for k in range(K))
        np.testing.assert_array_equal(got, a.astype(np.int64) @ b.astype(np.int64).T)


def test_gemm_int32_bound():
    """K = 131056, the largest multiple of 16 with 128^2 K <= 2^31 - 1, is the largest K for which no int8 codes
    (-128 included) can overflow int32: the oracle's int64 sums stay in range there and leave it 16 columns on."""
    K = ((2 ** 31 - 1) // (128 * 128)) // 16 * 16
    assert K == 131056
    a = np.full((1, K), -128, dtype=np.int8)
    assert oracle.gemm_i8(a, a)[0, 0] == 128 * 128 * K
    a2 = np.full((1, K + 16), -128, dtype=np.int8)
    with pytest.raises(oracle.OracleError):
        oracle.gemm_i8(a2, a2)


# ---------------------------------------------------------------- whole path

def test_lossless_path_reproduces_exact_product():
    """X rows = d_t * integers and W rows = c_n * integers, both with max |k| = 127 and
    power-of-two steps: quantization is lossless, so the dequantized output equals X W^T exactly.
    A wrong scale axis, a transposed operand or a dropped scale breaks equality."""
    rng = np.random.default_rng(16)
    T, K, N = 9, 64, 13
    kx = rng.integers(-127, 128, (T, K))
    kx[:, 3] = 127
    kw = rng.integers(-127, 128, (N, K))
    kw[:, 10] = -127
    dt = 2.0 ** rng.integers(-8, 3, T)
    cn = 2.0 ** rng.integers(-14, -4, N)
    x = (kx * dt[:, None]).astype(np.float32)
    w = (kw * cn[:, None]).astype(np.float32)
    out = oracle.run_linear([x], w, x, smooth=False)
    np.testing.assert_array_equal(out["S"], cn.astype(np.float32))
    np.testing.assert_array_equal(out["delta"], dt.astype(np.float32))
    np.testing.assert_array_equal(out["y"], x.astype(np.float64) @ w.astype(np.float64).T)


def test_smoothing_helps_on_outlier_activations():
    """The SmoothQuant article's claim on the tiny outlier workload: smoothing lowers the W8A8 error."""
    c = synth.cases("tiny")[0]
    x = synth.widen(c.x_batch(0))
    w = synth.widen(c.w())
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    e = {}
    for sm in (False, True):
        y = oracle.run_linear([x], w, x, alpha=0.5, smooth=sm)["y"]
        e[sm] = np.max(np.abs(y - ref)) / np.max(np.abs(ref))
    assert e[True] < e[False]
    assert e[True] < 2e-2


# ------------------------------------------------- epilogue fusion, static scales (NEXT-2..4)

def test_bf16_rounding_table_and_library():
    """Round to nearest even at the bf16 grid: hand-checked values, and torch's own fp32 -> bf16 conversion."""
    table = [(1.0, 0x3F80), (1.00390625, 0x3F80), (1.01171875, 0x3F82), (1.0078125, 0x3F81), (-2.5, 0xC020),
             (0.0, 0x0000), (-0.0, 0x8000), (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81), (65504.0, 0x4780)]
    for f, want in table:
        assert oracle.bf16_rne(f) == want, (f, hex(oracle.bf16_rne(f)), hex(want))
    import torch
    x = (np.random.default_rng(40).standard_normal(5000) * np.exp(np.random.default_rng(41).uniform(-20, 20, 5000)))
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_rne(v) for v in x], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_epilogue_dequant_matches_fp64_within_two_roundings():
    rng = np.random.default_rng(42)
    acc = rng.integers(-2 ** 30, 2 ** 30, (7, 9))
    ts = rng.uniform(1e-3, 1, 7).astype(np.float32)
    cs = rng.uniform(1e-4, 1e-2, 9).astype(np.float32)
    y = oracle.epilogue(acc, ts, cs).astype(np.float64)
    y64 = acc * ts.astype(np.float64)[:, None] * cs.astype(np.float64)[None, :]
    assert np.all(np.abs(y - y64) <= 3 * U * np.abs(y64))


def test_epilogue_bias_then_activation():
    acc = np.array([[-4, 4, 0, 10]])
    ts, cs = np.array([0.25], np.float32), np.ones(4, np.float32)
    b = np.array([2.0, -3.0, 0.0, -2.5], np.float32)
    np.testing.assert_array_equal(oracle.epilogue(acc, ts, cs, b), [[1.0, -2.0, 0.0, 0.0]])
    relu = oracle.epilogue(acc, ts, cs, b, act=oracle.ACT_RELU)
    np.testing.assert_array_equal(relu, [[1.0, 0.0, 0.0, 0.0]])  # relu(v + b), not relu(v) + b
    assert not np.signbit(relu).any()  # relu returns +0


def test_epilogue_gelu_closed_form():
    """GELU(v) = v * Phi(v): Phi(1) = 0.841344746..., Phi(-1) = 0.158655253..., and scipy's erf elsewhere."""
    from scipy.special import erf
    acc = np.array([[0, 1, -1, 10, -10]])
    g = oracle.epilogue(acc, np.ones(1, np.float32), np.ones(5, np.float32), act=oracle.ACT_GELU)[0]
    np.testing.assert_allclose(g, [0.0, 0.8413447460685429, -0.15865525393145707, 10.0, 0.0], atol=2e-7)
    rng = np.random.default_rng(43)
    acc = rng.integers(-6000, 6000, (1, 4000))
    v = acc[0] * np.float32(1e-3)
    g = oracle.epilogue(acc, np.array([1e-3], np.float32), np.ones(4000, np.float32), act=oracle.ACT_GELU)[0]
    ref = v.astype(np.float64) * 0.5 * (1.0 + erf(v.astype(np.float64) / np.sqrt(2.0)))
    assert np.max(np.abs(g - ref)) <= 4e-7 * max(1.0, np.max(np.abs(ref)))


def test_epilogue_bf16_and_int8_outputs():
    acc = np.array([[5, -5, 7, 600, -600, 3]])
    ts = np.array([0.5], np.float32)
    cs = np.ones(6, np.float32)
    bf = oracle.epilogue(acc, ts, cs, out=oracle.OUT_BF16)
    assert bf.dtype == np.uint16 and bf[0, 0] == 0x4020 and bf[0, 1] == 0xC020  # +-2.5
    # int8 with out_scale 1: v = 2.5 -> 2 (ties to even), -2.5 -> -2, 3.5 -> 4, saturation at +-127
    q = oracle.epilogue(acc, ts, cs, out=oracle.OUT_I8, out_scale=1.0)
    np.testing.assert_array_equal(q, [[2, -2, 4, 127, -127, 2]])
    # with the next layer's fold: x_hat = v / s_next, s_next = 0.5 doubles the codes before rounding
    ns = np.full(6, 0.5, np.float32)
    q2 = oracle.epilogue(acc, ts, cs, out=oracle.OUT_I8, next_s=ns, out_scale=2.0)
    np.testing.assert_array_equal(q2, [[2, -2, 4, 127, -127, 2]])
    # relu before requantisation
    q3 = oracle.epilogue(acc, ts, cs, act=oracle.ACT_RELU, out=oracle.OUT_I8, out_scale=1.0)
    np.testing.assert_array_equal(q3, [[2, 0, 4, 127, 0, 2]])


@pytest.mark.parametrize("fold", [0, 1, 2])
def test_absmax_tensor_and_column_identity(fold):
    """Tensor absmax of the folded tensor (numpy fp32 arithmetic as the independent reference), and the
    identity the GPU path relies on: max_t |fl32(x_tj * r)| = fl32(max_t |x_tj| * r) for r > 0."""
    rng = np.random.default_rng(44 + fold)
    x = (rng.standard_normal((300, 96)) * np.exp(rng.uniform(-3, 3, 96))).astype(np.float32)
    s = np.exp(rng.uniform(-2, 2, 96)).astype(np.float32)
    if fold == 1:
        xf = x * (np.float32(1) / s)
    elif fold == 2:
        xf = x * s
    else:
        xf = x
    assert oracle.absmax_tensor(x, s if fold else None, fold) == np.max(np.abs(xf))
    colmax = np.max(np.abs(x), axis=0)
    r = (np.float32(1) / s) if fold == 1 else (s if fold == 2 else np.ones(96, np.float32))
    np.testing.assert_array_equal(np.max(np.abs(xf), axis=0), (colmax * r).astype(np.float32))


def test_moving_average_closed_forms():
    assert oracle.ema_update(None, 4.0, 0.9, True) == 4.0  # the first batch sets the state
    assert oracle.ema_update(4.0, 8.0, 0.5, False) == 6.0
    assert oracle.ema_update(4.0, 8.0, 0.0, False) == 8.0  # momentum 0: the last batch
    st = np.float32(3.0)
    for _ in range(50):
        st = oracle.ema_update(st, 3.0, 0.9, False)
    assert abs(st - 3.0) <= 8 * U * 3.0  # a constant range stays put (up to fp32 rounding)
    st = np.float32(0.0)
    for b in range(200):
        st = oracle.ema_update(st, 5.0, 0.9, b == 0)
    assert abs(st - 5.0) < 1e-5
    with pytest.raises(oracle.OracleError):
        oracle.ema_update(1.0, 2.0, 1.0, False)  # momentum must lie in [0, 1)
    assert oracle.act_static_scale(127.0) == 1.0 and oracle.act_static_scale(0.0) == 1.0
    assert oracle.act_static_scale(63.5) == np.float32(0.5)
    assert oracle.weight_scale_per_tensor(1.27) == np.float32(np.float32(1.27) / np.float32(127))
    assert oracle.weight_scale_per_tensor(1e-4) == np.float32(1e-5)


def test_quant_static_half_step_and_saturation():
    rng = np.random.default_rng(45)
    x = (rng.standard_normal((64, 128)) * 3).astype(np.float32)
    S = np.float32(0.05)
    q = oracle.quant_static(x, S)
    inside = np.abs(x) < 127 * S
    assert np.all(np.abs(x[inside] - S * q[inside].astype(np.float64)) <= S * (0.5 + 1e-6))
    assert np.all(q[x >= 127.5 * S] == 127) and np.all(q[x <= -127.5 * S] == -127)
    assert np.all(np.abs(q) <= 127)
    # S a power of two: the code is numpy's rint of x / S, clipped
    q2 = oracle.quant_static(x, np.float32(0.0625))
    np.testing.assert_array_equal(q2, np.clip(np.rint(x / np.float32(0.0625)), -127, 127).astype(np.int8))


def test_granularity_error_ordering_on_outlier_layer():
    """The pages' per-layer vs per-channel comparison, on a synthetic layer with outlier input channels and
    rows of different ranges: the W8A8 output error of (a) per-tensor weight + static per-tensor
    activation exceeds (b) per-channel weight + per-token activation; SSZ (c) is not worse than MinMax (b)
    per channel; smoothing (d) helps on outlier activations.  Reported numbers, not a pin of the pages'
    percentages (those are model accuracies)."""
    rng = np.random.default_rng(46)
    T, K, N = 64, 256, 96
    x = rng.standard_normal((T, K)).astype(np.float32)
    x[:, [3, 77, 200]] *= 40
    w = (rng.standard_normal((N, K)) * 0.02 * np.exp(rng.uniform(np.log(0.05), 0, N))[:, None]).astype(np.float32)
    ref = x.astype(np.float64) @ w.astype(np.float64).T

    def err(y):
        return np.max(np.abs(y - ref)) / np.max(np.abs(ref))

    # (a) per-tensor weight, per-tensor activation (the batch's own range as the static scale)
    Sw = oracle.weight_scale_per_tensor(oracle.absmax_tensor(w))
    wq = oracle.quant_static(w, Sw)
    Sx = oracle.act_static_scale(oracle.ema_update(None, oracle.absmax_tensor(x), 0.9, True))
    xq = oracle.quant_static(x, Sx)
    ya = oracle.dequant(oracle.gemm_i8(xq, wq), np.full(T, Sx, np.float32), np.full(N, Sw, np.float32))
    # (b) per-channel MinMax + per-token; (c) per-channel SSZ + per-token; (d) SSZ + smoothing
    xq_t, d = oracle.quant_per_token(x)
    mm = oracle.ssz(w, None, 8, max_iter=0)
    yb = oracle.dequant(oracle.gemm_i8(xq_t, mm["q"]), d, mm["S"])
    sz = oracle.ssz(w, None, 8)
    yc = oracle.dequant(oracle.gemm_i8(xq_t, sz["q"]), d, sz["S"])
    s = oracle.smooth_factors(oracle.absmax_cols(x), oracle.absmax_cols(w), 0.5)
    xq_s, d_s = oracle.quant_per_token(x, s)
    sz_s = oracle.ssz(w, s, 8)
    yd = oracle.dequant(oracle.gemm_i8(xq_s, sz_s["q"]), d_s, sz_s["S"])
    ea, eb, ec, ed = err(ya), err(yb), err(yc), err(yd)
    print(f"\nW8A8 output error: per-tensor {ea:.3e}, per-channel MinMax {eb:.3e}, per-channel SSZ {ec:.3e}, "
          f"+ smoothing {ed:.3e}")
    assert ea > eb and ec <= eb * 1.05 and ed < ec


def _reading_rows(seed, N=96, K=256):
    """Rows of mixed size with a few heavy entries, plus the special rows: all-zero, exact grid, one element."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K)) * 0.02 * np.exp(rng.uniform(np.log(0.02), 0, N))[:, None]
    w[rng.random((N, K)) < 0.004] *= 20
    w[0] = 0.0
    w[1] = 2.0 ** -9 * rng.integers(-127, 128, K)
    w[2] = 0.0
    w[2, 5] = 0.3
    return w.astype(np.float32)


def test_ssz_reading_variants_default_is_the_oracle():
    """The diagnostic search with the used readings (OR, mean, per row) reproduces o_ssz exactly, int8 and int4."""
    w = _reading_rows(71)
    s = np.exp(np.random.default_rng(72).uniform(-0.5, 0.5, w.shape[1])).astype(np.float32)
    for bits in (8, 4):
        for ss in (None, s):
            ref = oracle.ssz(w, ss, bits)
            v = oracle.ssz_variant(w, ss, bits)
            np.testing.assert_array_equal(v["S"], ref["S"])
            np.testing.assert_array_equal(v["iters"], ref["iters"])
            np.testing.assert_array_equal(v["mse"], ref["mse"])


def test_ssz_reading_variants_properties():
    """AND stops no earlier than OR and follows the same steps until OR stops; rows iterating until all
    have converged all take the same number of steps, and a row whose own search ended on a rejected
    candidate (a fixed point) keeps its scale; the summed error only weakens the absolute test."""
    w = _reading_rows(73)
    ref = oracle.ssz(w, None, 8, hist=True)
    a = oracle.ssz_variant(w, None, 8, conv_and=True)
    assert np.all(a["iters"] >= ref["iters"])
    same = a["iters"] == ref["iters"]
    np.testing.assert_array_equal(a["S"][same], ref["S"][same])
    assert np.all(a["mse"] <= ref["mse"])  # it only ever keeps improvements

    g = oracle.ssz_variant(w, None, 8, global_loop=True)
    assert g["iters"][0] == 1  # the all-zero row has nothing to fit
    assert np.all(g["iters"][1:] == g["iters"].max())
    h = ref["hist"]
    it = ref["iters"]
    rejected_last = np.array([it[n] > 0 and h[n, it[n]] == h[n, it[n] - 1] for n in range(w.shape[0])])
    assert rejected_last.sum() >= 3
    np.testing.assert_array_equal(g["S"][rejected_last], ref["S"][rejected_last])

    m = oracle.ssz_variant(w, None, 8, err_sum=True)
    assert np.mean(m["iters"] >= ref["iters"]) >= 0.99
    assert m["iters"].mean() > ref["iters"].mean()


def test_folded_overflow_is_refused():
    """A folded value that overflows fp32 (x / s_j or w * s_j beyond the largest float) has no code: the path
    requires finite folded values, and the oracle refuses such input instead of converting a NaN quotient."""
    x = np.ones((2, 16), np.float32)
    x[1, 3] = np.float32(3e38)
    s = np.ones(16, np.float32)
    s[3] = np.float32(0.5)
    with pytest.raises(oracle.OracleError):
        oracle.quant_per_token(x, s)
    with pytest.raises(oracle.OracleError):
        oracle.ssz(x, 1.0 / s)
    with pytest.raises(oracle.OracleError):
        oracle.ssz_asym(x, 1.0 / s)
    # the same rows without the overflowing factor are accepted
    s[3] = np.float32(1.0)
    oracle.quant_per_token(x, s)
    oracle.ssz(x, s)
