"""GPU parity on the five workloads, whole path per linear layer:
calibrate over the seeded batches -> smoothing factors -> MinMax + SSZ weight
quantization -> per-token activation quantization -> int8 GEMM + dequant.

Small workloads are compared in full.  At full size the GPU runs every row
(the launch configuration the bench times) and the oracle recomputes sampled
rows from the same seeded inputs: calibration is checked in full (it is
cheap), the weight quantization on sampled output channels, the activation
quantization on sampled tokens, and the GEMM on the sampled tokens x channels.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import (announce, assert_scales, assert_y, compare_ssz, compare_ssz_asym, dev, host, sample_rows,
                         unpack_int4)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_int8_quantization_amd as m
    return m


def run_case(pq, case, alpha, bits=8, w_sample=None, x_sample=None):
    """GPU whole path for one linear case; oracle on (sampled) rows; compare every stage."""
    tag = f"{case.name} alpha={alpha} bits={bits}"
    w_host = case.w()
    w_f = synth.widen(w_host)
    wdev = dev(w_host)

    # calibration: running max over the calibration batches (GPU and oracle both see every batch)
    ax_ref = None
    ax = None
    for b in range(case.calib_batches):
        xb = case.x_batch(b)
        ax_ref = oracle.absmax_cols(synth.widen(xb), ax_ref)
        announce(f"{tag}: sq_absmax_calib batch {b}")
        ax = pq.sq_absmax_calib(dev(xb), ax, accumulate=b > 0)
        del xb
    aw_ref = oracle.absmax_cols(w_f)
    announce(f"{tag}: sq_absmax_calib weight")
    aw = pq.sq_absmax_calib(wdev)
    np.testing.assert_array_equal(host(ax), ax_ref, err_msg=tag + " a_x")
    np.testing.assert_array_equal(host(aw), aw_ref, err_msg=tag + " a_w")

    s_ref = oracle.smooth_factors(ax_ref, aw_ref, alpha)
    announce(f"{tag}: sq_smooth_factors")
    s = pq.sq_smooth_factors(ax, aw, alpha)
    s_h = host(s)
    assert_scales(s_h, s_ref, tag + " s")
    assert np.array_equal(s_h, s_ref), f"{tag}: {np.sum(s_h != s_ref)} smoothing factors differ in the last bit"

    # weight quantization (all rows on the GPU; oracle on the sample)
    rows = np.arange(case.N) if w_sample is None else sample_rows(case.N, w_sample, 11)
    ref_w = oracle.ssz(w_f[rows], s_ref, bits)
    announce(f"{tag}: ssz_weight_qparams N={case.N} K={case.K}")
    S, wq, it, mse = pq.ssz_weight_qparams(wdev, s, bits=bits)
    codes = host(wq) if bits == 8 else unpack_int4(host(wq))
    compare_ssz(host(S)[rows], codes[rows], host(it)[rows], host(mse)[rows], ref_w, tag + " ssz")
    if bits != 8:
        return

    # activation quantization of the forward batch
    x_eval = case.x_batch(case.eval_index())
    toks = np.arange(case.T) if x_sample is None else sample_rows(case.T, x_sample, 13)
    xq_ref, d_ref = oracle.quant_per_token(synth.widen(x_eval)[toks], s_ref)
    announce(f"{tag}: quant_per_token_i8 T={case.T}")
    xq, d = pq.quant_per_token_i8(dev(x_eval), s)
    np.testing.assert_array_equal(host(d)[toks], d_ref, err_msg=tag + " tok_scale")
    np.testing.assert_array_equal(host(xq)[toks], xq_ref, err_msg=tag + " xq")

    # GEMM + dequant: full launch on the GPU, sampled block of outputs on the oracle
    acc_ref = oracle.gemm_i8(xq_ref, ref_w["q"])
    y_ref = oracle.dequant(acc_ref, d_ref, ref_w["S"])
    announce(f"{tag}: w8a8_gemm_dequant M={case.T} N={case.N} K={case.K}")
    y, acc = pq.w8a8_gemm_dequant(xq, wq, d, S, want_acc=True)
    acc_full = host(acc)
    acc_h = acc_full[np.ix_(toks, rows)]
    np.testing.assert_array_equal(acc_h, acc_ref, err_msg=tag + " acc")
    err = assert_y(host(y)[np.ix_(toks, rows)], y_ref, tag + " y")
    # every output, by properties that hold at any size: the int32 sums pass Freivalds' test (C v = A (B^T v)
    # exactly in int64, three random integer vectors; a wrong sum escapes one draw with probability ~1/2001), and
    # y is the epilogue fl32(acc) * fl32(ts * cs) of those sums, element for element
    a64 = acc_full.astype(np.int64)
    xq64 = host(xq).astype(np.int64)
    wq64 = host(wq).astype(np.int64)
    rng = np.random.default_rng(41)
    for _ in range(3):
        v = rng.integers(-1000, 1001, case.N).astype(np.int64)
        assert np.array_equal(a64 @ v, xq64 @ (wq64.T @ v)), tag + ": int32 sums fail Freivalds' test"
    del xq64, wq64
    y_all = acc_full.astype(np.float32) * (host(d)[:, None] * host(S)[None, :])
    np.testing.assert_array_equal(host(y), y_all, err_msg=tag + " y (every element) from acc")
    del a64, y_all
    # accuracy of the whole W8A8 layer against the unquantized product (reported; parity unpinned)
    full = synth.widen(x_eval)[toks].astype(np.float64) @ w_f[rows].astype(np.float64).T
    rel = np.max(np.abs(host(y)[np.ix_(toks, rows)] - full)) / np.max(np.abs(full))
    announce(f"{tag}: y parity {err:.2e}; W8A8 vs fp64 product {rel:.3e}")


def test_tiny(pq):
    for case in synth.cases("tiny"):
        run_case(pq, case, 0.5)


@pytest.mark.parametrize("idx", range(4))
def test_gpt345m(pq, idx):
    run_case(pq, synth.cases("gpt345m")[idx], 0.5, w_sample=None, x_sample=None)


def test_decode(pq):
    run_case(pq, synth.cases("decode")[0], 0.5, w_sample=512)


@pytest.mark.parametrize("alpha", [0.5, 0.8])
@pytest.mark.parametrize("idx", [0, 1])
def test_opt67b(pq, idx, alpha):
    run_case(pq, synth.cases("opt67b")[idx], alpha, w_sample=256, x_sample=64)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("layer", [0, 31])
def test_ssz_scale(pq, layer, bits):
    for case in synth.cases("ssz_scale")[4 * layer: 4 * layer + 4]:
        w_host = case.w()
        rows = sample_rows(case.N, 384, 17 + layer)
        ref = oracle.ssz(synth.widen(w_host)[rows], None, bits)
        announce(f"{case.name}: ssz_weight_qparams int{bits} N={case.N} K={case.K}")
        S, wq, it, mse = pq.ssz_weight_qparams(dev(w_host), None, bits=bits)
        codes = host(wq) if bits == 8 else unpack_int4(host(wq))
        compare_ssz(host(S)[rows], codes[rows], host(it)[rows], host(mse)[rows], ref, case.name)


@pytest.mark.parametrize("bits", [8, 4])
def test_ssz_scale_all_rows_properties(pq, bits):
    """Every row of a model-scale layer (its 4 matrices, 36864 rows) at full size, by properties that hold at any
    size ([SSZ] 算法流程, 收敛判断, 算法参数): scales at or above the 1e-5 floor, 1 to 20 steps, the codes are the
    quantizer's codes for the returned scale, the reported error is those codes' error, and no row ends worse than
    its MinMax start."""
    qmax = 127 if bits == 8 else 7
    floor = np.float32(1e-5)
    for case in synth.cases("ssz_scale")[:4]:
        w_host = case.w()
        announce(f"{case.name}: ssz_weight_qparams int{bits} N={case.N} K={case.K}, every row")
        S, wq, it, mse = pq.ssz_weight_qparams(dev(w_host), None, bits=bits)
        S, it, mse = host(S), host(it), host(mse)
        codes = host(wq) if bits == 8 else unpack_int4(host(wq))
        assert S.min() >= floor and it.min() >= 1 and it.max() <= 20, case.name
        w = synth.widen(w_host)
        for r0 in range(0, case.N, 1024):
            r1 = min(r0 + 1024, case.N)
            wr, Sr, cr = w[r0:r1], S[r0:r1], codes[r0:r1]
            q = np.clip(np.rint(wr / Sr[:, None]), -qmax, qmax)
            np.testing.assert_array_equal(q, cr, err_msg=f"{case.name} rows {r0}..{r1}: codes of the returned scale")
            e = ((wr.astype(np.float64) - Sr.astype(np.float64)[:, None] * cr) ** 2).mean(axis=1)
            rel = np.abs(mse[r0:r1] - e) / np.maximum(e, 1e-300)
            rel[e == 0] = np.abs(mse[r0:r1][e == 0])
            assert rel.max() <= 1e-9, f"{case.name} rows {r0}..{r1}: reported error {rel.max():.2e} off"
            S0 = np.maximum((np.abs(wr).max(axis=1) / np.float32(qmax)).astype(np.float32), floor)
            q0 = np.clip(np.rint(wr / S0[:, None]), -qmax, qmax)
            e0 = ((wr.astype(np.float64) - S0.astype(np.float64)[:, None] * q0) ** 2).mean(axis=1)
            assert np.all(mse[r0:r1] <= e0 * (1 + 1e-9)), f"{case.name} rows {r0}..{r1}: worse than MinMax"


@pytest.mark.parametrize("idx", [0, 1])
def test_opt67b_smoothed_ssz_all_rows_properties(pq, idx):
    """Every row of the smoothed hidden-4096 weight (fc1 [16384,4096] or fc2 [4096,16384], alpha 0.5 -- the rows
    that run the most steps: 5147 of fc1's run all 20) at full size, by the properties of the method: the floor,
    1 to 20 steps, codes equal to the quantizer's codes of the returned scale on the folded weight, the reported
    error equal to those codes' error, and no row worse than its MinMax start.  The smoothing factors are the
    oracle's (the GPU's are bit-identical to them in the other tests)."""
    case = synth.cases("opt67b")[idx]
    w_host = case.w()
    ax = None
    for b in range(case.calib_batches):
        ax = oracle.absmax_cols(synth.widen(case.x_batch(b)), ax)
    w = synth.widen(w_host)
    s = oracle.smooth_factors(ax, oracle.absmax_cols(w), 0.5)
    announce(f"{case.name}: ssz_weight_qparams int8 smoothed N={case.N} K={case.K}, every row")
    S, wq, it, mse = pq.ssz_weight_qparams(dev(w_host), dev(s), bits=8)
    S, it, mse, codes = host(S), host(it), host(mse), host(wq)
    assert S.min() >= np.float32(1e-5) and it.min() >= 1 and it.max() <= 20, case.name
    for r0 in range(0, case.N, 1024):
        r1 = min(r0 + 1024, case.N)
        wr = oracle.fold_weight(w[r0:r1], s)
        Sr, cr = S[r0:r1], codes[r0:r1]
        q = np.clip(np.rint(wr / Sr[:, None]), -127, 127)
        np.testing.assert_array_equal(q, cr, err_msg=f"{case.name} rows {r0}..{r1}: codes of the returned scale")
        e = ((wr.astype(np.float64) - Sr.astype(np.float64)[:, None] * cr) ** 2).mean(axis=1)
        rel = np.abs(mse[r0:r1] - e) / np.maximum(e, 1e-300)
        assert rel.max() <= 1e-9, f"{case.name} rows {r0}..{r1}: reported error {rel.max():.2e} off"
        S0 = np.maximum((np.abs(wr).max(axis=1) / np.float32(127)).astype(np.float32), np.float32(1e-5))
        q0 = np.clip(np.rint(wr / S0[:, None]), -127, 127)
        e0 = ((wr.astype(np.float64) - S0.astype(np.float64)[:, None] * q0) ** 2).mean(axis=1)
        assert np.all(mse[r0:r1] <= e0 * (1 + 1e-9)), f"{case.name} rows {r0}..{r1}: worse than MinMax"


@pytest.mark.parametrize("layer", [0, 31])
def test_ssz_scale_asym(pq, layer):
    """Asymmetric int8 SSZ at full size on the 4 matrices of a layer (sampled rows on the oracle)."""
    for case in synth.cases("ssz_scale")[4 * layer: 4 * layer + 4]:
        w_host = case.w()
        rows = sample_rows(case.N, 256, 19 + layer)
        ref = oracle.ssz_asym(synth.widen(w_host)[rows], None)
        announce(f"{case.name}: ssz_weight_qparams_asym N={case.N} K={case.K}")
        S, Z, wq, it, mse = pq.ssz_weight_qparams_asym(dev(w_host), None)
        compare_ssz_asym(host(S)[rows], host(Z)[rows], host(wq)[rows], host(it)[rows], host(mse)[rows], ref,
                         case.name + " asym")


@pytest.mark.parametrize("idx", [0, 1])
def test_opt67b_asym_weights(pq, idx):
    """Asymmetric int8 SSZ of the smoothed hidden-4096 weights (alpha 0.5), sampled rows on the oracle."""
    case = synth.cases("opt67b")[idx]
    w_host = case.w()
    w_f = synth.widen(w_host)
    ax = None
    for b in range(case.calib_batches):
        ax = oracle.absmax_cols(synth.widen(case.x_batch(b)), ax)
    s_ref = oracle.smooth_factors(ax, oracle.absmax_cols(w_f), 0.5)
    rows = sample_rows(case.N, 256, 23 + idx)
    ref = oracle.ssz_asym(w_f[rows], s_ref)
    announce(f"{case.name}: ssz_weight_qparams_asym N={case.N} K={case.K} smoothed")
    S, Z, wq, it, mse = pq.ssz_weight_qparams_asym(dev(w_host), dev(s_ref))
    compare_ssz_asym(host(S)[rows], host(Z)[rows], host(wq)[rows], host(it)[rows], host(mse)[rows], ref,
                     case.name + " asym")


def test_mlp_block_static_chain(pq):
    """The hidden-4096 MLP block with static activation scales and the fused epilogue, end to end.
    fc1: smoothing and a moving-average static activation scale from its 8 calibration batches.  fc2:
    smoothing and static scale from fc1's own W8A8 ReLU outputs on 64 tokens of each calibration batch
    (so the int8 intermediate is calibrated on what it will carry).  Forward: static fc1 input codes,
    fc1 GEMM + ReLU writing fc2's int8 input (fc2's fold and static scale in the epilogue), fc2 GEMM.
    GPU at full size; the oracle quantizes all of fc1's weight (fc2 reads every fc1 channel) and checks
    sampled tokens and fc2 channels, every stage bit for bit."""
    c1, c2 = synth.cases("opt67b")
    T = c1.T
    toks = sample_rows(T, 32, 29)
    rows2 = sample_rows(c2.N, 128, 37)
    momentum = 0.9
    ct = 64  # calibration tokens per batch for fc2
    w1, w2 = c1.w(), c2.w()
    w1f, w2f = synth.widen(w1), synth.widen(w2)
    xs = [c1.x_batch(b) for b in range(c1.calib_batches)]

    # fc1 calibration
    ax1 = None
    for xb in xs:
        ax1 = oracle.absmax_cols(synth.widen(xb), ax1)
    s1 = oracle.smooth_factors(ax1, oracle.absmax_cols(w1f), 0.5)
    st1_ref = None
    st1 = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    d1 = None
    for b, xb in enumerate(xs):
        st1_ref = oracle.ema_update(st1_ref, oracle.absmax_tensor(synth.widen(xb), s1, oracle.FOLD_DIV), momentum,
                                    b == 0)
        announce(f"mlp chain: fc1 activation scale, batch {b}")
        _, d1, _ = pq.sq_act_scale_ema(pq.sq_absmax_calib(dev(xb)), dev(s1), momentum, first=b == 0, state=st1)
    d1_ref = oracle.act_static_scale(st1_ref)
    assert host(d1)[0] == d1_ref
    announce("mlp chain: ssz fc1")
    S1, wq1, _, _ = pq.ssz_weight_qparams(dev(w1), dev(s1), bits=8)
    r1 = oracle.ssz(w1f, s1, 8)
    np.testing.assert_array_equal(host(S1), r1["S"])

    # fc2 calibration on fc1's W8A8 ReLU outputs
    hs_ref, hs = [], []
    for b, xb in enumerate(xs):
        xc = xb[:ct]
        q_ref = oracle.quant_static(synth.widen(xb[:ct]), d1_ref, s1, oracle.FOLD_DIV)
        hs_ref.append(oracle.epilogue(oracle.gemm_i8(q_ref, r1["q"]), np.full(ct, d1_ref, np.float32), r1["S"],
                                      act=oracle.ACT_RELU))
        announce(f"mlp chain: fc1 on fc2 calibration tokens, batch {b}")
        q, rsc = pq.quant_static_i8(dev(np.ascontiguousarray(xc)), d1, dev(s1), "div")
        hs.append(pq.w8a8_gemm_fused(q, wq1, rsc, S1, act="relu", out="f32"))
        np.testing.assert_array_equal(host(hs[-1]), hs_ref[-1])
    ax2 = None
    for h in hs_ref:
        ax2 = oracle.absmax_cols(h, ax2)
    s2 = oracle.smooth_factors(ax2, oracle.absmax_cols(w2f), 0.5)
    st2_ref = None
    st2 = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    d2 = None
    for b, (h_ref, h) in enumerate(zip(hs_ref, hs)):
        st2_ref = oracle.ema_update(st2_ref, oracle.absmax_tensor(h_ref, s2, oracle.FOLD_DIV), momentum, b == 0)
        _, d2, _ = pq.sq_act_scale_ema(pq.sq_absmax_calib(h), dev(s2), momentum, first=b == 0, state=st2)
    d2_ref = oracle.act_static_scale(st2_ref)
    assert host(d2)[0] == d2_ref
    announce("mlp chain: ssz fc2")
    S2, wq2, _, _ = pq.ssz_weight_qparams(dev(w2), dev(s2), bits=8)
    r2 = oracle.ssz(w2f[rows2], s2, 8)
    np.testing.assert_array_equal(host(S2)[rows2], r2["S"])
    del xs, hs

    # forward
    x = c1.x_batch(c1.eval_index())
    announce("mlp chain: quant_static_i8 fc1 input")
    xq1, rs1 = pq.quant_static_i8(dev(x), d1, dev(s1), "div")
    xq1_ref = oracle.quant_static(synth.widen(x)[toks], d1_ref, s1, oracle.FOLD_DIV)
    np.testing.assert_array_equal(host(xq1)[toks], xq1_ref)
    announce("mlp chain: fc1 GEMM + ReLU -> int8 (fc2 fold, static scale)")
    h = pq.w8a8_gemm_fused(xq1, wq1, rs1, S1, act="relu", out="i8", next_s=dev(s2), out_scale=d2)
    h_ref = oracle.epilogue(oracle.gemm_i8(xq1_ref, r1["q"]), np.full(len(toks), d1_ref, np.float32), r1["S"],
                            act=oracle.ACT_RELU, out=oracle.OUT_I8, next_s=s2, out_scale=d2_ref)
    np.testing.assert_array_equal(host(h)[toks], h_ref)
    announce("mlp chain: fc2 GEMM")
    rs2 = torch.full((T,), float(d2_ref), dtype=torch.float32, device="cuda:0")
    y = pq.w8a8_gemm_dequant(h, wq2, rs2, S2)
    y_ref = oracle.epilogue(oracle.gemm_i8(h_ref, r2["q"]), np.full(len(toks), d2_ref, np.float32), r2["S"])
    np.testing.assert_array_equal(host(y)[np.ix_(toks, rows2)], y_ref)
    # accuracy of the chained static int8 block against the fp64 block on the same tokens (reported, unpinned)
    h64 = np.maximum(synth.widen(x)[toks].astype(np.float64) @ w1f.astype(np.float64).T, 0.0)
    y64 = h64 @ w2f[rows2].astype(np.float64).T
    rel = np.max(np.abs(y_ref - y64)) / np.max(np.abs(y64))
    announce(f"mlp chain: static W8A8 block vs fp64 block {rel:.3e}")


def _rel_errors(y, full):
    d = host(y).astype(np.float64) - full
    return float(np.max(np.abs(d)) / np.max(np.abs(full))), float(np.linalg.norm(d) / np.linalg.norm(full))


@pytest.mark.parametrize("config,alpha", [("gpt345m", 0.5), ("opt67b", 0.5), ("opt67b", 0.8)])
def test_accuracy_report(pq, config, alpha):
    """End-to-end error of the W8A8 layer through the GPU path against the fp64 product of the unquantized
    bf16 inputs, on 256 tokens of the forward batch and every output channel -- for the path and for the
    alternatives the pages discuss: no smoothing ([SQ]), MinMax without the least-squares refits ([SSZ]),
    one weight scale per tensor ([PTQ] per-layer vs per-channel), and one static activation scale from the
    calibration batches' moving-average maximum ([INT8] 2.1).  The pages print no values for these
    workloads, so the numbers are reported, not pinned; two claims are checked in kind: smoothing lowers the
    error on these outlier-channel activations, and per-channel weight scales do no worse than one per tensor."""
    n_tok = 256
    rows = []
    for case in synth.cases(config):
        tag = f"{case.name} alpha={alpha}"
        w_host = case.w()
        wd = dev(w_host)
        ax = None
        state = torch.zeros(1, dtype=torch.float32, device="cuda:0")
        col = []
        for b in range(case.calib_batches):
            xb = dev(case.x_batch(b))
            announce(f"accuracy {tag}: calibration batch {b}")
            ax = pq.sq_absmax_calib(xb, ax, accumulate=b > 0)
            col.append(pq.sq_absmax_calib(xb))
            del xb
        aw = pq.sq_absmax_calib(wd)
        s = pq.sq_smooth_factors(ax, aw, alpha)
        x_eval = np.ascontiguousarray(case.x_batch(case.eval_index())[:n_tok])
        xd = dev(x_eval)
        full = synth.widen(x_eval).astype(np.float64) @ synth.widen(w_host).astype(np.float64).T
        err = {}

        announce(f"accuracy {tag}: per-channel SSZ weights, per-token activations, smoothed")
        S, wq, _, _ = pq.ssz_weight_qparams(wd, s, bits=8, want_stats=False)
        xq, d = pq.quant_per_token_i8(xd, s)
        err["path"] = _rel_errors(pq.w8a8_gemm_dequant(xq, wq, d, S), full)

        announce(f"accuracy {tag}: no smoothing")
        S0, wq0, _, _ = pq.ssz_weight_qparams(wd, None, bits=8, want_stats=False)
        xq0, d0 = pq.quant_per_token_i8(xd, None)
        err["no smoothing"] = _rel_errors(pq.w8a8_gemm_dequant(xq0, wq0, d0, S0), full)

        announce(f"accuracy {tag}: MinMax weight scales")
        Sm, wqm, _, _ = pq.ssz_weight_qparams(wd, s, bits=8, max_iter=0, want_stats=False)
        err["MinMax weights"] = _rel_errors(pq.w8a8_gemm_dequant(xq, wqm, d, Sm), full)

        announce(f"accuracy {tag}: one weight scale per tensor")
        st, ch = pq.weight_scale_per_tensor(aw, s, n=case.N)
        wqt, _ = pq.quant_static_i8(wd, st, s, "mul", want_row_scale=False)
        err["per-tensor weights"] = _rel_errors(pq.w8a8_gemm_dequant(xq, wqt, d, ch), full)

        announce(f"accuracy {tag}: one static activation scale")
        for b, c in enumerate(col):
            _, da, _ = pq.sq_act_scale_ema(c, s, 0.9, first=b == 0, state=state)
        xqs, rs = pq.quant_static_i8(xd, da, s, "div")
        err["static activations"] = _rel_errors(pq.w8a8_gemm_dequant(xqs, wq, rs, S), full)

        rows.append((case.name, err))
        assert err["path"][1] < err["no smoothing"][1], f"{tag}: smoothing did not lower the error: {err}"
        assert err["path"][1] <= err["per-tensor weights"][1], f"{tag}: per-channel worse than per-tensor: {err}"
        del col

    names = list(rows[0][1])
    announce(f"accuracy report, {config} alpha {alpha}: relative error vs fp64 (max-normalised / Frobenius)")
    for layer, err in rows:
        announce(f"  {layer:16s} " + "  ".join(f"{n}: {err[n][0]:.2e} / {err[n][1]:.2e}" for n in names))


# case count and seed of the random-shape sweep; larger sweeps: PTQ_RANDOM_CASES=5000 PTQ_RANDOM_SEED=11
_RANDOM_CASES = int(os.environ.get("PTQ_RANDOM_CASES", "64"))
_RANDOM_SEED = int(os.environ.get("PTQ_RANDOM_SEED", "2024"))


def _random_shapes(n=_RANDOM_CASES, seed=_RANDOM_SEED):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = int(rng.choice([1, 3, 5, 16, 17, 31, 33, 64, 65, 100, 257, 512, 700]))
        K = 16 * int(rng.integers(1, 260))
        N = int(rng.integers(1, 1200))
        dt = synth.BF16 if rng.random() < 0.7 else synth.F32
        smooth = bool(rng.random() < 0.7)
        alpha = float(rng.choice([0.0, 0.3, 0.5, 0.8, 1.0]))
        std = float(rng.choice([0.002, 0.02, 0.5]))
        out.append((seed, i, T, K, N, dt, smooth, alpha, std))
    return out


# Two cases of earlier sweeps whose SSZ rows hold a candidate one fp32 step from the kept scale, with errors
# 1.15e-12 relative apart (seed 22 case 55, row 515; seed 25 case 1315, row 306): kept as fixed cases.
_TIED_ROW_CASES = [_random_shapes(56, 22)[55], _random_shapes(1316, 25)[1315]]


@pytest.mark.parametrize("seed,i,T,K,N,dtype,smooth,alpha,std", _TIED_ROW_CASES + _random_shapes())
def test_random_shapes_whole_path(pq, seed, i, T, K, N, dtype, smooth, alpha, std):
    """The whole path on seeded random shapes (ragged tokens, widths of 16 to ~4 K, any channel count, both input
    types, three weight spreads with heavy-tailed entries, with and without smoothing), every output against the
    oracle: codes, scales, iteration counts, int32 sums bit for bit, y within the tolerance; and on the same
    weights the int4 and the asymmetric int8 SSZ."""
    tag = f"random {seed}/{i}: T={T} K={K} N={N} dtype={dtype} smooth={smooth} alpha={alpha} std={std}"
    x_h = synth.activation(f"random/{seed}/{i}/x", T, K, dtype,
                           synth.pick_channels(f"random/{seed}/{i}/ch", K, max(1, K // 50)), 40.0)
    w_h = synth.weight(f"random/{seed}/{i}/w", N, K, dtype, std, 0.05, 1.0, 0.001, 20.0)
    xf, wf = synth.widen(x_h), synth.widen(w_h)
    announce(tag)
    xd, wd = dev(x_h), dev(w_h)
    if smooth:
        s_ref = oracle.smooth_factors(oracle.absmax_cols(xf), oracle.absmax_cols(wf), alpha)
        s = pq.sq_smooth_factors(pq.sq_absmax_calib(xd), pq.sq_absmax_calib(wd), alpha)
        np.testing.assert_array_equal(host(s), s_ref, err_msg=tag + " s")
    else:
        s_ref, s = None, None
    ref = oracle.ssz(wf, s_ref, 8)
    S, wq, it, mse = pq.ssz_weight_qparams(wd, s, bits=8)
    compare_ssz(host(S), host(wq), host(it), host(mse), ref, tag)
    xq_ref, d_ref = oracle.quant_per_token(xf, s_ref)
    xq, d = pq.quant_per_token_i8(xd, s)
    np.testing.assert_array_equal(host(xq), xq_ref, err_msg=tag + " xq")
    np.testing.assert_array_equal(host(d), d_ref, err_msg=tag + " tok_scale")
    acc_ref = oracle.gemm_i8(xq_ref, ref["q"])
    y, acc = pq.w8a8_gemm_dequant(xq, wq, d, S, want_acc=True)
    np.testing.assert_array_equal(host(acc), acc_ref, err_msg=tag + " acc")
    assert_y(host(y), oracle.dequant(acc_ref, d_ref, ref["S"]), tag + " y")
    r4 = oracle.ssz(wf, s_ref, 4)
    S4, q4, it4, m4 = pq.ssz_weight_qparams(wd, s, bits=4)
    compare_ssz(host(S4), unpack_int4(host(q4)), host(it4), host(m4), r4, tag + " int4")
    ra = oracle.ssz_asym(wf, s_ref)
    Sa, Za, qa, ita, ma = pq.ssz_weight_qparams_asym(wd, s)
    compare_ssz_asym(host(Sa), host(Za), host(qa), host(ita), host(ma), ra, tag + " asym")
