"""GPU parity, stage by stage: each entry point of the C ABI against the oracle on
seeded inputs, over shapes that span several tiles and a ragged tail, plus the
degenerate cases of the method.  Integers are compared bit for bit; floats to
the tolerances in parity_util.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import (announce, assert_scales, assert_y, compare_ssz, compare_ssz_asym, dev, host,
                         unpack_int4)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_int8_quantization_amd as m
    return m


def _x(name, T, K, dtype, factor=40.0, frac=0.01):
    ch = synth.pick_channels(name, K, max(1, round(frac * K)))
    return synth.activation(name, T, K, dtype, ch, factor)


def _w(name, N, K, dtype, tail=0.0):
    return synth.weight(name, N, K, dtype, 0.02, 0.05, 1.0, tail, 20.0)


# ------------------------------------------------------------------ calibration

@pytest.mark.parametrize("rows,cols,dtype,batches", [
    (16, 64, synth.F32, 1), (1, 16, synth.BF16, 1), (300, 1040, synth.BF16, 3), (257, 4112, synth.F32, 2),
    (4096, 4096, synth.BF16, 2), (2048, 16384, synth.BF16, 1), (28672, 8192, synth.BF16, 1)])
def test_absmax_calib(pq, rows, cols, dtype, batches):
    ref = None
    amax = None
    for b in range(batches):
        x = _x(f"cal/{rows}x{cols}/b{b}", rows, cols, dtype)
        ref = oracle.absmax_cols(synth.widen(x), ref)
        announce(f"sq_absmax_calib rows={rows} cols={cols} dtype={dtype} batch={b}")
        amax = pq.sq_absmax_calib(dev(x), amax, accumulate=b > 0)
    np.testing.assert_array_equal(host(amax), ref)


def test_absmax_calib_accumulate_keeps_larger(pq):
    x = _x("cal/acc", 64, 256, synth.F32)
    big = torch.full((256,), 1e6, device="cuda:0")
    announce("sq_absmax_calib accumulate into large values")
    out = pq.sq_absmax_calib(dev(x), big.clone(), accumulate=True)
    assert torch.all(out == 1e6)


# ------------------------------------------------------------------ smoothing factors

@pytest.mark.parametrize("alpha", [0.0, 0.5, 0.8, 1.0])
def test_smooth_factors(pq, alpha):
    K = 4096 + 16
    rng = np.random.default_rng(3)
    ax = np.exp(rng.uniform(-3, 5, K)).astype(np.float32)
    aw = np.exp(rng.uniform(-7, 0, K)).astype(np.float32)
    ax[5] = 0.0
    aw[9] = 0.0
    ref = oracle.smooth_factors(ax, aw, alpha)
    announce(f"sq_smooth_factors K={K} alpha={alpha}")
    s = host(pq.sq_smooth_factors(dev(ax), dev(aw), alpha))
    assert s[5] == 1.0 and s[9] == 1.0
    assert_scales(s, ref, "s")
    assert np.sum(s != ref) <= 2  # fp64 pow may differ in the last bit before the single rounding


# ------------------------------------------------------------------ per-token quantization

@pytest.mark.parametrize("T,K,dtype,smooth", [
    (16, 64, synth.F32, True), (1, 16, synth.BF16, False), (257, 1040, synth.BF16, True),
    (300, 4096, synth.BF16, True), (300, 4096, synth.F32, False), (33, 16384, synth.BF16, True),
    (5, 8192, synth.BF16, False), (64, 3072, synth.BF16, True), (9, 36864, synth.BF16, True),
    (3, 65536 + 16, synth.BF16, True), (2, 131072, synth.BF16, True), (2, 131072, synth.F32, False)])
def test_quant_per_token(pq, T, K, dtype, smooth):
    x = _x(f"q/{T}x{K}", T, K, dtype)
    if T > 2:
        x[2] = 0  # all-zero token
    s = np.exp(np.random.default_rng(K).uniform(-2, 2, K)).astype(np.float32) if smooth else None
    xq_ref, d_ref = oracle.quant_per_token(synth.widen(x), s)
    announce(f"quant_per_token_i8 T={T} K={K} dtype={dtype} smooth={smooth}")
    xq, d = pq.quant_per_token_i8(dev(x), None if s is None else dev(s))
    np.testing.assert_array_equal(host(d), d_ref)
    np.testing.assert_array_equal(host(xq), xq_ref)
    if T > 2:
        assert host(d)[2] == 1.0


# ------------------------------------------------------------------ SSZ weight quantization

def _edge_rows(K, qmax):
    rows = np.zeros((4, K), dtype=np.float32)
    k = (np.arange(K) % (2 * qmax + 1)) - qmax
    rows[1] = k * 2.0 ** -9            # exact grid: lossless
    rows[2, K // 3] = -0.37             # a single non-zero element
    rows[3] = 6e-6                      # refit falls under the 1e-5 floor
    return rows


def _bf16_bits(a):
    """fp32 -> bf16 bit patterns (uint16), round to nearest even; finite inputs (test input preparation)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("N,K,dtype,bits,smooth,tail", [
    (128, 64, synth.F32, 8, True, 0.0), (300, 1040, synth.BF16, 8, True, 0.001),
    (300, 1040, synth.BF16, 4, False, 0.001), (96, 4096, synth.BF16, 8, False, 0.001),
    (96, 4096, synth.BF16, 4, True, 0.0), (40, 16384, synth.BF16, 8, True, 0.001),
    (40, 16384, synth.BF16, 4, False, 0.001), (23, 8192, synth.BF16, 8, True, 0.0),
    (17, 2064, synth.F32, 4, True, 0.002), (6, 36864, synth.BF16, 8, False, 0.001),
    (3, 131072, synth.BF16, 8, True, 0.001), (3, 131072, synth.BF16, 4, False, 0.001),
    # short rows, several per wave: 1, 2, 4, 8, 16 and 32 lanes per row (row counts that leave the
    # last wave partly empty), and the widths just past them on the one-wave row kernel
    (13, 16, synth.F32, 8, True, 0.0), (130, 32, synth.BF16, 4, True, 0.001),
    (67, 48, synth.F32, 4, False, 0.0), (301, 112, synth.BF16, 8, True, 0.001),
    (257, 256, synth.F32, 4, True, 0.002), (1023, 512, synth.BF16, 8, False, 0.001),
    (45, 528, synth.BF16, 4, True, 0.001), (99, 1024, synth.F32, 8, True, 0.0)])
def test_ssz(pq, N, K, dtype, bits, smooth, tail):
    w = _w(f"ssz/{N}x{K}", N, K, dtype, tail)
    wf = synth.widen(w).copy()
    edge = _edge_rows(K, 127 if bits == 8 else 7)[:min(4, N)]
    if dtype == synth.F32:
        wf[:len(edge)] = edge
        w = wf
    else:
        w = w.copy()
        w[:len(edge)] = _bf16_bits(edge)
        wf = synth.widen(w).copy()
    s = np.exp(np.random.default_rng(N + K).uniform(-1, 1, K)).astype(np.float32) if smooth else None
    ref = oracle.ssz(wf, s, bits)
    announce(f"ssz_weight_qparams N={N} K={K} dtype={dtype} bits={bits} smooth={smooth}")
    S, wq, it, mse = pq.ssz_weight_qparams(dev(w), None if s is None else dev(s), bits=bits)
    codes = host(wq) if bits == 8 else unpack_int4(host(wq))
    compare_ssz(host(S), codes, host(it), host(mse), ref, f"ssz {N}x{K} int{bits}")


@pytest.mark.parametrize("K", [1024, 256])
@pytest.mark.parametrize("max_iter", [0, 1, 3])
def test_ssz_max_iter(pq, max_iter, K):
    w = _w(f"ssz/iter/{K}", 64, K, synth.BF16, 0.001)
    ref = oracle.ssz(synth.widen(w), None, 4, max_iter=max_iter)
    announce(f"ssz_weight_qparams K={K} max_iter={max_iter}")
    S, wq, it, mse = pq.ssz_weight_qparams(dev(w), None, bits=4, max_iter=max_iter)
    compare_ssz(host(S), unpack_int4(host(wq)), host(it), host(mse), ref, f"K={K} max_iter={max_iter}")


def test_ssz_outputs_optional(pq):
    w = _w("ssz/opt", 32, 512, synth.BF16)
    ref = oracle.ssz(synth.widen(w), None, 8)
    announce("ssz_weight_qparams scale only")
    S, wq, it, mse = pq.ssz_weight_qparams(dev(w), None, bits=8, want_codes=False, want_stats=False)
    assert wq is None and it is None
    np.testing.assert_array_equal(host(S), ref["S"])


# Thresholds that make the relative convergence test decide: on weights scaled to mean errors above 1,
# a threshold of 1e-3 leaves accepted improvements d > 0 with |d| >= thr and d / best near thr (the
# kernels take the fp64 quotient only there); threshold 0 leaves only d < 0 (a rejected step) to stop
# a row early.
@pytest.mark.parametrize("N,K,bits,mag,thr", [
    (64, 4096, 8, 1e4, 1e-3), (64, 4096, 4, 1e3, 1e-3), (256, 256, 8, 1e4, 1e-3), (256, 256, 4, 1e4, 1e-3),
    (16, 16384, 8, 1e4, 1e-3), (64, 1024, 8, 1.0, 0.0), (256, 128, 4, 1.0, 0.0)])
def test_ssz_thresholds(pq, N, K, bits, mag, thr):
    w = (synth.widen(_w(f"ssz/thr/{N}x{K}", N, K, synth.F32, 0.001)) * np.float32(mag)).astype(np.float32)
    ref = oracle.ssz(w, None, bits, thr=thr)
    announce(f"ssz_weight_qparams N={N} K={K} bits={bits} magnitude={mag:g} threshold={thr:g}")
    S, wq, it, mse = pq.ssz_weight_qparams(dev(w), None, bits=bits, threshold=thr)
    codes = host(wq) if bits == 8 else unpack_int4(host(wq))
    compare_ssz(host(S), codes, host(it), host(mse), ref, f"ssz thr={thr:g} {N}x{K} int{bits}")


@pytest.mark.parametrize("N,K,mag,thr", [(64, 4096, 1e4, 1e-3), (48, 512, 1e3, 1e-3), (32, 2048, 1.0, 0.0)])
def test_ssz_asym_thresholds(pq, N, K, mag, thr):
    w = (synth.widen(_w(f"ssza/thr/{N}x{K}", N, K, synth.F32, 0.001)) * np.float32(mag)).astype(np.float32)
    ref = oracle.ssz_asym(w, None, thr=thr)
    announce(f"ssz_weight_qparams_asym N={N} K={K} magnitude={mag:g} threshold={thr:g}")
    S, Z, wq, it, mse = pq.ssz_weight_qparams_asym(dev(w), None, threshold=thr)
    compare_ssz_asym(host(S), host(Z), host(wq), host(it), host(mse), ref, f"asym thr={thr:g} {N}x{K}")


# ------------------------------------------------------------------ asymmetric SSZ

def _edge_rows_asym(K):
    rows = np.zeros((6, K), dtype=np.float32)
    k = (np.arange(K) % 256) - 128
    rows[1] = (k - 37) * 2.0 ** -9      # exact grid with offset 37: lossless
    rows[2, K // 3] = -0.37             # a single non-zero element
    rows[3] = 0.5                       # constant: floor scale, saturated offset, nothing to fit
    rows[4] = np.linspace(0.0, 1.0, K)  # one-sided: offset at the bottom of the range
    rows[5] = -np.linspace(0.0, 1.0, K)
    return rows


@pytest.mark.parametrize("N,K,dtype,smooth,tail,shift", [
    (128, 64, synth.F32, True, 0.0, 0.0), (300, 1040, synth.BF16, True, 0.001, 0.01),
    (96, 4096, synth.BF16, False, 0.001, 0.0), (96, 4096, synth.F32, True, 0.0, 0.005),
    (40, 16384, synth.BF16, True, 0.001, 0.0), (23, 8192, synth.BF16, False, 0.0, 0.02),
    (17, 2064, synth.F32, False, 0.002, 0.0), (9, 16, synth.F32, False, 0.0, 0.0),
    (6, 36864, synth.BF16, True, 0.001, 0.0), (3, 131072, synth.BF16, False, 0.001, 0.0)])
def test_ssz_asym(pq, N, K, dtype, smooth, tail, shift):
    w = _w(f"ssza/{N}x{K}", N, K, dtype, tail)
    wf = synth.widen(w).copy()
    wf[::2] += np.float32(shift)
    edge = _edge_rows_asym(K)[:min(6, N)]
    wf[:len(edge)] = edge
    if dtype == synth.F32:
        w = wf
    else:
        w = _bf16_bits(wf)
        wf = synth.widen(w).copy()
    s = np.exp(np.random.default_rng(N * 3 + K).uniform(-1, 1, K)).astype(np.float32) if smooth else None
    ref = oracle.ssz_asym(wf, s)
    announce(f"ssz_weight_qparams_asym N={N} K={K} dtype={dtype} smooth={smooth}")
    S, Z, wq, it, mse = pq.ssz_weight_qparams_asym(dev(w), None if s is None else dev(s))
    compare_ssz_asym(host(S), host(Z), host(wq), host(it), host(mse), ref, f"ssz asym {N}x{K}")


@pytest.mark.parametrize("max_iter", [0, 1, 3])
def test_ssz_asym_max_iter(pq, max_iter):
    w = _w("ssza/iter", 64, 1024, synth.BF16, 0.001)
    ref = oracle.ssz_asym(synth.widen(w), None, max_iter=max_iter)
    announce(f"ssz_weight_qparams_asym max_iter={max_iter}")
    S, Z, wq, it, mse = pq.ssz_weight_qparams_asym(dev(w), None, max_iter=max_iter)
    compare_ssz_asym(host(S), host(Z), host(wq), host(it), host(mse), ref, f"asym max_iter={max_iter}")


def test_ssz_asym_scale_only(pq):
    w = _w("ssza/opt", 32, 512, synth.BF16)
    ref = oracle.ssz_asym(synth.widen(w), None)
    announce("ssz_weight_qparams_asym scale and offset only")
    S, Z, wq, it, mse = pq.ssz_weight_qparams_asym(dev(w), None, want_codes=False, want_stats=False)
    assert wq is None and it is None and mse is None
    np.testing.assert_array_equal(host(S), ref["S"])
    np.testing.assert_array_equal(host(Z), ref["Z"])


# ------------------------------------------------------------------ GEMM + dequant

@pytest.mark.parametrize("M,N,K", [
    (16, 128, 64), (1, 1, 16), (7, 33, 48), (16, 1000, 8192), (5, 1000, 8208), (20, 700, 272), (31, 4000, 4112),
    (33, 77, 160), (64, 300, 4096), (64, 16448, 1040), (65, 130, 1040),
    (300, 520, 1040), (257, 259, 4096), (512, 768, 2048), (256, 256, 16), (1024, 1024, 4096),
    (1900, 3100, 1040), (3100, 1900, 1040)])
def test_gemm_dequant(pq, M, N, K):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    a = rng.integers(-127, 128, (M, K)).astype(np.int8)
    b = rng.integers(-127, 128, (N, K)).astype(np.int8)
    ts = rng.uniform(0.01, 1.0, M).astype(np.float32)
    cs = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    acc_ref = oracle.gemm_i8(a, b)
    y_ref = oracle.dequant(acc_ref, ts, cs)
    announce(f"w8a8_gemm_dequant M={M} N={N} K={K}")
    y, acc = pq.w8a8_gemm_dequant(dev(a), dev(b), dev(ts), dev(cs), want_acc=True)
    np.testing.assert_array_equal(host(acc), acc_ref)
    assert_y(host(y), y_ref, f"y {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,act,out,want_acc", [
    (1, 1, 4096, "none", "f32", True), (5, 17, 4096, "relu", "bf16", False), (16, 4096, 4096, "gelu", "i8", False),
    (16, 9000, 4096, "none", "f32", True), (2, 16, 8192, "none", "i8", True), (16, 4100, 8192, "relu", "f32", False),
    (13, 28672, 8192, "none", "f32", True), (16, 28688, 8192, "gelu", "bf16", True)])
def test_gemm_decode_streaming(pq, M, N, K, act, out, want_acc):
    """The streaming decode kernel (at most 16 tokens, K of 4 or 8 KB): persistent blocks over groups of 16
    weight rows -- one group, fewer groups than blocks, more (ragged last group, blocks taking one or two more
    groups), the full decode shape -- every output type, against the oracle."""
    _fused_case(pq, M, N, K, act, out, want_acc, M * 31 + N + K)


def test_gemm_max_k_extremes(pq):
    """K = 131056 (the largest multiple of 16 with 2^14 K < 2^31) with all-extreme codes, -128 included: exact
    int32 at the largest magnitudes any int8 codes reach (+2^14 K and -127 * 128 K)."""
    K = 131056
    a = np.full((3, K), -128, dtype=np.int8)
    a[1] = 127
    b = np.full((20, K), -128, dtype=np.int8)
    b[7] = 127
    ref = oracle.gemm_i8(a, b)
    assert ref.max() == 128 * 128 * K and ref.min() == -127 * 128 * K
    ts = np.ones(3, np.float32)
    cs = np.ones(20, np.float32)
    announce("w8a8_gemm_dequant K=131056 extremes (decode kernel)")
    y, acc = pq.w8a8_gemm_dequant(dev(a), dev(b), dev(ts), dev(cs), want_acc=True)
    np.testing.assert_array_equal(host(acc), ref)
    a2 = np.tile(a, (40, 1))[:100]
    ref2 = oracle.gemm_i8(a2, b)
    announce("w8a8_gemm_dequant K=131056 extremes (prefill kernel)")
    y2, acc2 = pq.w8a8_gemm_dequant(dev(a2), dev(b), dev(np.ones(100, np.float32)), dev(cs), want_acc=True)
    np.testing.assert_array_equal(host(acc2), ref2)


@pytest.mark.parametrize("M,N", [(4096, 4096), (2048, 3072), (3072, 2048), (2048, 2048)])
def test_gemm_max_k_tiles(pq, M, N):
    """K = 131056 on the prefill tile shapes (256x256, 128x256, 256x128, 128x128 grids): rows of all -128 or all
    127 codes make every int32 sum 128^2 K, -127 * 128 K or 127^2 K -- the largest magnitudes the bound admits
    (closed form)."""
    K = 131056
    va = torch.where(torch.arange(M, device="cuda:0") % 3 == 0, -128, 127).to(torch.int8)
    vb = torch.where(torch.arange(N, device="cuda:0") % 5 == 0, -128, 127).to(torch.int8)
    a = (va[:, None] * torch.ones((M, K), dtype=torch.int8, device="cuda:0")).contiguous()
    b = (vb[:, None] * torch.ones((N, K), dtype=torch.int8, device="cuda:0")).contiguous()
    ones_m = torch.ones(M, dtype=torch.float32, device="cuda:0")
    ones_n = torch.ones(N, dtype=torch.float32, device="cuda:0")
    announce(f"w8a8_gemm_dequant K=131056 extremes M={M} N={N}")
    y, acc = pq.w8a8_gemm_dequant(a, b, ones_m, ones_n, want_acc=True)
    del a, b
    expect = np.outer(host(va).astype(np.int64), host(vb).astype(np.int64)) * K
    np.testing.assert_array_equal(host(acc).astype(np.int64), expect)
    np.testing.assert_array_equal(host(y), expect.astype(np.float32))


def test_gemm_deterministic(pq):
    rng = np.random.default_rng(5)
    a = dev(rng.integers(-127, 128, (700, 1024)).astype(np.int8))
    b = dev(rng.integers(-127, 128, (900, 1024)).astype(np.int8))
    ts = dev(rng.uniform(0.1, 1, 700).astype(np.float32))
    cs = dev(rng.uniform(0.1, 1, 900).astype(np.float32))
    announce("w8a8_gemm_dequant run twice")
    y1 = pq.w8a8_gemm_dequant(a, b, ts, cs)
    y2 = pq.w8a8_gemm_dequant(a, b, ts, cs)
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("M,N,K", [(16, 1000, 8192), (65, 130, 1040), (300, 520, 1040), (257, 259, 4096),
                                   (1024, 1024, 4096), (512, 4352, 1024), (4352, 4096, 64), (4300, 4100, 80),
                                   (1900, 3104, 1040), (3100, 1904, 1040)])
@pytest.mark.parametrize("out", ["f32", "bf16", "i8"])
def test_gemm_plain_epilogue(pq, M, N, K, out):
    """No bias, no activation, no int32 copy: the prefill kernel's separate plain-dequantization loop,
    bit-exact against the oracle's fp32 epilogue (also with the int8 output's next-layer fold)."""
    rng = np.random.default_rng(M * 13 + N * 7 + K + len(out))
    a = rng.integers(-127, 128, (M, K)).astype(np.int8)
    b = rng.integers(-127, 128, (N, K)).astype(np.int8)
    ts = rng.uniform(0.002, 0.02, M).astype(np.float32)
    cs = rng.uniform(1e-4, 1e-3, N).astype(np.float32)
    ns = np.exp(rng.uniform(-1, 1, N)).astype(np.float32) if out == "i8" and M % 2 == 1 else None
    acc_ref = oracle.gemm_i8(a, b)
    code = {"f32": oracle.OUT_F32, "bf16": oracle.OUT_BF16, "i8": oracle.OUT_I8}[out]
    y32 = oracle.epilogue(acc_ref, ts, cs, None, oracle.ACT_NONE)
    osc = np.float32(np.max(np.abs(y32)) / 100.0) if out == "i8" else 1.0
    if out == "i8" and not osc > 0:  # an all-zero output (tiny shapes): any positive scale will do
        osc = np.float32(1.0)
    ref = oracle.epilogue(acc_ref, ts, cs, None, oracle.ACT_NONE, code, ns, osc)
    announce(f"w8a8_gemm_fused plain M={M} N={N} K={K} out={out} next_s={ns is not None}")
    y = pq.w8a8_gemm_fused(dev(a), dev(b), dev(ts), dev(cs), None, "none", out, None if ns is None else dev(ns),
                           dev(np.array([osc], np.float32)) if out == "i8" else None)
    got = host(y.view(torch.int16)).view(np.uint16) if out == "bf16" else host(y)
    np.testing.assert_array_equal(got, ref)
    if out == "f32":
        announce(f"w8a8_gemm_dequant plain M={M} N={N} K={K}")
        y2 = pq.w8a8_gemm_dequant(dev(a), dev(b), dev(ts), dev(cs))
        np.testing.assert_array_equal(host(y2), ref)


# ------------------------------------------------------------------ fused epilogue

@pytest.mark.parametrize("M,N,K", [(16, 1000, 8192), (5, 77, 160), (64, 300, 4096), (300, 520, 1040),
                                   (257, 259, 4096), (1024, 1024, 4096), (700, 4352, 1024)])
@pytest.mark.parametrize("act", ["none", "relu", "gelu"])
@pytest.mark.parametrize("out", ["f32", "bf16", "i8"])
@pytest.mark.parametrize("want_acc", [True, False])
def test_gemm_fused(pq, M, N, K, act, out, want_acc):
    """With the int32 copy the prefill kernel stores element by element; without it (and 16-byte output
    rows) its epilogue goes through LDS as whole-row pieces: both against the oracle."""
    _fused_case(pq, M, N, K, act, out, want_acc, M * 11 + N * 5 + K + len(act) + len(out))


# case count and seed of the random-shape sweep; larger sweeps: PTQ_RANDOM_CASES=2000 PTQ_RANDOM_SEED=11
_RANDOM_CASES = int(os.environ.get("PTQ_RANDOM_CASES", "64"))
_RANDOM_SEED = int(os.environ.get("PTQ_RANDOM_SEED", "2024"))


def _random_fused(n=_RANDOM_CASES, seed=_RANDOM_SEED):
    rng = np.random.default_rng(seed + 1)
    out = []
    while len(out) < n:
        M = int(rng.choice([1, 2, 7, 16, 17, 32, 33, 63, 64, 65, 100, 255, 256, 300, 513, 1024, 1100]))
        N = int(rng.integers(1, 2300))
        K = 16 * int(rng.integers(1, 400))
        if M * N * K > 2_000_000_000:  # keeps the oracle's GEMM to a second or two
            continue
        out.append((seed, len(out), M, N, K, str(rng.choice(["none", "relu", "gelu"])),
                    str(rng.choice(["f32", "bf16", "i8"])), bool(rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("seed,i,M,N,K,act,out,want_acc", _random_fused())
def test_gemm_fused_random_shapes(pq, seed, i, M, N, K, act, out, want_acc):
    """The fused epilogue on seeded random shapes: every GEMM kernel the dispatch picks (decode kernel, 64x64 to
    256x256 tiles, ragged edges on all three sides), every activation and output type, against the oracle."""
    _fused_case(pq, M, N, K, act, out, want_acc, seed * 100_003 + i)


def _fused_case(pq, M, N, K, act, out, want_acc, seed):
    rng = np.random.default_rng(seed)
    a = rng.integers(-127, 128, (M, K)).astype(np.int8)
    b = rng.integers(-127, 128, (N, K)).astype(np.int8)
    ts = rng.uniform(0.002, 0.02, M).astype(np.float32)
    cs = rng.uniform(1e-4, 1e-3, N).astype(np.float32)
    bias = rng.normal(0, 0.5, N).astype(np.float32) if (M + N) % 2 else None
    ns = np.exp(rng.uniform(-1, 1, N)).astype(np.float32) if out == "i8" and M % 2 == 0 else None
    acc_ref = oracle.gemm_i8(a, b)
    code = {"f32": oracle.OUT_F32, "bf16": oracle.OUT_BF16, "i8": oracle.OUT_I8}[out]
    # a static output scale near the output range, so that the int8 codes use the whole range
    y32 = oracle.epilogue(acc_ref, ts, cs, bias, oracle.ACT_RELU if act == "relu" else oracle.ACT_NONE)
    osc = np.float32(np.max(np.abs(y32)) / 100.0) if out == "i8" else 1.0
    ref = oracle.epilogue(acc_ref, ts, cs, bias, {"none": 0, "relu": 1, "gelu": 2}[act], code, ns, osc)
    announce(f"w8a8_gemm_fused M={M} N={N} K={K} act={act} out={out} bias={bias is not None} "
             f"next_s={ns is not None} want_acc={want_acc}")
    r = pq.w8a8_gemm_fused(dev(a), dev(b), dev(ts), dev(cs), None if bias is None else dev(bias), act, out,
                           None if ns is None else dev(ns),
                           dev(np.array([osc], np.float32)) if out == "i8" else None, want_acc=want_acc)
    if want_acc:
        y, acc = r
        np.testing.assert_array_equal(host(acc), acc_ref)
    else:
        y = r
    if out == "bf16":
        got = host(y.view(torch.int16)).view(np.uint16)
    else:
        got = host(y)
    if act != "gelu":
        np.testing.assert_array_equal(got, ref)  # exact: the same fp32 operations in the same order
        return
    n_amb, n_diff = gelu_check(got, ref, acc_ref, ts, cs, bias, out, ns, osc)
    if out == "f32":
        announce(f"  gelu f32: {n_diff} of {got.size} outputs differ from the oracle's, all within the bound")
    else:
        announce(f"  gelu {out}: {n_diff} of {got.size} outputs on the other side of a rounding boundary "
                 f"({n_amb} within the erf fit's bound of one)")


# The device takes erf from a published erfc fit (relative error below 1.2e-7); the oracle takes the C library's
# erff (within an ulp).  GELU(u) = 0.5 u (1 + erf(u / sqrt 2)): for u < 0 the sum 1 + erf cancels on both
# sides, so the two fp32 values agree within an absolute amount proportional to |u| (about 6e-8 |u| per
# rounding near erf = -1, plus the fit's 1.2e-7 relative to erfc), not relative to the result.  Bound:
# GELU_EPS |u| + GELU_TINY (the last for results that underflow), a few times the sum of those terms.
GELU_EPS, GELU_TINY = 1e-6, 1e-37


def gelu_check(got, ref, acc_ref, ts, cs, bias, out, ns, osc):
    """Every GELU output must equal the oracle's, except where the oracle's fp32 GELU value v lies within the
    bound e = GELU_EPS |u| + GELU_TINY (u the pre-activation value) of a rounding boundary of the output format --
    where v - e and v + e give different outputs; there the output may be any value between those two.  Returns
    the count of such elements and of those that do differ."""
    v = oracle.epilogue(acc_ref, ts, cs, bias, oracle.ACT_GELU)  # fp32 GELU values of the oracle
    u = oracle.epilogue(acc_ref, ts, cs, bias, oracle.ACT_NONE)  # the pre-activation values
    e = np.abs(u.astype(np.float64)) * GELU_EPS + GELU_TINY
    v_lo, v_hi = (v - e).astype(np.float32), (v + e).astype(np.float32)
    if out == "f32":
        assert np.all(np.abs(got.astype(np.float64) - v) <= e), "gelu f32 beyond the erf fit's bound"
        return 0, int(np.sum(got != v))
    if out == "bf16":
        to_bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).float().numpy()  # noqa: E731
        lo, hi = to_bf(v_lo), to_bf(v_hi)
        g = (got.astype(np.uint32) << 16).view(np.float32)
        same = (got == ref)
    else:
        def code(x):
            xh = x / ns[None, :] if ns is not None else x
            return np.clip(np.rint(xh / np.float32(osc)), -127, 127)
        lo, hi = code(v_lo), code(v_hi)
        g = got.astype(np.float32)
        same = (got == ref)
    amb = lo != hi
    assert np.all(same | amb), f"gelu {out}: {int(np.sum(~same & ~amb))} outputs differ away from a boundary"
    assert np.all((g >= lo) & (g <= hi) | ~amb), f"gelu {out}: an output beyond the boundary's two sides"
    return int(np.sum(amb)), int(np.sum(~same))


# ------------------------------------------------------------------ static per-tensor scales

@pytest.mark.parametrize("T,K,dtype,smooth", [(16, 64, synth.F32, True), (300, 1040, synth.BF16, True),
                                              (257, 4096, synth.BF16, False), (64, 16384, synth.F32, True)])
def test_act_scale_ema(pq, T, K, dtype, smooth):
    s = np.exp(np.random.default_rng(T + K).uniform(-1, 1, K)).astype(np.float32) if smooth else None
    state_ref = None
    state = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    for b in range(5):
        x = _x(f"ema/{T}x{K}/{b}", T, K, dtype, factor=40.0 if b != 2 else 200.0)
        a = oracle.absmax_tensor(synth.widen(x), s, oracle.FOLD_DIV)
        state_ref = oracle.ema_update(state_ref, a, 0.9, b == 0)
        announce(f"sq_act_scale_ema T={T} K={K} batch {b}")
        col = pq.sq_absmax_calib(dev(x))
        st, sc, rs = pq.sq_act_scale_ema(col, None if s is None else dev(s), 0.9, first=b == 0, state=state, rows=T)
        assert host(st)[0] == state_ref, (b, host(st)[0], state_ref)
        assert host(sc)[0] == oracle.act_static_scale(state_ref)
        assert np.all(host(rs) == host(sc)[0])


@pytest.mark.parametrize("N,K,smooth", [(128, 64, True), (300, 1040, False), (4096, 4096, True)])
def test_weight_scale_per_tensor(pq, N, K, smooth):
    w = _w(f"wpt/{N}x{K}", N, K, synth.BF16, 0.001)
    s = np.exp(np.random.default_rng(N + K).uniform(-1, 1, K)).astype(np.float32) if smooth else None
    S_ref = oracle.weight_scale_per_tensor(oracle.absmax_tensor(synth.widen(w), s, oracle.FOLD_MUL))
    announce(f"weight_scale_per_tensor N={N} K={K}")
    col = pq.sq_absmax_calib(dev(w))
    sc, ch = pq.weight_scale_per_tensor(col, None if s is None else dev(s), n=N)
    assert host(sc)[0] == S_ref
    assert np.all(host(ch) == S_ref)
    tiny = np.zeros(64, np.float32)
    sc0, _ = pq.weight_scale_per_tensor(dev(tiny))
    assert host(sc0)[0] == np.float32(1e-5)  # the floor


@pytest.mark.parametrize("R,C,dtype,fold", [(16, 64, synth.F32, "div"), (300, 1040, synth.BF16, "div"),
                                            (257, 4096, synth.BF16, "mul"), (33, 16384, synth.F32, "mul"),
                                            (5, 8192, synth.BF16, None), (1, 16, synth.F32, None),
                                            (2, 131072, synth.BF16, "div")])
def test_quant_static(pq, R, C, dtype, fold):
    x = _x(f"qs/{R}x{C}", R, C, dtype)
    s = np.exp(np.random.default_rng(R + C).uniform(-1, 1, C)).astype(np.float32) if fold else None
    fcode = {"div": oracle.FOLD_DIV, "mul": oracle.FOLD_MUL, None: oracle.FOLD_NONE}[fold]
    S = np.float32(oracle.absmax_tensor(synth.widen(x), s, fcode) / 150.0)  # the largest codes saturate
    ref = oracle.quant_static(synth.widen(x), S, s, fcode)
    announce(f"quant_static_i8 R={R} C={C} fold={fold}")
    q, rs = pq.quant_static_i8(dev(x), dev(np.array([S], np.float32)), None if s is None else dev(s),
                               fold or "div")
    np.testing.assert_array_equal(host(q), ref)
    assert np.all(host(rs) == S)
    assert np.any(np.abs(ref) == 127)


def _random_quant(n=_RANDOM_CASES, seed=_RANDOM_SEED):
    rng = np.random.default_rng(seed + 2)
    out = []
    for i in range(n):
        R = int(rng.choice([1, 2, 3, 16, 31, 64, 100, 257, 600, 2048]))
        C = 16 * int(rng.integers(1, 1300))
        out.append((seed, i, R, C, synth.BF16 if rng.random() < 0.7 else synth.F32,
                    [None, "div", "mul"][int(rng.integers(0, 3))]))
    return out


@pytest.mark.parametrize("seed,i,R,C,dtype,fold", _random_quant())
def test_quantizers_random_shapes(pq, seed, i, R, C, dtype, fold):
    """Per-token, per-tensor weight and static quantization on seeded random shapes (1 to 2048 rows, widths of 16
    to ~21 K, both input types, each fold), bit for bit against the oracle."""
    x = _x(f"rq/{seed}/{i}", R, C, dtype)
    s = np.exp(np.random.default_rng(seed * 7 + i).uniform(-1, 1, C)).astype(np.float32) if fold else None
    xf = synth.widen(x)
    sd = None if s is None else dev(s)
    announce(f"random quantizers {seed}/{i}: R={R} C={C} dtype={dtype} fold={fold}")
    xd = dev(x)
    if fold != "mul":  # per-token quantization folds by division or not at all
        xq_ref, d_ref = oracle.quant_per_token(xf, s)
        xq, d = pq.quant_per_token_i8(xd, sd)
        np.testing.assert_array_equal(host(xq), xq_ref)
        np.testing.assert_array_equal(host(d), d_ref)
    fcode = {"div": oracle.FOLD_DIV, "mul": oracle.FOLD_MUL, None: oracle.FOLD_NONE}[fold]
    a = oracle.absmax_tensor(xf, s, fcode)
    if fold != "div":  # the per-tensor weight scale folds by multiplication or not at all
        sc, _ = pq.weight_scale_per_tensor(pq.sq_absmax_calib(xd), sd)
        assert host(sc)[0] == oracle.weight_scale_per_tensor(a)
    S = np.float32(a / 150.0) if a > 0 else np.float32(1.0)
    q, _ = pq.quant_static_i8(xd, dev(np.array([S], np.float32)), sd, fold or "div")
    np.testing.assert_array_equal(host(q), oracle.quant_static(xf, S, s, fcode))


# ------------------------------------------------------------------ streams, graphs, determinism

def test_repeatable_bit_for_bit(pq):
    """Every kernel is deterministic: two runs give identical bits (no order-dependent float sums)."""
    x = dev(_x("det/x", 300, 4096, synth.BF16))
    w = dev(_w("det/w", 200, 4096, synth.BF16, 0.001))
    s = dev(np.exp(np.random.default_rng(7).uniform(-1, 1, 4096)).astype(np.float32))
    announce("repeatability: calib, ssz, ssz_asym, quant, static quant")
    r1 = (pq.sq_absmax_calib(x), pq.ssz_weight_qparams(w, s), pq.ssz_weight_qparams_asym(w, s),
          pq.quant_per_token_i8(x, s))
    r2 = (pq.sq_absmax_calib(x), pq.ssz_weight_qparams(w, s), pq.ssz_weight_qparams_asym(w, s),
          pq.quant_per_token_i8(x, s))
    flat = lambda r: [t for item in r for t in (item if isinstance(item, tuple) else (item,)) if t is not None]
    for a, b in zip(flat(r1), flat(r2)):
        assert torch.equal(a, b)


def test_side_stream_ordering(pq):
    """Work enqueued on a caller's stream runs in order on that stream and matches the default stream."""
    x = _x("strm/x", 257, 4096, synth.BF16)
    w = _w("strm/w", 384, 4096, synth.BF16)
    ref_S = oracle.ssz(synth.widen(w), None, 8)["S"]
    side = torch.cuda.Stream()
    announce("side stream: calib -> smooth -> ssz -> quant -> gemm")
    with torch.cuda.stream(side):
        xd, wd = dev(x), dev(w)
        ax = pq.sq_absmax_calib(xd, stream=side)
        aw = pq.sq_absmax_calib(wd, stream=side)
        sm = pq.sq_smooth_factors(ax, aw, 0.5, stream=side)
        S, wq, _, _ = pq.ssz_weight_qparams(wd, None, stream=side)
        xq, d = pq.quant_per_token_i8(xd, sm, stream=side)
        y = pq.w8a8_gemm_dequant(xq, wq, d, S, stream=side)
    side.synchronize()
    np.testing.assert_array_equal(host(S), ref_S)
    y0 = pq.w8a8_gemm_dequant(xq, wq, d, S)
    assert torch.equal(y, y0)


def test_graph_replay_matches_eager(pq):
    """The whole path captured once in a HIP graph and replayed several times, with eager work and
    synchronisation between replays; every replay equals the eager result (the path clears its own
    outputs with fill kernels, no memset nodes)."""
    x = dev(_x("graph/x", 512, 4096, synth.BF16))
    w = dev(_w("graph/w", 1024, 4096, synth.BF16, 0.001))
    ax = torch.empty(4096, dtype=torch.float32, device="cuda:0")
    aw = torch.empty_like(ax)
    s = torch.empty_like(ax)
    S = torch.empty(1024, dtype=torch.float32, device="cuda:0")
    wq = torch.empty((1024, 4096), dtype=torch.int8, device="cuda:0")
    xq = torch.empty((512, 4096), dtype=torch.int8, device="cuda:0")
    d = torch.empty(512, dtype=torch.float32, device="cuda:0")
    y = torch.empty((512, 1024), dtype=torch.float32, device="cuda:0")

    def path(stream):
        pq.sq_absmax_calib(x, ax, stream=stream)
        pq.sq_absmax_calib(w, aw, stream=stream)
        pq.sq_smooth_factors(ax, aw, 0.5, s=s, stream=stream)
        pq.ssz_weight_qparams(w, s, scale=S, wq=wq, want_stats=False, stream=stream)
        pq.quant_per_token_i8(x, s, xq=xq, tok_scale=d, stream=stream)
        pq.w8a8_gemm_fused(xq, wq, d, S, act="relu", out="f32", y=y, stream=stream)

    announce("graph: eager reference")
    path(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        path(cap)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    announce("graph: capture")
    with torch.cuda.graph(g, stream=cap):
        path(cap)
    for r in range(4):
        for t in (ax, aw, s, S, wq, xq, d, y):
            t.fill_(7)  # eager work between replays
        torch.cuda.synchronize()
        announce(f"graph: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {r}"


# ------------------------------------------------------------------ quotient domain edges and deferred rows
# The kernels take fl32(R / S) as a corrected product with the IEEE reciprocal where that is proven equal to
# the IEEE quotient, and the IEEE division elsewhere; SSZ rows they cannot certify go to the exact search.
# These cases drive every such path against the oracle.

def _scaled_rows(rng, N, K, scales):
    """fp32 rows ~N(0, 0.02) times a per-row scale taken in turn from `scales`."""
    w = rng.standard_normal((N, K)) * 0.02
    return (w * np.resize(np.asarray(scales, np.float64), N)[:, None]).astype(np.float32)


@pytest.mark.parametrize("K", [64, 320, 1024, 2048, 4096, 8192, 16384])
@pytest.mark.parametrize("bits", [8, 4])
def test_ssz_deferred_scales(pq, K, bits):
    """Rows whose scale leaves [2^-100, 2^100] (tiny rows under a tiny floor, huge rows) mixed with ordinary
    rows: those rows are searched again exactly, the others keep the fast path; every row as the oracle.  K spans
    the short-row kernel (64, 320), the row kernels that search such rows themselves (1024 to 8192: one, two and
    four chunks per lane, one and two waves per row) and one that leaves them to the separate exact launch
    (16384)."""
    rng = np.random.default_rng(K + bits)
    w = _scaled_rows(rng, 96, K, [1.0, 1e-33, 3.0, 1e32, 0.5])
    w[7] = 0.0
    ref = oracle.ssz(w, None, bits, min_scale=1e-38)
    announce(f"ssz_weight_qparams deferred scales K={K} int{bits}")
    S, wq, it, mse = pq.ssz_weight_qparams(dev(w), None, bits=bits, min_scale=1e-38)
    codes = host(wq) if bits == 8 else unpack_int4(host(wq))
    compare_ssz(host(S), codes, host(it), host(mse), ref, f"deferred scales K={K} int{bits}")


@pytest.mark.parametrize("K", [1024, 4096])
def test_ssz_asym_deferred_scales(pq, K):
    rng = np.random.default_rng(K + 1)
    w = _scaled_rows(rng, 64, K, [1.0, 1e-33, 1e32, 2.0])
    w[::5] += np.float32(0.01)
    ref = oracle.ssz_asym(w, None, min_scale=1e-38)
    announce(f"ssz_weight_qparams_asym deferred scales K={K}")
    S, Z, wq, it, mse = pq.ssz_weight_qparams_asym(dev(w), None, min_scale=1e-38)
    compare_ssz_asym(host(S), host(Z), host(wq), host(it), host(mse), ref, f"asym deferred scales K={K}")


@pytest.mark.parametrize("K", [32768, 65536])
def test_ssz_deferred_wide_uniform_rows(pq, K):
    """Uniform rows this wide have sum w q past the exactness certificate of a pass (large codes everywhere):
    they are searched again with double-double sums.  Gaussian rows of the same width stay on the fast path."""
    rng = np.random.default_rng(K)
    w = rng.uniform(-1.0, 1.0, (12, K)).astype(np.float32)
    w[::3] = (rng.standard_normal((4, K)) * 0.02).astype(np.float32)
    for bits in (8, 4):
        ref = oracle.ssz(w, None, bits)
        announce(f"ssz_weight_qparams wide uniform rows K={K} int{bits}")
        S, wq, it, mse = pq.ssz_weight_qparams(dev(w), None, bits=bits)
        codes = host(wq) if bits == 8 else unpack_int4(host(wq))
        compare_ssz(host(S), codes, host(it), host(mse), ref, f"wide uniform K={K} int{bits}")
    ra = oracle.ssz_asym(w, None)
    announce(f"ssz_weight_qparams_asym wide uniform rows K={K}")
    Sa, Za, qa, ita, ma = pq.ssz_weight_qparams_asym(dev(w), None)
    compare_ssz_asym(host(Sa), host(Za), host(qa), host(ita), host(ma), ra, f"asym wide uniform K={K}")


def _near_grid_rows(rng, N, K, qmax, noise, asym=False):
    """Rows fl32(S (q + noise u)) on a random grid S (not a power of two) with integer codes q that reach the end
    of the range: the least-squares refit of the MinMax scale lands on the same codes, often one or two ulps
    away, so the candidate's pass sums equal the kept ones and the two errors differ by ~1e-11 relative or
    less.  asym: codes over [-128, 127] with a random offset."""
    S = rng.uniform(0.003, 0.03, N)
    lo, hi = (-128, 127) if asym else (-qmax, qmax)
    q = rng.integers(lo, hi + 1, (N, K)).astype(np.float64)
    q[:, 0] = hi
    q[:, 1] = lo
    if asym:
        q -= rng.integers(-40, 41, (N, 1))
    u = rng.uniform(-1.0, 1.0, (N, K))
    return (S[:, None] * (q + noise * u)).astype(np.float32)


def _same_sums_rows(w, qmax, min_scale=1e-5):
    """Rows whose first refit keeps the MinMax codes under a different scale (oracle helpers only)."""
    n = 0
    for row in w:
        S0 = max(np.float32(np.max(np.abs(row)) / np.float32(qmax)), np.float32(min_scale))
        q0 = oracle.quant_row(row, S0, qmax)
        S1 = max(np.float32(oracle.lsq_scale(row, q0)), np.float32(min_scale))
        n += int(S1 != S0 and np.array_equal(oracle.quant_row(row, S1, qmax), q0))
    return n


@pytest.mark.parametrize("K", [48, 320, 1024, 4096, 16384])
@pytest.mark.parametrize("bits", [8, 4])
def test_ssz_same_codes_candidates(pq, K, bits):
    """Candidates with the kept codes under a neighbouring scale: the two errors share one quadratic, and the
    decision between them is taken from its exact difference (on every row as the oracle decides it)."""
    qmax = 127 if bits == 8 else 7
    rng = np.random.default_rng(K * 5 + bits)
    N = 96
    w = np.concatenate([_near_grid_rows(rng, N // 4, K, qmax, noise) for noise in (0.0, 1e-6, 1e-4, 1e-2)])
    assert _same_sums_rows(w, qmax) >= N // 4, "the rows do not exercise same-codes candidates"
    s = np.exp(rng.uniform(-0.5, 0.5, K)).astype(np.float32)
    for smooth in (False, True):
        # smoothing: the folded rows fl32(w s) sit on the grid again (the division by s undone)
        wi = (w / s).astype(np.float32) if smooth else w
        ref = oracle.ssz(wi, s if smooth else None, bits)
        announce(f"ssz_weight_qparams same-codes candidates K={K} int{bits} smooth={smooth}")
        S, wq, it, mse = pq.ssz_weight_qparams(dev(wi), dev(s) if smooth else None, bits=bits)
        codes = host(wq) if bits == 8 else unpack_int4(host(wq))
        compare_ssz(host(S), codes, host(it), host(mse), ref, f"same codes K={K} int{bits} smooth={smooth}")


@pytest.mark.parametrize("K", [64, 1024, 4096])
def test_ssz_asym_same_codes_candidates(pq, K):
    rng = np.random.default_rng(K * 7)
    w = np.concatenate([_near_grid_rows(rng, 16, K, 127, noise, asym=True) for noise in (0.0, 1e-6, 1e-4)])
    ref = oracle.ssz_asym(w, None)
    announce(f"ssz_weight_qparams_asym same-codes candidates K={K}")
    S, Z, wq, it, mse = pq.ssz_weight_qparams_asym(dev(w), None)
    compare_ssz_asym(host(S), host(Z), host(wq), host(it), host(mse), ref, f"asym same codes K={K}")


def _hash3(seed, a, b):
    """The probes' operand hash, on the host (uint32 arithmetic)."""
    m = 0xFFFFFFFF
    h = ((seed * 0x9E3779B9) & m) ^ ((a * 0x85EBCA6B + b * 0xC2B2AE35 + 0x27D4EB2F) & m)
    h ^= h >> 15
    h = (h * 0x2C1B3C6D) & m
    h ^= h >> 12
    h = (h * 0x297A2D39) & m
    h ^= h >> 15
    return h - (1 << 32) if h & 0x80000000 else h


def test_valu_probe_runs_the_search_loop(pq):
    """The VALU probe's SSZ-loop kind computes what it claims: lane 0 of each block returns P + R2 summed over the
    iterations, P = sum w q (exact in fp64), R2 = sum q^2, q = clamp(rint(fl32(w / s))) -- recomputed here with
    numpy's fp32 division.  The other kinds run and report plausible rates."""
    seed, iters, blocks = 7, 5, 3
    r = pq.probe_valu("ssz_loop", blocks=blocks, iters=iters, seed=seed)
    out = torch.zeros(3 * blocks, dtype=torch.int64, device="cuda")
    assert pq.lib.ptq_probe_valu(0, blocks, iters, seed, out.data_ptr(), None) == 0
    torch.cuda.synchronize()
    got = out.view(blocks, 3)[:, 2].cpu().numpy().view(np.float64)
    s0 = np.float32(np.float32(0.125) / np.float32(127.0))
    s1 = np.float32(s0 * np.float32(1.0009765625))
    for b in range(blocks):
        t = b * 64
        w = np.array([np.float32(np.float32(_hash3(seed, t, i) >> 8) * np.float32(2.0 ** -26)) for i in range(64)],
                     dtype=np.float32)
        P, R2 = 0.0, np.float32(0.0)
        for it in range(iters):
            q = np.clip(np.rint(w / (s1 if it & 1 else s0)), -127, 127).astype(np.float32)
            P += float(np.sum(w.astype(np.float64) * q.astype(np.float64)))
            R2 = np.float32(R2 + np.float32(np.sum(q.astype(np.float64) ** 2)))
        assert got[b] == P + float(R2), (b, got[b], P + float(R2))
    assert r["lane_ops_per_s"] > 0 and r["clock_GHz"] > 0.5
    for kind in ("ssz_loop_reduce", "fma_f32", "fma_f64"):
        announce(f"probe_valu {kind}")
        q = pq.probe_valu(kind, blocks=2048, iters=200)  # two waves per SIMD: every SIMD busy
        assert q["lane_ops_per_s"] > 0 and 1.0 < q["simd_cycles_per_wave_op"] < 64.0, q


def test_stream_probe_reads_and_copies_every_byte(pq):
    """The HBM stream probe behind the bench's measured peak touches every byte: a copy reproduces the buffer,
    and a read's combined xor is the xor of every 32-bit word (whole rounds of 64 KB over two blocks plus a
    tail)."""
    n16 = 3 * 256 * 16 + 5
    g = torch.Generator(device="cuda:0").manual_seed(3)
    src = torch.randint(0, 256, (16 * n16,), dtype=torch.uint8, device="cuda:0", generator=g)
    dst = torch.zeros_like(src)
    announce("probe_stream copy and read")
    pq.probe_stream("copy", src, dst, blocks=2)
    assert torch.equal(dst, src)
    r = pq.probe_stream("read", src, blocks=2)
    assert r["xor"] == int(np.bitwise_xor.reduce(host(src).view(np.uint32)))
    assert r["bytes"] == src.numel()


@pytest.mark.parametrize("T,K", [(40, 64), (33, 1040), (24, 4096), (9, 16384)])
@pytest.mark.parametrize("smooth", ["none", "ok", "tiny_s"])
def test_quant_per_token_domain_edges(pq, T, K, smooth):
    """Per-token quantization of rows the corrected quotient does not cover -- all-zero, tiny (max under 2^-60),
    subnormal and huge rows, subnormal elements inside ordinary rows -- and smoothing factors below 2^-20, which
    send the whole launch to the IEEE division: codes and token scales bit for bit."""
    rng = np.random.default_rng(T * K + len(smooth))
    x = _scaled_rows(rng, T, K, [1.0, 1e-25, 1e-38 / 0.02, 1e25, 7.0, 1e-15])
    x[3] = 0.0
    x[4, ::7] = np.float32(1e-40)  # subnormal elements in an ordinary row
    s = None
    if smooth != "none":
        s = np.exp(rng.uniform(-3, 3, K)).astype(np.float32)
        if smooth == "tiny_s":
            s[K // 3] = np.float32(1e-7)
    xq_ref, d_ref = oracle.quant_per_token(x, s)
    announce(f"quant_per_token_i8 domain edges T={T} K={K} smooth={smooth}")
    xq, d = pq.quant_per_token_i8(dev(x), None if s is None else dev(s))
    np.testing.assert_array_equal(host(d), d_ref)
    np.testing.assert_array_equal(host(xq), xq_ref)


@pytest.mark.parametrize("scale", [1e-25, 3e-3, 1e35])
@pytest.mark.parametrize("fold", ["div", "mul"])
def test_quant_static_domain_edges(pq, scale, fold):
    rng = np.random.default_rng(int(scale > 1) + 2 * len(fold))
    x = _scaled_rows(rng, 21, 1040, [1.0, 1e-30, 1e30])
    s = np.exp(rng.uniform(-2, 2, 1040)).astype(np.float32)
    S = np.float32(scale)
    ref = oracle.quant_static(x, S, s, oracle.FOLD_DIV if fold == "div" else oracle.FOLD_MUL)
    announce(f"quant_static_i8 domain edges scale={scale} fold={fold}")
    q, _ = pq.quant_static_i8(dev(x), dev(np.array([S], np.float32)), dev(s), fold)
    np.testing.assert_array_equal(host(q), ref)


@pytest.mark.parametrize("M,N,K", [(16, 300, 512), (300, 520, 1040), (1024, 1024, 256)])
@pytest.mark.parametrize("edge", ["tiny_next_s", "tiny_out_scale", "huge_out_scale"])
def test_gemm_int8_output_domain_edges(pq, M, N, K, edge):
    """The int8 output's quotients with a next-layer factor below 2^-20 or a static scale outside
    [2^-60, 2^100]: those tiles take the IEEE division; codes bit for bit."""
    rng = np.random.default_rng(M + N + K + len(edge))
    a = rng.integers(-127, 128, (M, K)).astype(np.int8)
    b = rng.integers(-127, 128, (N, K)).astype(np.int8)
    ts = rng.uniform(0.002, 0.02, M).astype(np.float32)
    cs = rng.uniform(1e-4, 1e-3, N).astype(np.float32)
    ns = np.exp(rng.uniform(-1, 1, N)).astype(np.float32)
    acc_ref = oracle.gemm_i8(a, b)
    y32 = oracle.epilogue(acc_ref, ts, cs, None, oracle.ACT_NONE)
    osc = np.float32(np.max(np.abs(y32)) / 100.0)
    if edge == "tiny_next_s":
        ns[N // 2] = np.float32(3e-7)
    elif edge == "tiny_out_scale":
        osc, y32 = np.float32(1e-20), None
        ns *= np.float32(1e18)
    else:
        # a static scale of 1e35 with next-layer factors small enough that the codes still span the range
        ns *= np.float32(float(osc) / 1e35)
        osc = np.float32(1e35)
    ref = oracle.epilogue(acc_ref, ts, cs, None, oracle.ACT_NONE, oracle.OUT_I8, ns, osc)
    announce(f"w8a8_gemm_fused int8 output domain edge {edge} M={M} N={N} K={K}")
    y = pq.w8a8_gemm_fused(dev(a), dev(b), dev(ts), dev(cs), None, "none", "i8", dev(ns),
                           dev(np.array([osc], np.float32)))
    np.testing.assert_array_equal(host(y), ref)
    assert np.unique(ref).size > 50, "the case should exercise many codes"
