"""Helpers for the GPU parity tests: moving seeded inputs to the device, sampling
rows of large outputs, and the comparisons the tests share.

The expected values always come from the oracle run on the same seeded host
inputs; nothing computed on the GPU is ever fed to the oracle.
"""
import numpy as np
import torch

DEV = "cuda:0"

# tolerances the checks use (floating point); integer outputs are compared exactly
SCALE_RTOL = 1e-6     # smoothing factors and scales
Y_TOL = 1e-3          # max |y_gpu - y_ref| / max |y_ref|
MSE_RTOL = 1e-9       # fp64 quantization error, summed in a different order


# line writer to the real terminal, installed by the test session (conftest): test modules import this
# module by name, but pytest loads conftest under its own module object, so it hands its writer over
_SAY = None


def set_writer(fn):
    global _SAY
    _SAY = fn


def announce(msg: str):
    """Name the case on the terminal before a GPU step (bypasses pytest capture, so the line is on record
    even if the process dies during the step)."""
    line = f"[gpu-case] {msg}"
    if _SAY is not None:
        _SAY(line)
    else:
        print(line, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    """Host array -> device tensor; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def sample_rows(n: int, k: int, seed: int) -> np.ndarray:
    """k distinct sorted row indices of n, always including the first and the last row."""
    if k >= n:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    pick = rng.choice(np.arange(1, n - 1), size=k - 2, replace=False)
    return np.sort(np.concatenate([[0, n - 1], pick]))


def unpack_int4(p: np.ndarray) -> np.ndarray:
    """[N, K/2] bytes -> [N, K] codes (low nibble first, two's complement)."""
    p = p.astype(np.uint8)
    lo = (p & 0xF).astype(np.int8)
    hi = (p >> 4).astype(np.int8)
    lo = np.where(lo > 7, lo - 16, lo)
    hi = np.where(hi > 7, hi - 16, hi)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def assert_scales(got, want, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    rel = np.abs(got - want) / np.maximum(np.abs(want), 1e-30)
    assert np.max(rel) <= SCALE_RTOL, f"{what}: max rel err {np.max(rel):.3e} at {int(np.argmax(rel))}"


def assert_y(y_gpu, y_ref, what):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    den = np.max(np.abs(y_ref))
    err = np.max(np.abs(y_gpu - y_ref)) / (den if den > 0 else 1.0)
    assert err <= Y_TOL, f"{what}: normalised max error {err:.3e}"
    return err


def compare_ssz(g_scale, g_codes, g_iters, g_mse, ref, what):
    """SSZ parity: scales, iteration counts and codes identical on every row; reported errors within 1e-9
    (the GPU's final error is an fp64 sum in another order)."""
    S_ref = ref["S"]
    diff = np.nonzero(g_scale != S_ref)[0]
    assert diff.size == 0, f"{what}: {diff.size} rows with a different scale, first {diff[:10]}"
    if g_iters is not None:
        bad = np.nonzero(g_iters != ref["iters"])[0]
        assert bad.size == 0, f"{what}: iteration counts differ on rows {bad[:10]}"
    if g_codes is not None:
        np.testing.assert_array_equal(g_codes, ref["q"], err_msg=what + " codes")
    if g_mse is not None:
        rel = np.abs(g_mse - ref["mse"]) / np.maximum(ref["mse"], 1e-300)
        rel[ref["mse"] == 0] = np.abs(g_mse[ref["mse"] == 0])
        assert np.max(rel) <= MSE_RTOL, f"{what}: mse rel err {np.max(rel):.3e}"


def compare_ssz_asym(g_scale, g_zp, g_codes, g_iters, g_mse, ref, what):
    """Asymmetric SSZ parity: as compare_ssz, plus zero points identical on every row."""
    diff = np.nonzero((g_scale != ref["S"]) | (g_zp != ref["Z"]))[0]
    assert diff.size == 0, f"{what}: {diff.size} rows with a different scale or zero point, first {diff[:10]}"
    if g_iters is not None:
        bad = np.nonzero(g_iters != ref["iters"])[0]
        assert bad.size == 0, f"{what}: iteration counts differ on rows {bad[:10]}"
    if g_codes is not None:
        np.testing.assert_array_equal(g_codes, ref["q"], err_msg=what + " codes")
    if g_mse is not None:
        rel = np.abs(g_mse - ref["mse"]) / np.maximum(ref["mse"], 1e-300)
        rel[ref["mse"] == 0] = np.abs(g_mse[ref["mse"] == 0])
        assert np.max(rel) <= MSE_RTOL, f"{what}: mse rel err {np.max(rel):.3e}"
