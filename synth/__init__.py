"""Seeded synthetic inputs for the W8A8 quantized-linear path.

This module draws tensors and nothing else: it holds none of the
quantization arithmetic.  Tests, the oracle checks and the bench all take
their inputs from here, so the GPU path and the CPU oracle see the same bits.

The shapes and value structure stand in for the workloads the pages talk
about (GPT-345M with hidden 1024; an OPT-6.7B-sized layer with hidden 4096,
32 layers; a decode step), whose checkpoints and datasets are not used:

* activations ~ N(0,1) with a fixed set of outlier channels multiplied by a
  factor (the activation outliers the SmoothQuant article describes; the same
  channels in every calibration batch of a layer, since such outliers are
  channel-persistent);
* weights ~ N(0, sigma) with a per-row log-uniform scale (rows of very
  different range: the per-layer vs per-channel example of the PTQ tutorial),
  optionally with rare heavy-tail entries (the uneven weight distributions the
  SSZ document targets).

Random stream: SplitMix64, counter based (see synth.c).  Seeds are derived from
a tensor name with 64-bit FNV-1a, so each tensor is reproducible on its own.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

F32, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile libsynth.so in place (gcc, OpenMP)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.synth_u64.argtypes = [u64, u64, i64, vp]
        lib.synth_uniform.argtypes = [u64, u64, i64, vp]
        lib.synth_fill.argtypes = [u64, i64, i64, dbl, vp, vp, u64, dbl, dbl, ctypes.c_int, vp]
        _lib = lib
    return _lib


def seed_of(name: str) -> int:
    """64-bit FNV-1a hash of a tensor name: the seed of that tensor's stream."""
    h = 0xCBF29CE484222325
    for b in name.encode():
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def u64_stream(seed: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_u64(seed, first, n, out.ctypes.data)
    return out


def uniform_stream(seed: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniform(seed, first, n, out.ctypes.data)
    return out


def pick_channels(name: str, K: int, count: int) -> np.ndarray:
    """`count` distinct channels of K by a seeded partial Fisher-Yates shuffle."""
    count = int(count)
    if count <= 0:
        return np.zeros(0, dtype=np.int64)
    r = u64_stream(seed_of(name + "/channels"), count)
    perm = np.arange(K, dtype=np.int64)
    for i in range(count):
        j = i + int(r[i] % np.uint64(K - i))
        perm[i], perm[j] = perm[j], perm[i]
    return np.sort(perm[:count])


def log_uniform_rows(name: str, rows: int, lo: float, hi: float) -> np.ndarray:
    """Per-row scale exp(ln lo + u (ln hi - ln lo)), u uniform in (0,1)."""
    u = uniform_stream(seed_of(name + "/rowscale"), rows)
    return np.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))


def tensor(name: str, rows: int, cols: int, std: float, dtype: int, row_scale=None, col_mult=None,
           tail_p: float = 0.0, tail_mult: float = 1.0) -> np.ndarray:
    """Draw a row-major [rows, cols] tensor; float32 array, or uint16 bf16 bits."""
    lib = _load()
    out = np.empty((rows, cols), dtype=np.float32 if dtype == F32 else np.uint16)
    rs = None if row_scale is None else np.ascontiguousarray(row_scale, dtype=np.float64)
    cm = None if col_mult is None else np.ascontiguousarray(col_mult, dtype=np.float64)
    lib.synth_fill(seed_of(name), rows, cols, float(std),
                   None if rs is None else rs.ctypes.data, None if cm is None else cm.ctypes.data,
                   seed_of(name + "/tail"), float(tail_p), float(tail_mult), dtype, out.ctypes.data)
    return out


def widen(a: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) -> float32 (exact); float32 passes through."""
    if a.dtype == np.float32:
        return a
    assert a.dtype == np.uint16
    return (a.astype(np.uint32) << 16).view(np.float32)


def activation(name: str, T: int, K: int, dtype: int, outlier_channels, factor: float) -> np.ndarray:
    """X ~ N(0,1) [T,K] with the given channels multiplied by `factor`."""
    cm = np.ones(K, dtype=np.float64)
    cm[np.asarray(outlier_channels, dtype=np.int64)] = factor
    return tensor(name, T, K, 1.0, dtype, col_mult=cm)


def weight(name: str, N: int, K: int, dtype: int, std: float, lo: float, hi: float,
           tail_p: float = 0.0, tail_mult: float = 1.0) -> np.ndarray:
    """W ~ N(0,std) [N,K], row n scaled by a log-uniform[lo,hi] factor, optional heavy tail."""
    return tensor(name, N, K, std, dtype, row_scale=log_uniform_rows(name, N, lo, hi),
                  tail_p=tail_p, tail_mult=tail_mult)


from .configs import CONFIGS, LinearCase, cases  # noqa: E402,F401
