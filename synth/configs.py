"""The five synthetic workloads of the quantized-linear path.

Each workload is a list of linear layers ("cases").  A case names its token
count T, input width K, output width N, storage dtype, the activation outlier
structure, the weight distribution, the number of calibration batches and the
smoothing strengths alpha to run.

* tiny       : X fp32 [16,64], channels 3 and 41 x50; W fp32 [128,64] ~N(0,0.02)
               x per-row logU[0.1,1]; alpha 0.5; one batch serves calibration and
               the forward.
* gpt345m    : hidden 1024 (GPT-345M shapes); X bf16 [2048,K] with 1% channels x40;
               QKV [3072,1024], out [1024,1024], fc1 [4096,1024], fc2 [1024,4096];
               alpha 0.5; 8 calibration batches.
* decode     : X bf16 [16,8192] with 0.5% channels x60; W [28672,8192] ~N(0,0.015)
               x logU[0.05,1]; alpha 0.5; 8 calibration batches.
* opt67b     : hidden 4096 (OPT-6.7B shapes, 32 layers on the PaddleNLP 6.7B
               config); X bf16 [4096,4096] and fc2 input [4096,16384], 1% channels
               x60; fc1 W [16384,4096], fc2 W [4096,16384]; alpha 0.5 and 0.8;
               8 calibration batches.
* ssz_scale  : weight quantization only, 32 layers x {QKV [12288,4096], out
               [4096,4096], fc1 [16384,4096], fc2 [4096,16384]} ~N(0,0.02) x
               logU[0.05,1] with 0.1% heavy-tail entries x20; no smoothing;
               int8 and int4.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import BF16, F32, activation, pick_channels, weight


@dataclass(frozen=True)
class LinearCase:
    name: str
    T: int
    K: int
    N: int
    dtype: int
    x_factor: float = 1.0
    x_outlier_frac: float = 0.0
    x_fixed_channels: tuple = ()
    w_std: float = 0.02
    w_lo: float = 0.1
    w_hi: float = 1.0
    w_tail_p: float = 0.0
    w_tail_mult: float = 1.0
    calib_batches: int = 8
    alphas: tuple = (0.5,)
    smooth: bool = True
    bits: tuple = (8,)
    shared_calib_eval: bool = False
    has_activations: bool = True

    def x_channels(self) -> np.ndarray:
        if self.x_fixed_channels:
            return np.asarray(self.x_fixed_channels, dtype=np.int64)
        return pick_channels(self.name + "/X", self.K, round(self.x_outlier_frac * self.K))

    def x_batch(self, b: int, T: int | None = None) -> np.ndarray:
        """Calibration batch b (b < calib_batches) or the forward batch (b = calib_batches)."""
        if self.shared_calib_eval:
            b = 0
        return activation(f"{self.name}/X/b{b}", self.T if T is None else T, self.K, self.dtype,
                          self.x_channels(), self.x_factor)

    def eval_index(self) -> int:
        return 0 if self.shared_calib_eval else self.calib_batches

    def w(self) -> np.ndarray:
        return weight(f"{self.name}/W", self.N, self.K, self.dtype, self.w_std, self.w_lo, self.w_hi,
                      self.w_tail_p, self.w_tail_mult)


def _tiny():
    return [LinearCase("tiny/lin", 16, 64, 128, F32, x_factor=50.0, x_fixed_channels=(3, 41),
                       calib_batches=1, shared_calib_eval=True)]


def _gpt345m():
    common = dict(T=2048, dtype=BF16, x_factor=40.0, x_outlier_frac=0.01, w_std=0.02, w_lo=0.1, w_hi=1.0)
    return [LinearCase("gpt345m/qkv", K=1024, N=3072, **common),
            LinearCase("gpt345m/out", K=1024, N=1024, **common),
            LinearCase("gpt345m/fc1", K=1024, N=4096, **common),
            LinearCase("gpt345m/fc2", K=4096, N=1024, **common)]


def _decode():
    return [LinearCase("decode/mlp", T=16, K=8192, N=28672, dtype=BF16, x_factor=60.0, x_outlier_frac=0.005,
                       w_std=0.015, w_lo=0.05, w_hi=1.0)]


def _opt67b():
    common = dict(T=4096, dtype=BF16, x_factor=60.0, x_outlier_frac=0.01, w_std=0.02, w_lo=0.1, w_hi=1.0,
                  alphas=(0.5, 0.8))
    return [LinearCase("opt67b/fc1", K=4096, N=16384, **common),
            LinearCase("opt67b/fc2", K=16384, N=4096, **common)]


SSZ_SHAPES = (("qkv", 12288, 4096), ("out", 4096, 4096), ("fc1", 16384, 4096), ("fc2", 4096, 16384))


def _ssz_scale(layers: int = 32):
    out = []
    for layer in range(layers):
        for nm, N, K in SSZ_SHAPES:
            out.append(LinearCase(f"ssz_scale/L{layer}/{nm}", T=0, K=K, N=N, dtype=BF16, w_std=0.02, w_lo=0.05,
                                  w_hi=1.0, w_tail_p=0.001, w_tail_mult=20.0, smooth=False, bits=(8, 4),
                                  calib_batches=0, has_activations=False))
    return out


CONFIGS = {"tiny": _tiny, "gpt345m": _gpt345m, "decode": _decode, "opt67b": _opt67b, "ssz_scale": _ssz_scale}


def cases(config: str):
    return CONFIGS[config]()
