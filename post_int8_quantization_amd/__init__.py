"""Python binding of libptq, the gfx950 W8A8 post-training-quantized linear layer.

Argument marshalling only: every step runs in the HIP kernels of libptq.so,
called through its C ABI (include/ptq.h) with ctypes.  PyTorch supplies
device memory and the current stream.  There is no CPU fallback: importing
this module fails if libptq.so is missing, and each call raises PtqError on a
non-OK status.

Entry points (same names as the C ABI):
  sq_absmax_calib(x, amax=None, accumulate=False) -> amax[K] fp32
  sq_smooth_factors(act_amax, w_amax, alpha) -> s[K] fp32
  ssz_weight_qparams(w, s=None, bits=8, ...) -> (scale[N], wq, iters[N], mse[N])
  quant_per_token_i8(x, s=None) -> (xq[T,K] int8, tok_scale[T] fp32)
  w8a8_gemm_dequant(xq, wq, tok_scale, ch_scale, want_acc=False) -> y[M,N] fp32 (, acc int32)
  w8a8_gemm_fused(xq, wq, tok_scale, ch_scale, bias=None, act="none", out="f32", next_s=None,
                  out_scale=None) -> out[M,N] fp32 / bf16 / int8
  sq_act_scale_ema(col_amax, s=None, momentum=0.9, first=False, state=None, rows=0) -> (state, scale, row_scale)
  weight_scale_per_tensor(col_amax, s=None, min_scale=1e-5, n=0) -> (scale[1], ch_scale[n] or None)
  quant_static_i8(x, scale, s=None, fold="div") -> (q int8, row_scale)

Measurement aid (include/ptq_probe.h, not a step of the method):
  probe_mfma(kind, blocks=256, iters=2000, seed=1) -> dict with the loop's shader clock and int8 throughput
  probe_valu(kind, blocks=2048, iters=2000, seed=1) -> dict with the VALU loop's clock and lane-operation rate
  probe_stream(kind, src, dst=None, blocks=1024) -> dict with the bytes read (or copied) per second
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libptq.so")

PTQ_F32, PTQ_BF16 = 0, 1
SSZ_MAX_ITER = 20
SSZ_THRESHOLD = 1e-10
SSZ_MIN_SCALE = 1e-5
GEMM_MAX_K = 131056

STATUS = {0: "PTQ_OK", 1: "PTQ_ERR_NULL", 2: "PTQ_ERR_SHAPE", 3: "PTQ_ERR_DTYPE", 4: "PTQ_ERR_UNSUPPORTED",
          5: "PTQ_ERR_ARG", 6: "PTQ_ERR_ALIGN", 7: "PTQ_ERR_HIP"}

EXPORTS = ("ptq_abi_version", "ptq_last_error", "ptq_status_string", "sq_absmax_calib", "sq_smooth_factors",
           "ssz_weight_qparams", "ssz_weight_qparams_asym", "quant_per_token_i8", "w8a8_gemm_dequant",
           "w8a8_gemm_fused", "sq_act_scale_ema", "weight_scale_per_tensor", "quant_static_i8", "ptq_probe_mfma",
           "ptq_probe_stream", "ptq_probe_valu",
           "ptq_probe_last_error")

PROBE_KINDS = {"mfma16_random": 0, "mfma32_random": 1, "mfma16_lds_random": 2, "mfma16_zero": 3}
STREAM_KINDS = {"read": 0, "copy": 1}
VALU_KINDS = {"ssz_loop": 0, "ssz_loop_reduce": 1, "fma_f32": 2, "fma_f64": 3}
VALU_ELEMS_PER_ITER = 64   # kinds 0, 1: element-passes per lane and iteration
VALU_FMAS_PER_ITER = 128   # kinds 2, 3: multiply-adds per lane and iteration
PROBE_MACS_PER_BLOCK_ITER = 8 * 64 * 16 * 16 * 64


class PtqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libptq.so not built at {LIB_PATH}; run `python post_int8_quantization_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, ci, f32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
    lib.ptq_abi_version.restype = ci
    lib.ptq_abi_version.argtypes = []
    lib.ptq_last_error.restype = ctypes.c_char_p
    lib.ptq_last_error.argtypes = []
    lib.ptq_status_string.restype = ctypes.c_char_p
    lib.ptq_status_string.argtypes = [ci]
    lib.sq_absmax_calib.argtypes = [vp, ci, i64, i64, vp, ci, vp]
    lib.sq_smooth_factors.argtypes = [vp, vp, i64, f32, vp, vp]
    lib.ssz_weight_qparams.argtypes = [vp, ci, i64, i64, vp, ci, ci, ci, f64, f32, vp, vp, vp, vp, vp]
    lib.ssz_weight_qparams_asym.argtypes = [vp, ci, i64, i64, vp, ci, f64, f32, vp, vp, vp, vp, vp, vp]
    lib.quant_per_token_i8.argtypes = [vp, ci, i64, i64, vp, vp, vp, vp]
    lib.w8a8_gemm_dequant.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, vp]
    lib.w8a8_gemm_fused.argtypes = [vp, vp, vp, vp, vp, ci, ci, vp, vp, i64, i64, i64, vp, vp, vp]
    lib.sq_act_scale_ema.argtypes = [vp, vp, i64, f32, ci, vp, vp, vp, i64, vp]
    lib.weight_scale_per_tensor.argtypes = [vp, vp, i64, f32, vp, vp, i64, vp]
    lib.quant_static_i8.argtypes = [vp, ci, i64, i64, vp, ci, vp, vp, vp, vp]
    lib.ptq_probe_mfma.argtypes = [ci, ci, ci, ctypes.c_uint32, vp, vp]
    lib.ptq_probe_mfma.restype = ci
    lib.ptq_probe_valu.argtypes = [ci, ci, ci, ctypes.c_uint32, vp, vp]
    lib.ptq_probe_valu.restype = ci
    lib.ptq_probe_stream.argtypes = [ci, vp, ctypes.c_uint64, vp, ci, vp, vp]
    lib.ptq_probe_stream.restype = ci
    lib.ptq_probe_last_error.argtypes = []
    lib.ptq_probe_last_error.restype = ctypes.c_char_p
    for fn in ("sq_absmax_calib", "sq_smooth_factors", "ssz_weight_qparams", "ssz_weight_qparams_asym",
               "quant_per_token_i8", "w8a8_gemm_dequant", "w8a8_gemm_fused", "sq_act_scale_ema",
               "weight_scale_per_tensor", "quant_static_i8"):
        getattr(lib, fn).restype = ci
    return lib


lib = _load()


def _check(st: int):
    if st != 0:
        raise PtqError(st, lib.ptq_last_error().decode(errors="replace"))


# The current stream's raw handle without building a Stream object (a tenth of the host time of
# torch.cuda.current_stream(), which is most of a short call's overhead); the public route where torch lacks it.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_cur_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream(stream):
    if stream is None:
        if _raw_stream is not None and _cur_device is not None:
            return ctypes.c_void_p(_raw_stream(_cur_device()))
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtypes=None, numel=None, ndim=None, device=None):
    """Checks a tensor argument: type, dtype, dimensions, size, layout, and the device it shares with the call's
    other tensors.  The kernels read and write exactly these sizes, so a short buffer is an error here rather
    than an out-of-bounds access on the device."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _gpu(*ts):
    """Every tensor argument lives on the GPU (checked after all sizes and types)."""
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensor arguments must be GPU tensors")


def _opt(t, name, dtype, numel, device):
    """An optional argument (None passes through)."""
    return None if t is None else _dev(t, name, (dtype,), numel=numel, device=device)


def _dtype_code(t):
    return PTQ_BF16 if t.dtype == torch.bfloat16 else PTQ_F32


_FLOATS = (torch.float32, torch.bfloat16)


def sq_absmax_calib(x, amax=None, accumulate=False, stream=None):
    _dev(x, "x", _FLOATS, ndim=2)
    rows, cols = x.shape
    if amax is None:
        amax = torch.empty(cols, dtype=torch.float32, device=x.device)
        accumulate = False
    _dev(amax, "amax", (torch.float32,), numel=cols, device=x.device)
    _gpu(x, amax)
    _check(lib.sq_absmax_calib(_ptr(x), _dtype_code(x), rows, cols, _ptr(amax), int(bool(accumulate)),
                               _stream(stream)))
    return amax


def sq_smooth_factors(act_amax, w_amax, alpha, s=None, stream=None):
    _dev(act_amax, "act_amax", (torch.float32,))
    K = act_amax.numel()
    _dev(w_amax, "w_amax", (torch.float32,), numel=K, device=act_amax.device)
    if s is None:
        s = torch.empty(K, dtype=torch.float32, device=act_amax.device)
    _dev(s, "s", (torch.float32,), numel=K, device=act_amax.device)
    _gpu(act_amax, w_amax, s)
    _check(lib.sq_smooth_factors(_ptr(act_amax), _ptr(w_amax), K, float(alpha), _ptr(s), _stream(stream)))
    return s


def ssz_weight_qparams(w, s=None, bits=8, symmetric=True, max_iter=SSZ_MAX_ITER, threshold=SSZ_THRESHOLD,
                       min_scale=SSZ_MIN_SCALE, want_codes=True, want_stats=True, scale=None, wq=None, iters=None,
                       mse=None, stream=None):
    """Returns (scale[N] fp32, wq (int8 [N,K] or uint8 [N,K/2] for int4) or None, iters or None, mse or None).
    Output tensors may be passed in preallocated."""
    _dev(w, "w", _FLOATS, ndim=2)
    N, K = w.shape
    dev = w.device
    _opt(s, "s", torch.float32, K, dev)
    if scale is None:
        scale = torch.empty(N, dtype=torch.float32, device=dev)
    if wq is None and want_codes:
        wq = torch.empty((N, K), dtype=torch.int8, device=dev) if bits == 8 else \
            torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    if want_stats:
        iters = torch.empty(N, dtype=torch.int32, device=dev) if iters is None else iters
        mse = torch.empty(N, dtype=torch.float64, device=dev) if mse is None else mse
    _dev(scale, "scale", (torch.float32,), numel=N, device=dev)
    if wq is not None:
        _dev(wq, "wq", (torch.int8, torch.uint8), numel=N * K if bits == 8 else N * (K // 2), device=dev)
    _opt(iters, "iters", torch.int32, N, dev)
    _opt(mse, "mse", torch.float64, N, dev)
    _gpu(w, s, scale, wq, iters, mse)
    _check(lib.ssz_weight_qparams(_ptr(w), _dtype_code(w), N, K, _ptr(s), int(bits), int(bool(symmetric)),
                                  int(max_iter), float(threshold), float(min_scale), _ptr(scale), _ptr(wq),
                                  _ptr(iters), _ptr(mse), _stream(stream)))
    return scale, wq, iters, mse


def ssz_weight_qparams_asym(w, s=None, max_iter=SSZ_MAX_ITER, threshold=SSZ_THRESHOLD, min_scale=SSZ_MIN_SCALE,
                            want_codes=True, want_stats=True, scale=None, zero_point=None, wq=None, iters=None,
                            mse=None, stream=None):
    """Asymmetric int8.  Returns (scale[N] fp32, zero_point[N] int32, wq int8 [N,K] or None, iters or None,
    mse or None).  Output tensors may be passed in preallocated."""
    _dev(w, "w", _FLOATS, ndim=2)
    N, K = w.shape
    dev = w.device
    _opt(s, "s", torch.float32, K, dev)
    if scale is None:
        scale = torch.empty(N, dtype=torch.float32, device=dev)
    if zero_point is None:
        zero_point = torch.empty(N, dtype=torch.int32, device=dev)
    if wq is None and want_codes:
        wq = torch.empty((N, K), dtype=torch.int8, device=dev)
    if want_stats:
        iters = torch.empty(N, dtype=torch.int32, device=dev) if iters is None else iters
        mse = torch.empty(N, dtype=torch.float64, device=dev) if mse is None else mse
    _dev(scale, "scale", (torch.float32,), numel=N, device=dev)
    _dev(zero_point, "zero_point", (torch.int32,), numel=N, device=dev)
    _opt(wq, "wq", torch.int8, N * K, dev)
    _opt(iters, "iters", torch.int32, N, dev)
    _opt(mse, "mse", torch.float64, N, dev)
    _gpu(w, s, scale, zero_point, wq, iters, mse)
    _check(lib.ssz_weight_qparams_asym(_ptr(w), _dtype_code(w), N, K, _ptr(s), int(max_iter), float(threshold),
                                       float(min_scale), _ptr(scale), _ptr(zero_point), _ptr(wq), _ptr(iters),
                                       _ptr(mse), _stream(stream)))
    return scale, zero_point, wq, iters, mse


def quant_per_token_i8(x, s=None, xq=None, tok_scale=None, stream=None):
    _dev(x, "x", _FLOATS, ndim=2)
    T, K = x.shape
    _opt(s, "s", torch.float32, K, x.device)
    if xq is None:
        xq = torch.empty((T, K), dtype=torch.int8, device=x.device)
    if tok_scale is None:
        tok_scale = torch.empty(T, dtype=torch.float32, device=x.device)
    _dev(xq, "xq", (torch.int8,), numel=T * K, device=x.device)
    _dev(tok_scale, "tok_scale", (torch.float32,), numel=T, device=x.device)
    _gpu(x, s, xq, tok_scale)
    _check(lib.quant_per_token_i8(_ptr(x), _dtype_code(x), T, K, _ptr(s), _ptr(xq), _ptr(tok_scale),
                                  _stream(stream)))
    return xq, tok_scale


def w8a8_gemm_dequant(xq, wq, tok_scale, ch_scale, want_acc=False, y=None, stream=None):
    _dev(xq, "xq", (torch.int8,), ndim=2)
    M, K = xq.shape
    dev = xq.device
    _dev(wq, "wq", (torch.int8,), ndim=2, device=dev)
    N, K2 = wq.shape
    if K2 != K:
        raise ValueError("xq and wq differ in K")
    _dev(tok_scale, "tok_scale", (torch.float32,), numel=M, device=dev)
    _dev(ch_scale, "ch_scale", (torch.float32,), numel=N, device=dev)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    _dev(y, "y", (torch.float32,), numel=M * N, device=dev)
    _gpu(xq, wq, tok_scale, ch_scale, y)
    acc = torch.empty((M, N), dtype=torch.int32, device=xq.device) if want_acc else None
    _check(lib.w8a8_gemm_dequant(_ptr(xq), _ptr(wq), _ptr(tok_scale), _ptr(ch_scale), M, N, K, _ptr(y), _ptr(acc),
                                 _stream(stream)))
    return (y, acc) if want_acc else y


ACT = {"none": 0, "relu": 1, "gelu": 2}
OUT = {"f32": (0, torch.float32), "bf16": (1, torch.bfloat16), "i8": (2, torch.int8)}


def w8a8_gemm_fused(xq, wq, tok_scale, ch_scale, bias=None, act="none", out="f32", next_s=None, out_scale=None,
                    want_acc=False, y=None, stream=None):
    """GEMM + dequant + bias + activation, output fp32, bf16 or int8 (the next layer's static quantization:
    next_s [N] its smoothing factors or None, out_scale a 1-element device tensor, its static scale)."""
    _dev(xq, "xq", (torch.int8,), ndim=2)
    M, K = xq.shape
    dev = xq.device
    _dev(wq, "wq", (torch.int8,), ndim=2, device=dev)
    N, K2 = wq.shape
    if K2 != K:
        raise ValueError("xq and wq differ in K")
    _dev(tok_scale, "tok_scale", (torch.float32,), numel=M, device=dev)
    _dev(ch_scale, "ch_scale", (torch.float32,), numel=N, device=dev)
    _opt(bias, "bias", torch.float32, N, dev)
    _opt(next_s, "next_s", torch.float32, N, dev)
    _opt(out_scale, "out_scale", torch.float32, 1, dev)
    if act not in ACT or out not in OUT:
        raise ValueError(f"act must be one of {tuple(ACT)} and out one of {tuple(OUT)}")
    code, dt = OUT[out]
    if y is None:
        y = torch.empty((M, N), dtype=dt, device=xq.device)
    _dev(y, "y", (dt,), numel=M * N, device=dev)
    _gpu(xq, wq, tok_scale, ch_scale, bias, next_s, out_scale, y)
    acc = torch.empty((M, N), dtype=torch.int32, device=xq.device) if want_acc else None
    _check(lib.w8a8_gemm_fused(_ptr(xq), _ptr(wq), _ptr(tok_scale), _ptr(ch_scale), _ptr(bias), ACT[act], code,
                               _ptr(next_s), _ptr(out_scale), M, N, K, _ptr(y), _ptr(acc), _stream(stream)))
    return (y, acc) if want_acc else y


FOLD = {"div": 1, "mul": 2}


def sq_act_scale_ema(col_amax, s=None, momentum=0.9, first=False, state=None, scale=None, rows=0, row_scale=None,
                     stream=None):
    """Moving-average static activation scale from one batch's column maxima.  state / scale are
    1-element fp32 device tensors (created when None); row_scale [rows] is filled with the scale."""
    _dev(col_amax, "col_amax", (torch.float32,))
    K = col_amax.numel()
    dev = col_amax.device
    _opt(s, "s", torch.float32, K, dev)
    if state is None:
        state = torch.zeros(1, dtype=torch.float32, device=dev)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=dev)
    if row_scale is None and rows > 0:
        row_scale = torch.empty(rows, dtype=torch.float32, device=dev)
    _dev(state, "state", (torch.float32,), numel=1, device=dev)
    _dev(scale, "scale", (torch.float32,), numel=1, device=dev)
    if row_scale is not None:
        _dev(row_scale, "row_scale", (torch.float32,), device=dev)
    n = row_scale.numel() if row_scale is not None else 0
    _gpu(col_amax, s, state, scale, row_scale)
    _check(lib.sq_act_scale_ema(_ptr(col_amax), _ptr(s), K, float(momentum), int(bool(first)), _ptr(state),
                                _ptr(scale), _ptr(row_scale), n, _stream(stream)))
    return state, scale, row_scale


def weight_scale_per_tensor(col_amax, s=None, min_scale=SSZ_MIN_SCALE, n=0, scale=None, ch_scale=None, stream=None):
    """Per-tensor weight scale from the weight's column maxima; ch_scale [n] gets it for every channel."""
    _dev(col_amax, "col_amax", (torch.float32,))
    K = col_amax.numel()
    dev = col_amax.device
    _opt(s, "s", torch.float32, K, dev)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=dev)
    if ch_scale is None and n > 0:
        ch_scale = torch.empty(n, dtype=torch.float32, device=dev)
    _dev(scale, "scale", (torch.float32,), numel=1, device=dev)
    if ch_scale is not None:
        _dev(ch_scale, "ch_scale", (torch.float32,), device=dev)
    nn = ch_scale.numel() if ch_scale is not None else 0
    _gpu(col_amax, s, scale, ch_scale)
    _check(lib.weight_scale_per_tensor(_ptr(col_amax), _ptr(s), K, float(min_scale), _ptr(scale), _ptr(ch_scale),
                                       nn, _stream(stream)))
    return scale, ch_scale


def quant_static_i8(x, scale, s=None, fold="div", q=None, row_scale=None, want_row_scale=True, stream=None):
    """Int8 codes of x with one static scale (1-element device tensor); fold "div" (activations) or "mul"
    (weights) when s is given."""
    _dev(x, "x", _FLOATS, ndim=2)
    R, C = x.shape
    dev = x.device
    _dev(scale, "scale", (torch.float32,), numel=1, device=dev)
    _opt(s, "s", torch.float32, C, dev)
    if fold not in FOLD:
        raise ValueError(f"fold must be one of {tuple(FOLD)}")
    if q is None:
        q = torch.empty((R, C), dtype=torch.int8, device=x.device)
    if row_scale is None and want_row_scale:
        row_scale = torch.empty(R, dtype=torch.float32, device=x.device)
    _dev(q, "q", (torch.int8,), numel=R * C, device=dev)
    _opt(row_scale, "row_scale", torch.float32, R, dev)
    _gpu(x, scale, s, q, row_scale)
    _check(lib.quant_static_i8(_ptr(x), _dtype_code(x), R, C, _ptr(s), FOLD[fold] if s is not None else 0,
                               _ptr(scale), _ptr(q), _ptr(row_scale), _stream(stream)))
    return q, row_scale


def probe_mfma(kind, blocks=256, iters=2000, seed=1, stream=None):
    """Matrix-core clock probe (include/ptq_probe.h): runs `kind` ("mfma16_random", "mfma32_random",
    "mfma16_lds_random", "mfma16_zero" or its code) on `blocks` blocks of 512 threads and returns the elapsed
    time, the mean shader clock wave 0 of each block saw, and the int8 throughput (2 operations per
    multiply-add)."""
    k = PROBE_KINDS.get(kind, kind)
    if not isinstance(k, int):
        raise ValueError(f"unknown probe kind {kind!r}")
    if stream is not None and not isinstance(stream, torch.cuda.Stream):
        raise ValueError("probe_mfma takes a torch.cuda.Stream or None")
    out = torch.zeros(3 * blocks, dtype=torch.int64, device="cuda")
    st = _stream(stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s = torch.cuda.current_stream() if stream is None else stream
    e0.record(s)
    rc = lib.ptq_probe_mfma(k, blocks, iters, seed, _ptr(out), st)
    if rc != 0:
        raise PtqError(rc, lib.ptq_probe_last_error().decode(errors="replace"))
    e1.record(s)
    e1.synchronize()
    us = e0.elapsed_time(e1) * 1e3
    rec = out.view(blocks, 3).cpu().double()
    cycles, ticks = rec[:, 0], rec[:, 1]
    ops = 2.0 * PROBE_MACS_PER_BLOCK_ITER * iters * blocks
    return {"kind": k, "us": us, "clock_GHz": float((cycles / (ticks * 10.0)).mean()),
            "wave_cycles": float(cycles.mean()), "TOPS": ops / us / 1e6}


def probe_valu(kind, blocks=2048, iters=2000, seed=1, stream=None):
    """VALU probe (include/ptq_probe.h): runs `kind` ("ssz_loop", "ssz_loop_reduce", "fma_f32", "fma_f64" or its
    code) on `blocks` one-wave blocks and returns the elapsed time, the mean shader clock wave 0 of each block saw,
    the lane operations per second (element-passes for the SSZ loop kinds, multiply-adds for the others) and the
    SIMD cycles one wave's unit of work took on average (all SIMDs of the device busy)."""
    k = VALU_KINDS.get(kind, kind)
    if k not in (0, 1, 2, 3):
        raise ValueError(f"unknown VALU probe kind {kind!r}")
    if stream is not None and not isinstance(stream, torch.cuda.Stream):
        raise ValueError("probe_valu takes a torch.cuda.Stream or None")
    out = torch.zeros(3 * blocks, dtype=torch.int64, device="cuda")
    st = _stream(stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s = torch.cuda.current_stream() if stream is None else stream
    e0.record(s)
    rc = lib.ptq_probe_valu(k, blocks, iters, seed, _ptr(out), st)
    if rc != 0:
        raise PtqError(rc, lib.ptq_probe_last_error().decode(errors="replace"))
    e1.record(s)
    e1.synchronize()
    us = e0.elapsed_time(e1) * 1e3
    rec = out.view(blocks, 3).cpu().double()
    cycles, ticks = rec[:, 0], rec[:, 1]
    clock = float((cycles / (ticks * 10.0)).mean())
    per_lane = VALU_ELEMS_PER_ITER if k <= 1 else VALU_FMAS_PER_ITER
    lane_ops = float(blocks) * 64 * iters * per_lane
    simds = 4 * torch.cuda.get_device_properties(out.device).multi_processor_count
    return {"kind": k, "us": us, "clock_GHz": clock, "lane_ops_per_s": lane_ops / (us * 1e-6),
            "simd_cycles_per_wave_op": us * 1e-6 * clock * 1e9 * simds / (lane_ops / 64)}


def probe_stream(kind, src, dst=None, blocks=1024, stream=None):
    """HBM stream probe (include/ptq_probe.h): reads every byte of the device tensor `src` once ("read"), or copies
    it into `dst` ("copy"), on `blocks` blocks of 256 threads; returns the elapsed time and the bytes moved per
    second (read bytes, or read plus written bytes for a copy)."""
    k = STREAM_KINDS.get(kind, kind)
    if k not in (0, 1):
        raise ValueError(f"unknown stream probe kind {kind!r}")
    if stream is not None and not isinstance(stream, torch.cuda.Stream):
        raise ValueError("probe_stream takes a torch.cuda.Stream or None")
    _dev(src, "src")
    nbytes = src.numel() * src.element_size()
    if k == 1:
        _dev(dst, "dst", device=src.device)
        if dst.numel() * dst.element_size() < nbytes:
            raise ValueError("dst is smaller than src")
    out = torch.zeros(blocks, dtype=torch.int32, device=src.device) if k == 0 else None
    st = _stream(stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s = torch.cuda.current_stream() if stream is None else stream
    e0.record(s)
    rc = lib.ptq_probe_stream(k, _ptr(src), nbytes, _ptr(dst) if k == 1 else None, blocks, _ptr(out), st)
    if rc != 0:
        raise PtqError(rc, lib.ptq_probe_last_error().decode(errors="replace"))
    e1.record(s)
    e1.synchronize()
    us = e0.elapsed_time(e1) * 1e3
    moved = nbytes * (2 if k == 1 else 1)
    res = {"kind": k, "us": us, "bytes": moved, "GBps": moved / us / 1e3}
    if k == 0:  # the xor of every 32-bit word read (the blocks' partial xors combined)
        res["xor"] = int(np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)))
    return res
