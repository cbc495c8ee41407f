"""The C ABI without a GPU: the library loads, exports every declared symbol, and
rejects every invalid argument on the host before any launch.

Every call here fails validation, so no kernel is ever enqueued: pointers are
either NULL or deliberately misaligned host-side integers that are never
dereferenced because validation stops first.
"""
import ctypes
import glob
import math
import os
import re

import pytest

from conftest import ROOT, read_golden

HEADER = os.path.join(ROOT, "include", "ptq.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
LIB = os.path.join(ROOT, "post_int8_quantization_amd", "libptq.so")

OK, NULL, SHAPE, DTYPE, UNSUP, ARG, ALIGN, HIP = range(8)
F32, BF16 = 0, 1
P = 0x10000  # a 16-byte-aligned stand-in pointer, only ever paired with an argument that fails validation
MIS = 0x10001  # misaligned stand-in pointer


def _ensure_built():
    if not os.path.exists(LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location("ptq_build", os.path.join(ROOT, "post_int8_quantization_amd",
                                                                                 "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


@pytest.fixture(scope="module")
def lib():
    _ensure_built()
    L = ctypes.CDLL(LIB)
    vp, i64, ci, f32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
    L.sq_absmax_calib.argtypes = [vp, ci, i64, i64, vp, ci, vp]
    L.sq_smooth_factors.argtypes = [vp, vp, i64, f32, vp, vp]
    L.ssz_weight_qparams.argtypes = [vp, ci, i64, i64, vp, ci, ci, ci, f64, f32, vp, vp, vp, vp, vp]
    L.ssz_weight_qparams_asym.argtypes = [vp, ci, i64, i64, vp, ci, f64, f32, vp, vp, vp, vp, vp, vp]
    L.quant_per_token_i8.argtypes = [vp, ci, i64, i64, vp, vp, vp, vp]
    L.w8a8_gemm_dequant.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, vp]
    L.w8a8_gemm_fused.argtypes = [vp, vp, vp, vp, vp, ci, ci, vp, vp, i64, i64, i64, vp, vp, vp]
    L.sq_act_scale_ema.argtypes = [vp, vp, i64, f32, ci, vp, vp, vp, i64, vp]
    L.weight_scale_per_tensor.argtypes = [vp, vp, i64, f32, vp, vp, i64, vp]
    L.quant_static_i8.argtypes = [vp, ci, i64, i64, vp, ci, vp, vp, vp, vp]
    L.ptq_last_error.restype = ctypes.c_char_p
    L.ptq_status_string.restype = ctypes.c_char_p
    return L


def header_functions():
    """Every function declared in include/*.h (PTQ_API in ptq.h, PTQ_PROBE_API in ptq_probe.h)."""
    names = []
    for h in HEADERS:
        names += re.findall(r"PTQ_(?:PROBE_)?API\s+[\w\s\*]+?\b(\w+)\s*\(", open(h).read())
    return names


def header_define(name):
    m = re.search(r"#define\s+%s\s+(\S+)" % name, open(HEADER).read())
    return m.group(1)


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == {"ptq_abi_version", "ptq_last_error", "ptq_status_string", "sq_absmax_calib",
                          "sq_smooth_factors", "ssz_weight_qparams", "ssz_weight_qparams_asym",
                          "quant_per_token_i8", "w8a8_gemm_dequant", "w8a8_gemm_fused", "sq_act_scale_ema",
                          "weight_scale_per_tensor", "quant_static_i8", "ptq_probe_mfma", "ptq_probe_stream", "ptq_probe_valu",
                          "ptq_probe_last_error"}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.ptq_abi_version() == int(header_define("PTQ_ABI_VERSION"))


def test_header_constants_match_pages():
    g = {k: float(v) for k, v in read_golden("ssz_constants.txt")}
    assert int(header_define("PTQ_SSZ_MAX_ITER")) == g["SCALE_SEARCH_ITER_NUM"]
    assert float(header_define("PTQ_SSZ_THRESHOLD")) == g["SCALE_SEARCH_CONVERGE_THRESHOLD"]
    assert float(header_define("PTQ_SSZ_MIN_SCALE").rstrip("f")) == g["SCALE_SEARCH_MIN_SCALE"]
    assert int(header_define("PTQ_GEMM_MAX_K")) == (2 ** 31 - 1) // 128 ** 2 // 16 * 16


def test_status_strings(lib):
    for code, name in enumerate(["PTQ_OK", "PTQ_ERR_NULL", "PTQ_ERR_SHAPE", "PTQ_ERR_DTYPE", "PTQ_ERR_UNSUPPORTED",
                                 "PTQ_ERR_ARG", "PTQ_ERR_ALIGN", "PTQ_ERR_HIP"]):
        assert lib.ptq_status_string(code).decode() == name


def _expect(lib, status, want, needle=None):
    assert status == want, (status, want, lib.ptq_last_error())
    msg = lib.ptq_last_error().decode()
    assert msg
    if needle:
        assert needle in msg, msg


def test_calib_errors(lib):
    c = lib.sq_absmax_calib
    _expect(lib, c(None, BF16, 4, 16, P, 0, None), NULL)
    _expect(lib, c(P, BF16, 4, 16, None, 0, None), NULL)
    _expect(lib, c(P, 7, 4, 16, P, 0, None), DTYPE)
    _expect(lib, c(P, BF16, 0, 16, P, 0, None), SHAPE)
    _expect(lib, c(P, BF16, 4, 0, P, 0, None), SHAPE)
    _expect(lib, c(P, BF16, 4, 24, P, 0, None), SHAPE, "multiple of 16")
    _expect(lib, c(MIS, BF16, 4, 16, P, 0, None), ALIGN)
    _expect(lib, c(P, F32, 4, 16, MIS, 1, None), ALIGN)


def test_smooth_errors(lib):
    c = lib.sq_smooth_factors
    _expect(lib, c(None, P, 16, 0.5, P, None), NULL)
    _expect(lib, c(P, P, 16, 0.5, None, None), NULL)
    _expect(lib, c(P, P, 0, 0.5, P, None), SHAPE)
    for a in (-0.01, 1.01, math.nan, math.inf):
        _expect(lib, c(P, P, 16, a, MIS, None), ARG, "alpha")


def test_ssz_errors(lib):
    c = lib.ssz_weight_qparams

    def call(w=P, dt=BF16, N=8, K=64, s=None, bits=8, sym=1, it=20, thr=1e-10, ms=1e-5, scale=P, wq=P):
        return c(w, dt, N, K, s, bits, sym, it, thr, ms, scale, wq, None, None, None)

    _expect(lib, call(w=None), NULL)
    _expect(lib, call(scale=None), NULL)
    _expect(lib, call(dt=2), DTYPE)
    _expect(lib, call(N=0), SHAPE)
    _expect(lib, call(K=40), SHAPE)
    _expect(lib, call(K=131072 + 16), SHAPE)
    _expect(lib, call(bits=2), UNSUP)
    _expect(lib, call(bits=16), UNSUP)
    _expect(lib, call(sym=0), UNSUP, "ssz_weight_qparams_asym")
    _expect(lib, call(it=-1), ARG)
    _expect(lib, call(it=21), ARG)
    _expect(lib, call(thr=-1.0), ARG)
    _expect(lib, call(thr=math.nan), ARG)
    _expect(lib, call(ms=0.0), ARG)
    _expect(lib, call(ms=-1e-5), ARG)
    _expect(lib, call(w=MIS), ALIGN)
    _expect(lib, call(s=MIS), ALIGN)
    _expect(lib, call(wq=MIS), ALIGN)


def test_ssz_asym_errors(lib):
    c = lib.ssz_weight_qparams_asym

    def call(w=P, dt=BF16, N=8, K=64, s=None, it=20, thr=1e-10, ms=1e-5, scale=P, zp=P, wq=P):
        return c(w, dt, N, K, s, it, thr, ms, scale, zp, wq, None, None, None)

    _expect(lib, call(w=None), NULL)
    _expect(lib, call(scale=None), NULL)
    _expect(lib, call(zp=None), NULL, "zero_point")
    _expect(lib, call(dt=2), DTYPE)
    _expect(lib, call(N=0), SHAPE)
    _expect(lib, call(K=40), SHAPE)
    _expect(lib, call(K=131072 + 16), SHAPE)
    _expect(lib, call(it=-1), ARG)
    _expect(lib, call(it=21), ARG)
    _expect(lib, call(thr=math.inf), ARG)
    _expect(lib, call(ms=0.0), ARG)
    _expect(lib, call(w=MIS), ALIGN)
    _expect(lib, call(s=MIS), ALIGN)
    _expect(lib, call(wq=MIS), ALIGN)


def test_quant_errors(lib):
    c = lib.quant_per_token_i8
    _expect(lib, c(None, BF16, 4, 64, None, P, P, None), NULL)
    _expect(lib, c(P, BF16, 4, 64, None, None, P, None), NULL)
    _expect(lib, c(P, BF16, 4, 64, None, P, None, None), NULL)
    _expect(lib, c(P, 5, 4, 64, None, P, P, None), DTYPE)
    _expect(lib, c(P, BF16, 0, 64, None, P, P, None), SHAPE)
    _expect(lib, c(P, BF16, 4, 72, None, P, P, None), SHAPE)
    _expect(lib, c(MIS, BF16, 4, 64, None, P, P, None), ALIGN)
    _expect(lib, c(P, BF16, 4, 64, None, MIS, P, None), ALIGN)
    _expect(lib, c(P, F32, 4, 64, MIS, P, P, None), ALIGN)


def test_gemm_errors(lib):
    c = lib.w8a8_gemm_dequant
    _expect(lib, c(None, P, P, P, 4, 4, 64, P, None, None), NULL)
    _expect(lib, c(P, P, None, P, 4, 4, 64, P, None, None), NULL)
    _expect(lib, c(P, P, P, P, 4, 4, 64, None, None, None), NULL)
    _expect(lib, c(P, P, P, P, 0, 4, 64, P, None, None), SHAPE)
    _expect(lib, c(P, P, P, P, 4, 0, 64, P, None, None), SHAPE)
    _expect(lib, c(P, P, P, P, 4, 4, 40, P, None, None), SHAPE)
    _expect(lib, c(P, P, P, P, 4, 4, 133152, P, None, None), SHAPE, "overflow")
    _expect(lib, c(MIS, P, P, P, 4, 4, 64, P, None, None), ALIGN)
    _expect(lib, c(P, P, P, P, 4, 4, 64, MIS, None, None), ALIGN)
    _expect(lib, c(P, P, P, P, 4, 4, 64, P, MIS, None), ALIGN)


def test_gemm_fused_errors(lib):
    c = lib.w8a8_gemm_fused

    def call(xq=P, act=0, out=0, ns=None, osc=None, M=4, N=4, K=64, y=P, acc=None, bias=None):
        return c(xq, P, P, P, bias, act, out, ns, osc, M, N, K, y, acc, None)

    _expect(lib, call(xq=None), NULL)
    _expect(lib, call(y=None), NULL)
    _expect(lib, call(act=3), UNSUP, "act")
    _expect(lib, call(out=3), DTYPE, "out_type")
    _expect(lib, call(out=2), NULL, "out_scale")
    _expect(lib, call(out=0, osc=P), ARG, "int8 output only")
    _expect(lib, call(out=1, ns=P), ARG, "int8 output only")
    _expect(lib, call(M=0), SHAPE)
    _expect(lib, call(K=40), SHAPE)
    _expect(lib, call(K=133152), SHAPE, "overflow")
    _expect(lib, call(xq=MIS), ALIGN)
    _expect(lib, call(out=2, osc=P, y=MIS), ALIGN)


def test_static_scale_errors(lib):
    e = lib.sq_act_scale_ema
    _expect(lib, e(None, None, 16, 0.9, 1, P, P, None, 0, None), NULL)
    _expect(lib, e(P, None, 16, 0.9, 1, None, P, None, 0, None), NULL)
    _expect(lib, e(P, None, 0, 0.9, 1, P, P, None, 0, None), SHAPE)
    _expect(lib, e(P, None, 16, 0.9, 1, P, P, P, 0, None), SHAPE)
    for m in (-0.1, 1.0, math.nan):
        _expect(lib, e(P, None, 16, m, 0, P, P, None, 0, None), ARG, "momentum")
    w = lib.weight_scale_per_tensor
    _expect(lib, w(None, None, 16, 1e-5, P, None, 0, None), NULL)
    _expect(lib, w(P, None, 16, 1e-5, None, None, 0, None), NULL)
    _expect(lib, w(P, None, 0, 1e-5, P, None, 0, None), SHAPE)
    _expect(lib, w(P, None, 16, 1e-5, P, P, 0, None), SHAPE)
    _expect(lib, w(P, None, 16, 0.0, P, None, 0, None), ARG)
    q = lib.quant_static_i8
    _expect(lib, q(None, BF16, 4, 64, None, 0, P, P, None, None), NULL)
    _expect(lib, q(P, BF16, 4, 64, None, 0, None, P, None, None), NULL)
    _expect(lib, q(P, 9, 4, 64, None, 0, P, P, None, None), DTYPE)
    _expect(lib, q(P, BF16, 4, 40, None, 0, P, P, None, None), SHAPE)
    _expect(lib, q(P, BF16, 4, 64, P, 0, P, P, None, None), ARG, "fold")
    _expect(lib, q(P, BF16, 4, 64, P, 3, P, P, None, None), ARG, "fold")
    _expect(lib, q(MIS, BF16, 4, 64, None, 0, P, P, None, None), ALIGN)


def test_binding_rejects_host_tensors():
    _ensure_built()
    import torch
    import post_int8_quantization_amd as pq
    x = torch.zeros(4, 16)
    with pytest.raises(ValueError, match="GPU tensor"):
        pq.sq_absmax_calib(x)
    with pytest.raises(ValueError):
        pq.quant_per_token_i8(x)
    assert set(pq.EXPORTS) == set(header_functions())


def _binding_cases(torch):
    """(call, message) pairs: every vector and preallocated output of the binding with a wrong length, dtype
    or shape.  Host tensors stand in for device ones: the size checks run before the GPU check."""
    f32, bf, i8, i32, f64 = torch.float32, torch.bfloat16, torch.int8, torch.int32, torch.float64
    x = torch.zeros(4, 32, dtype=bf)
    w = torch.zeros(8, 32, dtype=bf)
    xq, wq = torch.zeros(4, 32, dtype=i8), torch.zeros(8, 32, dtype=i8)
    v = lambda n, dt=f32: torch.zeros(n, dtype=dt)  # noqa: E731
    return [
        (lambda pq: pq.sq_absmax_calib(x, amax=v(31)), "amax has 31 elements"),
        (lambda pq: pq.sq_absmax_calib(x, amax=v(32, f64)), "amax has dtype"),
        (lambda pq: pq.sq_absmax_calib(torch.zeros(32, dtype=bf)), "x must be 2-D"),
        (lambda pq: pq.sq_smooth_factors(v(32), v(31), 0.5), "w_amax has 31 elements"),
        (lambda pq: pq.sq_smooth_factors(v(32), v(32), 0.5, s=v(16)), "s has 16 elements"),
        (lambda pq: pq.ssz_weight_qparams(w, s=v(31)), "s has 31 elements"),
        (lambda pq: pq.ssz_weight_qparams(w, scale=v(7)), "scale has 7 elements"),
        (lambda pq: pq.ssz_weight_qparams(w, wq=torch.zeros(8, 31, dtype=i8)), "wq has 248 elements"),
        (lambda pq: pq.ssz_weight_qparams(w, bits=4, wq=torch.zeros(8, 32, dtype=torch.uint8)), "wq has 256"),
        (lambda pq: pq.ssz_weight_qparams(w, iters=v(8, torch.int64)), "iters has dtype"),
        (lambda pq: pq.ssz_weight_qparams(w, mse=v(8, f32)), "mse has dtype"),
        (lambda pq: pq.ssz_weight_qparams(w, mse=v(9, f64)), "mse has 9 elements"),
        (lambda pq: pq.ssz_weight_qparams_asym(w, zero_point=v(8, f32)), "zero_point has dtype"),
        (lambda pq: pq.ssz_weight_qparams_asym(w, wq=torch.zeros(8, 16, dtype=i8)), "wq has 128 elements"),
        (lambda pq: pq.quant_per_token_i8(x, s=v(30)), "s has 30 elements"),
        (lambda pq: pq.quant_per_token_i8(x, xq=torch.zeros(4, 16, dtype=i8)), "xq has 64 elements"),
        (lambda pq: pq.quant_per_token_i8(x, tok_scale=v(3)), "tok_scale has 3 elements"),
        (lambda pq: pq.w8a8_gemm_dequant(xq, wq, v(3), v(8)), "tok_scale has 3 elements"),
        (lambda pq: pq.w8a8_gemm_dequant(xq, wq, v(4), v(7)), "ch_scale has 7 elements"),
        (lambda pq: pq.w8a8_gemm_dequant(xq, wq, v(4), v(8), y=v(31)), "y has 31 elements"),
        (lambda pq: pq.w8a8_gemm_dequant(xq, torch.zeros(8, 16, dtype=i8), v(4), v(8)), "differ in K"),
        (lambda pq: pq.w8a8_gemm_fused(xq, wq, v(4), v(8), bias=v(7)), "bias has 7 elements"),
        (lambda pq: pq.w8a8_gemm_fused(xq, wq, v(4), v(8), out="i8", next_s=v(9), out_scale=v(1)),
         "next_s has 9 elements"),
        (lambda pq: pq.w8a8_gemm_fused(xq, wq, v(4), v(8), out="i8", out_scale=v(2)), "out_scale has 2"),
        (lambda pq: pq.w8a8_gemm_fused(xq, wq, v(4), v(8), out="bf16", y=v(32)), "y has dtype"),
        (lambda pq: pq.w8a8_gemm_fused(xq, wq, v(4), v(8), act="tanh"), "act must be one of"),
        (lambda pq: pq.sq_act_scale_ema(v(32), s=v(16)), "s has 16 elements"),
        (lambda pq: pq.sq_act_scale_ema(v(32), state=v(2)), "state has 2 elements"),
        (lambda pq: pq.sq_act_scale_ema(v(32), row_scale=v(4, f64)), "row_scale has dtype"),
        (lambda pq: pq.weight_scale_per_tensor(v(32), scale=v(3)), "scale has 3 elements"),
        (lambda pq: pq.quant_static_i8(x, v(1), s=v(31)), "s has 31 elements"),
        (lambda pq: pq.quant_static_i8(x, v(2)), "scale has 2 elements"),
        (lambda pq: pq.quant_static_i8(x, v(1), q=torch.zeros(4, 31, dtype=i8)), "q has 124 elements"),
        (lambda pq: pq.quant_static_i8(x, v(1), row_scale=v(5)), "row_scale has 5 elements"),
        (lambda pq: pq.quant_static_i8(x, v(1), s=v(32), fold="pow"), "fold must be one of"),
    ]


def test_binding_checks_sizes_and_types():
    """ValueError before any launch for a wrong-length vector, a short or mistyped preallocated output, a wrong
    rank; with every size right, the GPU check is what remains."""
    _ensure_built()
    import torch
    import post_int8_quantization_amd as pq
    cases = _binding_cases(torch)
    for call, msg in cases:
        with pytest.raises(ValueError, match=re.escape(msg)):
            call(pq)
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        pq.quant_per_token_i8(x, s=torch.ones(32), xq=torch.zeros(4, 32, dtype=torch.int8),
                              tok_scale=torch.zeros(4))


def test_gemm_k_bound_is_the_int8_worst_case(lib):
    """K one step past 2^14 K < 2^31 (-128 codes) is rejected; the bound itself passes the K checks."""
    c = lib.w8a8_gemm_dequant
    _expect(lib, c(P, P, P, P, 4, 4, 131072, P, None, None), SHAPE, "overflow")
    _expect(lib, c(MIS, P, P, P, 4, 4, 131056, P, None, None), ALIGN)


def test_probe_rejects_bad_arguments(lib):
    """The clock probe validates on the host: nothing is launched for a bad kind, size, count or buffer."""
    f = lib.ptq_probe_mfma
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    lib.ptq_probe_last_error.restype = ctypes.c_char_p
    for args in [(4, 256, 10, 1, P), (-1, 256, 10, 1, P), (0, 0, 10, 1, P), (0, 65537, 10, 1, P), (0, 256, 0, 1, P),
                 (0, 256, 1000001, 1, P), (0, 256, 10, 1, None), (0, 256, 10, 1, MIS)]:
        assert f(*args, None) == ARG, args
        assert lib.ptq_probe_last_error().decode().startswith("ptq_probe_mfma")


def test_valu_probe_rejects_bad_arguments(lib):
    """The VALU probe validates on the host: nothing is launched for a bad kind, size, count or buffer."""
    f = lib.ptq_probe_valu
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    lib.ptq_probe_last_error.restype = ctypes.c_char_p
    for args in [(4, 2048, 10, 1, P), (-1, 2048, 10, 1, P), (0, 0, 10, 1, P), (0, 65537, 10, 1, P), (0, 2048, 0, 1, P),
                 (0, 2048, 1000001, 1, P), (0, 2048, 10, 1, None), (0, 2048, 10, 1, MIS)]:
        assert f(*args, None) == ARG, args
        assert lib.ptq_probe_last_error().decode().startswith("ptq_probe_valu")


def test_stream_probe_rejects_bad_arguments(lib):
    """The stream probe validates on the host: nothing is launched for a bad kind, size, block count or buffer."""
    f = lib.ptq_probe_stream
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p]
    lib.ptq_probe_last_error.restype = ctypes.c_char_p
    for args in [(2, P, 1024, P, 16, P), (-1, P, 1024, P, 16, P), (0, P, 0, P, 16, P), (0, P, 1000, P, 16, P),
                 (0, P, 1024, P, 0, P), (0, P, 1024, P, 65537, P), (0, None, 1024, P, 16, P),
                 (0, P, 1024, None, 16, None), (1, P, 1024, None, 16, P), (0, MIS, 1024, P, 16, P),
                 (1, P, 1024, MIS, 16, P), (0, P, 1024, None, 16, MIS)]:
        assert f(*args, None) == ARG, args
        assert lib.ptq_probe_last_error().decode().startswith("ptq_probe_stream")

