"""Memory and undefined-behaviour checks of the host code, on the CPU.

* The oracle (oracle/ptq_oracle.c) under gcc's AddressSanitizer and UndefinedBehaviorSanitizer (float-to-int
  overflow included), driven through every entry point on seeded inputs and on the edge inputs the quantizers
  meet: zero, subnormal, tiny, huge and mixed rows, extreme scales and zero points (tests/sanitize/oracle_driver.c).
* The C ABI's host code (csrc/capi.hip, compiled for the host only) under clang's AddressSanitizer and
  UndefinedBehaviorSanitizer, with the kernel launchers replaced by stand-ins: every invalid-argument class of
  every entry point, every valid call reaching its launcher, and a failed launch (tests/sanitize/abi_driver.cpp).

No GPU is used; the sanitizers apply to host code only (each -fsanitize is passed with -Xarch_host on the hipcc
lines, and the device side is not compiled at all).
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\nrc={r.returncode}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "ptq_oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([exe], env=env, timeout=600)
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "oracle sanitizer driver:" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_c_abi_host_code_under_asan_ubsan(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["-O1", "-g", "-std=c++17", *san, "-I", os.path.join(ROOT, "include")]
    objs = []
    for src, host_only in ((os.path.join(ROOT, "post_int8_quantization_amd", "csrc", "capi.hip"), True),
                           (os.path.join(HERE, "launch_stubs.cpp"), True),
                           (os.path.join(HERE, "abi_driver.cpp"), False)):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        lang = ["-x", "hip", "--offload-host-only"] if host_only else []
        _run([HIPCC, *lang, *common, "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, *san, *objs, "-o", exe])
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1"),
             timeout=300)
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert ", 0 failed" in r.stdout, r.stdout
