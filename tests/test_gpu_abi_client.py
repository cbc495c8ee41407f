"""The C ABI from a C++ program with no Python or torch (tests/abi_c/ptq_path.cpp: hipMalloc'd memory, its own
stream, the five calls of the path), run as its own process on seeded inputs; every output against the oracle."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth
from parity_util import announce, assert_y

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "abi_c", "ptq_path")


def _case(name):
    if name == "tiny":
        c = synth.cases("tiny")[0]
        return synth.widen(c.x_batch(0)), synth.widen(c.w())
    c = {x.name: x for x in synth.cases("gpt345m")}[name]
    return synth.widen(c.x_batch(0)), synth.widen(c.w())


@pytest.mark.parametrize("name", ["tiny", "gpt345m/out"])
def test_c_client_whole_path(tmp_path, name):
    if not os.path.exists(CLIENT):
        pytest.fail("the C client is not built: run __graft_entry__.build()")
    x, w = _case(name)
    T, K = x.shape
    N = w.shape[0]
    np.ascontiguousarray(x, np.float32).tofile(tmp_path / "x.f32")
    np.ascontiguousarray(w, np.float32).tofile(tmp_path / "w.f32")
    announce(f"C client {name}: T={T} K={K} N={N}")
    r = subprocess.run([CLIENT, str(tmp_path), str(T), str(K), str(N), "0.5"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    ref = oracle.run_linear([x], w, x, alpha=0.5, smooth=True, bits=8)
    rd = lambda f, dt: np.fromfile(tmp_path / f, dtype=dt)
    np.testing.assert_array_equal(rd("ax.f32", np.float32), ref["ax"])
    np.testing.assert_array_equal(rd("aw.f32", np.float32), ref["aw"])
    np.testing.assert_array_equal(rd("s.f32", np.float32), ref["s"])
    np.testing.assert_array_equal(rd("S.f32", np.float32), ref["S"])
    np.testing.assert_array_equal(rd("it.i32", np.int32), ref["iters"])
    np.testing.assert_array_equal(rd("wq.i8", np.int8).reshape(N, K), ref["wq"])
    np.testing.assert_array_equal(rd("xq.i8", np.int8).reshape(T, K), ref["xq"])
    np.testing.assert_array_equal(rd("d.f32", np.float32), ref["delta"])
    np.testing.assert_array_equal(rd("acc.i32", np.int32).reshape(T, N), ref["acc"])
    assert_y(rd("y.f32", np.float32).reshape(T, N), ref["y"], f"C client {name} y")
