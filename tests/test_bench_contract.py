"""Host-side checks of the benchmark script (no GPU): the one-GPU guard and the traffic-record key."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_key_ignores_comments_and_layout_only():
    b = _bench()
    code = "int f(int a) {\n  return a + 1;  // add\n}\n/* block\n comment */\n"
    assert b._code_only(code) == b._code_only("int f(int a) { return a + 1; }")
    assert b._code_only(code) != b._code_only("int f(int a) { return a + 2; }")


def test_every_traffic_record_names_a_known_kernel():
    b = _bench()
    import json
    import re
    seen = 0
    for f in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        if "counters" not in f:
            continue
        for m in re.finditer(r"traffic-record:\s*(\{.*\})", open(os.path.join(ROOT, "profiles", f)).read()):
            rec = json.loads(m.group(1))
            assert rec["kernel"] in b.KERNEL_SOURCES, f
            assert rec["traffic_bytes_per_launch"] > 0 and rec["dispatches"] > 0
            seen += 1
    assert seen > 0


def test_traffic_records_are_of_the_current_kernel_sources():
    """The committed HBM-traffic records were taken on the kernels as they are now (a record whose source hash no
    longer matches is ignored by the bench, which then reports traffic as null)."""
    b = _bench()
    import json
    import re
    stale = []
    for f in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        if "counters" not in f:
            continue
        for m in re.finditer(r"traffic-record:\s*(\{.*\})", open(os.path.join(ROOT, "profiles", f)).read()):
            rec = json.loads(m.group(1))
            if rec["source_sha"] != b.kernel_source_sha(rec["kernel"]):
                stale.append((f, rec["kernel"], rec["workload"]))
    assert not stale, stale
