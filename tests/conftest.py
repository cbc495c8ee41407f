import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def read_golden(name):
    """Rows of a whitespace-separated golden file, comments (#) dropped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def golden():
    return read_golden


_CONFIG = None


def pytest_sessionstart(session):
    global _CONFIG
    _CONFIG = session.config
    import parity_util
    parity_util.set_writer(say)


def say(msg):
    """Write a line to the real terminal right away (not captured), so the case a
    GPU step belongs to is on record even if the process dies during the step."""
    tr = _CONFIG.pluginmanager.getplugin("terminalreporter") if _CONFIG else None
    if tr is not None:
        # inside a test, output capture is on: suspend it around the write (as pytest's live logging does)
        capman = _CONFIG.pluginmanager.getplugin("capturemanager")
        if capman is not None:
            with capman.global_and_fixture_disabled():
                tr.write_line(msg)
                tr._tw.flush() if hasattr(tr, "_tw") else None
        else:
            tr.write_line(msg)
            tr._tw.flush() if hasattr(tr, "_tw") else None
    else:
        sys.__stderr__.write(msg + "\n")
        sys.__stderr__.flush()


def pytest_runtest_logstart(nodeid, location):
    if "gpu" in nodeid.split("::")[0]:
        say(f"[gpu-test] start {nodeid}")
