import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


# A host-only build of the C ABI (sanitized, no GPU) can stand in for libkvq.so: see
# tests/test_sanitized_host.py, which sets this variable for its child test run.
if os.environ.get("KVQ_TEST_LIBRARY"):
    import rotate_then_bit_amd as _kvq

    _kvq._LIB_PATH = os.environ["KVQ_TEST_LIBRARY"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    """The 1e-5 bound on code mismatches at rounding ties, over every code compared in the
    session (each comparison also holds it, rounded up to one tie).  Runs whatever subset
    of the tests was collected, so it cannot be skipped by selection or ordering."""
    par = sys.modules.get("tests.parity")
    if par is None or par.SESSION["codes"] == 0:
        return
    s = par.SESSION
    msg = f"[parity] {s['tie_mismatches']} code mismatches at rounding ties in {s['codes']} codes compared"
    ok = s["tie_mismatches"] <= par.CODE_MISMATCH_MAX * s["codes"]
    rep = session.config.pluginmanager.get_plugin("terminalreporter")
    if rep is not None:
        rep.write_line(msg + ("" if ok else f": above the bound {par.CODE_MISMATCH_MAX}"), red=not ok)
    if not ok:
        session.exitstatus = pytest.ExitCode.TESTS_FAILED


GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([p.strip() for p in line.split("|")])
    return rows
