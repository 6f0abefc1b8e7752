import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="session")
def golden():
    return load_golden


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One line per GPU output check: elements compared, how many fall in the
    output format's exception set, how many lie beyond the flat tolerance
    (all of them in that set), and the largest error. Printed under -q too."""
    mod = sys.modules.get("tests.test_gpu_parity")
    records = getattr(mod, "GATE_RECORDS", None) if mod else None
    if not records:
        return
    n = sum(r[1] for r in records)
    exc = sum(r[2] for r in records)
    beyond = sum(r[3] for r in records)
    terminalreporter.write_sep("-", "output gate")
    terminalreporter.write_line(f"{len(records)} checks, {n} elements: {exc} in the format's exception set, "
                                f"{beyond} beyond the flat tolerance (all inside that set)")
    for what, size, n_exc, n_beyond, err in records:
        if n_exc or n_beyond:
            terminalreporter.write_line(f"  {what}: {n_exc} excepted, {n_beyond} beyond flat, of {size}; "
                                        f"max abs err {err:.3e}")
