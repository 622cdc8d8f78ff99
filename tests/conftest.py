import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle.build(force=False)
    return oracle.lib()


def pytest_terminal_summary(terminalreporter):
    """Parity headroom of the GPU checks that recorded it: max |err| and max err/tol
    against the oracle (err/tol <= 1 passes), per check and workload."""
    try:
        from gpu_util import PARITY
    except Exception:
        return
    if not PARITY:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity against the oracle (max |err|, max err/tol; tol = 1e-2 + 1e-3 |ref|)")
    for (check, workload, detail), (err, ratio, rows) in sorted(PARITY.items()):
        if check == "select":  # index overlap; disagreements' distance to the k-th score / the tie-gap limit
            tr.write_line(f"[parity] {check:8s} {workload:30s} rows {rows:>10s}  {detail}  "
                          f"worst disagreement {ratio:.3f} of the tie-gap limit")
        else:
            tr.write_line(f"[parity] {check:8s} {workload:30s} rows {rows:>10s}  {detail}"
                          f"max|err| {err:.3e}  max err/tol {ratio:.3f}")
