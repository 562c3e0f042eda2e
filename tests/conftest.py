import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter):
    """List the parity records of the full-size workloads run in this session
    (elements, failed count, max ulp, floor-judged count; dw's normwise and
    relative errors), and write them to $TN_PARITY_DIR when it is set."""
    from tests import parity
    lines = parity.format_records()
    if not lines:
        return
    terminalreporter.write_sep("=", "parity records of the full-size workloads")
    for ln in lines:
        terminalreporter.write_line(ln)
    out = os.environ.get("TN_PARITY_DIR")
    if out:
        os.makedirs(out, exist_ok=True)
        for workload, reps in parity.RECORDS:
            path = os.path.join(out, f"parity_{workload}.txt")
            fresh = not os.path.exists(path)
            with open(path, "a") as f:
                if fresh:
                    f.write(f"# GPU library against the float64 oracle, workload {workload}, full size\n"
                            "# written by the GPU test session (rules: tests/parity.py):\n"
                            "#   TN_PARITY_DIR=<dir> python -m pytest tests -m gpu\n")
                for r in reps:
                    if r.n:
                        f.write(str(r) + "\n")
