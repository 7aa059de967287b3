import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload on the GPU")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the errors the parity tests measured (max|gpu-ref|/max|ref| per
    output, mismatch counts), one line per case, and also write them to the
    file that the environment variable MOE_PARITY_ERRORS names, if set."""
    try:
        import gpu_cases
    except Exception:
        return
    if not gpu_cases.RESULTS:
        return
    lines = []
    for test, errs in gpu_cases.RESULTS:
        vals = " ".join(f"{k}={v:.2e}" if isinstance(v, float) else f"{k}={v}"
                        for k, v in errs.items())
        lines.append(f"{test}: {vals}")
    terminalreporter.write_sep("-", "measured parity errors")
    for line in lines:
        terminalreporter.write_line(line)
    path = os.environ.get("MOE_PARITY_ERRORS")
    if path:
        with open(path, "w") as fh:
            fh.write("\n".join(lines) + "\n")
