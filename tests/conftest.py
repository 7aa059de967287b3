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
    output, mismatch counts), one line per case, and keep them in
    gpurun_out/parity_errors.txt when that folder exists."""
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
    out = os.path.join(ROOT, "gpurun_out")
    if os.path.isdir(out):
        with open(os.path.join(out, "parity_errors.txt"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
