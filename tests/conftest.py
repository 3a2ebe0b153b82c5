import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionfinish(session, exitstatus):
    """With PALU_PARITY_SUMMARY set, write every GPU-vs-oracle comparison of
    the session (max-abs error, the share of the element bar it uses, the
    relative L2 error and its share of the relative bar) as a markdown table."""
    path = os.environ.get("PALU_PARITY_SUMMARY")
    if not path:
        return
    try:
        import palu_cases
    except ImportError:
        return
    rows = palu_cases.RESULTS
    if not rows:
        return
    with open(path, "w") as f:
        f.write("| case | fmt | elements | max abs err | of element bar | rel L2 err | of rel bar |\n")
        f.write("|---|---|---|---|---|---|---|\n")
        for what, fmt, n, mx, used, rel, relused in rows:
            f.write(f"| {what} | {fmt} | {n} | {mx:.3e} | {used:.1%} | {rel:.3e} | {relused:.1%} |\n")
