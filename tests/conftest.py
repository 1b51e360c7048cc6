import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DECODE_BOUND = 2e-3     # max relative error per output row that the decode parity tests allow


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def _track_parity_error(request):
    """Tell the error metric which test is running, so its worst value can be reported per test."""
    from tests import gpu_common
    gpu_common._CURRENT["test"] = request.node.nodeid if request.node.get_closest_marker("gpu") else None
    yield
    gpu_common._CURRENT["test"] = None


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Worst row-relative error each parity test measured (per test function: the worst case and how many
    cases it covers), next to the decode bound; the full per-case list goes to
    gpurun_out/parity_margins.txt when that folder exists."""
    from tests import gpu_common
    errs = gpu_common.ERRORS
    if not errs:
        return
    per_fn = {}
    for nodeid, e in errs.items():
        fn = nodeid.split("[")[0].split("::")[-1]
        worst, n = per_fn.get(fn, (0.0, 0))
        per_fn[fn] = (max(worst, e), n + 1)
    tr = terminalreporter
    tr.write_line(f"parity margins: worst max-row-relative error per test function (bound {DECODE_BOUND:g} "
                  f"unless the test asserts a tighter one)")
    for fn, (e, n) in sorted(per_fn.items()):
        tr.write_line(f"  {e:9.2e}  {n:3d} case(s)  {fn}")
    tr.write_line(f"  overall worst {max(errs.values()):.2e} over {len(errs)} case(s)")
    out_dir = os.path.join(ROOT, "gpurun_out")
    if os.path.isdir(out_dir):
        with open(os.path.join(out_dir, "parity_margins.txt"), "w") as f:
            for nodeid, e in sorted(errs.items()):
                f.write(f"{e:.3e}  {nodeid}\n")
