import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    # Name the case on stderr, flushed, before any GPU work starts, so that a
    # run which dies inside a kernel still says which case it was in.
    if request.node.get_closest_marker("gpu") is not None:
        sys.stderr.write(f"\n[gpu case] {request.node.nodeid}\n")
        sys.stderr.flush()
    yield


def pytest_terminal_summary(terminalreporter):
    # Parity margins of every GPU-versus-oracle comparison made in this
    # session: the worst err / bound per test (1.0 = at the bar), under the
    # bar the tests use (2e-3 + (2e-3 + u_dtype) |ref|) and under the plain
    # 2e-3 + 2e-3 |ref|.  Also written as JSON when PA_MARGINS_JSON names a
    # file.
    from tests import harness

    if not harness.MARGINS:
        return
    per = {}
    for m in harness.MARGINS:
        k = (m["test"], m["dtype"])
        cur = per.get(k)
        if cur is None:
            per[k] = dict(m, calls=1)
        else:
            cur["calls"] += 1
            cur["n"] += m["n"]
            for f in ("max_abs_err", "max_err_over_bound", "max_err_over_plain_bound"):
                cur[f] = max(cur[f], m[f])
            cur["n_outside_plain_bound"] += m["n_outside_plain_bound"]
    tr = terminalreporter
    tr.write_sep("-", "parity margins (worst err/bound per test; 1.0 = at the bar)")
    for (test, dt), m in sorted(per.items()):
        tr.write_line(f"{m['max_err_over_bound']:.3f} bar  {m['max_err_over_plain_bound']:.3f} plain "
                      f"({m['n_outside_plain_bound']} of {m['n']} outside plain)  {dt:4s} "
                      f"max|err| {m['max_abs_err']:.2e}  {test}")
    out = os.environ.get("PA_MARGINS_JSON")
    if out:
        import json

        with open(out, "w") as f:
            json.dump(sorted(per.values(), key=lambda m: m["test"]), f, indent=1)
