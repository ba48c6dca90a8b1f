import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    oracle.build(force=False)
    return oracle


def pytest_terminal_summary(terminalreporter):
    """One line per gradient tensor kind: how many compared elements lie beyond the strict 2e-2 (they pass on
    the bf16 rounding term of parity.grad_bound) and the smallest |ref| among them."""
    try:
        import parity
    except ImportError:
        return
    if not parity.STRICT_LOG:
        return
    kinds = {}
    for name, n, over, min_ref, worst in parity.STRICT_LOG:
        k = kinds.setdefault(name, [0, 0, 0, None, 0.0])
        k[0] += 1
        k[1] += n
        k[2] += over
        if min_ref is not None:
            k[3] = min_ref if k[3] is None else min(k[3], min_ref)
        k[4] = max(k[4], worst)
    for name, (calls, n, over, min_ref, worst) in sorted(kinds.items()):
        terminalreporter.write_line(
            f"gradient parity {name}: {calls} compares, {n} elements, max|err| {worst:.3e}, beyond strict 2e-2: "
            f"{over}" + (f" (smallest |ref| among them {min_ref:.3f})" if over else ""))
