import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large workload parity (GPU)")


@pytest.fixture(scope="session")
def gpu_ok():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return True


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Worst parity figures of the GPU checks that ran (errors against the oracle, and
    each error over its tolerance where the tolerance is per element)."""
    try:
        from tests import gpu_check
    except Exception:  # pragma: no cover
        return
    if not gpu_check.WORST:
        return
    tr = terminalreporter
    tr.write_sep("-", "worst parity figures against the oracle")
    for tag in sorted(gpu_check.WORST):
        vals = gpu_check.WORST[tag]
        tr.write_line(f"{tag}: " + ", ".join(f"{k}={v:.3g}" for k, v in sorted(vals.items())))
