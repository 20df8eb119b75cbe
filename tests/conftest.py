import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_sessionfinish(session, exitstatus):
    """Writes the parity figures the GPU tests collected (nothing on a CPU-only run)."""
    import datetime
    import parity_log
    if not parity_log.LINES:
        return
    path = os.environ.get("LVQ_PARITY_RECORD") or os.path.join(ROOT, "gpurun_out", "parity_record.txt")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write("# GPU parity against the float64 oracle: per-case errors and near-tie listings\n")
        f.write(f"# written {datetime.datetime.now().isoformat(timespec='seconds')}, "
                f"pytest exit status {int(exitstatus)}\n")
        f.write("\n".join(parity_log.LINES) + "\n")


@pytest.fixture(scope="session")
def lvq_lib():
    """The built HIP library (GPU tests only); fails loudly when it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_bit_loop_amd import _abi
    return _abi.lib()
