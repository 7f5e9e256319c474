import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def _ensure_input_libs():
    import moe_inputs

    need = [os.path.join(os.path.dirname(moe_inputs.__file__), n)
            for n in ("libmoe_inputs_host.so", "libmoe_inputs_dev.so")]
    if all(os.path.exists(p) for p in need):
        return
    for cmd in moe_inputs.build_commands():
        subprocess.run(cmd, check=True, capture_output=True)


_ensure_input_libs()
