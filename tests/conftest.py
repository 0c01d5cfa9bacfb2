import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running oracle comparison")
    # The seeded input generator's C core; built here if this tree has none.
    so = os.path.join(ROOT, "synth", "_philox_words.so")
    if not os.path.exists(so):
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-shared", "-fPIC",
                               os.path.join(ROOT, "synth", "philox_words.c"), "-o", so, "-lm"])


@pytest.fixture(scope="session")
def gpu_available():
    import torch
    return torch.cuda.is_available()
