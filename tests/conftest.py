import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped, not failed, where no GPU is visible; the CPU suite is
    # run with -m "not gpu" anyway.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(scope="session")
def rocrand_ref(tmp_path_factory):
    """Philox4x32-10 blocks from rocRAND's host-callable engine, run as a library.

    Returns run(pairs) -> uint64 array [len(pairs), 4]: the four words of the block at
    counter c under seed s, for each (s, c).  An implementation of the SC'11 definition
    written independently of the oracle's."""
    import shutil
    import subprocess

    import numpy as np
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_kernel.h"):
        pytest.skip("hipcc / rocRAND headers not available")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_ref")
    subprocess.run([hipcc, "-O1", "-o", exe, os.path.join(ROOT, "tests", "pins", "philox_rocrand_ref.cpp")],
                   check=True, capture_output=True)

    def run(pairs):
        text = "".join(f"{s} {c}\n" for s, c in pairs)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return np.array([[int(w, 16) for w in line.split()] for line in out.strip().splitlines()],
                        dtype=np.uint64)
    return run
