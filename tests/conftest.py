import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    # a fresh checkout has no built library yet: build it (hipcc cross-compiles
    # for gfx950 without a GPU); a built one is used as it is.  (A copy of the
    # oracle and its pins alone, as the oracle mutation tests make, has nothing
    # to build.)
    if os.path.exists(os.path.join(ROOT, "__graft_entry__.py")):
        import __graft_entry__
        __graft_entry__.build_if_missing()


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def hip_lib():
    """The HIP library's Python binding; GPU tests fail loudly if it is not built."""
    import transformer_sequence_activation_amd as sp
    sp.load()  # raises if the shared library is missing
    return sp
