import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_host_libs():
    """Builds the gcc-built host libraries (oracle, input generator) only when
    they are missing; the usual flow builds everything first with
    __graft_entry__.build()."""
    from datagen import build as dg_build
    from oracle import build as or_build

    for mod, name in ((dg_build, "libdatagen.so"), (or_build, "liboracle.so")):
        if not os.path.exists(os.path.join(mod.HERE, name)):
            mod.build()


_ensure_host_libs()


@pytest.fixture(scope="session")
def vrl_lib():
    """The relayout library (ctypes), built with hipcc only if it is missing."""
    from head_relayout_amd import _lib, build as vrl_build

    if not os.path.exists(_lib.LIB_PATH):
        vrl_build.build()
    return _lib.lib()


@pytest.fixture(scope="session")
def gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("a gpu-marked test ran without a visible GPU")
    return torch.device("cuda:0")
