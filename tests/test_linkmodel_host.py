"""Host-side checks of the link-paced stand-in exchange
(harness/csrc/linkmodel.hip): every malformed call is refused before any HIP
call or launch, so these run without a GPU."""
import ctypes
import os

import pytest

from harness import build as lm_build
from harness import linkmodel


@pytest.fixture(scope="module", autouse=True)
def _library():
    """The library, built with hipcc only if it is missing."""
    if not os.path.exists(lm_build.LIB_PATH):
        lm_build.build()


def _blocks(*specs):
    arr = (linkmodel.Block * len(specs))()
    for i, (src, dst, n, paced) in enumerate(specs):
        arr[i] = linkmodel.Block(src, dst, n, paced)
    return arr


@pytest.mark.parametrize("blocks, n, rate, why", [
    (None, 1, 153.0, "1 to 64 blocks"),
    (_blocks((0x1000, 0x9000, 64, 1)), 0, 153.0, "1 to 64 blocks"),
    (_blocks((0x1000, 0x9000, 64, 1)), 65, 153.0, "1 to 64 blocks"),
    (_blocks((0x1000, 0x9000, 64, 1)), 1, 0.5, "link rate"),
    (_blocks((0x1000, 0x9000, 64, 1)), 1, 20000.0, "link rate"),
    (_blocks((0x1000, 0x9000, 64, 1)), 1, float("nan"), "link rate"),
    (_blocks((0, 0x9000, 64, 1)), 1, 153.0, "null pointer or no bytes"),
    (_blocks((0x1000, 0x9000, 0, 1)), 1, 153.0, "null pointer or no bytes"),
    (_blocks((0x1001, 0x9000, 64, 1)), 1, 153.0, "2-byte aligned"),
    (_blocks((0x1000, 0x9000, 63, 1)), 1, 153.0, "2-byte aligned"),
    (_blocks((0x1000, 0x1020, 64, 1)), 1, 153.0, "overlap"),
    (_blocks((0x1000, 0x9000, 64, 1), (0x20000, 0x20000, 64, 0)), 2, 153.0, "overlap"),
])
def test_malformed_exchanges_are_refused(blocks, n, rate, why):
    L = linkmodel.lib()
    ptr = None if blocks is None else ctypes.cast(blocks, ctypes.POINTER(linkmodel.Block))
    assert L.lm_exchange(ptr, n, rate, None) == 1
    assert why in L.lm_last_error().decode()
