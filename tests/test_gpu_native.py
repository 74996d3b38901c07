"""The C ABI driven from C++ alone: tests/native/abi_roundtrip.cpp (built by
__graft_entry__.build()) runs the whole path for six shapes, the
representative one included, with hipMalloc'd buffers and its own stream,
and checks the round trip and a few statuses."""
import os
import subprocess

import pytest

import __graft_entry__ as ge

pytestmark = pytest.mark.gpu


def test_native_abi_round_trip(gpu):
    if not os.path.exists(ge.NATIVE_TEST):
        pytest.fail(f"{ge.NATIVE_TEST} is not built; run __graft_entry__.build()")
    r = subprocess.run([ge.NATIVE_TEST], capture_output=True, text=True, timeout=180)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "C ABI round trip ok" in r.stdout
