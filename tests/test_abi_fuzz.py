"""The C ABI's host-side validation and launch planning under AddressSanitizer
and UBSan: tests/native/abi_fuzz.cpp links the library's host sources (not
the kernels) with stubs for the HIP runtime calls they make, then drives the
four relayouts with random, extreme and in-contract arguments.  Every call
must return a documented status, in-contract calls must be accepted and
planned, overlapping output columns refused, with no sanitizer report."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "head_relayout_amd", "csrc")


def _has_sanitizers():
    out = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return os.path.isabs(out) and os.path.exists(out)


@pytest.mark.skipif(not _has_sanitizers(), reason="libasan not available")
def test_abi_validation_fuzz_under_sanitizers(tmp_path):
    exe = tmp_path / "abi_fuzz"
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-Wall",
                           os.path.join(ROOT, "tests", "native", "abi_fuzz.cpp"),
                           os.path.join(CSRC, "vrl_api.cpp"), os.path.join(CSRC, "vrl_plan.cpp"),
                           "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "abi fuzz ok" in r.stdout, (r.stdout[-2000:], r.stderr[-3000:])
