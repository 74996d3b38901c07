"""Builds libvrl.so for gfx950 with hipcc, in place next to this file."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, "vrl_kernels.hip"), os.path.join(CSRC, "vrl_plan.cpp"),
           os.path.join(CSRC, "vrl_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    "-fvisibility=hidden",
    # no packed-FP32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(out: str | None = None) -> str:
    """Compiles the library (`out`: an alternative output path)."""
    out = out or os.path.join(HERE, "libvrl.so")
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag; that warning is noise
    noise = "'-packed-fp32-ops' is not a recognized feature"
    for line in (res.stdout + res.stderr).splitlines():
        if noise not in line:
            print(line)
    if res.returncode != 0:
        raise subprocess.CalledProcessError(res.returncode, cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
