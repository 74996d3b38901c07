"""Builds harness/liblinkmodel.so (the link-paced exchange) for gfx950 with
hipcc, in place next to this file."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "csrc", "linkmodel.hip")
LIB_PATH = os.path.join(HERE, "liblinkmodel.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    "-fvisibility=hidden",
    # no packed-FP32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build() -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, SOURCE]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    for line in (res.stdout + res.stderr).splitlines():
        if noise not in line:
            print(line)
    if res.returncode != 0:
        raise subprocess.CalledProcessError(res.returncode, cmd)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
