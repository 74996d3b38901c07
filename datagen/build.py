"""Builds libdatagen.so (plain C, gcc, OpenMP) next to this file."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build() -> str:
    src = os.path.join(HERE, "datagen.c")
    out = os.path.join(HERE, "libdatagen.so")
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
                           "-Wall", "-Wextra", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
