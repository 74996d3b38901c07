"""The oracle built with AddressSanitizer and UBSan (gcc, host code only) runs
its chains on tiny shapes of both chunk readings, views with padding and
head-major strides included, without a memory or undefined-behaviour error."""
import os
import subprocess
import sys
import textwrap

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _libasan():
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(_libasan() is None, reason="libasan not available")
def test_oracle_under_asan(tmp_path):
    so = tmp_path / "liboracle_asan.so"
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fopenmp", "-fPIC", "-shared", "-o", str(so), SRC])
    script = textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        import numpy as np
        import oracle
        from tests.test_oracle import _round_trip
        from tests.test_oracle_head_chunks import _path
        from tests.helpers import unique_fused, padded_view, unique_ids
        with oracle.library({str(so)!r}):
            for shape in [(2, 4, 10, 4, 8, 3), (3, 2, 7, 6, 8, 0), (1, 1, 1, 1, 1, 0)]:
                P, C, S_l, H, D, pad = shape
                _round_trip(P, C, S_l, H, D, unique_fused(P, S_l, H, D, pad))
                d = oracle.dims(P, C, S_l, H, D)
                out, _ = padded_view(S_l, H, D, head_major=True)
                oracle.head_merge(d, unique_ids(S_l * H * D), out, 0, 1)
            for shape in [(2, 2, 6, 8, 8, 1), (2, 4, 3, 8, 8, 0)]:
                P, C, S_l, H, D, pad = shape
                _path(P, C, S_l, H, D, unique_fused(P, S_l, H, D, pad), True)
        print("asan ok")
    """)
    preload = " ".join(x for x in (_libasan(), os.environ.get("LD_PRELOAD", "")) if x)
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0",
               OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, env=env,
                       timeout=300)
    assert r.returncode == 0 and "asan ok" in r.stdout, r.stderr[-3000:]
