"""Checks of the torch binding that need no GPU: wrong dtype, host tensors,
wrong shapes and wire sizes raise before the library is called; a missing
library raises; the device path and the oracle share no code."""
import os
import re
import subprocess
import sys

import pytest
import torch

import head_relayout_amd as vrl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_rejects_host_tensors_and_wrong_dtype():
    q = torch.zeros(4, 4, 8, dtype=torch.bfloat16)
    packed = torch.zeros(3 * 4 * 4 * 8, dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="HIP device"):
        vrl.qkv_pack(q, q, q, packed, 2, 2)
    with pytest.raises(TypeError, match="bfloat16"):
        vrl.qkv_pack(q.float(), q, q, packed, 2, 2)


def test_sizes_and_offsets():
    assert vrl.exchange_elems(vrl.VRL_EXCHANGE_QKV, 2, 4, 27707, 56, 128) == 595811328
    assert vrl.exchange_elems(vrl.VRL_EXCHANGE_ATTN, 2, 4, 27707, 56, 128) == 198603776
    assert [vrl.chunk_offset(c, 2, 4, 27707, 56, 128) for c in range(5)] == [0, 6927, 13854, 20781, 27707]
    assert vrl.chunk_offset(2, 2, 4, 27707, 56, 128, chunk_heads=True) == 14
    with pytest.raises(ValueError):
        vrl.exchange_elems(0, 3, 4, 27707, 56, 128)        # 56 heads over 3 ranks
    with pytest.raises(ValueError):
        vrl.chunk_offset(5, 2, 4, 27707, 56, 128)


def test_missing_library_raises_instead_of_falling_back():
    """With libvrl.so absent the binding raises on first use; there is no
    other path to take."""
    code = ("import head_relayout_amd._lib as L\n"
            "L.LIB_PATH = '/nonexistent/libvrl.so'\n"
            "L._lib = None\n"
            "import head_relayout_amd as vrl\n"
            "try:\n"
            "    vrl.exchange_elems(vrl.VRL_EXCHANGE_QKV, 2, 4, 16, 8, 8)\n"
            "except RuntimeError as e:\n"
            "    print('raised', e)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("raised") and "missing" in r.stdout


def test_product_and_oracle_share_no_code():
    """The device path (package and its C sources) never refers to the
    oracle, and the oracle never refers to the device path; both may use
    only the seeded input generator."""
    def sources(d):
        for dirpath, _, files in os.walk(os.path.join(ROOT, d)):
            for f in files:
                if f.endswith((".py", ".c", ".cpp", ".h", ".hip")):
                    yield os.path.join(dirpath, f)

    for path in sources("head_relayout_amd"):
        text = open(path).read()
        assert not re.search(r"\bimport oracle\b|\bfrom oracle\b|oracle\.h|oracle\.c", text), path
    for path in list(sources("oracle")) + list(sources("datagen")):
        text = open(path).read()
        assert "head_relayout_amd" not in text and "vrl.h" not in text and "vrl_" not in text, path
