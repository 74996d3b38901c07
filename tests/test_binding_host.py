"""Argument checks of the torch binding that need no GPU: wrong dtype, host
tensors, wrong shapes and wire sizes raise before the library is called."""
import pytest
import torch

import head_relayout_amd as vrl


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
