"""Checks of the seeded input generator (no GPU)."""
import numpy as np

import datagen
from datagen import PAD_SENTINEL, WORKLOADS


def _f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_splitmix64_published_sequence():
    # First outputs of SplitMix64 from state 0, as published with the
    # reference implementation (Vigna, splitmix64.c).
    got = datagen.splitmix64(3, 0)
    assert [int(x) for x in got] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_prefix_property():
    a = datagen.values(1001, "normal", seed=3, stream=7)
    b = datagen.values(1000, "normal", seed=3, stream=7)
    np.testing.assert_array_equal(a[:1000], b)
    u = datagen.values(999, "uniform8", seed=3, stream=7)
    np.testing.assert_array_equal(u, datagen.values(1500, "uniform8", seed=3, stream=7)[:999])


def test_streams_and_seeds_differ():
    a = datagen.values(4096, seed=1, stream=0)
    assert not np.array_equal(a, datagen.values(4096, seed=1, stream=1))
    assert not np.array_equal(a, datagen.values(4096, seed=2, stream=0))


def test_normal_moments():
    x = _f32(datagen.values(1 << 20, "normal", seed=1, stream=0)).astype(np.float64)
    assert abs(x.mean()) < 0.005
    assert abs(x.std() - 1.0) < 0.005
    assert np.isfinite(x).all()


def test_uniform8_range_and_specials():
    bits = datagen.values(1 << 20, "uniform8", seed=1, stream=0)
    x = _f32(bits)
    assert np.isfinite(x).all() and (x >= -8).all() and (x <= 8).all()
    special = (bits & 0x7F80) == 0
    frac = special.mean()
    assert abs(frac - 1 / 32) < 0.002
    assert (bits == 0x0000).any() and (bits == 0x8000).any()
    sub = special & ((bits & 0x7F) != 0)
    assert sub.any() and (bits[sub] >> 15).min() == 0 and (bits[sub] >> 15).max() == 1


def test_fused_source_layout():
    w = WORKLOADS[1]
    a0, a1 = datagen.fused_source(w, 0), datagen.fused_source(w, 1)
    assert a0.shape == (w.s_local, 3 * w.H * w.D)
    assert not np.array_equal(a0, a1)
    np.testing.assert_array_equal(a0, datagen.fused_source(w, 0))


def test_padding_rows_and_columns():
    from dataclasses import replace
    w = replace(WORKLOADS[4], s_local=40, H=4, D=8, total_tokens=75, row_pad=5)
    a1 = datagen.fused_source(w, 1)
    hd3 = 3 * w.H * w.D
    assert (a1[:, hd3:] == PAD_SENTINEL).all()
    assert (a1[35:, :hd3] == 0).all() and (a1[:35, :hd3] != 0).any()
    o = datagen.attention_output(w, 0)
    assert (o[75:] == 0).all()


def test_workload_shapes():
    assert WORKLOADS[3].S == 55414 and WORKLOADS[3].n_pad_tokens == 1 and WORKLOADS[3].G == 28
    assert WORKLOADS[4].row_stride == 21568
    assert WORKLOADS[5].S == 31008 and WORKLOADS[5].n_pad_tokens == 8 and WORKLOADS[5].G == 8
