"""The link-paced stand-in exchange (harness/csrc/linkmodel.hip) on the GPU:
a paced block takes its bytes / link rate (within a tolerance), blocks on
distinct links run at the same time, unpaced blocks run at copy speed, and
every block arrives bit for bit."""
import pytest
import torch

from harness import linkmodel
from tests.gpu_harness import say

pytestmark = pytest.mark.gpu

N = 38_250_000          # elements: 76.5 MB per block, 0.5 ms at 153 GB/s


def _time(pairs, rate):
    """Median of three timed calls after one untimed call (the first launch of
    a new grid size pays a one-off cost)."""
    linkmodel.exchange(pairs, rate)
    ts = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        linkmodel.exchange(pairs, rate)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return sorted(ts)[1]


def test_pacing_follows_the_link_rate(gpu):
    src = [torch.empty(N, dtype=torch.int16, device=gpu).random_(-30000, 30000) for _ in range(2)]
    dst = [torch.zeros(N, dtype=torch.int16, device=gpu) for _ in range(2)]
    target_ms = N * 2 / 153e9 * 1e3
    for rate in (153.0, 306.0):
        say(f"[link model] one paced block at {rate} GB/s")
        for d in dst:
            d.zero_()
        ms = _time([(src[0], dst[0], True)], rate)
        want = target_ms * 153.0 / rate
        assert 0.95 * want <= ms <= 1.15 * want, f"{ms:.3f} ms for one block at {rate} GB/s, expected {want:.3f}"
        assert torch.equal(dst[0], src[0])
    say("[link model] two paced blocks on two links")
    for d in dst:
        d.zero_()
    ms = _time([(src[0], dst[0], True), (src[1], dst[1], True)], 153.0)
    assert 0.95 * target_ms <= ms <= 1.15 * target_ms, f"{ms:.3f} ms for two links, expected {target_ms:.3f}"
    assert torch.equal(dst[0], src[0]) and torch.equal(dst[1], src[1])
    say("[link model] unpaced block")
    dst[0].zero_()
    ms = _time([(src[0], dst[0], False)], 153.0)
    assert ms < 0.8 * target_ms, f"an unpaced block took {ms:.3f} ms"
    assert torch.equal(dst[0], src[0])
    say("[link model] ok")
