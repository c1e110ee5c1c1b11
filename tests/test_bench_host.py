"""Host-side checks of bench.py's measurement set-up (no GPU needed)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("sizes", [
    # decode T=1: the gate/up launch, the down weights, the layer, 1 GiB
    [106_973_184, 53_477_376, 162_562_048, 1 << 30],
    # prefill T=2048: the gate/up launch (every expert) and the layer exceed 1 GiB;
    # a fixed 2 GiB buffer with two regions per size would end past the buffer
    [1_749_000_000, 874_500_000, 2_640_000_000, 1 << 30],
    [4096],
])
def test_probe_regions_stay_inside_the_buffer(sizes):
    total, regions = bench.probe_regions(sizes)
    assert total >= 2 << 30
    assert len(regions) == len(sizes)
    for (nbytes, nreg), s in zip(regions, sizes):
        assert nbytes % 4096 == 0 and 0 < nbytes <= s
        assert nreg >= 2, (nbytes, total)
        # every launch r reads [(r % nreg) * nbytes, + nbytes)
        assert (nreg - 1) * nbytes + nbytes <= total


def test_probe_regions_refuse_empty_sizes():
    with pytest.raises(ValueError):
        bench.probe_regions([100])
    with pytest.raises(ValueError):
        bench.probe_regions([])
