"""CPU checks of the work accounting behind bench.py's numbers: the visible
(query, key) pair counts that turn a measured time into algorithmic TFLOP/s
are compared with a count taken over the literal mask of the oracle, and the
committed HBM-traffic records are read back for the current kernel sources."""

import numpy as np
import pytest

import bench
from oracle.attention import visible


def _pairs_full(T, k):
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    return int(np.sum(visible(i, j, k)))


@pytest.mark.parametrize("T,k", [(1, 1), (7, 3), (100, 16), (97, 1), (50, 64), (34320 // 40, 1560 // 40)])
def test_full_pairs_match_mask(T, k):
    assert bench.full_pairs_per_head(T, k) == _pairs_full(T, k)


@pytest.mark.parametrize("kpf,C,prefix,B", [(4, 3, 7, 1), (5, 3, 0, 1), (3, 4, 2, 2), (6, 3, 1, 3), (2, 2, 5, 9)])
def test_stream_pairs_match_mask(kpf, C, prefix, B):
    Tq = C * kpf
    unit = min(B, C) * kpf
    i = np.arange(Tq)[:, None]
    j = np.arange(Tq)[None, :]
    literal = Tq * prefix * kpf + int(np.sum(visible(i, j, unit)))
    assert bench.stream_pairs_per_head(kpf, C, prefix, B) == literal


def test_headline_work_figures():
    # the Wan-1.3B step: 3 chunk frames of 1,560 tokens behind 7 cached frames
    assert bench.stream_pairs_per_head(1560, 3, 7) == 65_707_200
    assert 4 * 128 * 12 * 65_707_200 == 403_705_036_800  # 4.037e11 FLOP per step
    # the 34,320-token full form: 22 frames of 1,560 tokens
    assert bench.full_pairs_per_head(34_320, 1560) == 615_700_800


@pytest.mark.parametrize("workload", ["wan13b_stream_step", "full_block_causal", "wan14b_stream_step",
                                      "full_block_causal_bwd", "wan13b_stream_step_bwd"])
def test_traffic_records_parse(workload):
    """Each committed counter record parses to a positive byte count; a record
    taken on other kernel sources is reported as absent (bench.py then prints
    no traffic figure), which this test reports as a skip."""
    import os
    path = bench.TRAFFIC_FILE.format(workload=workload)
    assert os.path.exists(path)
    t = bench.read_traffic(workload)
    if t is None:
        pytest.skip("counter record predates the current kernel sources")
    assert t > 0
