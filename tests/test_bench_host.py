"""Host arithmetic of the benchmark (no GPU): the attended-pair count of the timed rows,
which sets the FLOPs of the cached call, against the oracle's token mask."""
import numpy as np
import pytest

import bench
import oracle


@pytest.mark.parametrize("n,c,local,stride", [(630, 210, 2, 4), (700, 64, 1, 3), (500, 499, 0, 2),
                                              (1000, 0, 3, 0), (777, 300, 64, 1)])
def test_attended_pairs_from(n, c, local, stride):
    for q_from in (0, c):
        rows = np.arange(q_from, n)
        ref = int(oracle.token_mask_rows(rows, n, c, local, stride).sum())
        assert bench.attended_pairs_from(n, c, local, stride, q_from) == ref
    assert bench.attended_pairs_from(n, c, local, stride, 0) == oracle.attended_pairs(n, c, local, stride)


def test_cpu_baselines_report_their_sample():
    """Both CPU figures of the benchmark run on the small workload and describe what they
    timed (the block-visiting form over whole query blocks)."""
    from lcv_inputs import WORKLOADS
    w = WORKLOADS["tiny"]
    dense = bench.cpu_baseline(w, 0.05)
    blocks = bench.cpu_baseline_blocks(w, 0.05)
    for r, kind in ((dense, "oracle"), (blocks, "oracle-block-visiting")):
        assert r["kind"] == kind and r["unit"] == "TFLOP/s" and r["value"] > 0 and r["cores"] >= 1
        assert w.name in r["sample"]
    assert "query blocks" in blocks["sample"]
