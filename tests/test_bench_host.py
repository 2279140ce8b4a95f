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
