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


def test_bench_refuses_several_gpus():
    """One GPU only: asking for more exits with a message and status 2, before any GPU work."""
    import subprocess
    import sys
    from pathlib import Path
    root = Path(__file__).resolve().parent.parent
    res = subprocess.run([sys.executable, str(root / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                         timeout=120, cwd=root)
    assert res.returncode == 2
    assert "one GPU" in res.stderr + res.stdout
