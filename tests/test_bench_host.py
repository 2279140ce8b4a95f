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


def _write_pmc(directory, counter, rows):
    import csv
    import os
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_traffic_calibration_uses_the_last_three_copies(tmp_path):
    """The HBM byte counts scale each counter by the 1 GiB calibration copies that end the
    run; a copy of another size earlier in the run (the plain copy of Q) must not enter it."""
    import json
    kib = bench.COPY_BYTES // 1024
    copy = "__amd_rocclr_copyBuffer"
    fetch = [(copy, 1.5), ("void lcv::bsa_fwd_kernel<true>", 1000.0), ("lcv::rope3d_kernel", 300.0),
             ("void lcv::qk_prologue_kernel<true>", 310.0)] + [(copy, 100.0)] * 5 + [(copy, kib / 2)] * 3
    write = [(copy, 0.03), ("void lcv::bsa_fwd_kernel<true>", 400.0), ("lcv::rope3d_kernel", 600.0),
             ("void lcv::qk_prologue_kernel<true>", 600.0)] + [(copy, 200.0)] * 5 + [(copy, kib)] * 3
    _write_pmc(tmp_path / "f", "FETCH_SIZE", fetch)
    _write_pmc(tmp_path / "w", "WRITE_SIZE", write)
    out = tmp_path / "t.json"
    assert bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(out)) == 0
    d = json.loads(out.read_text())
    assert d["bsa_fwd_kernel"]["fetch_bytes"] == 1000.0 * 2048
    assert d["bsa_fwd_kernel"]["write_bytes"] == 400.0 * 1024
    assert d["rope3d_kernel"]["bytes_per_launch"] == 300.0 * 2048 + 600.0 * 1024
    assert d["qk_prologue_kernel"]["FETCH_SIZE"]["copy_kib"] == kib / 2
    assert bench.traffic_from_profile(str(out), "rope3d_kernel") == 300.0 * 2048 + 600.0 * 1024


def test_traffic_calibration_refuses_disagreeing_copies(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    rows = [("void lcv::bsa_fwd_kernel<true>", 1.0), ("lcv::rope3d_kernel", 1.0),
            ("void lcv::qk_prologue_kernel<true>", 1.0), (copy, 100.0), (copy, 500.0), (copy, 500.0)]
    _write_pmc(tmp_path / "f", "FETCH_SIZE", rows)
    _write_pmc(tmp_path / "w", "WRITE_SIZE", rows)
    assert bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "t.json")) == 1


def test_counter_summary_per_kernel(tmp_path, capsys):
    """--summarize-counters: per-kernel means over the dispatches and the matrix-core share
    SQ_VALU_MFMA_BUSY_CYCLES / (128 * GRBM_GUI_ACTIVE)."""
    import csv
    import json
    d = tmp_path / "pmc"
    d.mkdir()
    with open(d / "p_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        name = "void lcv::(anonymous namespace)::bsa_fwd_kernel<true, false, false, false>(lcv::FwdParams)"
        for i, (busy, gui, mfma, valu) in enumerate(((1280.0, 20.0, 40.0, 250.0), (1920.0, 30.0, 60.0, 390.0))):
            for c, v in (("SQ_VALU_MFMA_BUSY_CYCLES", busy), ("GRBM_GUI_ACTIVE", gui), ("SQ_INSTS_MFMA", mfma),
                         ("SQ_INSTS_VALU", valu)):
                w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": c, "Counter_Value": v})
    assert bench.summarize_counters(str(d)) == 0
    out = [json.loads(l) for l in capsys.readouterr().out.splitlines()]
    assert len(out) == 1 and out[0]["kernel"] == "bsa_fwd_kernel<true, false, false, false>"
    assert out[0]["dispatches"] == 2
    assert out[0]["mfma_busy"] == round(1600.0 / (128 * 25.0), 4)
    assert out[0]["valu_per_mfma"] == round(320.0 / 50.0, 3)
