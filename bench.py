#!/usr/bin/env python3
"""Benchmark of LongCat-Video block-sparse 3D self-attention on one MI355X.

One step = one pass of the hot path over one batch of synthetic input: the attention
forward with the 3D-RoPE fused into its Q/K loads, over the prebuilt block layout (the
layout is built once per shape and reused; its build time is reported separately).
The default workload is T2V 720x1280, 93 frames: latent 24x45x80 = 86,400 tokens,
32 heads of 64 channels, bf16, local window 2 + global stride 4 blocks.

Prints one JSON line: effective attended TFLOP/s = 4 * 64 * attended token pairs *
heads / time, the MFMA roofline of the attention kernel and the fp64 oracle timed on the
host's cores over a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from lcv_inputs import WORKLOADS, bf16_bits_to_f64, workload_inputs  # noqa: E402

METRIC = "effective attended TFLOP/s + % MFMA peak, 720p 93-frame block-sparse attn"
MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# The kernels whose HBM traffic is taken from counters, with the sources each is built from:
# a counter summary is valid only for the kernel code it was taken on.
TRAFFIC_KERNELS = {
    "bsa_fwd_kernel": ("bsa_fwd_kernel.hip", "attn_tile.h", "lcv_internal.h", "rope_math.h"),
    "rope3d_kernel": ("rope3d_kernel.hip", "lcv_internal.h", "rope_math.h"),
    "qk_prologue_kernel": ("qk_prologue_kernel.hip", "lcv_internal.h", "rope_math.h"),
}


def kernel_source_hash(kernel: str = "bsa_fwd_kernel") -> str:
    """sha256 over a kernel's sources."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_attention_lcv_amd", "csrc")
    for name in TRAFFIC_KERNELS[kernel]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_from_profile(path: str | None, kernel: str = "bsa_fwd_kernel"):
    """HBM bytes per launch of a kernel from a committed counter summary (FETCH_SIZE +
    WRITE_SIZE scaled by the copy-kernel calibration); None when absent or taken on other
    kernel sources."""
    if not path or not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            data = json.load(f)[kernel]
        if data.get("kernel_source_sha256") != kernel_source_hash(kernel):
            return None
        return float(data["bytes_per_launch"])
    except Exception:
        return None


COPY_BYTES = 1 << 30


def _pmc_rows(directory: str, counter: str):
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"]),
                                 int(r.get("Dispatch_Id") or 0)))
    rows.sort(key=lambda r: r[2])
    return rows


def summarize_traffic(fetch_dir: str, write_dir: str, out_path: str) -> int:
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the attention kernel, the K RoPE pass and
    the QK prologue, each scaled by what the same counter reads for a plain copy of COPY_BYTES
    (read COPY_BYTES, write COPY_BYTES)."""
    result = {}
    for kernel in TRAFFIC_KERNELS:
        entry = {}
        for counter, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
            rows = _pmc_rows(directory, counter)
            vals = [v for name, v, _ in rows if kernel in name]
            if not vals and kernel != "bsa_fwd_kernel":
                break   # a side pass this run did not launch
            # the calibration copies are the last three copy dispatches of the run (bench.py
            # --copy-calibration issues them after everything else); other copies (the plain
            # copy of Q beside the RoPE pass) have other sizes
            copies = [v for name, v, _ in rows
                      if "copybuffer" in name.lower() or "copy_kernel" in name.lower()][-3:]
            if not vals or len(copies) < 3:
                print(f"no {counter} rows for {kernel} or the copy kernel in {directory}", file=sys.stderr)
                return 1
            if max(copies) > 1.01 * min(copies):
                print(f"{counter}: the last three copies disagree ({copies})", file=sys.stderr)
                return 1
            copy_kib = float(np.median(copies))
            scale = COPY_BYTES / (copy_kib * 1024.0)
            entry[counter] = {"kib_per_launch": float(np.median(vals)), "copy_kib": copy_kib,
                              "scale_bytes_per_kib": scale * 1024.0, "launches": len(vals)}
        if len(entry) < 2:
            continue
        fetch = entry["FETCH_SIZE"]["kib_per_launch"] * entry["FETCH_SIZE"]["scale_bytes_per_kib"]
        write = entry["WRITE_SIZE"]["kib_per_launch"] * entry["WRITE_SIZE"]["scale_bytes_per_kib"]
        entry.update({"bytes_per_launch": fetch + write, "fetch_bytes": fetch, "write_bytes": write,
                      "kernel_source_sha256": kernel_source_hash(kernel)})
        result[kernel] = entry
    with open(out_path, "w") as f:
        json.dump(result, f, indent=1)
    print(json.dumps(result))
    return 0


def summarize_counters(directory: str) -> int:
    """Per-kernel averages over the dispatches of every counter in a rocprofv3 --pmc run
    (one JSON object per kernel name), with the matrix-core utilisation where the run has
    the counters for it: SQ_VALU_MFMA_BUSY_CYCLES / (128 * GRBM_GUI_ACTIVE), the busy count
    being summed over the 1,024 SIMDs and GRBM_GUI_ACTIVE over the 8 XCDs."""
    import csv
    import glob
    import re
    acc: dict = {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                m = re.search(r"::(\w+_kernel(<[^>]*>)?)", r["Kernel_Name"])
                name = m.group(1) if m else r["Kernel_Name"][:60]
                acc.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    for name, counters in acc.items():
        out = {"kernel": name, "dispatches": max(len(v) for v in counters.values())}
        avg = {c: float(np.mean(v)) for c, v in counters.items()}
        out.update({c: round(v, 1) for c, v in avg.items()})
        if avg.get("GRBM_GUI_ACTIVE") and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            out["mfma_busy"] = round(avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (128 * avg["GRBM_GUI_ACTIVE"]), 4)
        if avg.get("SQ_VALU_MFMA_BUSY_CYCLES") and "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
            out["coexec_of_mfma_busy"] = round(avg["SQ_VALU_MFMA_COEXEC_CYCLES"] / avg["SQ_VALU_MFMA_BUSY_CYCLES"], 4)
        if avg.get("SQ_INSTS_MFMA") and "SQ_INSTS_VALU" in avg:
            out["valu_per_mfma"] = round(avg["SQ_INSTS_VALU"] / avg["SQ_INSTS_MFMA"], 3)
        print(json.dumps(out))
    return 0 if acc else 1


def cpu_baseline(w, seconds: float = 12.0) -> dict:
    """The fp64 oracle on a bounded sample: one head, as many query rows as fit the
    time budget (doubling from 256), scaled to effective attended TFLOP/s."""
    import oracle
    from lcv_inputs import qkv_bits
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    qb, kb, vb = qkv_bits(w.seed, 1, 1, w.n_tokens)
    q, k, v = bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb)
    rng = np.random.default_rng(0)
    rows_n = 256
    best = None
    t_total = 0.0
    while True:
        rows = np.sort(rng.choice(w.n_tokens, size=min(rows_n, w.n_tokens), replace=False))
        t0 = time.perf_counter()
        oracle.bsa_forward(q, k, v, w.grid, w.cond_len, w.local_blocks, w.global_stride, w.theta, rows=rows)
        dt = time.perf_counter() - t0
        t_total += dt
        mask = oracle.token_mask_rows(rows, w.n_tokens, w.cond_len, w.local_blocks, w.global_stride)
        flops = 4.0 * 64 * float(mask.sum())
        best = (rows.size, dt, flops)
        if t_total >= seconds or rows_n >= w.n_tokens or dt * 2 + t_total > 3 * seconds:
            break
        rows_n *= 2
    n_rows, dt, flops = best
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "cpu": cpu_model(), "sample": f"{w.name}: 1 of {w.heads} heads, {n_rows} random query rows of {w.n_tokens} "
                      f"(fp64 numpy oracle: RoPE + masked dense attention), {dt:.2f} s"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_blocks(w, seconds: float = 10.0) -> dict:
    """The oracle's block-visiting form (each query block attends only the key blocks its CSR
    row lists, fp64) on a bounded sample: one head, as many random query blocks as fit the
    time budget (doubling from 4), scaled to effective attended TFLOP/s: the like-for-like
    CPU analogue of a block-sparse CPU implementation."""
    import oracle
    from lcv_inputs import qkv_bits
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    qb, kb, vb = qkv_bits(w.seed, 1, 1, w.n_tokens)
    q, k, v = bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb)
    n_blocks = -(-w.n_tokens // 64)
    rng = np.random.default_rng(1)
    count = 4
    t_total = 0.0
    while True:
        blocks = rng.choice(n_blocks, size=min(count, n_blocks), replace=False)
        t0 = time.perf_counter()
        oracle.bsa_forward_blocks(q, k, v, w.grid, w.cond_len, w.local_blocks, w.global_stride, w.theta,
                                  q_blocks=blocks)
        dt = time.perf_counter() - t0
        t_total += dt
        rows = np.concatenate([np.arange(64 * i, min(64 * i + 64, w.n_tokens)) for i in blocks])
        flops = 4.0 * 64 * float(oracle.token_mask_rows(rows, w.n_tokens, w.cond_len, w.local_blocks,
                                                        w.global_stride).sum())
        best = (blocks.size, dt, flops)
        if t_total >= seconds or count >= n_blocks or dt * 2 + t_total > 3 * seconds:
            break
        count *= 2
    n_b, dt, flops = best
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle-block-visiting",
            "cpu": cpu_model(),
            "sample": f"{w.name}: 1 of {w.heads} heads, {n_b} random query blocks of {n_blocks} (fp64 numpy "
                      f"oracle visiting only the CSR's key blocks: RoPE + attention), {dt:.2f} s"}


def timed_launches(torch, stream, launch, count: int) -> float:
    """Average milliseconds per launch of `count` back-to-back launches, timed with HIP events
    on the launch stream.  The GPU is first held busy by a spin kernel (~20 ms) while the host
    queues every launch, so the events measure the kernels and not the host's launch rate
    (short kernels would otherwise wait for Python between launches)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(40_000_000)
    a.record(stream)
    for _ in range(count):
        launch()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / count


def measure_prologue(bsa, torch, q, k, w, steps: int, stream, traffic_json: str | None = None) -> dict:
    """The QK prologue (RMSNorm of each head's channels + 3D-RoPE) on this workload's Q and
    K, timed apart from the attention step: HBM-bound, algorithmic bytes = bf16 read + write
    of every element (4 B per element per launch)."""
    gen = torch.Generator(device="cpu").manual_seed(12)
    gq = (torch.rand(64, generator=gen) + 0.5).cuda()
    gk = (torch.rand(64, generator=gen) + 0.5).cuda()
    qn, kn = torch.empty_like(q), torch.empty_like(k)
    for _ in range(3):
        bsa.qk_rmsnorm_rope3d(q, gq, 1e-6, w.grid, out=qn)
        bsa.qk_rmsnorm_rope3d(k, gk, 1e-6, w.grid, out=kn)
    torch.cuda.synchronize()
    def both():
        bsa.qk_rmsnorm_rope3d(q, gq, 1e-6, w.grid, out=qn)
        bsa.qk_rmsnorm_rope3d(k, gk, 1e-6, w.grid, out=kn)
    ms = timed_launches(torch, stream, both, steps) / 2
    nbytes = 4.0 * q.numel()
    gbps = nbytes / (ms * 1e-3) / 1e9
    traffic = traffic_from_profile(traffic_json, "qk_prologue_kernel") if traffic_json else None
    # a plain device copy of the same tensor: the HBM rate a read + write stream reaches here
    for _ in range(3):
        qn.copy_(q)
    copy_gbps = nbytes / (timed_launches(torch, stream, lambda: qn.copy_(q), steps) * 1e-3) / 1e9
    log(f"[bench] QK prologue: {ms:.4f} ms per tensor, {gbps:.0f} GB/s ({100 * gbps / HBM_PEAK_GBS:.1f}% of HBM; "
        f"a plain copy of the tensor: {copy_gbps:.0f} GB/s)")
    del qn, kn
    return {"bound": "hbm", "kernel": "qk_prologue_kernel", "avg_launch_ms": round(ms, 4),
            "bytes_per_launch": nbytes, "achieved": round(gbps, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBS, 4), "launches": 2 * steps,
            "copy_reference_gbs": round(copy_gbps, 1), "traffic": traffic,
            "what": "RMSNorm over each head's 64 channels with a 64-value gain, then 3D-RoPE, on Q and on K"}


def measure_prologue_backward(bsa, torch, q, w, steps: int, stream) -> dict:
    """Backward of the QK prologue on this workload's Q shape, HBM-bound: algorithmic bytes =
    x and dy read, dx written (6 B per element); dgamma's partial sums are a few KB."""
    gen = torch.Generator(device="cpu").manual_seed(16)
    gq = (torch.rand(64, generator=gen) + 0.5).cuda()
    dy = torch.randn(q.shape, generator=gen, dtype=torch.float32).to(torch.bfloat16).cuda()
    dx = torch.empty_like(q)
    dg = torch.empty(64, dtype=torch.float32, device="cuda")
    n_tokens = q.shape[-2]
    n_outer = q.numel() // (64 * n_tokens)
    ws = torch.empty(int(bsa.lib().lcv_qk_rmsnorm_rope3d_backward_workspace(n_outer, n_tokens)),
                     dtype=torch.float32, device="cuda")
    for _ in range(3):
        bsa.qk_rmsnorm_rope3d_backward(q, dy, gq, 1e-6, w.grid, dx=dx, dgamma=dg, workspace=ws)
    ms = timed_launches(torch, stream,
                        lambda: bsa.qk_rmsnorm_rope3d_backward(q, dy, gq, 1e-6, w.grid, dx=dx, dgamma=dg, workspace=ws),
                        steps)
    nbytes = 6.0 * q.numel()
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] QK prologue backward: {ms:.4f} ms per tensor, {gbps:.0f} GB/s ({100 * gbps / HBM_PEAK_GBS:.1f}% of HBM)")
    del dy, dx, ws
    return {"bound": "hbm", "kernel": "qk_prologue_bwd_kernel", "avg_launch_ms": round(ms, 4),
            "bytes_per_launch": nbytes, "achieved": round(gbps, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBS, 4), "launches": steps,
            "what": "gradients dx and dgamma of RMSNorm + 3D-RoPE for one Q-shaped tensor"}


def measure_backward(bsa, torch, q, k, v, layout, w, fwd_flops: float, steps: int, stream) -> dict:
    """The attention backward (dQ, dK, dV from the forward's output and LSE) on this
    workload, timed apart from the forward step (q and k taken as already rotated).
    Effective rate by the usual convention: 2.5x the forward's FLOPs (five products of the
    attended pairs: S, dP, dV, dQ, dK); the kernels execute seven (S and dP are formed once
    for the query walk and once for the key walk), also reported."""
    out, lse = bsa.forward(q, k, v, layout, grid=None)
    gen = torch.Generator(device="cpu").manual_seed(13)
    do = torch.randn(q.shape, generator=gen, dtype=torch.float32).to(torch.bfloat16).cuda()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(bsa.backward_workspace(q.shape[0], q.shape[1], q.shape[2]), dtype=torch.float32, device="cuda")
    for _ in range(3):
        bsa.backward(q, k, v, out, lse, do, layout, dq=dq, dk=dk, dv=dv, workspace=ws)
    ms = timed_launches(torch, stream,
                        lambda: bsa.backward(q, k, v, out, lse, do, layout, dq=dq, dk=dk, dv=dv, workspace=ws),
                        steps)
    eff = 2.5 * fwd_flops / (ms * 1e-3) / 1e12
    executed = 3.5 * fwd_flops / (ms * 1e-3) / 1e12
    log(f"[bench] backward: {ms:.3f} ms, {eff:.1f} TFLOP/s effective (2.5x forward FLOPs), "
        f"{executed:.1f} TFLOP/s of executed matrix work")
    del out, lse, do, dq, dk, dv, ws
    return {"bound": "mfma", "kernels": ["bwd_dq_kernel", "bwd_dkdv_kernel"],
            "ms": round(ms, 4), "effective_flops": 2.5 * fwd_flops, "achieved": round(eff, 3),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(eff / MFMA_BF16_PEAK_TFLOPS, 4),
            "executed_tflops": round(executed, 3), "launches": steps,
            "what": "dQ, dK, dV of the block-sparse attention (query walk with the per-row D = rowsum(dO*O), "
                    "key walk)"}


def measure_cross(bsa, torch, q, w, steps: int, stream, with_backward: bool = True):
    """Cross-attention of this workload's video queries over 512 text tokens (32 heads), and
    its backward, timed apart from the self-attention step: algorithmic FLOPs of the forward
    = 4 * 64 * N * L * heads (dense).  Returns (forward, backward or None)."""
    from lcv_inputs import TEXT_LEN
    gen = torch.Generator(device="cpu").manual_seed(14)
    shape = (q.shape[0], q.shape[1], TEXT_LEN, 64)
    k = torch.randn(shape, generator=gen, dtype=torch.float32).to(torch.bfloat16).cuda()
    v = torch.randn(shape, generator=gen, dtype=torch.float32).to(torch.bfloat16).cuda()
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    for _ in range(3):
        bsa.cross_attention(q, k, v, out=out, lse=lse)
    ms = timed_launches(torch, stream, lambda: bsa.cross_attention(q, k, v, out=out, lse=lse), steps)
    flops = 4.0 * 64 * q.shape[2] * TEXT_LEN * q.shape[1] * q.shape[0]
    tf = flops / (ms * 1e-3) / 1e12
    nbytes = 2.0 * (2 * q.numel() + 2 * k.numel()) + 4.0 * lse.numel()
    log(f"[bench] cross-attention ({TEXT_LEN} text tokens): {ms:.4f} ms, {tf:.1f} TFLOP/s "
        f"({100 * tf / MFMA_BF16_PEAK_TFLOPS:.1f}% of MFMA peak; {nbytes / (ms * 1e-3) / 1e9:.0f} GB/s of Q, O, K, V, lse)")
    # up to 512 text tokens the library runs the text-resident kernel
    kernel = "bsa_cross_resident_kernel" if TEXT_LEN <= 512 else "bsa_fwd_kernel<cross>"
    fwd = {"bound": "mfma", "kernel": kernel, "ms": round(ms, 4), "text_tokens": TEXT_LEN,
           "flops": flops, "achieved": round(tf, 3), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
           "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "min_bytes": nbytes,
           "hbm_gbs_at_min_bytes": round(nbytes / (ms * 1e-3) / 1e9, 1), "launches": steps,
           "what": "video queries over 512 padded text tokens, dense softmax attention"}
    if not with_backward:
        del k, v, out, lse
        return fwd, None
    # backward: effective rate by the usual convention, 2.5x the forward's FLOPs (S, dP, dV,
    # dQ, dK); the kernels execute seven products (S and dP in both walks)
    do = torch.randn(q.shape, generator=gen, dtype=torch.float32).to(torch.bfloat16).cuda()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(bsa.cross_attention_backward_workspace(q.shape[0], q.shape[1], q.shape[2], TEXT_LEN),
                     dtype=torch.float32, device="cuda")

    def call():
        bsa.cross_attention_backward(q, k, v, out, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws)
    for _ in range(3):
        call()
    bms = timed_launches(torch, stream, call, steps)
    eff = 2.5 * flops / (bms * 1e-3) / 1e12
    executed = 3.5 * flops / (bms * 1e-3) / 1e12
    log(f"[bench] cross-attention backward: {bms:.4f} ms, {eff:.1f} TFLOP/s effective (2.5x forward FLOPs), "
        f"{executed:.1f} TFLOP/s of executed matrix work")
    del k, v, out, lse, do, dq, dk, dv, ws
    bwd = {"bound": "mfma", "kernels": ["bwd_dq_cross_resident_kernel", "bwd_dkdv_kernel<cross>",
                                        "bwd_cross_reduce_kernel"],
           "ms": round(bms, 4), "effective_flops": 2.5 * flops, "achieved": round(eff, 3),
           "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(eff / MFMA_BF16_PEAK_TFLOPS, 4),
           "executed_tflops": round(executed, 3), "launches": steps,
           "what": "dQ, dK, dV of the cross-attention over 512 text tokens (query chunks' fp32 partial dK, dV "
                   "added in a fixed order)"}
    return fwd, bwd


def measure_merge(bsa, torch, q, steps: int, stream) -> dict:
    """The merge of two partial attention results of this workload's shape (the combine step
    of ring attention over two key shards), HBM-bound: algorithmic bytes = both parts' bf16
    out and fp32 lse read, the merged out and lse written."""
    gen = torch.Generator(device="cpu").manual_seed(15)
    outs = [torch.randn(q.shape, generator=gen, dtype=torch.float32).to(torch.bfloat16).cuda() for _ in range(2)]
    lses = [(torch.rand(q.shape[:3], generator=gen) * 10).cuda() for _ in range(2)]
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    for _ in range(3):
        bsa.attn_merge(outs, lses, out=out, lse=lse)
    ms = timed_launches(torch, stream, lambda: bsa.attn_merge(outs, lses, out=out, lse=lse), steps)
    nbytes = 3.0 * (2 * q.numel() + 4 * lse.numel())
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] merge of 2 partial results: {ms:.4f} ms, {gbps:.0f} GB/s ({100 * gbps / HBM_PEAK_GBS:.1f}% of HBM)")
    del outs, lses, out, lse
    return {"bound": "hbm", "kernel": "attn_merge_kernel", "avg_launch_ms": round(ms, 4), "bytes_per_launch": nbytes,
            "achieved": round(gbps, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBS, 4),
            "launches": steps, "what": "merge of two partial attention results (bf16 out + fp32 lse each)"}


def attended_pairs_from(n_tokens: int, cond: int, local: int, stride: int, q_from: int) -> int:
    """Attended (query, key) token pairs of the query rows q >= q_from, counted per block pair
    of the layout rule: a noise row sees every key of an allowed block, a condition row only
    the block's condition keys (host arithmetic for the FLOP count of the cached call)."""
    n = -(-n_tokens // 64)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    mb = np.abs(i - j) <= local
    if stride >= 1:
        mb = mb | (j % stride == 0)
    blk_lo = np.arange(n, dtype=np.int64) * 64
    blk_hi = np.minimum(blk_lo + 64, n_tokens)
    lo = np.maximum(blk_lo, q_from)
    noise_rows = np.clip(blk_hi - np.maximum(lo, cond), 0, None)
    cond_rows = np.clip(np.minimum(blk_hi, cond) - lo, 0, None)
    keys_all = blk_hi - blk_lo
    keys_cond = np.clip(np.minimum(blk_hi, cond) - blk_lo, 0, None)
    return int((noise_rows[:, None] * (mb * keys_all[None, :])).sum()
               + (cond_rows[:, None] * (mb * keys_cond[None, :])).sum())


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="t2v720", choices=sorted(WORKLOADS))
    ap.add_argument("--rope-mode", default="k-pass", choices=["k-pass", "fused", "none"],
                    help="k-pass: K rotated by the standalone RoPE pass into a second buffer, Q rotated "
                         "inside the attention kernel (both timed); fused: Q and K rotated inside the "
                         "attention kernel; none: inputs taken as already rotated")
    ap.add_argument("--cached", action="store_true",
                    help="time the workload's second call: noise-token rows [C, N) with the condition K/V "
                         "taken from the cache (workloads with condition frames)")
    ap.add_argument("--shard-of", type=int, default=0, metavar="G",
                    help="time one device's share of a sequence-sharded call: the middle one of G block-aligned "
                         "query-row ranges (K/V of the whole sequence resident)")
    ap.add_argument("--local", type=int, default=None, help="override the layout's local window (blocks)")
    ap.add_argument("--stride", type=int, default=None, help="override the layout's global stride")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prologue", action="store_true",
                    help="skip the separate measurement of the QK prologue (RMSNorm + 3D-RoPE) kernel")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the separate measurement of the attention backward")
    ap.add_argument("--no-cross", action="store_true",
                    help="skip the separate measurement of the cross-attention over text tokens")
    ap.add_argument("--no-merge", action="store_true",
                    help="skip the separate measurement of the merge of partial attention results")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "t2v720_traffic.json"))
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of --copy-calibration into "
                         "HBM bytes per attention launch; writes --traffic-json and exits")
    ap.add_argument("--summarize-counters", metavar="PMC_DIR",
                    help="print per-kernel averages of every counter of one rocprofv3 --pmc run and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters)
    if args.summarize_traffic:
        return summarize_traffic(*args.summarize_traffic, args.traffic_json)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              f"the library has no multi-GPU path", file=sys.stderr)
        return 2

    import torch
    import block_sparse_attention_lcv_amd as bsa

    import dataclasses
    w = WORKLOADS[args.workload]
    if args.local is not None or args.stride is not None:
        w = dataclasses.replace(w, local_blocks=w.local_blocks if args.local is None else args.local,
                                global_stride=w.global_stride if args.stride is None else args.stride)
    if args.shard_of and args.cached:
        print("--shard-of and --cached are exclusive", file=sys.stderr)
        return 2
    if args.cached and w.cond_len == 0:
        print(f"--cached needs a workload with condition frames ({w.name} has none)", file=sys.stderr)
        return 2
    log(f"[bench] workload {w.name}: grid {w.grid} N={w.n_tokens} heads={w.heads} C={w.cond_len} "
        f"local {w.local_blocks} stride {w.global_stride}{' (cached second call)' if args.cached else ''}")
    torch.cuda.init()
    stream = torch.cuda.current_stream()

    # the first build also loads the library and its GPU code; the layout used is a second,
    # warm build, whose time is the per-shape cost
    t0 = time.perf_counter()
    bsa.build_layout(w.n_tokens, w.local_blocks, w.global_stride, w.cond_len).close()
    first_layout_ms = (time.perf_counter() - t0) * 1e3
    t0 = time.perf_counter()
    layout = bsa.build_layout(w.n_tokens, w.local_blocks, w.global_stride, w.cond_len)
    layout_ms = (time.perf_counter() - t0) * 1e3
    info = layout.info
    pairs = info["attended_pairs"]
    row0, row1 = 0, w.n_tokens
    if args.cached:
        pairs = attended_pairs_from(w.n_tokens, w.cond_len, w.local_blocks, w.global_stride, w.cond_len)
    elif args.shard_of:
        per = -(-w.n_blocks // args.shard_of) * 64
        g = args.shard_of // 2
        row0, row1 = g * per, min((g + 1) * per, w.n_tokens)
        pairs = (attended_pairs_from(w.n_tokens, w.cond_len, w.local_blocks, w.global_stride, row0)
                 - attended_pairs_from(w.n_tokens, w.cond_len, w.local_blocks, w.global_stride, row1))
    flops = 4.0 * 64 * pairs * w.heads * w.batch
    log(f"[bench] layout nnz={info['nnz']} pairs/head={info['attended_pairs']} (timed rows: {pairs}) "
        f"build {layout_ms:.2f} ms")

    qb, kb, vb = workload_inputs(w)

    def dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = dev(qb), dev(kb), dev(vb)
    del qb, kb, vb
    C = w.cond_len
    if args.cached:
        # the cache: condition K (rotated unless the attention kernel rotates K) and V of call 1;
        # call 2 brings fresh noise-token Q, K, V
        v_cond = v[:, :, :C].contiguous()
        k_cond = k[:, :, :C].contiguous()
        if args.rope_mode == "k-pass":
            k_cond = bsa.rope3d_apply(k_cond, w.grid)
        qb, kb, vb = workload_inputs(w, call=1)
        q, k, v = dev(qb), dev(kb), dev(vb)
        del qb, kb, vb
    q_full = q
    if args.shard_of:
        q = q[:, :, row0:row1].contiguous()
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    k_rot = torch.empty_like(k) if args.rope_mode == "k-pass" else None
    k_offset = C if args.cached else 0

    # one step; ev_mid (if given) is recorded between the RoPE pass and the attention kernel
    def step(ev_mid=None):
        if args.rope_mode == "k-pass":
            bsa.rope3d_apply(k, w.grid, token_offset=k_offset, out=k_rot)
        if ev_mid is not None:
            ev_mid.record(stream)
        grid = None if args.rope_mode == "none" else w.grid
        kk = k_rot if args.rope_mode == "k-pass" else k
        rk = args.rope_mode == "fused"
        if args.cached:
            bsa.forward_cached(q, kk, v, k_cond, v_cond, layout, grid=grid, rope_q=grid is not None, rope_k=rk,
                               out=out, lse=lse)
        elif args.shard_of:
            bsa.forward_rows(q, kk, v, layout, row0, row1, grid=grid, rope_q=grid is not None, rope_k=rk,
                             out=out, lse=lse)
        else:
            bsa.forward(q, kk, v, layout, grid=grid, rope_q=grid is not None, rope_k=rk, out=out, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record(stream)
    for i in range(args.steps):
        starts[i].record(stream)
        step(mids[i])
        ends[i].record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    total_ms = t_all0.elapsed_time(t_all1)
    attn_ms = [m.elapsed_time(e) for m, e in zip(mids, ends)]
    rope_ms = [s_.elapsed_time(m) for s_, m in zip(starts, mids)]
    ms_per_step = total_ms / args.steps
    avg_launch_ms = float(np.mean(attn_ms))
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    log(f"[bench] {ms_per_step:.3f} ms/step; attention kernel avg {avg_launch_ms:.3f} ms "
        f"(min {min(attn_ms):.3f}, max {max(attn_ms):.3f}); K RoPE pass avg {np.mean(rope_ms):.3f} ms; "
        f"{value:.1f} TFLOP/s effective per step")

    default_config = (args.workload == "t2v720" and not args.cached and not args.shard_of
                      and args.rope_mode == "k-pass" and args.local is None and args.stride is None)
    # the side passes as HBM-bound passes: the K RoPE pass (bf16 read + write of every
    # element of K, timed by the step's events) and the layout build (its outputs: the CSR,
    # the workgroup lists, the work order and the backward's key-side schedule, all written
    # once; timed on the host around a warm build: allocation, 9 kernels and one read-back)
    rope_pass = None
    if args.rope_mode == "k-pass":
        rope_avg = float(np.mean(rope_ms))
        rope_bytes = 4.0 * k.numel()
        rope_gbs = rope_bytes / (rope_avg * 1e-3) / 1e9
        rope_pass = {"bound": "hbm", "kernel": "rope3d_kernel", "avg_launch_ms": round(rope_avg, 4),
                     "bytes_per_launch": rope_bytes, "achieved": round(rope_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(rope_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(args.traffic_json, "rope3d_kernel") if default_config else None,
                     "what": "3D-RoPE of K (bf16 in, fp32 math, bf16 out) into a second buffer, every step"}
    n_st = -(-info["n_blocks"] // 4)
    # row_ptr, col_idx, the workgroup lists and counts, the work order, and the key groups'
    # blocks, counts and offsets (their column lists, at most nnz entries, are not counted)
    layout_bytes = 4.0 * ((info["n_blocks"] + 1) + 2 * info["nnz"] + 2 * n_st + 6 * n_st + 1)
    layout_gbs = layout_bytes / (layout_ms * 1e-3) / 1e9
    layout_build = {"bound": "launch", "ms": round(layout_ms, 4), "bytes": layout_bytes,
                    "achieved": round(layout_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(layout_gbs / HBM_PEAK_GBS, 6),
                    "what": "warm lcv_bsa_build_layout on the host clock: one allocation, 9 kernels (row counts, "
                            "scans, CSR fill, workgroup list unions, work order, key-group unions) and one "
                            "read-back; bytes = every array written once except the key groups' column lists"}
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {w.description}",
            "grid": list(w.grid), "tokens": w.n_tokens, "heads": w.heads, "head_dim": 64, "batch": w.batch,
            "cond_len": w.cond_len, "layout": f"block 64, local {w.local_blocks}, stride {w.global_stride}",
            "rope": {"k-pass": "Q rotated in the attention kernel's Q load, K by the standalone RoPE pass "
                               "(both inside the timed step)",
                     "fused": "Q and K rotated in the attention kernel's loads",
                     "none": "none (inputs taken as rotated)"}[args.rope_mode],
            "nnz": info["nnz"], "attended_pairs_per_head": info["attended_pairs"],
            "call": ("cached second call: noise rows [C, N), condition K/V from the cache" if args.cached
                     else f"rows [{row0}, {row1}): the middle of {args.shard_of} sequence shards" if args.shard_of
                     else "full call"),
            "timed_pairs_per_head": pairs,
            "effective_flops": flops,
        },
        "pct_mfma_peak": round(100.0 * value / MFMA_BF16_PEAK_TFLOPS, 2),
        "layout_build_ms": round(layout_ms, 3),
        "layout_first_build_ms": round(first_layout_ms, 3),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            # the committed counter summary covers the default configuration only
            "traffic": traffic_from_profile(args.traffic_json) if default_config else None,
            "kernel": "bsa_fwd_kernel",
            "avg_launch_ms": round(avg_launch_ms, 4),
        },
        "rope_pass_ms": round(float(np.mean(rope_ms)), 4) if args.rope_mode == "k-pass" else None,
        "rope_pass": rope_pass,
        "layout_build": layout_build,
    }
    # the other kernels are measured on the full call's tensors
    q = q_full
    extras = not args.cached and not args.shard_of
    if not args.no_prologue and extras:
        result["qk_prologue"] = measure_prologue(bsa, torch, q, k, w, args.steps, stream,
                                                 args.traffic_json if default_config else None)
    if not args.no_backward and extras:
        result["backward"] = measure_backward(bsa, torch, q, k, v, layout, w, flops, args.steps, stream)
        if not args.no_prologue:
            result["qk_prologue_backward"] = measure_prologue_backward(bsa, torch, q, w, args.steps, stream)
    if not args.no_cross and extras:
        result["cross_attention"], cross_bwd = measure_cross(bsa, torch, q, w, args.steps, stream,
                                                             with_backward=not args.no_backward)
        if cross_bwd is not None:
            result["cross_attention_backward"] = cross_bwd
    if not args.no_merge and extras:
        result["merge"] = measure_merge(bsa, torch, q, args.steps, stream)
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: 3 copies of {COPY_BYTES} bytes")
        del src, dst
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        log("[bench] timing the oracle's block-visiting form on the host")
        result["cpu_baseline_block_visiting"] = cpu_baseline_blocks(w, args.cpu_seconds / 2)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    layout.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
