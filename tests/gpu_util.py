"""Helpers of the GPU parity tests: device upload of bf16 bit patterns, error metrics."""
from __future__ import annotations

import sys

import numpy as np

from lcv_inputs import bf16_bits_to_f64

# Tolerances for bf16-in / fp32-accumulate outputs against the fp64 oracle.
OUT_MAX_ABS = 2e-2
OUT_REL_L2 = 1e-2
LSE_MAX_ABS = 1e-2


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def from_dev_f64(t) -> np.ndarray:
    import torch
    return bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def out_errors(got: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / denom if denom > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_out_close(got, ref, what=""):
    max_abs, rel = out_errors(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert max_abs <= OUT_MAX_ABS and rel <= OUT_REL_L2, f"{what}: max_abs {max_abs:.3e} rel_l2 {rel:.3e}"
    return max_abs, rel


def assert_lse_close(got, ref, what=""):
    finite = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), finite), f"{what}: lse finiteness differs"
    err = float(np.max(np.abs(got[finite] - ref[finite]))) if finite.any() else 0.0
    assert err <= LSE_MAX_ABS, f"{what}: lse max_abs {err:.3e}"
    return err
