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


# Error budget of the forward's LSE (natural units) from the arithmetic of its scores.  A
# score is sum_c k_c q'_c over bf16 operands: q' = bf16(q * log2(e)/8) (the scale rounded to
# bf16 after an fp32 product), and with the 3D-RoPE applied in the kernel also q and k are
# rotated in fp32 and rounded to bf16 first.  Each rounding moves a product q_c k_c by at most
# u = 2^-8 of itself (round to nearest even, 8 significant bits); the fp32 trigonometry of the
# rotation by at most ~2e-5 of the pair's norm; the fp32 sums and the final conversions by a
# few 2^-24.  The LSE, a smooth maximum of the scores, moves by at most the largest score
# error of its row, plus the relative error of the row sum of bf16-rounded probabilities (u)
# and of its fp32 accumulation.
U_BF16 = 2.0 ** -8
U_F32 = 2.0 ** -24


def lse_error_budget(q_rot: np.ndarray, k_rot: np.ndarray, mask: np.ndarray, lse_ref: np.ndarray,
                     rope: bool) -> tuple[np.ndarray, np.ndarray]:
    """Per-row bounds on |lse_gpu - lse_ref| for one head: (worst case, standard deviation).

    q_rot [R, 64], k_rot [N, 64]: the rotated operands in fp64 (as the oracle forms them);
    mask [R, N]: attended pairs; lse_ref [R]: the oracle's LSE.  rope: the kernel rotates Q
    and K (three bf16 roundings per product) or takes them as rotated (one: the scale).

    Worst case: max over the row's keys of (n_round u + 70 u32) sum_c |q_c k_c| / 8, plus
    4e-5 |q| |k| / 8 for the trigonometry when rotating, plus u + n_keys u32 for the row sum
    and 2^-21 |lse| for the fp32 conversions.

    Standard deviation, to first order: with P the row's probabilities the LSE error is
    sum_k P_k ds_k.  The query-side roundings (the rotation of q and the scale) are shared by
    all keys of a row: sum_c (q_c kbar_c / 8) e_c with kbar = sum_k P_k k; the key-side ones
    are per key: sum_k P_k sum_c (q_c k_c / 8) e_kc; the probability roundings sum_k P_k e_k.
    Round-to-nearest errors relative to values spread over binades have a variance of about
    0.18 u^2 each (uniform absolute error of half an ulp, mantissas spread log-uniformly)."""
    n_round = 3 if rope else 1
    absq, absk = np.abs(q_rot), np.abs(k_rot)
    a = (absq @ absk.T) / 8.0                                            # sum_c |q_c k_c| / 8
    norms = np.outer(np.linalg.norm(q_rot, axis=1), np.linalg.norm(k_rot, axis=1)) / 8.0
    per_key = (n_round * U_BF16 + 70 * U_F32) * a + (4e-5 * norms if rope else 0.0)
    per_key = np.where(mask, per_key, 0.0)
    n_keys = mask.sum(axis=1)
    worst = per_key.max(axis=1) + U_BF16 + n_keys * U_F32 + 2.0 ** -21 * np.abs(lse_ref) + 1e-6
    # probabilities of the exact scores
    s = np.where(mask, (q_rot @ k_rot.T) / 8.0, -np.inf)
    p = np.exp(s - lse_ref[:, None])
    var_e = 0.18 * U_BF16 ** 2
    kbar = p @ k_rot
    q_side = (2 if rope else 1) * var_e * np.sum((q_rot * kbar / 8.0) ** 2, axis=1)
    k_side = (var_e * ((p ** 2) @ (k_rot ** 2)) * (q_rot ** 2) / 64.0).sum(axis=1) if rope else 0.0
    p_round = var_e * np.sum(p ** 2, axis=1)
    sigma = np.sqrt(q_side + k_side + p_round)
    return worst, sigma


def score_rounding_sigma(q: np.ndarray, k: np.ndarray, mask: np.ndarray) -> float:
    """Standard deviation (natural units, root mean square over the attended pairs) of the
    score error that the one bf16 rounding of the query operand Q' = bf16(q * log2(e)/8)
    leaves when q and k are taken as rotated: each product q_c k_c / 8 moves by a
    round-to-nearest error of relative standard deviation ~0.425 u (u = 2^-8), independently
    per channel.  q [..., R, 64], k [..., N, 64] with matching leading axes, mask [R, N]."""
    q2 = np.asarray(q, dtype=np.float64) ** 2
    k2 = np.asarray(k, dtype=np.float64) ** 2
    var = (q2 @ np.swapaxes(k2, -1, -2)) / 64.0              # sum_c (q_c k_c / 8)^2
    m = np.broadcast_to(mask, var.shape)
    return 0.425 * U_BF16 * float(np.sqrt(np.mean(var[m])))
