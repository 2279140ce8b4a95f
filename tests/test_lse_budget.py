"""The forward's LSE error budget (tests/gpu_util.lse_error_budget) checked on the CPU against
a rounding model of the kernel's score arithmetic, so that the GPU tests' LSE bounds are
derived rather than fitted.

The model: rotated Q and K rounded to bf16 after an fp32 rotation (when the kernel rotates),
the query operand Q' = bf16(fp32(q) * fp32(log2(e)/8)), scores Q' K^T in log2 units, the
row's coarse reference (a multiple of 64), probabilities 2^(s - ref) rounded to bf16 and
summed, lse = (ref + log2 l) ln 2.  On the stress inputs of the GPU tests it must stay within
the worst case of every row, with errors near one predicted standard deviation (root mean
square over rows), and reproduce the errors the GPU shows on them (0.086 on the peaked input,
1.38 on the +-3072 offset input).  The same model with an exactly scaled query operand
(Q / 8, exact in bf16, and log2(e) applied in fp32) is the alternative form of the
arithmetic, compared here."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from lcv_inputs import bf16_bits_to_f64, qkv_bits, round_to_bf16_bits
from tests.gpu_util import lse_error_budget

GRID = (3, 10, 21)
N, HEADS, COND, LOCAL, STRIDE = 630, 2, 210, 2, 4


def _bf16(x):
    return bf16_bits_to_f64(round_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def _model_lse(qf, kf, mask, rope: bool, exact_scale: bool) -> np.ndarray:
    if rope:
        qr = _bf16(oracle.rope3d(qf, GRID).astype(np.float32))
        kr = _bf16(oracle.rope3d(kf, GRID).astype(np.float32))
    else:
        qr, kr = qf, kf
    if exact_scale:
        s = ((qr / 8.0) @ kr.T) * float(np.float32(1.4426950408889634))
    else:
        qs = _bf16(qr.astype(np.float32) * np.float32(1.4426950408889634 / 8.0))
        s = qs @ kr.T
    s = np.where(mask, s, -np.inf)
    ref = 64.0 * np.rint(s.max(axis=1) / 64.0)
    p = _bf16(np.exp2(s - ref[:, None]).astype(np.float32))
    return (ref + np.log2(p.sum(axis=1))) * np.log(2.0)


def _inputs(case: str):
    if case == "peaked":
        qb, kb, _ = qkv_bits(33, 1, HEADS, N, 8.0)
        return bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), True
    if case == "plain":
        qb, kb, _ = qkv_bits(31, 1, HEADS, N)
        return bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), True
    offset = 3072.0 if case == "offset+" else -3072.0
    qb, kb, _ = qkv_bits(38, 1, HEADS, N)
    qb, kb = qb.copy(), kb.copy()
    qb[..., 0] = np.uint16(np.float32(offset).view(np.uint32) >> 16)
    kb[..., 0] = np.uint16(np.float32(1.0).view(np.uint32) >> 16)
    return bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), False


def _errors(case: str, exact_scale: bool):
    qf, kf, rope = _inputs(case)
    mask = oracle.token_mask_rows(np.arange(N), N, COND, LOCAL, STRIDE)
    errs, worsts, sigmas = [], [], []
    for h in range(HEADS):
        qr = oracle.rope3d(qf[0, h], GRID) if rope else qf[0, h]
        kr = oracle.rope3d(kf[0, h], GRID) if rope else kf[0, h]
        _, lse_ref = oracle.masked_attention(qr, kr, np.zeros_like(kr), mask)
        worst, sigma = lse_error_budget(qr, kr, mask, lse_ref, rope)
        errs.append(np.abs(_model_lse(qf[0, h], kf[0, h], mask, rope, exact_scale) - lse_ref))
        worsts.append(worst)
        sigmas.append(sigma)
    return np.concatenate(errs), np.concatenate(worsts), np.concatenate(sigmas)


@pytest.mark.parametrize("case", ["plain", "peaked", "offset+", "offset-"])
def test_model_within_budget(case):
    err, worst, sigma = _errors(case, exact_scale=False)
    assert np.all(err <= worst), float(np.max(err / worst))
    z_rms = float(np.sqrt(np.mean((err / sigma) ** 2)))
    if case in ("plain", "peaked"):          # independent roundings: the variance model holds
        assert 0.5 <= z_rms <= 1.5, z_rms
    else:                                    # one rounding shared by every score of the row
        assert z_rms <= 3.0, z_rms


def test_model_reproduces_the_gpu_errors():
    """The largest LSE errors the GPU shows on the stress inputs (peaked: 0.084-0.086;
    offset: 1.383) come out of the rounding model: they are the arithmetic's, not a defect."""
    err, _, _ = _errors("peaked", exact_scale=False)
    assert 0.07 <= float(np.max(err)) <= 0.1
    err, _, _ = _errors("offset+", exact_scale=False)
    assert abs(float(np.max(err)) - 1.384) < 0.01


def test_exact_scale_form_compared():
    """The alternative arithmetic (Q / 8 exact, log2(e) in fp32) removes the offset input's
    error but barely changes the peaked one, where the rotations' roundings dominate."""
    peaked_rounded = float(np.max(_errors("peaked", False)[0]))
    peaked_exact = float(np.max(_errors("peaked", True)[0]))
    offset_exact = float(np.max(_errors("offset+", True)[0]))
    assert peaked_exact > 0.9 * peaked_rounded
    assert offset_exact < 1e-2
