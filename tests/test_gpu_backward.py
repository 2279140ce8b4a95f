"""GPU block-sparse attention backward (dq, dk, dv) against the fp64 oracle.

The forward runs on the GPU (its bf16 output and fp32 LSE are what the backward consumes);
the oracle differentiates the exact attention of the same bf16 inputs.  Small and medium
shapes are compared on every element; the full-size workloads on sampled query rows (dq)
and on sampled keys of local-only key blocks (dk, dv), whose attending rows the oracle can
enumerate.

Tolerance, from the arithmetic: P and dS enter the matrix cores rounded to bf16 (relative
2^-9 each, independent across terms), both walks score with the forward's query operand
Q * log2(e)/8 rounded to bf16 (a score error of ~2^-9 of each product, the same as the
forward's, so P agrees with the saved LSE), D = rowsum(dO * O) uses the bf16 output O of the
forward, and every gradient is rounded to bf16 once (2^-9 of its value).  Summed over
hundreds of terms with independent signs these stay near 2^-9 of the result in relative L2
(<= 1e-2 asserted) and below 2^-6 of the compared set's largest magnitude element-wise
(max-abs <= 2e-2 * max|ref| + 1e-6 asserted; at the workloads' sizes the gradients are
~1e-2, so the absolute floor only covers gradients that vanish exactly, e.g. a single key)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from lcv_inputs import WORKLOADS, bf16_bits_to_f64, grad_bits, qkv_bits, workload_inputs
from tests.gpu_util import from_dev_f64, out_errors, say, score_rounding_sigma, to_dev

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_ABS_FRAC = 2e-2


def _sync():
    import torch
    torch.cuda.synchronize()


def _close(got, ref, what):
    max_abs, rel = out_errors(got, ref)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    say(f"  {what}: max_abs {max_abs:.3e} (max|ref| {scale:.3e}) rel_l2 {rel:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    assert max_abs <= MAX_ABS_FRAC * scale + 1e-6 and rel <= REL_L2, f"{what}: max_abs {max_abs:.3e} rel_l2 {rel:.3e}"


def _run(lib, n, heads, cond, local, stride, seed, batch=1, q_scale=1.0):
    """GPU forward + backward; returns the bf16 inputs and the device gradients."""
    qb, kb, vb = qkv_bits(seed, batch, heads, n, q_scale)
    gb = grad_bits(seed, batch, heads, n)
    layout = lib.build_layout(n, local, stride, cond)
    q, k, v, do = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(gb)
    out, lse = lib.forward(q, k, v, layout, grid=None)
    dq, dk, dv = lib.backward(q, k, v, out, lse, do, layout)
    _sync()
    return (qb, kb, vb, gb), (q, k, v, do, out, lse), (dq, dk, dv), layout


CASES = [
    # name, N, heads, cond, local, stride, batch
    ("tiny", 512, 2, 0, 2, 4, 1),
    ("ragged-c210", 630, 3, 210, 2, 4, 1),
    ("ragged-allcond", 630, 2, 630, 2, 4, 1),
    ("ragged-w1s3", 630, 2, 210, 1, 3, 1),
    ("ragged-w0s0", 630, 2, 210, 0, 0, 1),
    ("ragged-dense", 630, 2, 210, 3, 1, 1),
    ("one-token", 1, 2, 0, 2, 4, 1),
    ("one-partial-block", 63, 2, 5, 2, 4, 1),
    ("65-tokens", 65, 2, 64, 0, 1, 1),
    ("multi-workgroup", 2048, 2, 1061, 2, 4, 1),
    ("cond-at-63", 300, 2, 63, 0, 3, 1),
    ("batch-two", 384, 3, 100, 2, 4, 2),
    ("long-columns", 7680, 1, 1920, 2, 4, 1),   # 120 blocks: global columns of ~120 blocks
]


@pytest.mark.parametrize("name,n,heads,cond,local,stride,batch", CASES, ids=[c[0] for c in CASES])
def test_backward_full(lib, name, n, heads, cond, local, stride, batch):
    say(f"[bwd] {name} N={n} heads={heads} C={cond} w={local} s={stride} batch={batch}")
    (qb, kb, vb, gb), _, (dq, dk, dv), layout = _run(lib, n, heads, cond, local, stride, seed=41, batch=batch)
    ref = oracle.bsa_backward(*(bf16_bits_to_f64(a) for a in (qb, kb, vb, gb)), cond, local, stride)
    for what, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        _close(from_dev_f64(got), r, f"{name} {what}")
    layout.close()


def _check_peaked(got, ref, sigma, what):
    """Bounds of a peaked-softmax stress input, derived from the one rounding left in the
    backward's scores (see test_backward_peaked_softmax): relative L2 <= 1.5 sigma and
    max-abs <= 4 sigma * max|ref|, sigma the score error's standard deviation."""
    g64 = from_dev_f64(got)
    max_abs, rel = out_errors(g64, ref)
    scale = float(np.max(np.abs(ref)))
    say(f"  {what}: max_abs {max_abs:.3e} (max|ref| {scale:.3e}) rel_l2 {rel:.3e} (sigma {sigma:.3e})")
    assert np.all(np.isfinite(g64)), what
    assert max_abs <= 4 * sigma * scale and rel <= 1.5 * sigma, (what, max_abs, rel, sigma)


def test_backward_peaked_softmax(lib):
    """Q scaled by 8: scores of standard deviation ~8 natural units, each row dominated by a
    few keys.  This stress input is not one of the workloads, so its bound is derived from
    the arithmetic.
    - Both walks recompute P from the forward's own score operands, so P agrees with the
      forward's LSE; what is left is the forward's rounding of Q * log2(e)/8 to bf16, which
      moves each product q_c k_c / 8 by a round-to-nearest error (relative standard deviation
      ~0.425 * 2^-8).  Here (|q_c| ~ 8, |k_c| ~ 1) a score moves by sigma ~ 0.013 natural units
      in standard deviation (score_rounding_sigma, computed from the inputs), and so does
      each probability, relatively.
    - Where one or two queries dominate a key's gradient these errors do not average out;
      dS = P (dP - D) subtracts two terms of similar size, and D takes the forward's bf16
      output.  The gradients' relative L2 error is therefore of the order of sigma:
      bound 1.5 sigma (~2e-2), and max-abs 4 sigma * max|ref|.
    - Measured: ~1e-2 relative L2 for dQ and dK, ~5e-3 for dV (when the key walk scored with
      K * log2(e)/8 rounded on its own the mismatch added an independent rounding and
      the LSE's: 1.6-2.3%).  A wrong index, sign or operand gives errors of order one."""
    n, heads, cond, local, stride = 630, 2, 210, 2, 4
    say("[bwd] peaked softmax (Q x 8)")
    (qb, kb, vb, gb), _, (dq, dk, dv), layout = _run(lib, n, heads, cond, local, stride, seed=47, q_scale=8.0)
    qf, kf = bf16_bits_to_f64(qb), bf16_bits_to_f64(kb)
    ref = oracle.bsa_backward(qf, kf, bf16_bits_to_f64(vb), bf16_bits_to_f64(gb), cond, local, stride)
    sigma = score_rounding_sigma(qf[0], kf[0], oracle.token_mask_rows(np.arange(n), n, cond, local, stride))
    for what, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        _check_peaked(got, r, sigma, f"peaked {what}")
    layout.close()


@pytest.mark.parametrize("offset", [3072.0, -3072.0], ids=["plus", "minus"])
def test_backward_score_offset_far_from_zero(lib, offset):
    """Every score of a row shifted by the same large amount (channel 0 of every key is 1, of
    every query +-3072: +-384 in natural units).  The softmax ignores a shift common to its
    row, so the gradients must match the oracle at the standard bounds.  The forward forms
    that shift from Q * log2(e)/8 rounded to bf16 (an error of ~1.4 natural units in the
    row's LSE); the backward recomputes P from the same rounded operand, so P = exp(S - lse)
    stays a probability distribution.  A walk that scored with another rounding of the same
    product (for instance K * log2(e)/8) would put a common factor of up to 2^3 on the row's
    probabilities.  dK takes the rounded query too, which moves its channel 0 (the largest
    gradient entries, 384 times the others) by at most 2^-8 relative."""
    import torch
    n, heads, cond, local, stride = 630, 2, 210, 2, 4
    qb, kb, vb = qkv_bits(39, 1, heads, n)
    gb = grad_bits(39, 1, heads, n)
    qb, kb = qb.copy(), kb.copy()
    qb[..., 0] = np.uint16(np.float32(offset).view(np.uint32) >> 16)      # +-3072 is exact in bf16
    kb[..., 0] = np.uint16(np.float32(1.0).view(np.uint32) >> 16)
    say(f"[bwd] score offset {offset:+.0f} on channel 0")
    layout = lib.build_layout(n, local, stride, cond)
    q, k, v, do = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(gb)
    out, lse = lib.forward(q, k, v, layout, grid=None)
    dq, dk, dv = lib.backward(q, k, v, out, lse, do, layout)
    _sync()
    ref = oracle.bsa_backward(*(bf16_bits_to_f64(a) for a in (qb, kb, vb, gb)), cond, local, stride)
    for what, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        _close(from_dev_f64(got), r, f"offset {offset:+.0f} {what}")
    layout.close()


def _gains(seed, lo, hi):
    return np.random.default_rng(seed).uniform(lo, hi, 64)


@pytest.mark.parametrize("glo,ghi", [(1.0, 2.0), (1.5, 2.5)], ids=["gains-1-2", "gains-1.5-2.5"])
def test_backward_after_qk_norm_large_gains(lib, glo, ghi):
    """Q and K through the QK prologue (RMSNorm with gains drawn from U(glo, ghi), then the
    3D-RoPE) on the GPU, then the forward and backward on the normalised tensors, against the
    oracle's backward of the same bf16 tensors.  Each channel of q and k is ~gain * N(0, 1),
    so scores have a standard deviation of ~E[gain^2] natural units (2.3 and 4.1 here): rows
    are peaked and many scores are large.  With the backward scoring from the forward's own
    rounded Q the only score error left is that rounding (relative 2^-8 per product at most,
    ~0.4 * 2^-8 in standard deviation), which moves each probability by ~0.17% * E[gain^2]
    (0.4% and 0.7% in standard deviation): the standard bounds hold at these gains."""
    import torch
    grid = (3, 10, 21)
    n, heads, cond, local, stride = 630, 2, 210, 2, 4
    say(f"[bwd] after QK norm, gains U({glo}, {ghi})")
    qb, kb, vb = qkv_bits(49, 1, heads, n)
    gb = grad_bits(49, 1, heads, n)
    gq = torch.from_numpy(_gains(5, glo, ghi).astype(np.float32)).cuda()
    gk = torch.from_numpy(_gains(6, glo, ghi).astype(np.float32)).cuda()
    layout = lib.build_layout(n, local, stride, cond)
    q = lib.qk_rmsnorm_rope3d(to_dev(qb), gq, 1e-6, grid)
    k = lib.qk_rmsnorm_rope3d(to_dev(kb), gk, 1e-6, grid)
    v, do = to_dev(vb), to_dev(gb)
    out, lse = lib.forward(q, k, v, layout, grid=None)
    dq, dk, dv = lib.backward(q, k, v, out, lse, do, layout)
    _sync()
    qn, kn = from_dev_f64(q), from_dev_f64(k)
    ref = oracle.bsa_backward(qn, kn, bf16_bits_to_f64(vb), bf16_bits_to_f64(gb), cond, local, stride)
    for what, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        _close(from_dev_f64(got), r, f"gains U({glo}, {ghi}) {what}")
    layout.close()


def test_backward_writes_everything_and_is_deterministic(lib):
    """Gradients pre-filled with NaN come back finite; a second call gives identical bits."""
    import torch
    say("[bwd] nan poison + determinism")
    n, heads = 630, 2
    _, (q, k, v, do, out, lse), (dq, dk, dv), layout = _run(lib, n, heads, 210, 2, 4, seed=42)
    poison = [torch.full_like(q, float("nan")) for _ in range(3)]
    ws = torch.full((lib.backward_workspace(1, heads, n),), float("nan"), dtype=torch.float32, device="cuda")
    lib.backward(q, k, v, out, lse, do, layout, dq=poison[0], dk=poison[1], dv=poison[2], workspace=ws)
    _sync()
    for a, b in zip((dq, dk, dv), poison):
        assert torch.isfinite(b.float()).all()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    layout.close()


def test_backward_argument_errors(lib):
    """Argument errors with a real layout are reported before launch."""
    import ctypes
    layout = lib.build_layout(630, 2, 4, 210)
    L = lib.lib()
    p = ctypes.c_void_p(4096)
    f = L.lcv_bsa_backward
    h = layout.handle
    big = 1 << 40
    need = L.lcv_bsa_backward_workspace(1, 2, 630)
    assert f(p, p, p, p, p, p, 1, 2, h, 0, p, p, p, p, big, None) == 5                       # cond mismatch
    assert f(p, p, p, p, p, p, 0, 2, h, 210, p, p, p, p, big, None) == 2                     # batch 0
    assert f(p, p, p, p, p, p, 1, 0, h, 210, p, p, p, p, big, None) == 2                     # heads 0
    assert f(ctypes.c_void_p(4104), p, p, p, p, p, 1, 2, h, 210, p, p, p, p, big, None) == 2  # misaligned q
    assert f(p, p, p, p, ctypes.c_void_p(4098), p, 1, 2, h, 210, p, p, p, p, big, None) == 2  # misaligned lse
    assert f(p, p, p, p, p, p, 1, 2, h, 210, p, p, p, ctypes.c_void_p(4100), big, None) == 2  # workspace not 16-aligned
    assert f(p, p, p, p, p, p, 1, 2, h, 210, p, p, p, p, need - 1, None) == 2                # workspace too small
    assert b"workspace" in L.lcv_last_error()
    layout.close()


def _local_only_keys(w, rng, n_blocks=4, per_block=3):
    """Keys of key blocks that no global column covers (seen by their local band only)."""
    cand = [j for j in range(w.n_blocks) if j % w.global_stride != 0]
    picks = [cand[0], cand[-1]] + list(rng.choice(cand, n_blocks - 2, replace=False))
    keys = []
    for j in picks:
        lo, hi = 64 * j, min(64 * j + 64, w.n_tokens)
        keys += [lo, hi - 1] + list(rng.integers(lo, hi, per_block - 2))
    if w.cond_len:
        keys += [w.cond_len - 1, w.cond_len]
        keys = [t for t in keys if (t // 64) % w.global_stride != 0]
    return np.unique(np.array(keys))


@pytest.mark.parametrize("name", ["t2v480", "i2v480", "t2v720"])
def test_backward_workload_sampled(lib, name):
    """Full-size backward (all heads, the workload's layout); dq at sampled rows and dk, dv at
    sampled local-only keys of two heads against the oracle, every gradient finite."""
    import torch
    w = WORKLOADS[name]
    say(f"[bwd] workload {name} N={w.n_tokens} heads={w.heads} C={w.cond_len}")
    qb, kb, vb = workload_inputs(w)
    gb = grad_bits(w.seed, w.batch, w.heads, w.n_tokens)
    layout = lib.build_layout(w.n_tokens, w.local_blocks, w.global_stride, w.cond_len)
    q, k, v, do = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(gb)
    out, lse = lib.forward(q, k, v, layout, grid=None)
    dq, dk, dv = lib.backward(q, k, v, out, lse, do, layout)
    _sync()
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    rng = np.random.default_rng(43)
    n = w.n_tokens
    rows = np.unique(np.concatenate([[0, 63, 64, n - 1], rng.integers(0, n, 24),
                                     [w.cond_len - 1, w.cond_len] if w.cond_len else []]).astype(np.int64))
    keys = _local_only_keys(w, rng)
    for h in (0, w.heads - 1):
        args = [bf16_bits_to_f64(a[:, h:h + 1]) for a in (qb, kb, vb, gb)]
        ref_dq = oracle.bsa_backward_rows(*args, w.cond_len, w.local_blocks, w.global_stride, rows)
        ref_dk, ref_dv = oracle.bsa_backward_keys(*args, w.cond_len, w.local_blocks, w.global_stride, keys)
        r = torch.from_numpy(rows).cuda()
        kk = torch.from_numpy(keys).cuda()
        _close(from_dev_f64(dq[:, h:h + 1, r]), ref_dq, f"{name} h{h} dq rows")
        _close(from_dev_f64(dk[:, h:h + 1, kk]), ref_dk, f"{name} h{h} dk keys")
        _close(from_dev_f64(dv[:, h:h + 1, kk]), ref_dv, f"{name} h{h} dv keys")
    layout.close()
