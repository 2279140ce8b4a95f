"""Tensors past 2^31 elements: the kernels' 64-bit offsets at the largest sizes.

The 720p workload with 13 batch items (13 x 32 heads x 86,400 tokens x 64 channels =
2.30e9 elements, 4.6 GB per bf16 tensor): every batch item but the last is zero, and the last
item's last two heads hold the seeded 720p inputs.  Checked against the fp64 oracle on
sampled rows (and sampled keys for dK, dV) of those two heads, which sit at the highest
offsets of every tensor, with the tolerances of the other tests; the zero items against
their closed forms: zero queries and keys make every attended key equally likely, so
lse = ln(number of attended keys of the row) and out = 0 (zero values), and with a zero
upstream gradient every gradient is exactly zero.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from lcv_inputs import WORKLOADS, bf16_bits_to_f64, grad_bits, qkv_bits
from tests.gpu_util import assert_lse_close, assert_out_close, from_dev_f64, out_errors, say, to_dev

pytestmark = pytest.mark.gpu

BATCH = 13
SEEDED_HEADS = 2


def _sync():
    import torch
    torch.cuda.synchronize()


def _big_inputs(w, bits_list):
    """[BATCH, heads, N, 64] bf16 device tensors: zeros, with bits (shaped [1, SEEDED_HEADS,
    N, 64]) in the last heads of the last batch item."""
    import torch
    out = []
    for bits in bits_list:
        t = torch.zeros((BATCH, w.heads, w.n_tokens, 64), dtype=torch.bfloat16, device="cuda")
        t[BATCH - 1, w.heads - SEEDED_HEADS:] = to_dev(bits)[0]
        out.append(t)
    return out


def test_large_offsets_forward_and_backward(lib):
    import torch
    w = WORKLOADS["t2v720"]
    assert BATCH * w.heads * w.n_tokens * 64 > 2 ** 31
    say(f"[large] t2v720 x {BATCH} batch items: {BATCH * w.heads * w.n_tokens * 64:.3e} elements per tensor")
    qb, kb, vb = qkv_bits(w.seed, 1, SEEDED_HEADS, w.n_tokens)
    gb = grad_bits(w.seed, 1, SEEDED_HEADS, w.n_tokens)
    layout = lib.build_layout(w.n_tokens, w.local_blocks, w.global_stride, w.cond_len)
    q, k, v = _big_inputs(w, (qb, kb, vb))
    rng = np.random.default_rng(71)
    n = w.n_tokens
    rows = np.unique(np.concatenate([[0, 63, 64, n - 65, n - 1], rng.integers(0, n, 20)]).astype(np.int64))
    r = torch.from_numpy(rows).cuda()
    args = [bf16_bits_to_f64(a) for a in (qb, kb, vb)]
    hs = slice(w.heads - SEEDED_HEADS, w.heads)

    # forward with the 3D-RoPE fused into the loads (the headline call)
    say("[large] forward, RoPE fused")
    out, lse = lib.forward(q, k, v, layout, grid=w.grid)
    _sync()
    ref_o, ref_l = oracle.bsa_forward(*args, w.grid, w.cond_len, w.local_blocks, w.global_stride, w.theta, rows=rows)
    assert_out_close(from_dev_f64(out[BATCH - 1:, hs][:, :, r]), ref_o, "large forward")
    assert_lse_close(lse[BATCH - 1:, hs][:, :, r].cpu().numpy().astype(np.float64), ref_l, "large forward")
    counts = oracle.token_mask_rows(rows, n, w.cond_len, w.local_blocks, w.global_stride).sum(axis=1)
    for b in (0, BATCH // 2):
        assert not out[b].view(torch.int16).any(), f"batch item {b}: out not zero"
        got_l = lse[b, :, r].cpu().numpy().astype(np.float64)
        assert np.max(np.abs(got_l - np.log(counts)[None, :])) < 1e-5 * np.log(counts).max()
    assert torch.isfinite(lse).all()
    del out, lse

    # backward on the scores' inputs (no RoPE: q and k as they enter the scores)
    say("[large] forward without RoPE, backward")
    out, lse = lib.forward(q, k, v, layout, grid=None)
    (do,) = _big_inputs(w, (gb,))
    dq, dk, dv = lib.backward(q, k, v, out, lse, do, layout)
    _sync()
    gargs = args + [bf16_bits_to_f64(gb)]
    keys = np.unique(np.concatenate([np.arange(64 * j, 64 * j + 64, 21)
                                     for j in (1, 2, w.n_blocks - 2, w.n_blocks - 1)]).astype(np.int64))
    keys = keys[(keys // 64) % w.global_stride != 0]
    kk = torch.from_numpy(keys).cuda()
    ref_dq = oracle.bsa_backward_rows(*gargs, w.cond_len, w.local_blocks, w.global_stride, rows)
    ref_dk, ref_dv = oracle.bsa_backward_keys(*gargs, w.cond_len, w.local_blocks, w.global_stride, keys)
    for got, ref, what in ((dq[BATCH - 1:, hs][:, :, r], ref_dq, "dq rows"), (dk[BATCH - 1:, hs][:, :, kk], ref_dk, "dk keys"),
                           (dv[BATCH - 1:, hs][:, :, kk], ref_dv, "dv keys")):
        g = from_dev_f64(got)
        max_abs, rel = out_errors(g, ref)
        scale = float(np.max(np.abs(ref)))
        say(f"  {what}: max_abs {max_abs:.3e} (max|ref| {scale:.3e}) rel_l2 {rel:.3e}")
        assert np.all(np.isfinite(g)) and max_abs <= 2e-2 * scale + 1e-6 and rel <= 1e-2, what
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        for b in (0, BATCH // 2):
            assert not t[b].view(torch.int16).any(), f"batch item {b}: {name} not zero"
    layout.close()
