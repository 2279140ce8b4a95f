"""Tensors past 2^31 elements: the kernels' 64-bit offsets at the largest sizes, for every entry point.

The 720p workload with 13 batch items (13 x 32 heads x 86,400 tokens x 64 channels =
2.30e9 elements, 4.6 GB per bf16 tensor): every batch item but the last is zero, and the last
item's last two heads hold the seeded 720p inputs.  Checked against the fp64 oracle on
sampled rows (and sampled keys for dK, dV) of those two heads, which sit at the highest
offsets of every tensor, with the tolerances of the other tests; the zero items against
their closed forms: zero queries and keys make every attended key equally likely, so
lse = ln(number of attended keys of the row) and out = 0 (zero values), and with a zero
upstream gradient every gradient is exactly zero (zeros of either sign: a rotated zero
pair can come out as -0).
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
        assert bool((out[b] == 0).all()), f"batch item {b}: out not zero"
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
            assert bool((t[b] == 0).all()), f"batch item {b}: {name} not zero"
    layout.close()


def _pair_close(got, ref, what):
    """Prologue bound (as in the prologue tests): fp32 math to a few 1e-7 of each channel
    pair's norm, plus half a bf16 ulp of the value."""
    pair_norm = np.repeat(np.hypot(ref[..., 0::2], ref[..., 1::2]), 2, axis=-1)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)) and np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-5 * pair_norm), what


def _grad_close(got, ref, what):
    max_abs, rel = out_errors(got, ref)
    scale = float(np.max(np.abs(ref)))
    say(f"  {what}: max_abs {max_abs:.3e} (max|ref| {scale:.3e}) rel_l2 {rel:.3e}")
    assert np.all(np.isfinite(got)) and max_abs <= 2e-2 * scale + 1e-6 and rel <= 1e-2, what


def test_large_offsets_prologue_merge_cross(lib):
    """The QK prologue and its backward, the merge and the cross-attention with its backward
    on the same 2.30e9-element tensors (zero items, seeded last heads of the last item)."""
    import torch
    from lcv_inputs import TEXT_LEN, text_kv_bits
    w = WORKLOADS["t2v720"]
    n = w.n_tokens
    eps = 1e-6
    xb, _, _ = qkv_bits(w.seed + 1, 1, SEEDED_HEADS, n)
    dyb = grad_bits(w.seed + 1, 1, SEEDED_HEADS, n)
    x, dy = _big_inputs(w, (xb, dyb))
    g = np.random.default_rng(3).uniform(0.5, 2.0, 64)
    gd = torch.from_numpy(g.astype(np.float32)).cuda()
    rng = np.random.default_rng(72)
    toks = np.unique(np.concatenate([[0, 1, n - 1], rng.integers(0, n, 20)]).astype(np.int64))
    t = torch.from_numpy(toks).cuda()
    hs = slice(w.heads - SEEDED_HEADS, w.heads)
    xs, dys = bf16_bits_to_f64(xb[:, :, toks]), bf16_bits_to_f64(dyb[:, :, toks])
    zero_items = (0, BATCH // 2)

    say("[large] QK prologue")
    y = lib.qk_rmsnorm_rope3d(x, gd, eps, w.grid)
    _sync()
    _pair_close(from_dev_f64(y[BATCH - 1:, hs][:, :, t]), oracle.rope3d_at(oracle.rmsnorm(xs, g, eps), toks, w.grid),
                "prologue rows")
    for b in zero_items:
        assert bool((y[b] == 0).all()), f"batch item {b}: prologue output not zero"

    say("[large] QK prologue backward")
    dx, dgamma = lib.qk_rmsnorm_rope3d_backward(x, dy, gd, eps, w.grid)
    _sync()
    ref_dx = np.zeros_like(xs)
    for i, tok in enumerate(toks):
        ref_dx[:, :, i:i + 1], _ = oracle.qk_norm_rope_backward(xs[:, :, i:i + 1], g, eps, w.grid, dys[:, :, i:i + 1],
                                                                token_offset=int(tok))
    _grad_close(from_dev_f64(dx[BATCH - 1:, hs][:, :, t]), ref_dx, "prologue dx rows")
    _, ref_dg = oracle.qk_norm_rope_backward(bf16_bits_to_f64(xb), g, eps, w.grid, bf16_bits_to_f64(dyb))
    got_dg = dgamma.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got_dg - ref_dg)) <= 1e-4 * float(np.max(np.abs(ref_dg))), "prologue dgamma"
    for b in zero_items:
        assert bool((dx[b] == 0).all()), f"batch item {b}: prologue dx not zero"
    del dx

    say("[large] merge of two parts")
    lse_bits = [np.random.default_rng(73 + i).uniform(-3.0, 3.0, (1, SEEDED_HEADS, n)).astype(np.float32)
                for i in range(2)]
    lses = []
    for lb in lse_bits:
        l = torch.zeros((BATCH, w.heads, n), dtype=torch.float32, device="cuda")
        l[BATCH - 1, hs] = torch.from_numpy(lb[0]).cuda()
        lses.append(l)
    out, lse = lib.attn_merge([x, y], lses)
    _sync()
    ys = from_dev_f64(y[BATCH - 1:, hs][:, :, t])
    ref_o, ref_l = oracle.merge_partials([xs, ys], [lb[:, :, toks].astype(np.float64) for lb in lse_bits])
    got = from_dev_f64(out[BATCH - 1:, hs][:, :, t])
    assert np.all(np.abs(got - ref_o) <= 2.0 ** -8 * np.abs(ref_o) + 1e-6 * max(np.max(np.abs(xs)), np.max(np.abs(ys))))
    assert np.max(np.abs(lse[BATCH - 1:, hs][:, :, t].cpu().numpy() - ref_l)) <= 1e-5 * max(1.0, np.max(np.abs(ref_l)))
    for b in zero_items:
        assert bool((out[b] == 0).all()), f"batch item {b}: merged out not zero"
        assert torch.allclose(lse[b], torch.full_like(lse[b], float(np.log(2.0))), rtol=0, atol=1e-6)
    del out, lse, lses, y

    say("[large] cross-attention and its backward")
    kb, vb = text_kv_bits(w.seed + 1, 1, SEEDED_HEADS)
    tk = torch.zeros((BATCH, w.heads, TEXT_LEN, 64), dtype=torch.bfloat16, device="cuda")
    tv = torch.zeros_like(tk)
    tk[BATCH - 1, hs] = to_dev(kb)[0]
    tv[BATCH - 1, hs] = to_dev(vb)[0]
    out, lse = lib.cross_attention(x, tk, tv)
    dq, dk, dv = lib.cross_attention_backward(x, tk, tv, out, lse, dy)
    _sync()
    kf, vf = bf16_bits_to_f64(kb), bf16_bits_to_f64(vb)
    ref_o, ref_l = oracle.cross_attention(bf16_bits_to_f64(xb), kf, vf, rows=toks)
    assert_out_close(from_dev_f64(out[BATCH - 1:, hs][:, :, t]), ref_o, "large cross")
    assert_lse_close(lse[BATCH - 1:, hs][:, :, t].cpu().numpy().astype(np.float64), ref_l, "large cross")
    rdq, _, _ = oracle.cross_attention_backward(xs, kf, vf, dys)
    _grad_close(from_dev_f64(dq[BATCH - 1:, hs][:, :, t]), rdq, "cross dq rows")
    _, rdk, rdv = oracle.cross_attention_backward(bf16_bits_to_f64(xb), kf, vf, bf16_bits_to_f64(dyb))
    _grad_close(from_dev_f64(dk[BATCH - 1:, hs]), rdk, "cross dk")
    _grad_close(from_dev_f64(dv[BATCH - 1:, hs]), rdv, "cross dv")
    for b in zero_items:
        assert bool((out[b] == 0).all()), f"batch item {b}: cross out not zero"
        assert torch.allclose(lse[b], torch.full_like(lse[b], float(np.log(TEXT_LEN))), rtol=1e-6, atol=0)
        for tt, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
            assert bool((tt[b] == 0).all()), f"batch item {b}: cross {name} not zero"
