"""End to end on the GPU: the attention sub-layer of a LoRA training step, forward and
backward, against the composition of the oracle's pinned pieces.

Forward: q = prologue(x_q), k = prologue(x_k) (RMSNorm + 3D-RoPE, bf16), attention of q, k, v
(layout with a condition frame), then for the upstream gradient dO: the attention backward
(dq, dk, dv) and the prologue backward (dx_q, dgamma_q, dx_k, dgamma_k).  The oracle runs
the same chain in fp64 from the same bf16 inputs; the GPU's intermediate q, k, O and dq, dk
are bf16, so each stage adds about 2^-9 of relative error: relative L2 <= 2e-2 for every
gradient (1e-2 per stage, two stages) and dgamma within 2e-2 of its largest entry."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from lcv_inputs import bf16_bits_to_f64, grad_bits, qkv_bits
from tests.gpu_util import from_dev_f64, out_errors, say, to_dev

pytestmark = pytest.mark.gpu

EPS = 1e-6


@pytest.mark.parametrize("grid,heads,cond", [((3, 10, 21), 2, 210), ((4, 8, 16), 3, 0)])
def test_attention_layer_forward_backward(lib, grid, heads, cond):
    import torch
    n = grid[0] * grid[1] * grid[2]
    say(f"[train step] grid={grid} heads={heads} C={cond}")
    xq_b, xk_b, v_b = qkv_bits(91, 1, heads, n)
    do_b = grad_bits(91, 1, heads, n)
    rng = np.random.default_rng(92)
    gq, gk = rng.uniform(0.5, 2.0, 64), rng.uniform(0.5, 2.0, 64)
    dgq_t = torch.from_numpy(gq.astype(np.float32)).cuda()
    dgk_t = torch.from_numpy(gk.astype(np.float32)).cuda()
    xq, xk, v, do = to_dev(xq_b), to_dev(xk_b), to_dev(v_b), to_dev(do_b)
    layout = lib.build_layout(n, 2, 4, cond)
    q = lib.qk_rmsnorm_rope3d(xq, dgq_t, EPS, grid)
    k = lib.qk_rmsnorm_rope3d(xk, dgk_t, EPS, grid)
    out, lse = lib.forward(q, k, v, layout, grid=None)
    dq, dk, dv = lib.backward(q, k, v, out, lse, do, layout)
    dxq, dgam_q = lib.qk_rmsnorm_rope3d_backward(xq, dq, dgq_t, EPS, grid)
    dxk, dgam_k = lib.qk_rmsnorm_rope3d_backward(xk, dk, dgk_t, EPS, grid)
    torch.cuda.synchronize()

    xq64, xk64, v64, do64 = (bf16_bits_to_f64(a) for a in (xq_b, xk_b, v_b, do_b))
    q64 = oracle.qk_norm_rope(xq64, gq, EPS, grid)
    k64 = oracle.qk_norm_rope(xk64, gk, EPS, grid)
    rdq, rdk, rdv = oracle.bsa_backward(q64, k64, v64, do64, cond, 2, 4)
    rdxq, rdgq = oracle.qk_norm_rope_backward(xq64, gq, EPS, grid, rdq)
    rdxk, rdgk = oracle.qk_norm_rope_backward(xk64, gk, EPS, grid, rdk)
    for what, got, ref in (("dv", dv, rdv), ("dx_q", dxq, rdxq), ("dx_k", dxk, rdxk)):
        max_abs, rel = out_errors(from_dev_f64(got), ref)
        say(f"  {what}: rel_l2 {rel:.3e} max_abs {max_abs:.3e} (max|ref| {float(np.max(np.abs(ref))):.3e})")
        assert np.all(np.isfinite(from_dev_f64(got)))
        assert rel <= 2e-2, (what, rel)
    for what, got, ref in (("dgamma_q", dgam_q, rdgq), ("dgamma_k", dgam_k, rdgk)):
        err = float(np.max(np.abs(got.cpu().numpy().astype(np.float64) - ref)))
        say(f"  {what}: max err {err:.3e} (max|ref| {float(np.max(np.abs(ref))):.3e})")
        assert err <= 2e-2 * float(np.max(np.abs(ref))), (what, err)
    layout.close()
