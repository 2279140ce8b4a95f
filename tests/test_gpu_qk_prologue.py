"""GPU QK prologue (RMSNorm + 3D-RoPE) against the oracle (bf16 in, fp32 math, bf16 out)."""
import numpy as np
import pytest

import oracle
from lcv_inputs import WORKLOADS, bf16_bits_to_f64, qkv_bits, round_to_bf16_bits
from tests.gpu_util import from_dev_f64, say, to_dev

pytestmark = pytest.mark.gpu

# The fp32 path (sum of 64 squares, square root, product with the gain, rotation) is accurate
# to a few 1e-7 of the pair norm; rounding the result to bf16 adds at most half an ulp, 2^-8
# of the value.
REL = 2.0 ** -8
ABS_PAIR = 1e-5
EPS = 1e-6


def _gamma(seed=3):
    return np.random.default_rng(seed).uniform(0.5, 2.0, 64)


def _dev_gamma(g):
    import torch
    return torch.from_numpy(g.astype(np.float32)).cuda()


def _check(got, ref):
    pair_norm = np.repeat(np.hypot(ref[..., 0::2], ref[..., 1::2]), 2, axis=-1)
    err = np.abs(got - ref)
    bound = REL * np.abs(ref) + ABS_PAIR * pair_norm
    assert np.all(np.isfinite(got))
    assert np.all(err <= bound), float(np.max(err - bound))
    nearest = bf16_bits_to_f64(round_to_bf16_bits(ref.astype(np.float32)))
    exact = np.mean(got == nearest)
    assert exact > 0.98, exact


@pytest.mark.parametrize("grid,heads,offset,n_tokens", [
    ((4, 8, 16), 2, 0, None),           # tiny workload grid
    ((3, 10, 21), 3, 0, None),          # 630 tokens: partial last 256-thread group
    ((3, 10, 21), 2, 210, 420),         # noise tokens of a one-frame condition
    ((24, 30, 52), 1, 0, None),         # 480p grid, one head
    ((24, 45, 80), 1, 0, None),         # 720p grid, one head
])
def test_prologue_parity(lib, grid, heads, offset, n_tokens):
    import torch
    total = grid[0] * grid[1] * grid[2]
    n = total - offset if n_tokens is None else n_tokens
    say(f"[qk-prologue] grid={grid} heads={heads} offset={offset} n={n}")
    x_bits, _, _ = qkv_bits(17, 1, heads, n)
    g = _gamma()
    x = to_dev(x_bits)
    y = lib.qk_rmsnorm_rope3d(x, _dev_gamma(g), EPS, grid, token_offset=offset)
    torch.cuda.synchronize()
    xf = bf16_bits_to_f64(x_bits)
    ref = oracle.qk_norm_rope(xf, g, EPS, grid, token_offset=offset)
    _check(from_dev_f64(y), ref)
    # in place gives the same bits
    x2 = x.clone()
    lib.qk_rmsnorm_rope3d(x2, _dev_gamma(g), EPS, grid, token_offset=offset, out=x2)
    torch.cuda.synchronize()
    assert torch.equal(x2.view(torch.int16), y.view(torch.int16))


def test_norm_only(lib):
    """Without a grid the call is the RMSNorm alone."""
    import torch
    say("[qk-prologue] norm only")
    x_bits, _, _ = qkv_bits(18, 2, 3, 333)
    g = _gamma(4)
    y = lib.qk_rmsnorm_rope3d(to_dev(x_bits), _dev_gamma(g), EPS)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(bf16_bits_to_f64(x_bits), g, EPS)
    _check(from_dev_f64(y), ref)


def test_magnitudes(lib):
    """Rows from 1e-30 to 1e30 (and a zero row): the kernel scales by a power of two before
    summing squares, so nothing overflows or underflows; rows far below sqrt(eps) give
    x / sqrt(eps)."""
    import torch
    say("[qk-prologue] magnitudes")
    grid = (2, 4, 8)
    rng = np.random.default_rng(19)
    base = rng.standard_normal((1, 1, 64, 64))
    scales = np.array([1e-30, 1e-20, 1e-6, 1e-3, 1.0, 1e3, 1e10, 1e20, 1e30, 3e37] * 6 + [1.0] * 3 + [0.0])
    x = (base * scales[None, None, :, None]).astype(np.float32)
    x_bits = round_to_bf16_bits(x)
    g = _gamma(5)
    for eps in (EPS, 0.0):
        y = lib.qk_rmsnorm_rope3d(to_dev(x_bits), _dev_gamma(g), eps, grid)
        torch.cuda.synchronize()
        got = from_dev_f64(y)
        xf = bf16_bits_to_f64(x_bits)
        nz = scales > 0
        with np.errstate(invalid="ignore", divide="ignore"):
            ref = oracle.qk_norm_rope(xf, g, eps, grid)
        _check(got[:, :, nz], ref[:, :, nz])
        zero_row = got[:, :, ~nz]
        if eps > 0:
            assert np.all(zero_row == 0.0)
        else:
            assert np.all(np.isnan(zero_row))   # 0 / sqrt(0), as the formula says


def test_workload_shapes(lib):
    """Full [1, 32, N, 64] tensor of the 720p workload: sampled tokens against the oracle."""
    import torch
    w = WORKLOADS["t2v720"]
    say("[qk-prologue] t2v720 full shape")
    x_bits, _, _ = qkv_bits(w.seed, 1, w.heads, w.n_tokens)
    g = _gamma(6)
    y = lib.qk_rmsnorm_rope3d(to_dev(x_bits), _dev_gamma(g), EPS, w.grid)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    toks = np.unique(np.concatenate([[0, 1, w.n_tokens - 1], rng.integers(0, w.n_tokens, 200)]))
    got = from_dev_f64(y[:, :, torch.from_numpy(toks).cuda()])
    xf = bf16_bits_to_f64(x_bits[:, :, toks])
    ref = oracle.rope3d_at(oracle.rmsnorm(xf, g, EPS), toks, w.grid)
    _check(got, ref)


def test_feeds_attention(lib):
    """Prologue on Q and K, then attention without fused RoPE, equals the oracle's attention
    of the normalised, rotated inputs (the intended use of the two entry points)."""
    import torch
    from tests.gpu_util import assert_out_close
    say("[qk-prologue] prologue + attention")
    grid = (3, 10, 21)
    n = grid[0] * grid[1] * grid[2]
    qb, kb, vb = qkv_bits(21, 1, 2, n)
    gq, gk = _gamma(7), _gamma(8)
    q = lib.qk_rmsnorm_rope3d(to_dev(qb), _dev_gamma(gq), EPS, grid)
    k = lib.qk_rmsnorm_rope3d(to_dev(kb), _dev_gamma(gk), EPS, grid)
    layout = lib.build_layout(n, 2, 4, 0)
    out, _ = lib.forward(q, k, to_dev(vb), layout, grid=None, rope_q=False, rope_k=False)
    torch.cuda.synchronize()
    qn = from_dev_f64(q)
    kn = from_dev_f64(k)
    ref, _ = oracle.bsa_forward(qn, kn, bf16_bits_to_f64(vb), grid, 0, 2, 4, rope_q=False, rope_k=False)
    assert_out_close(from_dev_f64(out), ref, "prologue + attention")
    layout.close()


# ----------------------------------------------------------------------------- backward
def _bwd_check(got_dx, got_dg, ref_dx, ref_dg, what):
    """dx: fp32 math rounded once to bf16 (relative L2 <= 1e-2, max-abs <= 2e-2 * max|ref|);
    dgamma: fp32 sums over many rows of exact bf16 products (relative error <= 1e-4 of the
    largest entry)."""
    from tests.gpu_util import out_errors
    max_abs, rel = out_errors(got_dx, ref_dx)
    scale = float(np.max(np.abs(ref_dx)))
    say(f"  {what}: dx max_abs {max_abs:.3e} (max|ref| {scale:.3e}) rel_l2 {rel:.3e}; "
        f"dgamma max err {float(np.max(np.abs(got_dg - ref_dg))):.3e} (max|ref| {float(np.max(np.abs(ref_dg))):.3e})")
    assert np.all(np.isfinite(got_dx)) and np.all(np.isfinite(got_dg))
    assert rel <= 1e-2 and max_abs <= 2e-2 * scale, (max_abs, rel)
    assert np.max(np.abs(got_dg - ref_dg)) <= 1e-4 * float(np.max(np.abs(ref_dg))) + 1e-6


@pytest.mark.parametrize("grid,heads,offset,n_tokens", [
    ((4, 8, 16), 2, 0, None),
    ((3, 10, 21), 3, 0, None),          # 630 tokens: partial token group
    ((3, 10, 21), 2, 210, 420),         # token offset
    ((2, 5, 7), 37, 0, None),           # 37 slices: 3 slice ranges, the last with 5 (odd) slices
    (None, 2, 0, 333),                  # RMSNorm alone
])
def test_prologue_backward_parity(lib, grid, heads, offset, n_tokens):
    import torch
    from lcv_inputs import grad_bits
    total = grid[0] * grid[1] * grid[2] if grid else n_tokens
    n = total - offset if n_tokens is None else n_tokens
    say(f"[qk-prologue bwd] grid={grid} heads={heads} offset={offset} n={n}")
    x_bits, _, _ = qkv_bits(23, 1, heads, n)
    dy_bits = grad_bits(23, 1, heads, n)
    g = _gamma(9)
    dx, dg = lib.qk_rmsnorm_rope3d_backward(to_dev(x_bits), to_dev(dy_bits), _dev_gamma(g), EPS, grid,
                                            token_offset=offset)
    torch.cuda.synchronize()
    ref_dx, ref_dg = oracle.qk_norm_rope_backward(bf16_bits_to_f64(x_bits), g, EPS, grid, bf16_bits_to_f64(dy_bits),
                                                  token_offset=offset)
    _bwd_check(from_dev_f64(dx), dg.cpu().numpy().astype(np.float64), ref_dx, ref_dg, "parity")
    # in place over dy gives the same bits; a second call the same dgamma bits
    dy2 = to_dev(dy_bits)
    _, dg2 = lib.qk_rmsnorm_rope3d_backward(to_dev(x_bits), dy2, _dev_gamma(g), EPS, grid, token_offset=offset,
                                            dx=dy2)
    torch.cuda.synchronize()
    assert torch.equal(dy2.view(torch.int16), dx.view(torch.int16))
    assert torch.equal(dg2, dg)


def test_prologue_backward_workload(lib):
    """Full [1, 32, N, 64] tensors of the 720p workload: dx on sampled tokens against the
    oracle; dgamma against the oracle over all rows of 4 heads (the same kernel path)."""
    import torch
    from lcv_inputs import grad_bits
    w = WORKLOADS["t2v720"]
    say("[qk-prologue bwd] t2v720 full shape")
    x_bits, _, _ = qkv_bits(w.seed, 1, w.heads, w.n_tokens)
    dy_bits = grad_bits(w.seed, 1, w.heads, w.n_tokens)
    g = _gamma(10)
    dx, _ = lib.qk_rmsnorm_rope3d_backward(to_dev(x_bits), to_dev(dy_bits), _dev_gamma(g), EPS, w.grid)
    torch.cuda.synchronize()
    assert torch.isfinite(dx.float()).all()
    rng = np.random.default_rng(11)
    toks = np.unique(np.concatenate([[0, 1, w.n_tokens - 1], rng.integers(0, w.n_tokens, 100)]))
    got = from_dev_f64(dx[:, :, torch.from_numpy(toks).cuda()])
    xs = bf16_bits_to_f64(x_bits[:, :, toks])
    dys = bf16_bits_to_f64(dy_bits[:, :, toks])
    # rows at arbitrary tokens: rotate back with the per-token positions
    ref_dx = np.zeros_like(xs)
    for i, t in enumerate(toks):
        ref_dx[:, :, i:i + 1], _ = oracle.qk_norm_rope_backward(xs[:, :, i:i + 1], g, EPS, w.grid, dys[:, :, i:i + 1],
                                                                token_offset=int(t))
    from tests.gpu_util import out_errors
    max_abs, rel = out_errors(got, ref_dx)
    assert rel <= 1e-2 and max_abs <= 2e-2 * float(np.max(np.abs(ref_dx))), (max_abs, rel)
    x4, dy4 = x_bits[:, :4], dy_bits[:, :4]
    _, dg4 = lib.qk_rmsnorm_rope3d_backward(to_dev(x4), to_dev(dy4), _dev_gamma(g), EPS, w.grid)
    torch.cuda.synchronize()
    _, ref_dg = oracle.qk_norm_rope_backward(bf16_bits_to_f64(x4), g, EPS, w.grid, bf16_bits_to_f64(dy4))
    got_dg = dg4.cpu().numpy().astype(np.float64)
    say(f"  dgamma over 4 heads: max err {float(np.max(np.abs(got_dg - ref_dg))):.3e} of {float(np.max(np.abs(ref_dg))):.3e}")
    assert np.max(np.abs(got_dg - ref_dg)) <= 1e-4 * float(np.max(np.abs(ref_dg)))
