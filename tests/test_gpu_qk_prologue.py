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
