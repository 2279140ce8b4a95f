"""GPU 3D-RoPE pass against the oracle (bf16 in, fp32 math, bf16 out)."""
import numpy as np
import pytest

import oracle
from lcv_inputs import WORKLOADS, bf16_bits_to_f64, qkv_bits, round_to_bf16_bits
from tests.gpu_util import from_dev_f64, say, to_dev

pytestmark = pytest.mark.gpu

# fp32 rotation error is ~1e-6 of the pair norm; rounding the result to bf16 adds at most
# half an ulp, i.e. 2^-8 of the value.
REL = 2.0 ** -8
ABS_PAIR = 1e-5


def _check(got, ref, x):
    pair_norm = np.repeat(np.hypot(x[..., 0::2], x[..., 1::2]), 2, axis=-1)
    err = np.abs(got - ref)
    bound = REL * np.abs(ref) + ABS_PAIR * pair_norm
    assert np.all(err <= bound), float(np.max(err - bound))
    # nearly every element is exactly the nearest bf16 of the fp64 result
    nearest = bf16_bits_to_f64(round_to_bf16_bits(ref.astype(np.float32)))
    exact = np.mean(got == nearest)
    assert exact > 0.99, exact


@pytest.mark.parametrize("grid,heads,offset,n_tokens", [
    ((4, 8, 16), 2, 0, None),           # tiny workload grid
    ((3, 10, 21), 3, 0, None),          # ragged (630 tokens)
    ((3, 10, 21), 2, 210, 420),         # noise tokens of a one-frame condition
    ((24, 30, 52), 1, 0, None),         # 480p grid, one head
    ((24, 45, 80), 1, 0, None),         # 720p grid, one head
])
def test_rope_parity(lib, grid, heads, offset, n_tokens):
    import torch
    total = grid[0] * grid[1] * grid[2]
    n = total - offset if n_tokens is None else n_tokens
    say(f"[rope] grid={grid} heads={heads} offset={offset} n={n}")
    x_bits, _, _ = qkv_bits(7, 1, heads, n)
    x = to_dev(x_bits)
    y = lib.rope3d_apply(x, grid, token_offset=offset)
    torch.cuda.synchronize()
    xf = bf16_bits_to_f64(x_bits)
    ref = oracle.rope3d(xf, grid, token_offset=offset)
    _check(from_dev_f64(y), ref, xf)
    # in place gives the same bits
    x2 = x.clone()
    lib.rope3d_apply(x2, grid, token_offset=offset, out=x2)
    torch.cuda.synchronize()
    assert torch.equal(x2.view(torch.int16), y.view(torch.int16))


def test_rope_workload_shapes(lib):
    """Full [1, 32, N, 64] tensors of the 720p workload: sampled tokens against the oracle."""
    import torch
    w = WORKLOADS["t2v720"]
    say(f"[rope] t2v720 full shape")
    x_bits, _, _ = qkv_bits(w.seed, 1, w.heads, w.n_tokens)
    y = lib.rope3d_apply(to_dev(x_bits), w.grid)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    toks = np.unique(np.concatenate([[0, 1, w.n_tokens - 1], rng.integers(0, w.n_tokens, 200)]))
    got = from_dev_f64(y[:, :, torch.from_numpy(toks).cuda()])
    xf = bf16_bits_to_f64(x_bits[:, :, toks])
    ref = oracle.rope3d_at(xf, toks, w.grid)
    _check(got, ref, xf)
