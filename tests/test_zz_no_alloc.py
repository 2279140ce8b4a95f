"""The allocation-free prologue backward (lcv_qk_rmsnorm_rope3d_backward_noalloc, the library's
static scratch instead of a caller's workspace) against the entry point with a workspace,
through the C ABI: bitwise equal dx and dgamma on two calls in a row, the second one smaller,
and sizes beyond the static scratch refused before anything runs."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

from lcv_inputs import grad_bits, qkv_bits
from tests.gpu_util import say, to_dev

EPS = 1e-6


def _gamma(seed):
    import torch
    g = np.random.default_rng(seed).uniform(0.5, 2.0, 64).astype(np.float32)
    return torch.from_numpy(g).cuda()


def _both(lib, x, dy, gamma, grid, token_offset):
    """(dx, dgamma) from the entry point with a workspace and from the allocation-free one."""
    import torch
    L = lib.lib()
    n_tokens = x.shape[-2]
    n_outer = x.numel() // (64 * n_tokens)
    g = lib.Rope3dGrid(*grid, 1e4) if grid is not None else None
    gp = ctypes.byref(g) if g is not None else None
    ws = torch.empty(max(int(L.lcv_qk_rmsnorm_rope3d_backward_workspace(n_outer, n_tokens)), 1), dtype=torch.float32,
                     device="cuda")
    dx_ws, dx_na = torch.empty_like(x), torch.full_like(x, float("nan"))
    dg_ws = torch.empty(64, dtype=torch.float32, device="cuda")
    dg_na = torch.full((64,), float("nan"), dtype=torch.float32, device="cuda")
    st = L.lcv_qk_rmsnorm_rope3d_backward(x.data_ptr(), dy.data_ptr(), gamma.data_ptr(), EPS, n_outer, n_tokens,
                                          token_offset, gp, dx_ws.data_ptr(), dg_ws.data_ptr(), ws.data_ptr(),
                                          ws.numel(), None)
    assert st == 0, L.lcv_last_error()
    st = L.lcv_qk_rmsnorm_rope3d_backward_noalloc(x.data_ptr(), dy.data_ptr(), gamma.data_ptr(), EPS, n_outer,
                                                  n_tokens, token_offset, gp, dx_na.data_ptr(), dg_na.data_ptr(),
                                                  None)
    assert st == 0, L.lcv_last_error()
    torch.cuda.synchronize()
    return (dx_ws, dg_ws), (dx_na, dg_na)


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point(lib):
    import torch
    cases = [
        # (grid, heads, token_offset, n_tokens): the second call is smaller than the first
        ((24, 45, 80), 8, 0, 86400),        # 720p grid, 8 heads: 512 x 1 workgroups of partials
        ((3, 10, 21), 3, 210, 420),         # 630-token grid, noise tokens only: 14 x 1 workgroups
    ]
    for grid, heads, offset, n in cases:
        say(f"[no-alloc] prologue backward grid {grid} heads {heads} tokens [{offset}, {offset + n})")
        xb, _, _ = qkv_bits(71, 1, heads, n)
        x, dy = to_dev(xb), to_dev(grad_bits(71, 1, heads, n))
        (dx_ws, dg_ws), (dx_na, dg_na) = _both(lib, x, dy, _gamma(9), grid, offset)
        assert torch.equal(dx_ws.view(torch.int16), dx_na.view(torch.int16))
        assert torch.equal(dg_ws.view(torch.int32), dg_na.view(torch.int32))
    # norm only (no grid), a third shape
    xb, _, _ = qkv_bits(72, 1, 2, 100)
    x, dy = to_dev(xb), to_dev(grad_bits(72, 1, 2, 100))
    (dx_ws, dg_ws), (dx_na, dg_na) = _both(lib, x, dy, _gamma(10), None, 0)
    assert torch.equal(dx_ws.view(torch.int16), dx_na.view(torch.int16))
    assert torch.equal(dg_ws.view(torch.int32), dg_na.view(torch.int32))


def test_noalloc_refuses_sizes_beyond_its_scratch():
    """Checked on the host before any device work: 1,048,576 scratch values hold 16,384
    workgroup partials (512 token groups x 32 slice ranges of 16 slices at full length)."""
    import block_sparse_attention_lcv_amd as bsa
    L = bsa.lib()
    p = ctypes.c_void_p(4096)
    need = L.lcv_qk_rmsnorm_rope3d_backward_workspace(16 * 33, 86400)
    assert need > (1 << 20)
    assert L.lcv_qk_rmsnorm_rope3d_backward_noalloc(p, p, p, EPS, 16 * 33, 86400, 0, None, p, p, None) == 6
    assert b"static scratch" in L.lcv_last_error()
    assert L.lcv_qk_rmsnorm_rope3d_backward_noalloc(None, p, p, EPS, 16, 64, 0, None, p, p, None) == 1
    assert L.lcv_qk_rmsnorm_rope3d_backward_noalloc(p, p, p, -1.0, 16, 64, 0, None, p, p, None) == 2
