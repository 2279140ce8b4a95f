"""The Python binding's argument checks, on the CPU: every wrong shape, dtype or length of a
tensor whose address the C ABI would receive is refused with ValueError before anything is
launched (the library only sees raw pointers, so a short output would be written out of
bounds).  CPU tensors stand in for device tensors: each check below fires before the
binding asks for a device address."""
from __future__ import annotations

import pytest
import torch

import block_sparse_attention_lcv_amd as bsa


class _StubLayout:
    """What the binding reads from a layout before the call (no GPU needed)."""
    n_tokens = 630
    cond_len = 210
    handle = None


B, H, N = 1, 2, 630


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def test_forward_rejects_wrong_token_count():
    q = _t(B, H, 600, 64)
    with pytest.raises(ValueError, match="the layout"):
        bsa.forward(q, q, q, _StubLayout(), grid=None)


def test_forward_rejects_short_out_and_lse():
    q = _t(B, H, N, 64)
    with pytest.raises(ValueError, match="out must have the shape"):
        bsa.forward(q, q, q, _StubLayout(), grid=None, out=_t(B, H, N - 1, 64))
    with pytest.raises(ValueError, match="lse must have the shape"):
        bsa.forward(q, q, q, _StubLayout(), grid=None, lse=_t(B, H, N - 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="float32 CUDA"):
        bsa.forward(q, q, q, _StubLayout(), grid=None, lse=_t(B, H, N, dtype=torch.float16))
    with pytest.raises(ValueError, match="float32 CUDA"):     # right shape and dtype, but host memory
        bsa.forward(q, q, q, _StubLayout(), grid=None, lse=_t(B, H, N, dtype=torch.float32))


def test_forward_rows_rejects_short_out_and_lse():
    q = _t(B, H, 100, 64)
    kv = _t(B, H, N, 64)
    with pytest.raises(ValueError, match="q_rows must be"):
        bsa.forward_rows(q, kv, kv, _StubLayout(), 0, 99, grid=None)
    with pytest.raises(ValueError, match="out must have the shape"):
        bsa.forward_rows(q, kv, kv, _StubLayout(), 0, 100, grid=None, out=_t(B, H, 99, 64))
    with pytest.raises(ValueError, match="lse must have the shape"):
        bsa.forward_rows(q, kv, kv, _StubLayout(), 0, 100, grid=None, lse=_t(B, H, 101, dtype=torch.float32))


def test_forward_cached_rejects_short_out_and_lse():
    m = N - _StubLayout.cond_len
    qn = _t(B, H, m, 64)
    kc = _t(B, H, _StubLayout.cond_len, 64)
    with pytest.raises(ValueError, match="N-C"):
        bsa.forward_cached(_t(B, H, m + 1, 64), _t(B, H, m + 1, 64), _t(B, H, m + 1, 64), kc, kc, _StubLayout())
    with pytest.raises(ValueError, match="out must have the shape"):
        bsa.forward_cached(qn, qn, qn, kc, kc, _StubLayout(), out=_t(B, H, m - 1, 64))
    with pytest.raises(ValueError, match="lse must have the shape"):
        bsa.forward_cached(qn, qn, qn, kc, kc, _StubLayout(), lse=_t(B, H, m - 1, dtype=torch.float32))


def test_backward_rejects_wrong_shapes():
    q = _t(B, H, N, 64)
    lse = _t(B, H, N, dtype=torch.float32)
    with pytest.raises(ValueError, match="q must be"):
        x = _t(B, H, 600, 64)
        bsa.backward(x, x, x, x, _t(B, H, 600, dtype=torch.float32), x, _StubLayout())
    with pytest.raises(ValueError, match="lse must be"):
        bsa.backward(q, q, q, q, _t(B, H, N - 1, dtype=torch.float32), q, _StubLayout())
    with pytest.raises(ValueError, match="dq must have the shape"):
        bsa.backward(q, q, q, q, lse, q, _StubLayout(), dq=_t(B, H, N - 1, 64))


def test_cross_attention_rejects_short_lse():
    q = _t(B, H, 100, 64)
    kv = _t(B, H, 77, 64)
    with pytest.raises(ValueError, match="lse must have the shape"):
        bsa.cross_attention(q, kv, kv, out=_t(B, H, 100, 64), lse=_t(B, H, 99, dtype=torch.float32))
    with pytest.raises(ValueError, match="out must have the shape"):
        bsa.cross_attention(q, kv, kv, out=_t(B, H, 99, 64))
