"""C-ABI library on the CPU: it loads, exports every declared symbol, its host-side
layout arithmetic matches the oracle, and argument errors are reported before anything
touches the GPU (no compute calls here)."""
import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

import block_sparse_attention_lcv_amd as bsa
import oracle
from lcv_inputs import WORKLOADS

HEADER = Path(__file__).resolve().parent.parent / "include" / "lcv_bsa.h"


def _declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lcv_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = bsa.lib()
    declared = _declared_functions()
    assert declared, "no declarations found"
    assert sorted(bsa.EXPORTED) == declared
    for name in declared:
        assert hasattr(L, name), name


def test_abi_version():
    assert bsa.lib().lcv_abi_version() == 11


QUERY_CASES = [
    (512, 0, 2, 4), (37440, 0, 2, 4), (37440, 1560, 2, 4), (86400, 0, 2, 4), (62400, 24960, 2, 4),
    (62400, 24960, 64, 3), (62400, 24960, 2, 16), (630, 210, 2, 4), (630, 630, 1, 3), (1, 0, 2, 4),
    (63, 5, 0, 0), (65, 64, 0, 1), (1000, 999, 3, 5), (4097, 100, 7, 0), (5000, 64 * 13, 100, 2),
    (300, 63, 0, 3), (300, 127, 1, 2),
]


@pytest.mark.parametrize("n,c,w,s", QUERY_CASES)
def test_layout_query_matches_oracle(n, c, w, s):
    info = bsa.layout_query(n, w, s, c)
    row_ptr, col_idx = oracle.csr(n, c, w, s)
    lens = np.diff(row_ptr)
    assert info["n_blocks"] == oracle.n_blocks_of(n)
    assert info["nnz"] == col_idx.size
    assert info["max_row_len"] == int(lens.max())
    assert info["attended_pairs"] == oracle.attended_pairs(n, c, w, s)


def test_workload_flop_counts():
    """Effective FLOPs (4 * 64 * attended pairs * heads) of the five workloads."""
    expected = {"tiny": 8.808e7, "t2v480": 2.959e12, "i2v480": 2.844e12, "t2v720": 1.548e13, "vc480": 6.194e12}
    for name, w in WORKLOADS.items():
        info = bsa.layout_query(w.n_tokens, w.local_blocks, w.global_stride, w.cond_len)
        flops = 4 * 64 * info["attended_pairs"] * w.heads * w.batch
        assert abs(flops / expected[name] - 1) < 1e-3, (name, flops)


def _status(fn, *args):
    return fn(*args)


def test_layout_param_errors():
    L = bsa.lib()
    info = bsa.LayoutInfo()
    bad = [
        (bsa.LayoutParams(0, 64, 2, 4, 0), 2),        # no tokens
        (bsa.LayoutParams(128, 32, 2, 4, 0), 2),      # block must be 64
        (bsa.LayoutParams(128, 64, -1, 4, 0), 2),     # negative window
        (bsa.LayoutParams(128, 64, 2, -4, 0), 2),     # negative stride
        (bsa.LayoutParams(128, 64, 2, 4, 129), 2),    # cond_len > N
        (bsa.LayoutParams(128, 64, 2, 4, -1), 2),
        (bsa.LayoutParams(2**30, 64, 2, 1, 0), 6),    # too many blocks
    ]
    for params, code in bad:
        assert L.lcv_bsa_layout_query(ctypes.byref(params), ctypes.byref(info)) == code
        assert L.lcv_last_error()
    # the build entry point rejects the same parameters before touching the GPU
    handle = ctypes.c_void_p(1234)
    assert L.lcv_bsa_build_layout(ctypes.byref(bad[0][0]), None, ctypes.byref(handle)) == 2
    assert handle.value is None
    assert L.lcv_bsa_build_layout(None, None, ctypes.byref(handle)) == 1
    assert L.lcv_bsa_layout_query(None, ctypes.byref(info)) == 1
    assert L.lcv_bsa_layout_query(ctypes.byref(bsa.LayoutParams(128, 64, 2, 4, 0)), None) == 1
    assert L.lcv_bsa_build_layout(ctypes.byref(bsa.LayoutParams(128, 64, 2, 4, 0)), None, None) == 1


def test_forward_requires_layout():
    L = bsa.lib()
    g = bsa.Rope3dGrid(1, 1, 64, 1e4)
    p = ctypes.c_void_p(4096)
    assert L.lcv_bsa_forward(p, p, p, 1, 1, None, 0, 3, ctypes.byref(g), p, None, None) == 1
    assert L.lcv_bsa_forward_cached(p, p, p, p, p, 1, 1, None, 0, 3, ctypes.byref(g), p, None, None) == 1
    assert L.lcv_bsa_layout_get_info(None, None) == 1
    assert L.lcv_bsa_layout_copy_csr(None, p, p, None) == 1
    assert L.lcv_bsa_forward_rows(p, p, p, 1, 1, None, 0, 3, ctypes.byref(g), 0, 64, p, None, None) == 1
    L.lcv_bsa_layout_destroy(None)   # no-op


def test_cross_attention_argument_errors():
    L = bsa.lib()
    p = ctypes.c_void_p(4096)
    f = L.lcv_cross_attention
    assert f(None, p, p, 1, 1, 64, 64, None, p, None, None) == 1
    assert f(p, p, p, 1, 1, 64, 64, None, None, None, None) == 1
    assert f(p, None, p, 1, 1, 64, 64, None, p, None, None) == 1
    assert f(None, None, None, 1, 1, 0, 64, None, None, None, None) == 0   # no query: nothing read
    assert f(p, p, p, 0, 1, 64, 64, None, p, None, None) == 2
    assert f(p, p, p, 1, 1, -1, 64, None, p, None, None) == 2
    assert f(p, p, p, 1, 1, 64, -5, None, p, None, None) == 2
    assert f(ctypes.c_void_p(4104), p, p, 1, 1, 64, 64, None, p, None, None) == 2
    assert f(p, p, p, 1, 1, 64, 64, None, p, ctypes.c_void_p(4098), None) == 2
    assert f(p, p, p, 1, 1, 64, 64, ctypes.c_void_p(4097), p, None, None) == 2
    assert f(p, p, p, 1, 1, 0, 64, None, p, None, None) == 0          # no query: nothing to do
    assert f(p, p, p, 65536, 65536, 64, 64, None, p, None, None) == 6


def _cross_bwd_workspace(batch, heads, n_q, kv_len):
    """Expected scratch size: 38 values per query row (the scaled Q as 64 bf16, lse and D, the
    three bf16 parts of each of those two in 8 bytes; rounded up to 4), then fp32 partial dK and dV per query chunk; chunks give about 512
    key-walk workgroups, at most 64 and at most one per query block, none empty."""
    bh = batch * heads
    nqb, nkb = -(-n_q // 64), -(-kv_len // 64)
    groups = -(-nkb // 4)
    chunks = 0
    if nqb and groups:
        chunks = min(-(-512 // (bh * groups)), 64, nqb)
        per = -(-nqb // chunks)
        chunks = -(-nqb // per)
    return -(-38 * bh * n_q // 4) * 4 + 2 * chunks * bh * kv_len * 64


def test_cross_backward_workspace_sizes():
    f = bsa.lib().lcv_cross_attention_backward_workspace
    for args in [(1, 1, 64, 64), (2, 3, 1000, 77), (1, 32, 58560, 512), (4, 2, 0, 512), (1, 1, 100, 0),
                 (3, 5, 4097, 300)]:
        assert f(*args) == _cross_bwd_workspace(*args), args
    assert f(1, 1, 64, 64) == 38 * 64 + 2 * 64 * 64
    assert f(0, 1, 64, 64) == -1 and f(1, 1, -1, 64) == -1 and f(1, 1, 64, -1) == -1


def test_cross_backward_argument_errors():
    L = bsa.lib()
    p = ctypes.c_void_p(4096)
    f = L.lcv_cross_attention_backward
    big = 1 << 40

    def call(q=p, lse=p, batch=1, heads=1, n_q=64, kv_len=64, kv_lens=None, ws=p, ws_n=big, dk=p):
        return f(q, p, p, p, lse, p, batch, heads, n_q, kv_len, kv_lens, p, dk, p, ws, ws_n, None)

    assert call(q=None) == 1
    assert call(lse=None) == 1
    assert call(ws=None) == 1
    assert call(dk=None) == 1
    assert call(q=None, lse=None, n_q=0, dk=None) == 1           # text side still needs dk
    assert call(q=None, lse=None, n_q=0, kv_len=0, dk=None, ws=None, ws_n=0) == 0
    assert call(batch=0) == 2
    assert call(n_q=-1) == 2
    assert call(kv_len=-3) == 2
    assert call(q=ctypes.c_void_p(4104)) == 2
    assert call(lse=ctypes.c_void_p(4098)) == 2
    assert call(ws=ctypes.c_void_p(4100)) == 2                  # workspace needs 16-byte alignment
    assert call(kv_lens=ctypes.c_void_p(4097)) == 2
    assert call(ws_n=L.lcv_cross_attention_backward_workspace(1, 1, 64, 64) - 1) == 2
    assert b"workspace" in L.lcv_last_error()
    assert call(n_q=0, kv_len=0) == 0                            # nothing to compute
    assert call(batch=65536, heads=65536, ws_n=1 << 62) == 6


def test_merge_argument_errors():
    L = bsa.lib()
    p = ctypes.c_void_p(4096)
    arr = (ctypes.c_void_p * 2)(4096, 8192)
    bad = (ctypes.c_void_p * 2)(4096, 4100)
    null_part = (ctypes.c_void_p * 2)(4096, None)
    f = L.lcv_attn_merge
    assert f(None, arr, 2, 10, p, None, None) == 1
    assert f(arr, arr, 2, 10, None, None, None) == 1
    assert f(arr, null_part, 2, 10, p, None, None) == 1
    assert f(arr, arr, 0, 10, p, None, None) == 2
    assert f(arr, arr, 9, 10, p, None, None) == 2
    assert f(arr, arr, 2, -1, p, None, None) == 2
    assert f(bad, arr, 2, 10, p, None, None) == 2
    assert f(arr, arr, 2, 10, p, ctypes.c_void_p(4098), None) == 2
    assert f(arr, arr, 2, 0, p, None, None) == 0          # no rows: nothing to do


def test_prologue_backward_argument_errors():
    L = bsa.lib()
    g = bsa.Rope3dGrid(2, 4, 8, 1e4)
    p = ctypes.c_void_p(4096)
    f = L.lcv_qk_rmsnorm_rope3d_backward
    need = L.lcv_qk_rmsnorm_rope3d_backward_workspace(32, 86400)
    assert need == 512 * 2 * 64                 # 512 token-group workgroups x 2 slice ranges
    assert L.lcv_qk_rmsnorm_rope3d_backward_workspace(3, 64) == 2 * 64     # 64 tokens = 2 token groups
    assert L.lcv_qk_rmsnorm_rope3d_backward_workspace(-1, 64) == -1
    assert f(None, p, p, 1e-6, 1, 64, 0, ctypes.byref(g), p, p, p, 64, None) == 1
    assert f(p, p, p, 1e-6, 1, 64, 0, ctypes.byref(g), p, p, None, 64, None) == 1
    assert f(p, p, p, -1.0, 1, 64, 0, ctypes.byref(g), p, p, p, 64, None) == 2
    assert f(p, p, ctypes.c_void_p(4100), 1e-6, 1, 64, 0, ctypes.byref(g), p, p, p, 64, None) == 2
    assert f(p, p, p, 1e-6, 1, 64, 0, ctypes.byref(g), p, p, p, 127, None) == 2     # workspace too small
    assert f(p, p, p, 1e-6, 1, 64, 1, ctypes.byref(g), p, p, p, 64, None) == 3      # 65 tokens > 64
    assert f(p, p, p, 1e-6, 2000000, 64, 0, None, p, p, p, 1 << 40, None) == 6


def test_backward_argument_errors():
    L = bsa.lib()
    p = ctypes.c_void_p(4096)
    f = L.lcv_bsa_backward
    big = 1 << 40
    assert f(p, p, p, p, p, p, 1, 1, None, 0, p, p, p, p, big, None) == 1          # no layout
    assert f(p, p, p, p, p, p, 1, 1, None, 0, p, p, p, None, big, None) == 1       # no workspace
    assert f(p, p, p, p, None, p, 1, 1, None, 0, p, p, p, p, big, None) == 1       # no lse
    assert f(p, p, p, p, p, None, 1, 1, None, 0, p, p, p, p, big, None) == 1       # no dout
    assert b"required" in L.lcv_last_error()


def test_backward_workspace_sizes():
    """152 bytes per query row: the scaled Q (64 bf16), two fp32 per-row terms and the three
    bf16 parts of each of them (8 bytes each)."""
    f = bsa.lib().lcv_bsa_backward_workspace
    assert f(1, 1, 64) == 38 * 64
    assert f(1, 32, 86400) == 38 * 32 * 86400
    assert f(2, 3, 631) == 38 * 6 * 631
    assert f(0, 1, 64) == -1 and f(1, 0, 64) == -1 and f(1, 1, 0) == -1


def test_rope_argument_errors():
    L = bsa.lib()
    g = bsa.Rope3dGrid(2, 4, 8, 1e4)
    p = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4098)
    assert L.lcv_rope3d_apply(None, p, 1, 64, 0, ctypes.byref(g), None) == 1
    assert L.lcv_rope3d_apply(p, p, 1, 64, 0, None, None) == 1
    assert L.lcv_rope3d_apply(mis, p, 1, 64, 0, ctypes.byref(g), None) == 2
    assert L.lcv_rope3d_apply(p, p, -1, 64, 0, ctypes.byref(g), None) == 2
    assert L.lcv_rope3d_apply(p, p, 1, 64, 1, ctypes.byref(g), None) == 3       # 65 tokens > 64
    bad_theta = bsa.Rope3dGrid(2, 4, 8, 0.0)
    assert L.lcv_rope3d_apply(p, p, 1, 64, 0, ctypes.byref(bad_theta), None) == 2
    bad_dims = bsa.Rope3dGrid(0, 4, 8, 1e4)
    assert L.lcv_rope3d_apply(p, p, 1, 64, 0, ctypes.byref(bad_dims), None) == 2


def test_qk_prologue_argument_errors():
    L = bsa.lib()
    g = bsa.Rope3dGrid(2, 4, 8, 1e4)
    p = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4098)
    f = L.lcv_qk_rmsnorm_rope3d
    assert f(None, p, p, 1e-6, 1, 64, 0, ctypes.byref(g), None) == 1
    assert f(p, None, p, 1e-6, 1, 64, 0, ctypes.byref(g), None) == 1
    assert f(p, p, None, 1e-6, 1, 64, 0, ctypes.byref(g), None) == 1
    assert f(mis, p, p, 1e-6, 1, 64, 0, ctypes.byref(g), None) == 2
    assert f(p, p, ctypes.c_void_p(4097), 1e-6, 1, 64, 0, ctypes.byref(g), None) == 2
    assert f(p, p, p, -1e-6, 1, 64, 0, ctypes.byref(g), None) == 2
    assert f(p, p, p, float("nan"), 1, 64, 0, ctypes.byref(g), None) == 2
    assert f(p, p, p, 1e-6, -1, 64, 0, ctypes.byref(g), None) == 2
    assert f(p, p, p, 1e-6, 1, 64, 1, ctypes.byref(g), None) == 3       # 65 tokens > 64
    bad_theta = bsa.Rope3dGrid(2, 4, 8, 0.0)
    assert f(p, p, p, 1e-6, 1, 64, 0, ctypes.byref(bad_theta), None) == 2
    assert f(p, p, p, 1e-6, 600000, 64, 0, None, None) == 6
    for code in (1, 2, 3, 6):
        assert L.lcv_last_error()
