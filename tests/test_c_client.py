"""The library used from plain C (tests/c_client/lcv_client.c, compiled with gcc against
include/lcv_bsa.h), outside the Python binding.

CPU: the client's host-only calls (ABI version, layout closed form) against the oracle's CSR
and attended-pair count.  GPU: the client's forward (layout build + RoPE-fused attention on
device memory it allocates itself) against the oracle, with the forward's bounds; the
cross-attention backward with no query and a NULL workspace of size 0, whose dK and dV
must come back as zeros (the gradient of an attention that no query reads)."""
from __future__ import annotations

import subprocess

import numpy as np
import pytest

import oracle
from lcv_inputs import bf16_bits_to_f64, qkv_bits
from tests.c_client import build_client
from tests.gpu_util import assert_lse_close, assert_out_close, say


def _client():
    if not build_client.CLIENT.exists():
        build_client.build()
    return str(build_client.CLIENT)


@pytest.mark.parametrize("n,local,stride,cond", [(86400, 2, 4, 0), (37440, 2, 4, 1560), (630, 1, 3, 210),
                                                 (512, 2, 4, 0)])
def test_c_client_layout_query(n, local, stride, cond):
    res = subprocess.run([_client(), "query", str(n), str(local), str(stride), str(cond)], capture_output=True,
                         text=True, timeout=60)
    assert res.returncode == 0, res.stderr
    got = dict(line.split() for line in res.stdout.strip().splitlines())
    import block_sparse_attention_lcv_amd as bsa
    assert int(got["abi_version"]) == bsa.lib().lcv_abi_version()
    row_ptr, _ = oracle.csr(n, cond, local, stride)
    assert int(got["n_blocks"]) == oracle.n_blocks_of(n)
    assert int(got["nnz"]) == int(row_ptr[-1])
    assert int(got["max_row_len"]) == int(np.max(np.diff(row_ptr)))
    assert int(got["attended_pairs"]) == oracle.attended_pairs(n, cond, local, stride)


def test_c_client_rejects_bad_arguments():
    res = subprocess.run([_client(), "query", "-5", "2", "4", "0"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 1 and "lcv_bsa_layout_query" in res.stderr
    res = subprocess.run([_client(), "nonsense"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 2 and "usage" in res.stderr


@pytest.mark.gpu
def test_c_client_forward(tmp_path):
    grid = (3, 10, 21)          # 630 tokens: ragged last block
    n, heads, cond, local, stride = 630, 2, 210, 2, 4
    say(f"[c client] forward grid {grid} heads {heads} C={cond}")
    qb, kb, vb = qkv_bits(81, 1, heads, n)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        for bits in (qb, kb, vb):
            f.write(np.ascontiguousarray(bits).astype(np.uint16).tobytes())
    res = subprocess.run([_client(), "forward", *map(str, grid), str(heads), str(local), str(stride), str(cond),
                          str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    raw = dst.read_bytes()
    n_out = heads * n * 64
    out = np.frombuffer(raw[:2 * n_out], dtype=np.uint16).reshape(1, heads, n, 64)
    lse = np.frombuffer(raw[2 * n_out:], dtype=np.float32).reshape(1, heads, n)
    ref_o, ref_l = oracle.bsa_forward(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), grid, cond,
                                      local, stride)
    assert_out_close(bf16_bits_to_f64(out), ref_o, "C client forward")
    assert_lse_close(lse.astype(np.float64), ref_l, "C client forward")


@pytest.mark.gpu
@pytest.mark.parametrize("heads,kv_len", [(2, 96), (3, 512)])
def test_c_client_cross_backward_without_queries(heads, kv_len):
    say(f"[c client] cross-attention backward, no query, heads {heads} text {kv_len}")
    res = subprocess.run([_client(), "cross_bwd_noquery", str(heads), str(kv_len)], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "zeros", res.stdout
