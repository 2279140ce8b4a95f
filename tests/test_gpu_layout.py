"""GPU layout build: the CSR is bit-exact against the oracle on every workload, the
density sweep and edge shapes."""
import numpy as np
import pytest

import oracle
from lcv_inputs import WORKLOADS
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

CASES = []
for _w in WORKLOADS.values():
    CASES.append((_w.name, _w.n_tokens, _w.cond_len, _w.local_blocks, _w.global_stride))
    for _l, _s in _w.sweep:
        CASES.append((f"{_w.name}-w{_l}s{_s}", _w.n_tokens, _w.cond_len, _l, _s))
CASES += [
    ("one-token", 1, 0, 2, 4), ("ragged", 630, 210, 2, 4), ("all-cond", 630, 630, 1, 3),
    ("no-global", 4097, 100, 7, 0), ("dense", 1000, 999, 3, 1), ("cond-at-63", 300, 63, 0, 3),
    ("wide-window", 5000, 13 * 64, 100, 2), ("window0-stride0", 777, 0, 0, 0),
]


@pytest.mark.parametrize("name,n,c,w,s", CASES, ids=[c[0] for c in CASES])
def test_csr_bit_exact(lib, name, n, c, w, s):
    say(f"[layout] {name} N={n} C={c} w={w} s={s}")
    layout = lib.build_layout(n, w, s, c)
    row_ptr, col_idx = layout.csr()
    import torch
    torch.cuda.synchronize()
    ref_ptr, ref_col = oracle.csr(n, c, w, s)
    assert np.array_equal(row_ptr.cpu().numpy(), ref_ptr)
    assert np.array_equal(col_idx.cpu().numpy(), ref_col)
    assert layout.info["nnz"] == ref_col.size
    assert layout.info["attended_pairs"] == oracle.attended_pairs(n, c, w, s)
    layout.close()
