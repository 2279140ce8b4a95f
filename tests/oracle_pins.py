"""Pins of the fp64 oracle: checks against facts fixed by the pages or by mathematics.

Each ``pin_*`` function takes an oracle implementation (the real ``oracle`` package or a
copy with a planted mistake) and raises AssertionError when the implementation breaks
the fact it pins.  None of them re-types the oracle's own formula: each uses a second,
independent formulation (complex arithmetic, brute-force loops with math.fsum, a
library routine, a hand-derived fixture or a closed form).
"""
from __future__ import annotations

import json
import math
from pathlib import Path

import numpy as np

GOLDEN = Path(__file__).resolve().parent / "golden"


# ----------------------------------------------------------------------------- RoPE
def pin_rope_norm(impl):
    """Rotations conserve the norm of every token (longcat-video-rs page, section 01
    studio readout "3D-RoPE norm conservation 1.00000"); fp64 holds it to 1e-12."""
    rng = np.random.default_rng(11)
    grid = (6, 9, 13)
    x = rng.standard_normal((3, 6 * 9 * 13, 64))
    y = impl.rope3d(x, grid)
    nx = np.linalg.norm(x, axis=-1)
    ny = np.linalg.norm(y, axis=-1)
    assert np.max(np.abs(ny / nx - 1.0)) < 1e-12
    # every adjacent channel pair is a rotation on its own: pair norms are conserved
    px = np.hypot(x[..., 0::2], x[..., 1::2])
    py = np.hypot(y[..., 0::2], y[..., 1::2])
    assert np.max(np.abs(px - py)) < 1e-12


def pin_rope_origin_identity(impl):
    """The token at (t, y, x) = (0, 0, 0) is left unchanged."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((1, 64))
    y = impl.rope3d(x, (4, 5, 6), token_offset=0)
    assert np.array_equal(x, y)


def _textbook_rope_1d(z: np.ndarray, pos: np.ndarray, dim: int, theta: float) -> np.ndarray:
    """Textbook rotary embedding of complex pairs z[..., dim/2] at integer positions:
    z_p * exp(i * pos * theta**(-2p/dim)), frequencies written as 1/theta**(arange(0,dim,2)/dim)."""
    inv_freq = 1.0 / theta ** (np.arange(0, dim, 2, dtype=np.float64) / dim)
    return z * np.exp(1j * np.outer(pos, inv_freq))


def pin_rope_sections_textbook(impl):
    """Each of the three sections is a textbook 1-D RoPE of its own axis: channels
    [0,16) follow t, [16,40) follow y, [40,64) follow x (longcat-video-rs page,
    section 03 "Partitioned 3D-RoPE (16T+24H+24W)"), with adjacent channels as the
    real and imaginary parts of one complex number."""
    rng = np.random.default_rng(13)
    grid = (5, 7, 11)
    theta = 10000.0
    n = grid[0] * grid[1] * grid[2]
    x = rng.standard_normal((n, 64))
    y = impl.rope3d(x, grid, theta)
    t, yy, xx = np.unravel_index(np.arange(n), grid)
    z = x[:, 0::2] + 1j * x[:, 1::2]
    ref = np.concatenate([
        _textbook_rope_1d(z[:, 0:8], t, 16, theta),
        _textbook_rope_1d(z[:, 8:20], yy, 24, theta),
        _textbook_rope_1d(z[:, 20:32], xx, 24, theta),
    ], axis=1)
    got = y[:, 0::2] + 1j * y[:, 1::2]
    assert np.max(np.abs(got - ref)) < 1e-12


def pin_rope_relative_position(impl):
    """<R(a) q, R(b) k> depends on a - b only: shifting both tokens by the same
    (dt, dy, dx) leaves the inner product unchanged (composition of rotations)."""
    rng = np.random.default_rng(14)
    grid = (9, 9, 9)
    q = rng.standard_normal((1, 64))
    k = rng.standard_normal((1, 64))

    def tok(t, y, x):
        return int(np.ravel_multi_index((t, y, x), grid))

    def dot(a, b):
        qa = impl.rope3d(q, grid, token_offset=a)
        kb = impl.rope3d(k, grid, token_offset=b)
        return float((qa * kb).sum())

    base = dot(tok(1, 2, 3), tok(4, 1, 0))
    for shift in ((2, 0, 0), (0, 3, 0), (0, 0, 5), (3, 4, 2)):
        a = tok(1 + shift[0], 2 + shift[1], 3 + shift[2])
        b = tok(4 + shift[0], 1 + shift[1], 0 + shift[2])
        assert abs(dot(a, b) - base) < 1e-11 * max(1.0, abs(base))


def pin_rope_closed_form_first_pair(impl):
    """Pair 0 of each section turns by exactly its axis position in radians
    (theta**0 = 1): the unit vector (1, 0) at position p maps to (cos p, sin p)."""
    grid = (8, 8, 8)
    for c0, axis in ((0, 0), (16, 1), (40, 2)):
        pos = [0, 0, 0]
        pos[axis] = 3
        x = np.zeros((1, 64))
        x[0, c0] = 1.0
        y = impl.rope3d(x, grid, token_offset=int(np.ravel_multi_index(pos, grid)))
        assert abs(y[0, c0] - math.cos(3.0)) < 1e-15 and abs(y[0, c0 + 1] - math.sin(3.0)) < 1e-15


# ----------------------------------------------------------------------------- QK prologue
def _rms_fsum(row) -> float:
    """Root mean square of one channel vector, summed with math.fsum."""
    return math.sqrt(math.fsum(float(v) * float(v) for v in row) / len(row))


def pin_rmsnorm_unit_rms(impl):
    """With unit gains and eps = 0 every normalised token has root mean square 1 and keeps
    its direction (myzaker article, technical principles: RMSNorm in self-attention)."""
    rng = np.random.default_rng(41)
    x = rng.standard_normal((5, 64)) * np.array([[0.01], [1.0], [3.0], [250.0], [1e-3]])
    y = impl.rmsnorm(x, np.ones(64), 0.0)
    for r in range(x.shape[0]):
        assert abs(_rms_fsum(y[r]) - 1.0) < 1e-13
        ratio = y[r] / x[r]
        assert np.max(np.abs(ratio - ratio[0])) < 1e-12 * abs(ratio[0]) and ratio[0] > 0


def pin_rmsnorm_scale_invariance(impl):
    """eps = 0: rmsnorm(c x) = rmsnorm(x) for c > 0 and rmsnorm(-x) = -rmsnorm(x)."""
    rng = np.random.default_rng(42)
    x = rng.standard_normal((3, 64))
    g = rng.uniform(0.5, 2.0, 64)
    base = impl.rmsnorm(x, g, 0.0)
    for c in (1e-3, 0.37, 12.0, 4096.0):
        assert np.max(np.abs(impl.rmsnorm(c * x, g, 0.0) - base)) < 1e-12
    assert np.max(np.abs(impl.rmsnorm(-x, g, 0.0) + base)) < 1e-13


def pin_rmsnorm_closed_form(impl):
    """Hand-computed case: x = (3, 4, 0, ..., 0) over 64 channels has mean square 25/64, so
    with eps = 0 the unit-gain result is (4.8, 6.4, 0, ...); eps = 25/64 doubles the mean
    square (divisor sqrt(50)/8); the gain multiplies channel by channel; a zero vector stays
    zero when eps > 0."""
    x = np.zeros((1, 64))
    x[0, 0], x[0, 1] = 3.0, 4.0
    y = impl.rmsnorm(x, np.ones(64), 0.0)
    assert abs(y[0, 0] - 4.8) < 1e-14 and abs(y[0, 1] - 6.4) < 1e-14 and np.all(y[0, 2:] == 0.0)
    y = impl.rmsnorm(x, np.ones(64), 25.0 / 64.0)
    assert abs(y[0, 0] - 3.0 * 8.0 / math.sqrt(50.0)) < 1e-14 and abs(y[0, 1] - 4.0 * 8.0 / math.sqrt(50.0)) < 1e-14
    g = np.arange(64, dtype=np.float64) + 0.5
    y = impl.rmsnorm(x, g, 0.0)
    assert abs(y[0, 0] - 4.8 * 0.5) < 1e-14 and abs(y[0, 1] - 6.4 * 1.5) < 1e-14
    z = impl.rmsnorm(np.zeros((2, 64)), g, 1e-6)
    assert np.all(z == 0.0)


def pin_qk_prologue_textbook(impl):
    """The prologue is RMSNorm (per token, gain applied channel by channel) followed by the
    textbook rotation of every section: checked with an fsum root mean square and complex
    rotations, on a non-uniform gain so that the order of the two steps matters."""
    rng = np.random.default_rng(43)
    grid = (3, 5, 7)
    theta = 10000.0
    off = 17   # rows are tokens off .. T*H*W-1, as for the noise rows of a cached call
    n = grid[0] * grid[1] * grid[2] - off
    x = rng.standard_normal((2, n, 64)) * 2.0
    g = rng.uniform(0.25, 3.0, 64)
    eps = 1e-5
    y = impl.qk_norm_rope(x, g, eps, grid, theta, token_offset=off)
    t, yy, xx = np.unravel_index(np.arange(off, off + n), grid)
    for b in range(2):
        inv = np.array([1.0 / math.sqrt(math.fsum(float(v) * float(v) for v in row) / 64.0 + eps) for row in x[b]])
        nx = x[b] * inv[:, None] * g[None, :]
        z = nx[:, 0::2] + 1j * nx[:, 1::2]
        ref = np.concatenate([
            _textbook_rope_1d(z[:, 0:8], t, 16, theta),
            _textbook_rope_1d(z[:, 8:20], yy, 24, theta),
            _textbook_rope_1d(z[:, 20:32], xx, 24, theta),
        ], axis=1)
        got = y[b][:, 0::2] + 1j * y[b][:, 1::2]
        assert np.max(np.abs(got - ref)) < 1e-12


def pin_qk_prologue_norm(impl):
    """Unit gains, eps = 0: every output token has Euclidean norm sqrt(64) = 8 exactly (the
    normalisation sets it, the rotation conserves it), at any token offset."""
    rng = np.random.default_rng(44)
    grid = (4, 6, 5)
    x = rng.standard_normal((3, 40, 64)) * 7.0
    y = impl.qk_norm_rope(x, np.ones(64), 0.0, grid, token_offset=60)
    assert np.max(np.abs(np.linalg.norm(y, axis=-1) - 8.0)) < 1e-12


# ----------------------------------------------------------------------------- layout
def _brute_token_mask(n_tokens, cond_len, local, stride):
    """Token mask by pure-Python loops over every (q, k)."""
    m = np.zeros((n_tokens, n_tokens), dtype=bool)
    for q in range(n_tokens):
        for k in range(n_tokens):
            i, j = q // 64, k // 64
            in_layout = abs(i - j) <= local or (stride >= 1 and j % stride == 0)
            m[q, k] = in_layout and (q >= cond_len or k < cond_len)
    return m


LAYOUT_CASES = [
    # (N, C, local, stride)
    (128, 0, 0, 0), (128, 0, 0, 2), (128, 37, 0, 2), (200, 0, 1, 3), (200, 64, 0, 4),
    (256, 100, 2, 4), (330, 130, 1, 2), (330, 330, 0, 3), (448, 65, 2, 0), (448, 1, 0, 1),
    (512, 0, 2, 4), (200, 63, 0, 3), (330, 329, 1, 4), (130, 127, 0, 2),
]


def pin_token_mask_brute_force(impl):
    """The token mask and the CSR equal brute-force enumeration of the rule on small
    inputs, including ragged N and condition lengths that split a block."""
    for n_tokens, cond, local, stride in LAYOUT_CASES:
        ref = _brute_token_mask(n_tokens, cond, local, stride)
        got = impl.token_mask_rows(np.arange(n_tokens), n_tokens, cond, local, stride)
        assert np.array_equal(got, ref), (n_tokens, cond, local, stride)
        n = -(-n_tokens // 64)
        blocks = np.zeros((n, n), dtype=bool)
        for i in range(n):
            for j in range(n):
                blocks[i, j] = ref[64 * i:64 * i + 64, 64 * j:64 * j + 64].any()
        row_ptr, col_idx = impl.csr(n_tokens, cond, local, stride)
        exp_ptr = [0]
        exp_col = []
        for i in range(n):
            cols = [j for j in range(n) if blocks[i, j]]
            exp_col += cols
            exp_ptr.append(len(exp_col))
        assert row_ptr.tolist() == exp_ptr and col_idx.tolist() == exp_col, (n_tokens, cond, local, stride)
        assert impl.attended_pairs(n_tokens, cond, local, stride) == int(ref.sum())


def pin_tiny_csr_golden(impl):
    """Hand-derived CSR of the 512-token, local 2, stride 4 layout (tests/golden)."""
    g = json.loads((GOLDEN / "tiny_csr.json").read_text())
    row_ptr, col_idx = impl.csr(g["n_tokens"], g["cond_len"], g["local_blocks"], g["global_stride"])
    assert row_ptr.tolist() == g["row_ptr"]
    assert col_idx.tolist() == [j for row in g["rows"] for j in row]


def pin_two_block_layouts(impl):
    """Two-block (N = 128) layouts over local in {0,1,2} and stride in {0,1,2},
    enumerated by hand: rows of attended key blocks."""
    expected = {
        (0, 0): [[0], [1]],
        (0, 1): [[0, 1], [0, 1]],
        (0, 2): [[0], [0, 1]],
    }
    for local in (0, 1, 2):
        for stride in (0, 1, 2):
            rows = expected.get((local, stride), [[0, 1], [0, 1]])
            row_ptr, col_idx = impl.csr(128, 0, local, stride)
            got = [col_idx[row_ptr[i]:row_ptr[i + 1]].tolist() for i in range(2)]
            assert got == rows, (local, stride, got)


def _nnz_closed_form(n_tokens, cond_len, local, stride):
    """Sum over query blocks of |band u multiples of s|, limited to key blocks that hold a
    condition key when every row of the query block is a condition row:
    |band| + ceil(lim/s) - #(multiples of s inside the band)."""
    n = -(-n_tokens // 64)
    jc = -(-cond_len // 64)          # key blocks holding at least one condition key
    total = 0
    for i in range(n):
        last_row = min(64 * i + 63, n_tokens - 1)
        lim = n if last_row >= cond_len else jc
        lo, hi = max(0, i - local), min(i + local, lim - 1)
        band = hi - lo + 1 if hi >= lo else 0
        if stride >= 1:
            mult_all = -(-lim // stride)
            mult_band = (hi // stride - (lo - 1) // stride) if band else 0
        else:
            mult_all = mult_band = 0
        total += band + mult_all - mult_band
    return total


CONFIG_LAYOUTS = [
    # (N, C) of the five workloads, layout (local, stride)
    (512, 0, 2, 4), (37440, 0, 2, 4), (37440, 1560, 2, 4), (86400, 0, 2, 4), (62400, 24960, 2, 4),
    (62400, 24960, 64, 3), (62400, 24960, 2, 3), (62400, 24960, 2, 8), (62400, 24960, 2, 12),
    (62400, 24960, 2, 16), (1000, 333, 3, 5),
]


def pin_nnz_closed_form(impl):
    """nnz of the CSR equals the closed form on every workload and density-sweep point."""
    for n_tokens, cond, local, stride in CONFIG_LAYOUTS:
        row_ptr, col_idx = impl.csr(n_tokens, cond, local, stride)
        assert int(row_ptr[-1]) == col_idx.size == _nnz_closed_form(n_tokens, cond, local, stride)


def pin_attended_pairs_closed_form(impl):
    """Attended pairs without condition tokens on a block-aligned N: nnz * 64 * 64."""
    for n_tokens, local, stride in ((37440, 2, 4), (86400, 2, 4), (62400, 2, 12)):
        assert impl.attended_pairs(n_tokens, 0, local, stride) == 4096 * _nnz_closed_form(n_tokens, 0, local, stride)


# ----------------------------------------------------------------------------- attention
def _brute_attention_row(qrow, keys, vals, allowed):
    """One row by pure-Python loops and math.fsum (fp64)."""
    scores = []
    for k in range(len(keys)):
        if allowed[k]:
            scores.append((k, math.fsum(qrow[d] * keys[k][d] for d in range(64)) / 8.0))
    if not scores:
        return [0.0] * 64, -math.inf
    m = max(s for _, s in scores)
    w = [(k, math.exp(s - m)) for k, s in scores]
    l = math.fsum(e for _, e in w)
    out = [math.fsum(e * vals[k][d] for k, e in w) / l for d in range(64)]
    return out, m + math.log(l)


def pin_two_block_brute_force(impl):
    """Two-block inputs (N = 128, local 0, strides 0 and 2) against a pure-Python
    attention with math.fsum, for condition lengths {0, 1, 37, 64, 100, 128}."""
    rng = np.random.default_rng(21)
    q = rng.standard_normal((1, 1, 128, 64))
    k = rng.standard_normal((1, 1, 128, 64))
    v = rng.standard_normal((1, 1, 128, 64))
    grid = (2, 4, 16)
    for stride in (0, 2):
        for cond in (0, 1, 37, 64, 100, 128):
            out, lse = impl.bsa_forward(q, k, v, grid, cond, 0, stride, rope_q=False, rope_k=False)
            for r in range(128):
                allowed = [(abs(r // 64 - c // 64) <= 0 or (stride and (c // 64) % stride == 0))
                           and (r >= cond or c < cond) for c in range(128)]
                ro, rl = _brute_attention_row(q[0, 0, r].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), allowed)
                assert np.max(np.abs(out[0, 0, r] - ro)) < 1e-12, (stride, cond, r)
                assert abs(lse[0, 0, r] - rl) < 1e-12, (stride, cond, r)


def pin_full_layout_is_dense_sdpa(impl):
    """With a layout that keeps every block pair (stride 1) and no condition tokens the
    method is plain softmax attention: compare with torch's scaled_dot_product_attention
    and logsumexp in float64 on the CPU."""
    import torch
    rng = np.random.default_rng(22)
    q = rng.standard_normal((2, 3, 300, 64))
    k = rng.standard_normal((2, 3, 300, 64))
    v = rng.standard_normal((2, 3, 300, 64))
    for local, stride in ((0, 1), (10, 0)):
        out, lse = impl.bsa_forward(q, k, v, (3, 10, 10), 0, local, stride, rope_q=False, rope_k=False)
        tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).numpy()
        ref_lse = torch.logsumexp(tq @ tk.transpose(-1, -2) / 8.0, dim=-1).numpy()
        assert np.max(np.abs(out - ref)) < 1e-12
        assert np.max(np.abs(lse - ref_lse)) < 1e-12


def pin_condition_isolation(impl):
    """Condition queries never see noise tokens (myzaker article, technical principles):
    replacing every noise Q/K/V leaves condition rows of out and lse bitwise unchanged."""
    rng = np.random.default_rng(23)
    grid = (4, 5, 13)            # 260 tokens, condition = first 1.5 frames = 97 tokens
    n = 260
    cond = 97
    q, k, v = (rng.standard_normal((1, 2, n, 64)) for _ in range(3))
    out1, lse1 = impl.bsa_forward(q, k, v, grid, cond, 1, 2)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for a in (q2, k2, v2):
        a[:, :, cond:] = rng.standard_normal(a[:, :, cond:].shape) * 3.0
    out2, lse2 = impl.bsa_forward(q2, k2, v2, grid, cond, 1, 2)
    assert np.array_equal(out1[:, :, :cond], out2[:, :, :cond])
    assert np.array_equal(lse1[:, :, :cond], lse2[:, :, :cond])
    assert not np.array_equal(out1[:, :, cond:], out2[:, :, cond:])


def pin_cached_equals_full(impl):
    """The cached call (condition K/V from the cache, noise rows only) equals rows [C, N)
    of the full call on the concatenated sequence."""
    rng = np.random.default_rng(24)
    grid = (3, 6, 20)
    n = 360
    for cond in (0, 120, 150):
        q, k, v = (rng.standard_normal((1, 2, n, 64)) for _ in range(3))
        full_o, full_l = impl.bsa_forward(q, k, v, grid, cond, 1, 3)
        o, l = impl.bsa_forward_cached(q[:, :, cond:], k[:, :, cond:], v[:, :, cond:], k[:, :, :cond],
                                       v[:, :, :cond], grid, cond, 1, 3)
        assert np.max(np.abs(o - full_o[:, :, cond:])) < 1e-13
        assert np.max(np.abs(l - full_l[:, :, cond:])) < 1e-13


def pin_rope_shift_invariance(impl):
    """Shifting every token's time position by the same amount leaves the attention
    output unchanged (RoPE scores depend on relative positions only)."""
    rng = np.random.default_rng(25)
    grid = (4, 6, 10)
    n = 240
    q, k, v = (rng.standard_normal((1, 1, n, 64)) for _ in range(3))
    out, _ = impl.bsa_forward(q, k, v, grid, 0, 1, 2)
    shift = 3 * 6 * 10      # three frames later
    qs = impl.rope3d(q, grid, token_offset=shift)
    ks = impl.rope3d(k, grid, token_offset=shift)
    out_s, _ = impl.bsa_forward(qs, ks, v, grid, 0, 1, 2, rope_q=False, rope_k=False)
    assert np.max(np.abs(out - out_s)) < 1e-12


def pin_sampled_rows_match_full(impl):
    """Evaluating a subset of rows gives the same values as the full evaluation."""
    rng = np.random.default_rng(26)
    grid = (3, 8, 12)
    n = 288
    q, k, v = (rng.standard_normal((1, 2, n, 64)) for _ in range(3))
    rows = np.array([0, 5, 63, 64, 100, 200, 287])
    out, lse = impl.bsa_forward(q, k, v, grid, 70, 2, 4)
    out_r, lse_r = impl.bsa_forward(q, k, v, grid, 70, 2, 4, rows=rows)
    assert np.max(np.abs(out[:, :, rows] - out_r)) < 1e-13
    assert np.max(np.abs(lse[:, :, rows] - lse_r)) < 1e-13


def pin_block_visiting_equals_masked_dense(impl):
    """Visiting only the attended key blocks gives the masked dense attention (to fp64
    rounding): with the condition boundary inside a block and a ragged last block, for every
    block and for an unordered subset; with no window and no global blocks it is dense
    softmax attention inside each block (written out with a textbook row softmax here)."""
    rng = np.random.default_rng(27)
    grid = (2, 15, 21)
    n = 630
    q, k, v = (rng.standard_normal((1, 2, n, 64)) for _ in range(3))
    out, lse = impl.bsa_forward(q, k, v, grid, 210, 2, 4)
    out_b, lse_b = impl.bsa_forward_blocks(q, k, v, grid, 210, 2, 4)
    assert np.max(np.abs(out - out_b)) < 1e-12 and np.max(np.abs(lse - lse_b)) < 1e-12
    blocks = [9, 0, 3]
    rows = np.concatenate([np.arange(64 * i, min(64 * i + 64, n)) for i in blocks])
    out_s, lse_s = impl.bsa_forward_blocks(q, k, v, grid, 210, 1, 3, q_blocks=blocks)
    out_r, lse_r = impl.bsa_forward(q, k, v, grid, 210, 1, 3, rows=rows)
    assert np.max(np.abs(out_s - out_r)) < 1e-12 and np.max(np.abs(lse_s - lse_r)) < 1e-12
    # no window, no global blocks, no condition: each block attends itself densely
    out_d, lse_d = impl.bsa_forward_blocks(q, k, v, grid, 0, 0, 0, q_blocks=[4, 9])
    qr = impl.rope3d(q[0, 0], grid)
    kr = impl.rope3d(k[0, 0], grid)
    at = 0
    for i in (4, 9):
        r = np.arange(64 * i, min(64 * i + 64, n))
        sc = qr[r] @ kr[r].T / 8.0
        mx = sc.max(axis=1, keepdims=True)
        w = np.exp(sc - mx)
        ref = (w / w.sum(axis=1, keepdims=True)) @ v[0, 0, r]
        assert np.max(np.abs(out_d[0, 0, at:at + r.size] - ref)) < 1e-12
        assert np.max(np.abs(lse_d[0, 0, at:at + r.size] - (mx[:, 0] + np.log(w.sum(axis=1))))) < 1e-12
        at += r.size


def pin_empty_row(impl):
    """A row with no attended key gives out = 0 and lse = -inf."""
    q = np.ones((2, 64))
    k = np.ones((3, 64))
    v = np.ones((3, 64))
    mask = np.array([[False, False, False], [True, False, False]])
    out, lse = impl.masked_attention(q, k, v, mask)
    assert np.all(out[0] == 0.0) and lse[0] == -np.inf
    assert np.allclose(out[1], 1.0) and abs(lse[1] - 8.0) < 1e-12


# ----------------------------------------------------------------------------- backward
def _bwd_case(seed, n_tokens=150, cond_len=70, heads=1):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((1, heads, n_tokens, 64)) for _ in range(4))
    return q, k, v, do, cond_len


def pin_backward_finite_differences(impl):
    """The gradients are the derivatives of L = sum(dout * out): central differences of the
    forward (step 1e-5, fp64) on sampled coordinates of q, k and v, on a layout with three
    blocks, a partial last block and the condition rule (C = 70)."""
    q, k, v, do, cond = _bwd_case(51)
    grid = (1, 10, 15)
    local, stride = 1, 2

    def loss(qq, kk, vv):
        out, _ = impl.bsa_forward(qq, kk, vv, grid, cond, local, stride, rope_q=False, rope_k=False)
        return math.fsum((out * do).ravel())

    dq, dk, dv = impl.bsa_backward(q, k, v, do, cond, local, stride)
    rng = np.random.default_rng(52)
    h = 1e-5
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(12):
            t, c = int(rng.integers(0, q.shape[2])), int(rng.integers(0, 64))
            args = [q.copy(), k.copy(), v.copy()]
            args[which][0, 0, t, c] += h
            lp = loss(*args)
            args[which][0, 0, t, c] -= 2 * h
            lm = loss(*args)
            num = (lp - lm) / (2 * h)
            assert abs(num - grad[0, 0, t, c]) < 1e-6 * max(1.0, abs(num)), (which, t, c, num, grad[0, 0, t, c])


def pin_backward_sums(impl):
    """Softmax is invariant to a shift of every key by one vector, so the key gradients of a
    head sum to zero; the value gradients sum to the sum of dout over the non-empty rows
    (each probability row sums to one)."""
    q, k, v, do, cond = _bwd_case(53, n_tokens=200, cond_len=64, heads=2)
    dq, dk, dv = impl.bsa_backward(q, k, v, do, cond, 2, 3)
    for h in range(2):
        assert np.max(np.abs(dk[0, h].sum(axis=0))) < 1e-10
        assert np.max(np.abs(dv[0, h].sum(axis=0) - do[0, h].sum(axis=0))) < 1e-10


def pin_backward_uniform_closed_form(impl):
    """q = 0 gives uniform probabilities over each row's allowed keys: dv[key] is the sum of
    dout[q] / (allowed count of q) over the rows q that see the key (brute-force loops)."""
    rng = np.random.default_rng(54)
    n, cond = 130, 64
    q = np.zeros((1, 1, n, 64))
    k, v, do = (rng.standard_normal((1, 1, n, 64)) for _ in range(3))
    _, _, dv = impl.bsa_backward(q, k, v, do, cond, 0, 0)
    allowed = _brute_token_mask(n, cond, 0, 0)
    ref = np.zeros((n, 64))
    for qi in range(n):
        keys = [kj for kj in range(n) if allowed[qi][kj]]
        for kj in keys:
            ref[kj] += do[0, 0, qi] / len(keys)
    assert np.max(np.abs(dv[0, 0] - ref)) < 1e-12


def pin_backward_sampled_match_full(impl):
    """dq at sampled rows and dk, dv at sampled keys (global, local-only, condition and last
    partial-block keys; row chunks smaller than a block) equal the full backward; the key
    subset's token mask equals the brute-force loops."""
    q, k, v, do, cond = _bwd_case(55, n_tokens=300, cond_len=100, heads=2)
    local, stride = 1, 3
    dq, dk, dv = impl.bsa_backward(q, k, v, do, cond, local, stride)
    rows = np.array([0, 63, 64, 99, 100, 180, 299])
    keys = np.array([0, 5, 64, 99, 100, 130, 192, 250, 299])
    assert np.allclose(impl.bsa_backward_rows(q, k, v, do, cond, local, stride, rows), dq[:, :, rows],
                       rtol=0, atol=1e-12)
    dks, dvs = impl.bsa_backward_keys(q, k, v, do, cond, local, stride, keys, row_chunk=37)
    assert np.allclose(dks, dk[:, :, keys], rtol=0, atol=1e-12)
    assert np.allclose(dvs, dv[:, :, keys], rtol=0, atol=1e-12)
    allowed = np.array(_brute_token_mask(300, cond, local, stride))
    assert np.array_equal(impl.token_mask(rows, keys, cond, local, stride), allowed[np.ix_(rows, keys)])


# ------------------------------------------------------------------------ prologue backward
def pin_rope_transpose(impl):
    """R^T is the adjoint and the inverse of the rotation: <R x, y> = <x, R^T y> and
    R^T R x = x, with a token offset."""
    rng = np.random.default_rng(81)
    grid = (3, 4, 5)
    x = rng.standard_normal((2, 40, 64))
    y = rng.standard_normal((2, 40, 64))
    rx = impl.rope3d(x, grid, token_offset=13)
    rty = impl.rope3d_transpose(y, grid, token_offset=13)
    assert abs(float(np.sum(rx * y)) - float(np.sum(x * rty))) < 1e-10
    assert np.max(np.abs(impl.rope3d_transpose(rx, grid, token_offset=13) - x)) < 1e-12


def pin_prologue_backward_finite_differences(impl):
    """dx and dgamma are the derivatives of L = sum(dy * qk_norm_rope(x)): central
    differences (step 1e-6, fp64) on sampled coordinates of x and gamma, with the 3D-RoPE
    (token offset 9) and without it (the RMSNorm alone), eps 1e-3 and 1e-6."""
    rng = np.random.default_rng(82)
    grid = (2, 3, 7)
    x = rng.standard_normal((2, 30, 64)) * rng.uniform(0.1, 3.0, (2, 30, 1))
    gamma = rng.uniform(0.5, 2.0, 64)
    dy = rng.standard_normal((2, 30, 64))
    h = 1e-6
    for g, eps in ((grid, 1e-6), (None, 1e-3)):
        def loss(xx, gg):
            y = impl.rmsnorm(xx, gg, eps) if g is None else impl.qk_norm_rope(xx, gg, eps, g, token_offset=9)
            return math.fsum((y * dy).ravel())
        dx, dgamma = impl.qk_norm_rope_backward(x, gamma, eps, g, dy, token_offset=9)
        for _ in range(12):
            i, t, c = int(rng.integers(0, 2)), int(rng.integers(0, 30)), int(rng.integers(0, 64))
            xp, xm = x.copy(), x.copy()
            xp[i, t, c] += h
            xm[i, t, c] -= h
            num = (loss(xp, gamma) - loss(xm, gamma)) / (2 * h)
            assert abs(num - dx[i, t, c]) < 1e-6 * max(1.0, abs(num)), (g, i, t, c, num, dx[i, t, c])
        for c in rng.choice(64, 8, replace=False):
            gp, gm = gamma.copy(), gamma.copy()
            gp[c] += h
            gm[c] -= h
            num = (loss(x, gp) - loss(x, gm)) / (2 * h)
            assert abs(num - dgamma[c]) < 1e-6 * max(1.0, abs(num)), (g, c, num, dgamma[c])


# ------------------------------------------------------------------------- cross-attention
def pin_cross_dense_sdpa(impl):
    """Without padding, cross-attention is plain softmax attention of the video queries over
    the text keys: torch's scaled_dot_product_attention and logsumexp in float64."""
    import torch
    rng = np.random.default_rng(61)
    q = rng.standard_normal((2, 3, 150, 64))
    k = rng.standard_normal((2, 3, 77, 64))
    v = rng.standard_normal((2, 3, 77, 64))
    out, lse = impl.cross_attention(q, k, v)
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).numpy()
    ref_lse = torch.logsumexp(tq @ tk.transpose(-1, -2) / 8.0, dim=-1).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12
    assert np.max(np.abs(lse - ref_lse)) < 1e-12


def pin_cross_padding(impl):
    """Padding: with kv_lens, batch item b equals the unpadded attention over its first
    kv_lens[b] text tokens, whatever the padded keys and values hold (bitwise); a length of
    zero gives out = 0, lse = -inf; sampled rows equal the full result (to rounding)."""
    rng = np.random.default_rng(62)
    q = rng.standard_normal((3, 2, 90, 64))
    k = rng.standard_normal((3, 2, 40, 64))
    v = rng.standard_normal((3, 2, 40, 64))
    lens = [40, 13, 0]
    out, lse = impl.cross_attention(q, k, v, kv_lens=lens)
    k2, v2 = k.copy(), v.copy()
    k2[1, :, 13:] = 1e3
    v2[1, :, 13:] = -7.0
    out2, lse2 = impl.cross_attention(q, k2, v2, kv_lens=lens)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    o1, l1 = impl.cross_attention(q[1:2], k[1:2, :, :13], v[1:2, :, :13])
    assert np.max(np.abs(out[1:2] - o1)) < 1e-12 and np.max(np.abs(lse[1:2] - l1)) < 1e-12
    o0, l0 = impl.cross_attention(q[0:1], k[0:1], v[0:1])
    assert np.array_equal(out[0:1], o0) and np.array_equal(lse[0:1], l0)
    assert np.all(out[2] == 0.0) and np.all(lse[2] == -np.inf)
    rows = np.array([0, 5, 89])
    orow, lrow = impl.cross_attention(q, k, v, kv_lens=lens, rows=rows)
    assert np.max(np.abs(orow - out[:, :, rows])) < 1e-12
    assert np.array_equal(lrow == -np.inf, lse[:, :, rows] == -np.inf)
    fin = np.isfinite(lrow)
    assert np.max(np.abs(lrow[fin] - lse[:, :, rows][fin])) < 1e-12


def pin_cross_brute_force(impl):
    """A few rows against a pure-Python attention with math.fsum (text length 9, padding 3)."""
    rng = np.random.default_rng(63)
    q = rng.standard_normal((1, 1, 5, 64))
    k = rng.standard_normal((1, 1, 12, 64))
    v = rng.standard_normal((1, 1, 12, 64))
    out, lse = impl.cross_attention(q, k, v, kv_lens=[9])
    for r in range(5):
        ro, rl = _brute_attention_row(q[0, 0, r].tolist(), k[0, 0].tolist(), v[0, 0].tolist(),
                                      [c < 9 for c in range(12)])
        assert np.max(np.abs(out[0, 0, r] - ro)) < 1e-12
        assert abs(lse[0, 0, r] - rl) < 1e-12


# ------------------------------------------------------------------------- partial merge
def pin_merge_of_key_partition(impl):
    """Softmax attention over a union of disjoint key sets equals the merge of the attention
    over each set (the identity context-parallel attention relies on): three sets of a
    block-sparse row mask (one of them empty for some rows), checked against the full
    masked attention; merging one part returns it unchanged."""
    rng = np.random.default_rng(71)
    n = 200
    q, k, v = (rng.standard_normal((n, 64)) for _ in range(3))
    mask = impl.token_mask_rows(np.arange(n), n, 37, 1, 2)
    key_set = np.where(np.arange(n) < 64, 1, 2 * rng.integers(0, 2, n))
    # the 37 condition rows see keys < 37 only, all in set 1: sets 0 and 2 are empty for them
    full_o, full_l = impl.masked_attention(q, k, v, mask)
    parts = [impl.masked_attention(q, k, v, mask & (key_set == i)[None, :]) for i in range(3)]
    assert np.any(~np.isfinite(parts[0][1]))    # some row sees none of set 0's keys
    out, lse = impl.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    assert np.max(np.abs(out - full_o)) < 1e-12 and np.max(np.abs(lse - full_l)) < 1e-12
    o1, l1 = impl.merge_partials([full_o], [full_l])
    assert np.max(np.abs(o1 - full_o)) < 1e-15 and np.array_equal(l1, full_l)


def pin_merge_closed_form(impl):
    """Two parts with lse 0 and log 3 weigh 1/4 and 3/4 (lse log 4); an empty part (lse -inf)
    weighs nothing; all parts empty give out = 0, lse = -inf."""
    o_a = np.full((1, 64), 4.0)
    o_b = np.full((1, 64), -8.0)
    out, lse = impl.merge_partials([o_a, o_b], [np.array([0.0]), np.array([math.log(3.0)])])
    assert np.max(np.abs(out - (0.25 * 4.0 + 0.75 * -8.0))) < 1e-14 and abs(lse[0] - math.log(4.0)) < 1e-15
    out, lse = impl.merge_partials([o_a, o_b], [np.array([2.5]), np.array([-np.inf])])
    assert np.array_equal(out, o_a) and lse[0] == 2.5
    out, lse = impl.merge_partials([o_a, o_b], [np.array([-np.inf]), np.array([-np.inf])])
    assert np.all(out == 0.0) and lse[0] == -np.inf


def pin_cross_backward(impl):
    """Cross-attention gradients are the derivatives of L = sum(dout * out): central
    differences on sampled coordinates of q, k and v with a padded batch item; padded text
    tokens get exactly zero gradients; without padding the key gradients of a head sum to zero
    and the value gradients to the sum of dout."""
    rng = np.random.default_rng(85)
    q = rng.standard_normal((2, 1, 40, 64))
    k = rng.standard_normal((2, 1, 20, 64))
    v = rng.standard_normal((2, 1, 20, 64))
    do = rng.standard_normal((2, 1, 40, 64))
    lens = [20, 13]
    dq, dk, dv = impl.cross_attention_backward(q, k, v, do, kv_lens=lens)

    def loss(qq, kk, vv):
        out, _ = impl.cross_attention(qq, kk, vv, kv_lens=lens)
        return math.fsum((out * do).ravel())
    h = 1e-5
    for which, grad, shape in ((0, dq, q.shape), (1, dk, k.shape), (2, dv, v.shape)):
        for _ in range(10):
            b, t, c = int(rng.integers(0, 2)), int(rng.integers(0, shape[2])), int(rng.integers(0, 64))
            args = [q.copy(), k.copy(), v.copy()]
            args[which][b, 0, t, c] += h
            lp = loss(*args)
            args[which][b, 0, t, c] -= 2 * h
            lm = loss(*args)
            num = (lp - lm) / (2 * h)
            assert abs(num - grad[b, 0, t, c]) < 1e-6 * max(1.0, abs(num)), (which, b, t, c, num, grad[b, 0, t, c])
    assert np.all(dk[1, :, 13:] == 0.0) and np.all(dv[1, :, 13:] == 0.0)
    assert np.max(np.abs(dk[0, 0].sum(axis=0))) < 1e-10
    assert np.max(np.abs(dv[0, 0].sum(axis=0) - do[0, 0].sum(axis=0))) < 1e-10



def pin_cross_no_text(impl):
    """Without any text token a query attends nothing: out = 0, lse = -inf and dq = 0, the
    same as a batch item whose valid length is 0; with no query, dk = dv = 0."""
    rng = np.random.default_rng(86)
    q = rng.standard_normal((1, 2, 30, 64))
    do = rng.standard_normal((1, 2, 30, 64))
    none = np.zeros((1, 2, 0, 64))
    out, lse = impl.cross_attention(q, none, none)
    assert out.shape == q.shape and np.all(out == 0.0) and np.all(lse == -np.inf)
    dq, dk, dv = impl.cross_attention_backward(q, none, none, do)
    assert np.all(dq == 0.0) and dk.shape == (1, 2, 0, 64) and dv.shape == (1, 2, 0, 64)
    k = rng.standard_normal((1, 2, 9, 64))
    dq0, dk0, dv0 = impl.cross_attention_backward(q, k, k, do, kv_lens=[0])
    assert np.all(dq0 == 0.0) and np.all(dk0 == 0.0) and np.all(dv0 == 0.0)
    _, dk1, dv1 = impl.cross_attention_backward(np.zeros((1, 2, 0, 64)), k, k, np.zeros((1, 2, 0, 64)))
    assert np.all(dk1 == 0.0) and np.all(dv1 == 0.0)


ALL_PINS = [
    pin_rope_norm, pin_rope_origin_identity, pin_rope_sections_textbook, pin_rope_relative_position,
    pin_rope_closed_form_first_pair, pin_token_mask_brute_force, pin_tiny_csr_golden,
    pin_two_block_layouts, pin_nnz_closed_form, pin_attended_pairs_closed_form,
    pin_two_block_brute_force, pin_full_layout_is_dense_sdpa, pin_condition_isolation,
    pin_cached_equals_full, pin_rope_shift_invariance, pin_sampled_rows_match_full, pin_block_visiting_equals_masked_dense, pin_empty_row,
    pin_rmsnorm_unit_rms, pin_rmsnorm_scale_invariance, pin_rmsnorm_closed_form, pin_qk_prologue_textbook,
    pin_qk_prologue_norm, pin_backward_finite_differences, pin_backward_sums, pin_backward_uniform_closed_form,
    pin_backward_sampled_match_full, pin_cross_dense_sdpa, pin_cross_padding, pin_cross_brute_force,
    pin_merge_of_key_partition, pin_merge_closed_form, pin_rope_transpose,
    pin_prologue_backward_finite_differences, pin_cross_backward, pin_cross_no_text,
]
