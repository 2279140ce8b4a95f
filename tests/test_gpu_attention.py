"""GPU block-sparse attention against the fp64 oracle.

Small and medium shapes (several query blocks and workgroups, ragged tails, condition
boundaries inside a block) are compared on every row; the five workloads at full size are
compared on sampled rows and checked for properties that hold at any size (every row
written, finite).  Tolerances: out max-abs <= 2e-2 and relative L2 <= 1e-2, lse max-abs
<= 1e-2 (bf16 inputs, fp32 accumulation)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from lcv_inputs import WORKLOADS, bf16_bits_to_f64, qkv_bits, workload_inputs
from tests.gpu_util import (assert_lse_close, assert_out_close, from_dev_f64, lse_error_budget, out_errors, say,
                            to_dev)

pytestmark = pytest.mark.gpu


def _sync():
    import torch
    torch.cuda.synchronize()


def _run_full(lib, grid, heads, cond, local, stride, seed, rope=True, q_scale=1.0, batch=1):
    n = grid[0] * grid[1] * grid[2]
    qb, kb, vb = qkv_bits(seed, batch, heads, n, q_scale)
    layout = lib.build_layout(n, local, stride, cond)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    out, lse = lib.forward(q, k, v, layout, grid=grid if rope else None)
    _sync()
    return layout, (qb, kb, vb), (q, k, v), out, lse


MEDIUM = [
    # name, grid, heads, cond, local, stride
    ("tiny", (4, 8, 16), 2, 0, 2, 4),
    ("ragged-c0", (3, 10, 21), 3, 0, 2, 4),
    ("ragged-c210", (3, 10, 21), 3, 210, 2, 4),
    ("ragged-allcond", (3, 10, 21), 2, 630, 2, 4),
    ("ragged-w1s3", (3, 10, 21), 2, 210, 1, 3),
    ("ragged-w0s0", (3, 10, 21), 2, 210, 0, 0),
    ("ragged-dense", (3, 10, 21), 2, 210, 3, 1),
    ("one-token", (1, 1, 1), 2, 0, 2, 4),
    ("one-partial-block", (1, 7, 9), 2, 5, 2, 4),
    ("65-tokens", (1, 5, 13), 2, 64, 0, 1),
    ("multi-workgroup", (2, 16, 64), 2, 1061, 2, 4),
    ("cond-at-63", (1, 10, 30), 2, 63, 0, 3),
]


@pytest.mark.parametrize("name,grid,heads,cond,local,stride", MEDIUM, ids=[m[0] for m in MEDIUM])
def test_full_rows(lib, name, grid, heads, cond, local, stride):
    say(f"[attn] {name} grid={grid} heads={heads} C={cond} w={local} s={stride}")
    layout, (qb, kb, vb), _, out, lse = _run_full(lib, grid, heads, cond, local, stride, seed=31)
    ref_o, ref_l = oracle.bsa_forward(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), grid,
                                      cond, local, stride)
    got_l = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_l)
    say(f"  lse err max {np.max(np.abs(got_l[fin] - ref_l[fin])):.3e} mean {np.mean(got_l[fin] - ref_l[fin]):.3e}")
    assert_out_close(from_dev_f64(out), ref_o, name)
    assert_lse_close(got_l, ref_l, name)


@pytest.mark.parametrize("name,grid,heads,cond,local,stride",
                         [m for m in MEDIUM if 0 < m[3] < m[1][0] * m[1][1] * m[1][2]],
                         ids=[m[0] for m in MEDIUM if 0 < m[3] < m[1][0] * m[1][1] * m[1][2]])
def test_cached_matches_full_bitwise(lib, name, grid, heads, cond, local, stride):
    """Condition K/V from the cache, noise rows only: identical bits to rows [C, N) of the
    full call, and within tolerance of the oracle's cached definition."""
    import torch
    say(f"[cached] {name}")
    layout, (qb, kb, vb), (q, k, v), out, lse = _run_full(lib, grid, heads, cond, local, stride, seed=32)
    oc, lc = lib.forward_cached(q[:, :, cond:].contiguous(), k[:, :, cond:].contiguous(), v[:, :, cond:].contiguous(),
                                k[:, :, :cond].contiguous(), v[:, :, :cond].contiguous(), layout, grid=grid)
    _sync()
    assert torch.equal(oc.view(torch.int16), out[:, :, cond:].view(torch.int16))
    assert torch.equal(lc, lse[:, :, cond:])
    qf, kf, vf = (bf16_bits_to_f64(a) for a in (qb, kb, vb))
    ref_o, ref_l = oracle.bsa_forward_cached(qf[:, :, cond:], kf[:, :, cond:], vf[:, :, cond:], kf[:, :, :cond],
                                             vf[:, :, :cond], grid, cond, local, stride)
    assert_out_close(from_dev_f64(oc), ref_o, name)
    assert_lse_close(lc.cpu().numpy().astype(np.float64), ref_l, name)


def _check_lse_budget(lse_gpu, qf, kf, cond, local, stride, grid, rope, what, z_rms_max=None):
    """Every row's LSE error within the worst case of the score arithmetic (lse_error_budget),
    and, where z_rms_max is given, the errors' size in units of their predicted standard
    deviation (root mean square over rows) below z_rms_max."""
    n = qf.shape[2]
    rows = np.arange(n)
    mask = oracle.token_mask_rows(rows, n, cond, local, stride)
    worst_ratio, zs = 0.0, []
    for h in range(qf.shape[1]):
        qr = oracle.rope3d(qf[0, h], grid) if rope else qf[0, h]
        kr = oracle.rope3d(kf[0, h], grid) if rope else kf[0, h]
        _, lse_ref = oracle.masked_attention(qr, kr, np.zeros_like(kr), mask)
        worst, sigma = lse_error_budget(qr, kr, mask, lse_ref, rope)
        err = np.abs(lse_gpu[0, h] - lse_ref)
        assert np.all(err <= worst), f"{what}: lse error {float(np.max(err - worst)):.3e} above its bound"
        worst_ratio = max(worst_ratio, float(np.max(err / worst)))
        zs.append(err / sigma)
    z_rms = float(np.sqrt(np.mean(np.concatenate(zs) ** 2)))
    say(f"  {what}: lse error at most {worst_ratio:.2f} of its worst case; {z_rms:.2f} predicted standard "
        f"deviations (root mean square)")
    if z_rms_max is not None:
        assert z_rms <= z_rms_max, f"{what}: lse errors {z_rms:.2f} standard deviations (rms)"


def test_peaked_softmax(lib):
    """Q scaled by 8 (scores of standard deviation 8, up to ~40): exercises the running-max
    rescaling.  This stress input is not one of the workloads, so its bounds are derived from
    the arithmetic.  Each score sum_d q_d k_d / 8 sees three bf16 roundings before the matrix
    cores (rotated Q, Q times log2(e)/8, rotated K): for the output, in a row dominated by two
    keys the output moves by a few percent of |v_a - v_b| (~3): max-abs <= 0.1, while the
    relative L2 error stays <= 1e-2.  For the LSE every row must stay within the worst case of
    those roundings (lse_error_budget: three times 2^-8 of the largest sum_c |q_c k_c| / 8 of
    the row's keys, plus the row sum's rounding), and the errors' root mean square must stay
    within 3 of their predicted standard deviations (a model of independent round-to-nearest
    errors; a correct kernel sits near 1, a missing or doubled rounding far above)."""
    grid = (3, 10, 21)
    say("[attn] peaked softmax")
    _, (qb, kb, vb), _, out, lse = _run_full(lib, grid, 2, 210, 2, 4, seed=33, q_scale=8.0)
    qf, kf, vf = bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb)
    ref_o, ref_l = oracle.bsa_forward(qf, kf, vf, grid, 210, 2, 4)
    got = from_dev_f64(out)
    max_abs, rel = out_errors(got, ref_o)
    got_l = lse.cpu().numpy().astype(np.float64)
    lse_err = float(np.max(np.abs(got_l - ref_l)))
    say(f"  peaked: max_abs {max_abs:.3e} rel_l2 {rel:.3e} lse {lse_err:.3e}")
    assert np.all(np.isfinite(got))
    assert max_abs <= 0.1 and rel <= 1e-2, (max_abs, rel)
    _check_lse_budget(got_l, qf, kf, 210, 2, 4, grid, True, "peaked", z_rms_max=3.0)


@pytest.mark.parametrize("offset", [3072.0, -3072.0], ids=["plus", "minus"])
def test_score_offset_far_from_zero(lib, offset):
    """Every score of a row shifted by the same large amount: channel 0 of every key is 1 and
    channel 0 of every query is +-3072, so each score gains +-384 (natural units, ~ +-554 in
    log2 units).  The softmax ignores a shift that is common to the row, so the output must
    match the oracle within the usual bounds.  This exercises the kernel's row reference far
    from 0 in both directions: each row's first block moves it to +-576, the subtraction runs on
    the vector ALU, and the probabilities stay within 2^+-32 of the row's largest one.
    The LSE carries the shift as the kernel forms it: the query operand is Q times log2(e)/8
    rounded to bf16, whose rounding moves a product by at most 2^-8 of itself, here up to
    1.5 natural units on the shift alone; every row must stay within that worst case
    (lse_error_budget with the one rounding of inputs taken as rotated).  No RoPE: a rotation
    would mix channel 0 into channel 1 with a per-token angle and break the common shift."""
    n, heads, cond, local, stride = 630, 2, 210, 2, 4
    qb, kb, vb = qkv_bits(38, 1, heads, n)
    q_bits = np.float32(offset).view(np.uint32) >> 16          # +-3072 is exact in bf16
    qb = qb.copy()
    kb = kb.copy()
    qb[..., 0] = np.uint16(q_bits)
    kb[..., 0] = np.uint16(np.float32(1.0).view(np.uint32) >> 16)
    say(f"[attn] score offset {offset:+.0f} on channel 0")
    layout = lib.build_layout(n, local, stride, cond)
    out, lse = lib.forward(to_dev(qb), to_dev(kb), to_dev(vb), layout, grid=None)
    _sync()
    qf, kf, vf = bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb)
    ref_o, ref_l = oracle.bsa_forward(qf, kf, vf, None, cond, local, stride, rope_q=False, rope_k=False)
    got = from_dev_f64(out)
    max_abs, rel = assert_out_close(got, ref_o, f"offset {offset:+.0f}")
    got_l = lse.cpu().numpy().astype(np.float64)
    say(f"  max_abs {max_abs:.3e} rel_l2 {rel:.3e} lse {float(np.max(np.abs(got_l - ref_l))):.3e}")
    _check_lse_budget(got_l, qf, kf, cond, local, stride, None, False, f"offset {offset:+.0f}")
    layout.close()


def test_batch_two(lib):
    grid = (2, 8, 24)
    say("[attn] batch 2")
    _, (qb, kb, vb), _, out, lse = _run_full(lib, grid, 3, 100, 2, 4, seed=34, batch=2)
    ref_o, ref_l = oracle.bsa_forward(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), grid,
                                      100, 2, 4)
    assert_out_close(from_dev_f64(out), ref_o, "batch2")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_l, "batch2")


def test_fused_rope_equals_prepass_and_is_deterministic(lib):
    """Fused Q/K RoPE gives the same bits as the standalone RoPE pass followed by an
    unrotated forward; two identical calls give identical bits."""
    import torch
    grid = (3, 10, 21)
    say("[attn] fused vs prepass")
    layout, _, (q, k, v), out, lse = _run_full(lib, grid, 3, 210, 2, 4, seed=35)
    qr = lib.rope3d_apply(q, grid)
    kr = lib.rope3d_apply(k, grid)
    out2, lse2 = lib.forward(qr, kr, v, layout, grid=None)
    out3, lse3 = lib.forward(q, k, v, layout, grid=grid)
    _sync()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse, lse2)
    assert torch.equal(out.view(torch.int16), out3.view(torch.int16))
    assert torch.equal(lse, lse3)
    # rope on one side only
    out4, _ = lib.forward(qr, k, v, layout, grid=grid, rope_q=False, rope_k=True)
    out5, _ = lib.forward(q, kr, v, layout, grid=grid, rope_q=True, rope_k=False)
    _sync()
    assert torch.equal(out.view(torch.int16), out4.view(torch.int16))
    assert torch.equal(out.view(torch.int16), out5.view(torch.int16))


def test_every_row_written(lib):
    """Outputs pre-filled with NaN come back finite everywhere."""
    import torch
    grid = (3, 10, 21)
    n = 630
    say("[attn] nan poison")
    qb, kb, vb = qkv_bits(36, 1, 2, n)
    layout = lib.build_layout(n, 2, 4, 210)
    out = torch.full((1, 2, n, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((1, 2, n), float("nan"), dtype=torch.float32, device="cuda")
    lib.forward(to_dev(qb), to_dev(kb), to_dev(vb), layout, grid=grid, out=out, lse=lse)
    _sync()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


def test_forward_argument_errors(lib):
    """Argument errors with a real layout are reported before launch."""
    import ctypes
    layout = lib.build_layout(630, 2, 4, 210)
    L = lib.lib()
    p = ctypes.c_void_p(4096)
    g_ok = lib.Rope3dGrid(3, 10, 21, 1e4)
    g_bad = lib.Rope3dGrid(3, 10, 20, 1e4)
    h = layout.handle
    assert L.lcv_bsa_forward(p, p, p, 1, 2, h, 0, 3, ctypes.byref(g_ok), p, None, None) == 5      # cond mismatch
    assert L.lcv_bsa_forward(p, p, p, 1, 2, h, 210, 3, ctypes.byref(g_bad), p, None, None) == 3   # grid != N
    assert L.lcv_bsa_forward(p, p, p, 1, 2, h, 210, 8, ctypes.byref(g_ok), p, None, None) == 2    # unknown flag
    assert L.lcv_bsa_forward(p, p, p, 0, 2, h, 210, 3, ctypes.byref(g_ok), p, None, None) == 2    # batch 0
    assert L.lcv_bsa_forward(p, p, p, 1, 2, h, 210, 3, None, p, None, None) == 1                  # grid missing
    assert L.lcv_bsa_forward(ctypes.c_void_p(4100), p, p, 1, 2, h, 210, 3, ctypes.byref(g_ok), p, None, None) == 2
    assert L.lcv_bsa_forward(p, p, p, 1, 2, h, 210, 3, ctypes.byref(g_ok), p, ctypes.c_void_p(4098), None) == 2
    assert L.lcv_bsa_forward_cached(p, p, p, None, p, 1, 2, h, 210, 3, ctypes.byref(g_ok), p, None, None) == 1
    big = lib.Rope3dGrid(1, 1, 630, 1e4)     # 8 + 12 + 12*630 table entries: too many for the fused path
    assert L.lcv_bsa_forward(p, p, p, 1, 2, h, 210, 3, ctypes.byref(big), p, None, None) == 6
    layout.close()


# ---------------------------------------------------------------- full-size workloads
def _sample_rows(n, cond, rng, extra=40):
    rows = [0, 1, 63, 64, n - 1, n - 2, n - 65]
    if cond:
        rows += [cond - 2, cond - 1, cond, cond + 1, cond + 63]
    rows += list(rng.integers(0, n, extra))
    rows = np.unique(np.clip(np.array(rows), 0, n - 1))
    return rows


def _check_rows(out, lse, ref_fn, rows, heads, what, row_offset=0):
    """Compare sampled rows (token index rows + row_offset in the tensors) of every head."""
    import torch
    idx = torch.from_numpy(rows).cuda()
    got_o = from_dev_f64(out[:, :, idx])
    got_l = lse[:, :, idx].cpu().numpy().astype(np.float64)
    ref_o, ref_l = ref_fn(rows)
    assert_out_close(got_o, ref_o, what)
    assert_lse_close(got_l, ref_l, what)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all(), f"{what}: non-finite output"


def _oracle_rows_full(qb, kb, vb, w, local, stride):
    def fn(rows):
        outs, lses = [], []
        for h in range(w.heads):
            q = bf16_bits_to_f64(qb[:, h:h + 1])
            k = bf16_bits_to_f64(kb[:, h:h + 1])
            v = bf16_bits_to_f64(vb[:, h:h + 1])
            o, l = oracle.bsa_forward(q, k, v, w.grid, w.cond_len, local, stride, w.theta, rows=rows)
            outs.append(o)
            lses.append(l)
        return np.concatenate(outs, axis=1), np.concatenate(lses, axis=1)
    return fn


WORKLOAD_MODES = [(name, "fused") for name in ("tiny", "t2v480", "i2v480", "t2v720", "vc480")] + \
                 [(name, "k-pass") for name in ("i2v480", "t2v720", "vc480")]


@pytest.mark.parametrize("name,mode", WORKLOAD_MODES, ids=[f"{n}-{m}" for n, m in WORKLOAD_MODES])
def test_workload_sampled_rows(lib, name, mode):
    """A workload at full size against the oracle on sampled rows of every head.  mode
    "fused": Q and K rotated inside the attention kernel; "k-pass": the configuration the
    benchmark times, K rotated by the standalone RoPE pass (the condition cache holding the
    rotated condition K) and Q inside the attention kernel."""
    import torch
    w = WORKLOADS[name]
    kpass = mode == "k-pass"
    say(f"[workload] {name} ({mode}) N={w.n_tokens} heads={w.heads} C={w.cond_len}")
    qb, kb, vb = workload_inputs(w)
    layout = lib.build_layout(w.n_tokens, w.local_blocks, w.global_stride, w.cond_len)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((w.batch, w.heads, w.n_tokens), float("nan"), dtype=torch.float32, device="cuda")
    if kpass:
        lib.forward(q, lib.rope3d_apply(k, w.grid), v, layout, grid=w.grid, rope_q=True, rope_k=False, out=out,
                    lse=lse)
    else:
        lib.forward(q, k, v, layout, grid=w.grid, out=out, lse=lse)
    _sync()
    rng = np.random.default_rng(w.seed)
    rows = _sample_rows(w.n_tokens, w.cond_len, rng)
    _check_rows(out, lse, _oracle_rows_full(qb, kb, vb, w, w.local_blocks, w.global_stride), rows, w.heads,
                f"{name}-{mode}")
    if not w.cached:
        return
    # second call: fresh noise tokens, condition K/V reused from the first call's inputs
    C = w.cond_len
    say(f"[workload] {name} ({mode}) cached call")
    nqb, nkb, nvb = workload_inputs(w, call=1)
    oc = torch.full((w.batch, w.heads, w.n_tokens - C, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    lc = torch.full((w.batch, w.heads, w.n_tokens - C), float("nan"), dtype=torch.float32, device="cuda")
    if kpass:
        k_cache = lib.rope3d_apply(k[:, :, :C].contiguous(), w.grid)
        nk = lib.rope3d_apply(to_dev(nkb), w.grid, token_offset=C)
        lib.forward_cached(to_dev(nqb), nk, to_dev(nvb), k_cache, v[:, :, :C].contiguous(), layout, grid=w.grid,
                           rope_q=True, rope_k=False, out=oc, lse=lc)
    else:
        lib.forward_cached(to_dev(nqb), to_dev(nkb), to_dev(nvb), k[:, :, :C].contiguous(), v[:, :, :C].contiguous(),
                           layout, grid=w.grid, out=oc, lse=lc)
    _sync()
    nrows = _sample_rows(w.n_tokens - C, 0, rng)

    def fn(rows_local):
        outs, lses = [], []
        for h in range(w.heads):
            o, l = oracle.bsa_forward_cached(
                bf16_bits_to_f64(nqb[:, h:h + 1]), bf16_bits_to_f64(nkb[:, h:h + 1]),
                bf16_bits_to_f64(nvb[:, h:h + 1]), bf16_bits_to_f64(kb[:, h:h + 1, :C]),
                bf16_bits_to_f64(vb[:, h:h + 1, :C]), w.grid, C, w.local_blocks, w.global_stride, w.theta,
                rows=rows_local)
            outs.append(o)
            lses.append(l)
        return np.concatenate(outs, axis=1), np.concatenate(lses, axis=1)

    _check_rows(oc, lc, fn, nrows, w.heads, f"{name}-{mode}-cached")


@pytest.mark.parametrize("local,stride", WORKLOADS["vc480"].sweep)
def test_vc_density_sweep(lib, local, stride):
    """Video-continuation grid over the density sweep, a few heads, sampled rows."""
    import torch
    w = WORKLOADS["vc480"]
    heads = 4
    say(f"[sweep] vc480 w={local} s={stride}")
    qb, kb, vb = qkv_bits(w.seed, 1, heads, w.n_tokens)
    layout = lib.build_layout(w.n_tokens, local, stride, w.cond_len)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    out, lse = lib.forward(q, k, v, layout, grid=w.grid)
    _sync()
    rows = _sample_rows(w.n_tokens, w.cond_len, np.random.default_rng(local * 100 + stride), extra=16)

    class _W:
        pass
    ww = _W()
    ww.heads, ww.grid, ww.cond_len, ww.theta = heads, w.grid, w.cond_len, w.theta
    _check_rows(out, lse, _oracle_rows_full(qb, kb, vb, ww, local, stride), rows, heads, f"sweep w{local} s{stride}")


@pytest.mark.parametrize("name,grid,heads,cond,ranges", [
    ("three-unaligned", (3, 10, 21), 2, 210, [(0, 200), (200, 413), (413, 630)]),
    ("eight-aligned", (2, 16, 64), 2, 1061, [(256 * i, 256 * (i + 1)) for i in range(8)]),
    ("single-rows", (1, 7, 9), 2, 5, [(0, 1), (1, 2), (2, 40), (40, 63)]),
])
def test_row_shards_match_full_bitwise(lib, name, grid, heads, cond, ranges):
    """Sequence-sharded calls (one device's rows each) reproduce the full call bit for bit."""
    import torch
    say(f"[rows] {name}")
    layout, _, (q, k, v), out, lse = _run_full(lib, grid, heads, cond, 2, 4, seed=37)
    for r0, r1 in ranges:
        o, l = lib.forward_rows(q[:, :, r0:r1].contiguous(), k, v, layout, r0, r1, grid=grid)
        _sync()
        assert torch.equal(o.view(torch.int16), out[:, :, r0:r1].view(torch.int16)), (r0, r1)
        assert torch.equal(l, lse[:, :, r0:r1]), (r0, r1)
    empty = torch.empty((1, heads, 0, 64), dtype=torch.bfloat16, device="cuda")
    mid = layout.n_tokens // 2
    lib.forward_rows(empty, k, v, layout, mid, mid, grid=grid)
    import ctypes
    p = ctypes.c_void_p(4096)
    g = lib.Rope3dGrid(*grid, 1e4)
    assert lib.lib().lcv_bsa_forward_rows(p, p, p, 1, heads, layout.handle, cond, 3, ctypes.byref(g), 5, 4, p, None,
                                          None) == 2
    assert lib.lib().lcv_bsa_forward_rows(p, p, p, 1, heads, layout.handle, cond, 3, ctypes.byref(g), 0,
                                          layout.n_tokens + 1, p, None, None) == 2
    layout.close()


def test_row_shard_workload_bitwise(lib):
    """One eighth of the 720p rows (the middle shard) against the same rows of the full call."""
    import torch
    w = WORKLOADS["t2v720"]
    say("[rows] t2v720 shard 4 of 8")
    qb, kb, vb = workload_inputs(w)
    layout = lib.build_layout(w.n_tokens, w.local_blocks, w.global_stride, w.cond_len)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    out, lse = lib.forward(q, k, v, layout, grid=w.grid)
    per = -(-w.n_blocks // 8) * 64
    r0, r1 = 4 * per, min(5 * per, w.n_tokens)
    o, l = lib.forward_rows(q[:, :, r0:r1].contiguous(), k, v, layout, r0, r1, grid=w.grid)
    _sync()
    assert torch.equal(o.view(torch.int16), out[:, :, r0:r1].view(torch.int16))
    assert torch.equal(l, lse[:, :, r0:r1])
    layout.close()
