"""GPU cross-attention backward (dq, dk, dv of video queries over padded text states) against
the fp64 oracle.

The forward runs on the GPU (its bf16 output and fp32 LSE are what the backward consumes); the
oracle differentiates the exact attention of the same bf16 inputs.  Small and medium shapes are
compared on every element; the 720p workload on sampled query rows of every head (dq) and on
every text key of two heads (dk, dv, each the sum over all 86,400 query rows).  Texts of at
most 512 tokens take the query walk with the text resident in LDS, longer ones the pipelined
walk; the cases cover both and the boundary.

Tolerance as for the self-attention backward, from the same arithmetic (P and dS rounded to
bf16 for the matrix cores, K * log2(e)/8 rounded to bf16 in the key walk, D from the bf16
output, one bf16 rounding of every gradient; the key walk's fp32 partial sums of the query
chunks add no bf16 rounding): relative L2 <= 1e-2 and max-abs <= 2e-2 * max|ref| + 1e-6."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from lcv_inputs import TEXT_LEN, WORKLOADS, bf16_bits_to_f64, grad_bits, qkv_bits, text_kv_bits
from tests.gpu_util import from_dev_f64, out_errors, say, score_rounding_sigma, to_dev

pytestmark = pytest.mark.gpu

REL_L2 = 1e-2
MAX_ABS_FRAC = 2e-2


def _sync():
    import torch
    torch.cuda.synchronize()


def _lens_dev(lens):
    import torch
    return None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")


def _close(got, ref, what):
    if ref.size == 0:
        assert got.size == 0
        return
    max_abs, rel = out_errors(got, ref)
    scale = float(np.max(np.abs(ref)))
    say(f"  {what}: max_abs {max_abs:.3e} (max|ref| {scale:.3e}) rel_l2 {rel:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    if scale == 0.0:   # a vanishing gradient (one key: dS = dP - D in fp32 with D from bf16 O)
        assert max_abs <= 1e-6, f"{what}: max_abs {max_abs:.3e} where the gradient vanishes"
        return
    assert max_abs <= MAX_ABS_FRAC * scale + 1e-6 and rel <= REL_L2, f"{what}: max_abs {max_abs:.3e} rel_l2 {rel:.3e}"


def _run(lib, seed, batch, heads, n_q, text_len, kv_lens, q_scale=1.0):
    qb, _, _ = qkv_bits(seed, batch, heads, n_q, q_scale)
    kb, vb = text_kv_bits(seed, batch, heads, text_len)
    gb = grad_bits(seed, batch, heads, n_q)
    q, k, v, do = to_dev(qb), to_dev(kb), to_dev(vb), to_dev(gb)
    lens = _lens_dev(kv_lens)
    out, lse = lib.cross_attention(q, k, v, kv_lens=lens)
    dq, dk, dv = lib.cross_attention_backward(q, k, v, out, lse, do, kv_lens=lens)
    _sync()
    return (qb, kb, vb, gb), (q, k, v, do, out, lse, lens), (dq, dk, dv)


CASES = [
    # name, batch, heads, n_q, text_len, kv_lens
    ("ragged-77", 1, 2, 630, 77, None),
    ("text-512-padded", 2, 3, 300, 512, [512, 100]),
    ("one-query-one-key", 1, 2, 1, 1, None),
    ("block-exact", 1, 2, 256, 64, None),
    ("block-plus-one", 1, 2, 257, 65, None),
    ("long-text", 1, 2, 200, 1000, None),           # past 512 text tokens: the pipelined query walk
    ("text-513", 2, 2, 300, 513, [513, 512]),     # one token past the resident-text limit
    ("many-chunks", 1, 2, 4097, 300, [7]),        # 33 query chunks of 2 blocks, last one ragged
    ("empty-text-item", 2, 2, 130, 96, [0, 96]),
    ("lens-clamped", 2, 1, 70, 40, [-3, 99]),
    # 256 (batch, head) pairs: one query range per head, 20 query blocks for the forward's 8
    # wavefronts and 20 units of 32 rows for the backward query walk's, handed out by the
    # workgroup's counter
    ("many-heads-long-ranges", 2, 128, 1221, 150, [150, 61]),
    ("no-query", 2, 2, 0, 100, [100, 30]),         # dk = dv = 0
    ("no-text", 1, 2, 100, 0, None),               # dq = 0
]
EXACT_ZERO = {"no-query": ("dk", "dv"), "no-text": ("dq",), "empty-text-item": ()}


@pytest.mark.parametrize("name,batch,heads,n_q,text_len,kv_lens", CASES, ids=[c[0] for c in CASES])
def test_cross_backward_full(lib, name, batch, heads, n_q, text_len, kv_lens):
    say(f"[cross-bwd] {name} B={batch} H={heads} N={n_q} L={text_len} lens={kv_lens}")
    (qb, kb, vb, gb), _, (dq, dk, dv) = _run(lib, 61, batch, heads, n_q, text_len, kv_lens)
    ref_lens = None if kv_lens is None else [min(max(x, 0), text_len) for x in kv_lens]
    rdq, rdk, rdv = oracle.cross_attention_backward(*(bf16_bits_to_f64(a) for a in (qb, kb, vb, gb)),
                                                    kv_lens=ref_lens)
    got = {"dq": from_dev_f64(dq), "dk": from_dev_f64(dk), "dv": from_dev_f64(dv)}
    for what, ref in (("dq", rdq), ("dk", rdk), ("dv", rdv)):
        _close(got[what], ref, f"{name} {what}")
    for what in EXACT_ZERO.get(name, ()):   # nothing attended: written as exact zeros
        assert not np.any(got[what]), f"{name}: {what} not zero"
    if name == "empty-text-item":           # batch item 0 has no text: its dq rows are zeros
        assert not np.any(got["dq"][0])


def test_cross_backward_peaked_softmax(lib):
    """Q scaled by 8 over 300 text tokens (200 valid in the second item): the same derivation
    and bounds as the self-attention backward's stress test (relative L2 <= 1.5 sigma,
    max-abs <= 4 sigma * max|ref|, sigma the standard deviation of the score error that the
    forward's bf16 rounding of Q * log2(e)/8 leaves, ~0.013 natural units here).  Measured:
    ~1e-2 relative L2 for dQ and dK, ~5e-3 for dV."""
    say("[cross-bwd] peaked softmax (Q x 8)")
    lens = [300, 200]
    (qb, kb, vb, gb), _, (dq, dk, dv) = _run(lib, 67, 2, 2, 500, 300, lens, q_scale=8.0)
    qf, kf = bf16_bits_to_f64(qb), bf16_bits_to_f64(kb)
    rdq, rdk, rdv = oracle.cross_attention_backward(qf, kf, *(bf16_bits_to_f64(a) for a in (vb, gb)), kv_lens=lens)
    sigma = score_rounding_sigma(qf[0], kf[0], np.ones((qf.shape[2], kf.shape[2]), dtype=bool))
    for what, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        g64 = from_dev_f64(got)
        max_abs, rel = out_errors(g64, ref)
        scale = float(np.max(np.abs(ref)))
        say(f"  peaked {what}: max_abs {max_abs:.3e} (max|ref| {scale:.3e}) rel_l2 {rel:.3e} (sigma {sigma:.3e})")
        assert np.all(np.isfinite(g64)), what
        assert max_abs <= 4 * sigma * scale and rel <= 1.5 * sigma, (what, max_abs, rel, sigma)


def test_cross_backward_padding_ignored_and_deterministic(lib):
    """Padded text keys/values change no gradient bit; padded rows of dk, dv are exactly zero;
    NaN-poisoned outputs are overwritten; two calls agree bitwise."""
    import torch
    say("[cross-bwd] padding invariance")
    _, (q, k, v, do, out, lse, lens), (dq, dk, dv) = _run(lib, 62, 2, 2, 700, 200, [200, 61])
    k2, v2 = k.clone(), v.clone()
    k2[1, :, 61:] = 50.0
    v2[1, :, 61:] = float("nan")
    poison = [torch.full_like(t, float("nan")) for t in (dq, dk, dv)]
    lib.cross_attention_backward(q, k2, v2, out, lse, do, kv_lens=lens, dq=poison[0], dk=poison[1], dv=poison[2])
    again = lib.cross_attention_backward(q, k, v, out, lse, do, kv_lens=lens)
    _sync()
    for a, b, c in zip((dq, dk, dv), poison, again):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    assert not dk[1, :, 61:].view(torch.int16).any() and not dv[1, :, 61:].view(torch.int16).any()


def test_cross_backward_workload_sampled(lib):
    """720p video queries (32 heads x 86,400 tokens) over 512 text tokens: dq on sampled rows
    of every head, dk and dv on every text key of the first and last head; every gradient
    finite."""
    import torch
    w = WORKLOADS["t2v720"]
    say(f"[cross-bwd] t2v720 N={w.n_tokens} heads={w.heads} L={TEXT_LEN}")
    (qb, kb, vb, gb), _, (dq, dk, dv) = _run(lib, w.seed, 1, w.heads, w.n_tokens, TEXT_LEN, None)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    rng = np.random.default_rng(63)
    rows = np.unique(np.concatenate([[0, 63, 64, w.n_tokens - 1], rng.integers(0, w.n_tokens, 40)]))
    qf, kf, vf, gf = (bf16_bits_to_f64(a) for a in (qb, kb, vb, gb))
    # a query row's dq needs only its own row: the oracle on the sampled rows is exact for them
    rdq, _, _ = oracle.cross_attention_backward(qf[:, :, rows], kf, vf, gf[:, :, rows])
    idx = torch.from_numpy(rows).cuda()
    _close(from_dev_f64(dq[:, :, idx]), rdq, "t2v720 dq rows")
    for h in (0, w.heads - 1):
        say(f"  head {h}: dk, dv over all {w.n_tokens} query rows")
        _, rdk, rdv = oracle.cross_attention_backward(qf[:, [h]], kf[:, [h]], vf[:, [h]], gf[:, [h]])
        _close(from_dev_f64(dk[:, [h]]), rdk, f"t2v720 dk head {h}")
        _close(from_dev_f64(dv[:, [h]]), rdv, f"t2v720 dv head {h}")
