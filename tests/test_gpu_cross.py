"""GPU cross-attention (video queries over padded text states) against the fp64 oracle.

Tolerances as for the self-attention (bf16 inputs, fp32 accumulation, P rounded to bf16):
out max-abs <= 2e-2 and relative L2 <= 1e-2, lse max-abs <= 1e-2."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from lcv_inputs import TEXT_LEN, WORKLOADS, bf16_bits_to_f64, qkv_bits, text_kv_bits
from tests.gpu_util import assert_lse_close, assert_out_close, from_dev_f64, lse_error_budget, say, to_dev

pytestmark = pytest.mark.gpu


def _sync():
    import torch
    torch.cuda.synchronize()


def _lens_dev(lens):
    import torch
    return None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")


CASES = [
    # name, batch, heads, n_q, text_len, kv_lens
    ("ragged-77", 1, 2, 630, 77, None),
    ("text-512-padded", 2, 3, 300, 512, [512, 100]),
    ("one-query-one-key", 1, 2, 1, 1, None),
    ("block-exact", 1, 2, 256, 64, None),
    ("block-plus-one", 1, 2, 257, 65, None),
    ("long-text", 1, 2, 200, 1000, None),
    ("many-workgroups", 1, 2, 4097, 300, [7]),
    ("empty-text-item", 2, 2, 130, 96, [0, 96]),
    ("lens-clamped", 2, 1, 70, 40, [-3, 99]),
    # 256 (batch, head) pairs: one query range per head, 20 query blocks for the forward's 8
    # wavefronts and 20 units of 32 rows for the backward query walk's, handed out by the
    # workgroup's counter
    ("many-heads-long-ranges", 2, 128, 1221, 150, [150, 61]),
]


@pytest.mark.parametrize("name,batch,heads,n_q,text_len,kv_lens", CASES, ids=[c[0] for c in CASES])
def test_cross_rows(lib, name, batch, heads, n_q, text_len, kv_lens):
    say(f"[cross] {name} B={batch} H={heads} N={n_q} L={text_len} lens={kv_lens}")
    qb, _, _ = qkv_bits(51, batch, heads, n_q)
    kb, vb = text_kv_bits(51, batch, heads, text_len)
    out, lse = lib.cross_attention(to_dev(qb), to_dev(kb), to_dev(vb), kv_lens=_lens_dev(kv_lens))
    _sync()
    ref_lens = None if kv_lens is None else [min(max(x, 0), text_len) for x in kv_lens]
    ref_o, ref_l = oracle.cross_attention(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb),
                                          kv_lens=ref_lens)
    assert_out_close(from_dev_f64(out), ref_o, name)
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_l, name)


def test_cross_padding_contents_ignored_and_deterministic(lib):
    """Padded text keys/values do not change a single output bit; two calls agree bitwise;
    NaN-poisoned outputs are fully overwritten."""
    import torch
    say("[cross] padding invariance")
    qb, _, _ = qkv_bits(52, 2, 2, 500)
    kb, vb = text_kv_bits(52, 2, 2, 200)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    lens = _lens_dev([200, 61])
    out, lse = lib.cross_attention(q, k, v, kv_lens=lens)
    k2, v2 = k.clone(), v.clone()
    k2[1, :, 61:] = 50.0
    v2[1, :, 61:] = float("nan")
    out_p = torch.full_like(out, float("nan"))
    lse_p = torch.full_like(lse, float("nan"))
    lib.cross_attention(q, k2, v2, kv_lens=lens, out=out_p, lse=lse_p)
    _sync()
    assert torch.equal(out.view(torch.int16), out_p.view(torch.int16))
    assert torch.equal(lse, lse_p)
    out3, lse3 = lib.cross_attention(q, k, v, kv_lens=lens)
    _sync()
    assert torch.equal(out.view(torch.int16), out3.view(torch.int16)) and torch.equal(lse, lse3)


def test_cross_workload_sampled_rows(lib):
    """720p video queries (32 heads x 86,400 tokens) over 512 text tokens: sampled rows of every
    head against the oracle, every output finite."""
    import torch
    w = WORKLOADS["t2v720"]
    say(f"[cross] t2v720 N={w.n_tokens} heads={w.heads} L={TEXT_LEN}")
    qb, _, _ = qkv_bits(w.seed, 1, w.heads, w.n_tokens)
    kb, vb = text_kv_bits(w.seed, 1, w.heads)
    out, lse = lib.cross_attention(to_dev(qb), to_dev(kb), to_dev(vb))
    _sync()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(53)
    rows = np.unique(np.concatenate([[0, 63, 64, w.n_tokens - 1], rng.integers(0, w.n_tokens, 40)]))
    idx = torch.from_numpy(rows).cuda()
    ref_o, ref_l = oracle.cross_attention(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb),
                                          rows=rows)
    assert_out_close(from_dev_f64(out[:, :, idx]), ref_o, "t2v720 cross")
    assert_lse_close(lse[:, :, idx].cpu().numpy().astype(np.float64), ref_l, "t2v720 cross")


def _bf16(x: float) -> np.uint16:
    return np.uint16(np.float32(x).view(np.uint32) >> 16)   # the values used here are exact in bf16


@pytest.mark.parametrize("text_len", [307, 700], ids=["text-in-lds", "text-streamed"])
def test_cross_reference_moves(lib, text_len):
    """Text blocks whose scores lie far apart: channel 0 of the keys is constant per 64-key
    block (2, 6, -30, 0, 3, repeated) and channel 0 of the queries cycles through 0, 64, -64,
    16, -256 and 128, so a row's blocks are shifted against each other by up to ~1,000
    (natural units).  This walks the transitions of the lazy row reference: rows whose
    reference stays 0 (0, 16), rows that move it up in a later block by a large step (64),
    past an fp32 overflow of the exponentials (-64: scores ~346 in log2 units against the
    reference 0), and rows whose first block sets it far below (-256) or above (128) zero and
    a later block moves it up again.  Outputs against the oracle at the usual bounds; the LSE within
    the worst case of its score arithmetic (lse_error_budget: the one bf16 rounding of the
    query operand moves the dominant block's shift by up to 2^-8 of itself).  307 text tokens
    stay in LDS (the last block partly masked), 700 are streamed."""
    batch, heads, n_q = 1, 2, 390
    say(f"[cross] reference moves L={text_len}")
    qb, _, _ = qkv_bits(57, batch, heads, n_q)
    kb, vb = text_kv_bits(57, batch, heads, text_len)
    qb, kb = qb.copy(), kb.copy()
    q0 = [0.0, 64.0, -64.0, 16.0, -256.0, 128.0]
    k0 = [2.0, 6.0, -30.0, 0.0, 3.0]
    for r in range(n_q):
        qb[:, :, r, 0] = _bf16(q0[r % len(q0)])
    for key in range(text_len):
        kb[:, :, key, 0] = _bf16(k0[(key // 64) % len(k0)])
    out, lse = lib.cross_attention(to_dev(qb), to_dev(kb), to_dev(vb))
    _sync()
    qf, kf, vf = bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb)
    ref_o, ref_l = oracle.cross_attention(qf, kf, vf)
    assert_out_close(from_dev_f64(out), ref_o, f"reference moves L={text_len}")
    got_l = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got_l))
    mask = np.ones((n_q, text_len), dtype=bool)
    for h in range(heads):
        worst, _ = lse_error_budget(qf[0, h], kf[0, h], mask, ref_l[0, h], rope=False)
        err = np.abs(got_l[0, h] - ref_l[0, h])
        assert np.all(err <= worst), f"L={text_len} head {h}: lse error {float(np.max(err - worst)):.3e} above its bound"
