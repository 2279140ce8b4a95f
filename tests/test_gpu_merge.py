"""GPU merge of attention results over disjoint key sets against the fp64 oracle.

Direct: random bf16 parts and fp32 LSEs (with empty parts and rows empty in every part)
against `oracle.merge_partials` of the same values: fp32 weights and sums, one bf16 rounding,
so each element is within half a bf16 ulp of the exact merge plus a few fp32 ulps
(|err| <= 2^-8 |ref| + 1e-6 |max part| asserted), lse within 1e-5.
End to end: cross-attention over split text states (ring attention over two or three key
shards on one GPU), merged, against the oracle's attention over the whole text (self-attention
bounds: out max-abs <= 2e-2, rel-L2 <= 1e-2, lse <= 1e-2)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from lcv_inputs import bf16_bits_to_f64, qkv_bits, round_to_bf16_bits, text_kv_bits
from tests.gpu_util import assert_lse_close, assert_out_close, from_dev_f64, say, to_dev

pytestmark = pytest.mark.gpu


def _sync():
    import torch
    torch.cuda.synchronize()


def _parts(seed, n_parts, shape):
    rng = np.random.default_rng(seed)
    outs = [round_to_bf16_bits(rng.standard_normal(shape + (64,)).astype(np.float32)) for _ in range(n_parts)]
    lses = [rng.uniform(-5.0, 30.0, shape).astype(np.float32) for _ in range(n_parts)]
    # empty parts in some rows, and some rows empty in every part
    for i, l in enumerate(lses):
        l[..., i::7] = -np.inf
    for l in lses:
        l[..., 3::11] = -np.inf
    return outs, lses


@pytest.mark.parametrize("n_parts,shape", [(1, (1, 2, 100)), (2, (2, 3, 333)), (3, (1, 1, 4097)), (8, (1, 2, 65))])
def test_merge_random_parts(lib, n_parts, shape):
    import torch
    say(f"[merge] parts={n_parts} shape={shape}")
    outs, lses = _parts(70 + n_parts, n_parts, shape)
    d_outs = [to_dev(o) for o in outs]
    d_lses = [torch.from_numpy(l).cuda() for l in lses]
    out, lse = lib.attn_merge(d_outs, d_lses)
    _sync()
    ref_o, ref_l = oracle.merge_partials([bf16_bits_to_f64(o) for o in outs], [l.astype(np.float64) for l in lses])
    got = from_dev_f64(out)
    got_l = lse.cpu().numpy().astype(np.float64)
    big = max(float(np.max(np.abs(bf16_bits_to_f64(o)))) for o in outs)
    assert np.all(np.abs(got - ref_o) <= 2.0 ** -8 * np.abs(ref_o) + 1e-6 * big)
    assert np.array_equal(np.isfinite(got_l), np.isfinite(ref_l))
    fin = np.isfinite(ref_l)
    assert np.max(np.abs(got_l[fin] - ref_l[fin])) <= 1e-5 * max(1.0, float(np.max(np.abs(ref_l[fin]))))
    assert np.all(got[~fin] == 0.0)
    # in place into the first part gives the same bits
    lib.attn_merge(d_outs, d_lses, out=d_outs[0], lse=d_lses[0])
    _sync()
    assert torch.equal(d_outs[0].view(torch.int16), out.view(torch.int16))
    assert torch.equal(d_lses[0], lse)


@pytest.mark.parametrize("splits,kv_lens", [((256, 256), None), ((100, 212, 200), None), ((300, 212), [512, 250])])
def test_merge_ring_cross_attention(lib, splits, kv_lens):
    """Cross-attention over the text split into shards (each shard's padding length follows
    from kv_lens), merged, equals the attention over the whole text."""
    import torch
    say(f"[merge] ring over text shards {splits} lens={kv_lens}")
    batch, heads, n_q, L = (2 if kv_lens else 1), 2, 700, sum(splits)
    qb, _, _ = qkv_bits(75, batch, heads, n_q)
    kb, vb = text_kv_bits(75, batch, heads, L)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    outs, lses = [], []
    start = 0
    for size in splits:
        lens = None
        if kv_lens is not None:
            lens = torch.tensor([min(max(x - start, 0), size) for x in kv_lens], dtype=torch.int32, device="cuda")
        o, l = lib.cross_attention(q, k[:, :, start:start + size].contiguous(), v[:, :, start:start + size].contiguous(),
                                   kv_lens=lens)
        outs.append(o)
        lses.append(l)
        start += size
    out, lse = lib.attn_merge(outs, lses)
    _sync()
    ref_o, ref_l = oracle.cross_attention(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb),
                                          kv_lens=kv_lens)
    assert_out_close(from_dev_f64(out), ref_o, f"ring {splits}")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), ref_l, f"ring {splits}")
