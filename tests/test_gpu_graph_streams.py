"""Capture in a HIP graph, and concurrent streams on one layout.

Every compute entry point only launches kernels on the caller's stream (no allocation, copy,
memset or synchronisation), so a whole training chain can be captured once and replayed: the
QK prologue on Q and K, the attention forward and backward, the prologue backward on both,
and the cross-attention with its backward.  The graph is replayed several times, with eager
work of the program and new input values between the replays, and every replay is compared
bitwise with eager calls on the same inputs.  A layout is immutable, so two streams may run
on it at once: each stream's results are bitwise those of the serial calls."""
from __future__ import annotations

import numpy as np
import pytest

from lcv_inputs import grad_bits, qkv_bits, text_kv_bits
from tests.gpu_util import say, to_dev

pytestmark = pytest.mark.gpu

GRID = (3, 10, 21)   # 630 tokens: ragged last block
N = 630
HEADS = 2
COND = 210
EPS = 1e-6


def _gains():
    import torch
    rng = np.random.default_rng(91)
    return [torch.from_numpy(rng.uniform(0.5, 2.0, 64).astype(np.float32)).cuda() for _ in range(2)]


class Chain:
    """Static buffers of one training chain and the calls that fill them."""

    def __init__(self, lib, layout):
        import torch
        self.lib, self.layout = lib, layout
        shape = (1, HEADS, N, 64)
        self.q, self.k, self.v, self.do = (torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in range(4))
        self.tk, self.tv = (torch.empty((1, HEADS, 96, 64), dtype=torch.bfloat16, device="cuda") for _ in range(2))
        self.lens = torch.tensor([77], dtype=torch.int32, device="cuda")
        self.gq, self.gk = _gains()
        e = lambda: torch.empty(shape, dtype=torch.bfloat16, device="cuda")   # noqa: E731
        self.qn, self.kn, self.out, self.dq, self.dk, self.dv, self.dxq, self.dxk = (e() for _ in range(8))
        self.xo, self.xdq = e(), e()
        self.xdk, self.xdv = torch.empty_like(self.tk), torch.empty_like(self.tv)
        self.lse = torch.empty((1, HEADS, N), dtype=torch.float32, device="cuda")
        self.xlse = torch.empty_like(self.lse)
        self.dgq, self.dgk = (torch.empty(64, dtype=torch.float32, device="cuda") for _ in range(2))
        self.ws = torch.empty(lib.backward_workspace(1, HEADS, N), dtype=torch.float32, device="cuda")
        self.pws = torch.empty(lib.lib().lcv_qk_rmsnorm_rope3d_backward_workspace(HEADS, N), dtype=torch.float32,
                               device="cuda")
        self.xws = torch.empty(lib.cross_attention_backward_workspace(1, HEADS, N, 96), dtype=torch.float32,
                               device="cuda")

    def set_inputs(self, seed):
        qb, kb, vb = qkv_bits(seed, 1, HEADS, N)
        tkb, tvb = text_kv_bits(seed, 1, HEADS, 96)
        for dst, bits in ((self.q, qb), (self.k, kb), (self.v, vb), (self.do, grad_bits(seed, 1, HEADS, N)),
                          (self.tk, tkb), (self.tv, tvb)):
            dst.copy_(to_dev(bits))

    def run(self, stream=None):
        lib = self.lib
        lib.qk_rmsnorm_rope3d(self.q, self.gq, EPS, GRID, out=self.qn, stream=stream)
        lib.qk_rmsnorm_rope3d(self.k, self.gk, EPS, GRID, out=self.kn, stream=stream)
        lib.forward(self.qn, self.kn, self.v, self.layout, grid=None, out=self.out, lse=self.lse, stream=stream)
        lib.backward(self.qn, self.kn, self.v, self.out, self.lse, self.do, self.layout, dq=self.dq, dk=self.dk,
                     dv=self.dv, workspace=self.ws, stream=stream)
        lib.qk_rmsnorm_rope3d_backward(self.q, self.dq, self.gq, EPS, GRID, dx=self.dxq, dgamma=self.dgq,
                                       workspace=self.pws, stream=stream)
        lib.qk_rmsnorm_rope3d_backward(self.k, self.dk, self.gk, EPS, GRID, dx=self.dxk, dgamma=self.dgk,
                                       workspace=self.pws, stream=stream)
        lib.cross_attention(self.q, self.tk, self.tv, kv_lens=self.lens, out=self.xo, lse=self.xlse, stream=stream)
        lib.cross_attention_backward(self.q, self.tk, self.tv, self.xo, self.xlse, self.do, kv_lens=self.lens,
                                     dq=self.xdq, dk=self.xdk, dv=self.xdv, workspace=self.xws, stream=stream)

    def outputs(self):
        return [t.clone() for t in (self.qn, self.kn, self.out, self.lse, self.dq, self.dk, self.dv, self.dxq,
                                    self.dxk, self.dgq, self.dgk, self.xo, self.xlse, self.xdq, self.xdk, self.xdv)]


def _same(a, b, what):
    import torch
    for i, (x, y) in enumerate(zip(a, b)):
        xv = x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)
        yv = y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)
        assert torch.equal(xv, yv), f"{what}: output {i} differs"


def test_graph_capture_and_replay(lib):
    import torch
    layout = lib.build_layout(N, 2, 4, COND)
    chain = Chain(lib, layout)
    eager = {}
    for seed in (5, 6, 7):
        chain.set_inputs(seed)
        chain.run()
        torch.cuda.synchronize()
        eager[seed] = chain.outputs()
    say("[graph] capture the training chain")
    chain.set_inputs(5)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chain.run()          # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        chain.run()
    torch.cuda.synchronize()
    other = Chain(lib, layout)
    for replay, seed in enumerate((5, 6, 5, 7, 7)):
        chain.set_inputs(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(chain.outputs(), eager[seed], f"replay {replay} (inputs {seed})")
        # eager work of the program between replays, on other buffers and the same layout
        other.set_inputs(100 + replay)
        other.run()
        torch.cuda.synchronize()
    say("[graph] 5 replays bitwise equal to eager")
    del g
    layout.close()


def test_two_streams_share_a_layout(lib):
    import torch
    layout = lib.build_layout(N, 2, 4, COND)
    chains = [Chain(lib, layout) for _ in range(2)]
    serial = []
    for i, c in enumerate(chains):
        c.set_inputs(20 + i)
        c.run()
        torch.cuda.synchronize()
        serial.append(c.outputs())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for c in chains:
            for t in (c.qn, c.kn, c.out, c.dq, c.dk, c.dv, c.xo, c.xdq):
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        for c, st in zip(chains, streams):
            c.run(stream=st)
        torch.cuda.synchronize()
        for i, c in enumerate(chains):
            _same(c.outputs(), serial[i], f"stream {i}, round {rep}")
    say("[streams] two streams on one layout, 3 rounds bitwise equal to serial")
    layout.close()
