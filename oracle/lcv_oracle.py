"""Plain fp64 CPU oracle of LongCat-Video block-sparse 3D self-attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run this
module: only the test-suite, the smoke check of the graft entry point and the
``cpu_baseline`` leg of the benchmark use it.  It shares no code with the HIP path
(only the seeded input generator in ``lcv_inputs`` feeds both).

What it computes is the plain definition of the method, written out with no blocking,
fusion or reordering beyond what that definition states:

* token -> (t, y, x) map of the patchified latent grid, row-major in t, y, x;
* partitioned 3D-RoPE: channels [0,16) rotate with t, [16,40) with y, [40,64) with x,
  interleaved channel pairs treated as complex numbers, pair p of a section of width
  d rotating by pos * theta**(-2p/d)  [longcat-video-rs page, section 03 "Partitioned
  3D-RoPE (16T+24H+24W)"; myzaker article, section on technical principles: 3D RoPE
  on visual tokens];
* block mask over 64-token blocks: query block i sees key block j iff |i-j| <= local
  (sliding window) or j is a multiple of the global stride  [longcat-video-rs page,
  section 02 benchmark table "block=64, local=2, stride=4" and section 03
  "Block-Sparse & Multi-Audio": local sliding-window blocks plus strided global
  key/value blocks; zhichai.net post, section "Block Sparse Attention": dense inside
  a block, sparse between blocks];
* condition isolation at token level: a condition query (q < C) sees only condition
  keys (k < C)  [myzaker article, section on technical principles: block attention
  with a KV cache keeps condition tokens unaffected by noise tokens];
* softmax attention with scale 1/sqrt(64) and the natural-log LSE of the scaled scores;
* the CSR of attended key blocks per query block, and the attention evaluated block by
  block over only the key blocks the CSR lists (the CPU block-sparse form);
* the query/key prologue: RMSNorm over each head's 64 channels with a per-channel gain,
  then the 3D-RoPE  [myzaker article, section on technical principles: RMSNorm in the
  self-attention module, 3D RoPE on visual tokens];
* cross-attention of the video tokens' queries over the text states' keys and values (the
  second attention of every DiT block  [myzaker article, technical principles: each block is
  3D self-attention, cross-attention and a SwiGLU feed-forward network]): dense softmax
  attention over the first kv_len[b] text tokens of each batch item (the rest is padding);
* the merge of attention results computed over disjoint key sets (context-parallel ring
  attention [myzaker article, technical principles: context-parallel ring block-sparse
  attention for high resolution]): with L = log(sum_i exp(lse_i)), out = sum_i exp(lse_i - L)
  out_i, which is softmax attention over the union of the sets;
* the gradients of the attention with respect to q, k, v (the backward pass that LoRA
  training of the model needs  [myzaker article, technical principles: the LoRA-trained
  refinement expert; SimpleTuner quickstart "LongCat-Video Edit", LoRA training]) by the
  chain rule through the row softmax.

Readings taken where the pages are silent (each listed in the design notes): local is
a radius; global blocks are key columns j % s == 0 (s == 0 disables them); blocks are
64 consecutive tokens of the flattened (t, y, x) order; condition tokens are the first
C tokens; noise rows attend by the layout alone; RoPE pairs are adjacent channels,
integer positions from 0, theta = 1e4; attention is bidirectional; a row with no
attended key yields out = 0 and lse = -inf; RMSNorm works per head over its 64 channels
with one 64-value gain and is applied before the rotation; cross-attention has no RoPE and
no block sparsity, and text tokens past a batch item's length are padding.

Every function is pinned by the CPU tests (tests/test_oracle_*.py) to properties fixed
by the pages or by mathematics; nothing here is unpinned.
"""
from __future__ import annotations

import math

import numpy as np

HEAD_DIM = 64
BLOCK = 64
# (first channel, section width, axis) with axis 0 = t, 1 = y, 2 = x.
ROPE_SECTIONS = ((0, 16, 0), (16, 24, 1), (40, 24, 2))
SOFTMAX_SCALE = 1.0 / math.sqrt(HEAD_DIM)


# --------------------------------------------------------------------------- grid
def token_coords(token_index: np.ndarray, grid) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Flattened token index -> (t, y, x) of a row-major (T, H, W) latent grid."""
    _, h, w = grid
    n = np.asarray(token_index, dtype=np.int64)
    return n // (h * w), (n // w) % h, n % w


# --------------------------------------------------------------------------- RoPE
def rope3d(x: np.ndarray, grid, theta: float = 10000.0, token_offset: int = 0) -> np.ndarray:
    """Rotate x[..., N, 64] (float64) by the partitioned 3D-RoPE of tokens
    token_offset .. token_offset+N-1."""
    n_tokens = np.shape(x)[-2]
    return rope3d_at(x, np.arange(n_tokens) + token_offset, grid, theta)


def rope3d_at(x: np.ndarray, tokens: np.ndarray, grid, theta: float = 10000.0) -> np.ndarray:
    """Rotate the rows x[..., R, 64] that sit at token indices ``tokens`` [R]."""
    x = np.asarray(x, dtype=np.float64)
    coords = token_coords(tokens, grid)
    out = x.copy()
    for c0, width, axis in ROPE_SECTIONS:
        pos = coords[axis].astype(np.float64)
        for p in range(width // 2):
            phi = pos * theta ** (-2.0 * p / width)
            cos, sin = np.cos(phi), np.sin(phi)
            a = x[..., c0 + 2 * p]
            b = x[..., c0 + 2 * p + 1]
            out[..., c0 + 2 * p] = a * cos - b * sin
            out[..., c0 + 2 * p + 1] = a * sin + b * cos
    return out


# --------------------------------------------------------------------------- QK prologue (RMSNorm + RoPE)
def rmsnorm(x: np.ndarray, gamma, eps: float) -> np.ndarray:
    """RMS normalisation over the channel (last) axis with a per-channel gain:
    y = x / sqrt(mean(x**2) + eps) * gamma  [myzaker article, section on technical
    principles: RMSNorm in the self-attention module].  Reading taken: it normalises each
    head's 64 query or key channels on their own, with one gain vector of 64 values."""
    x = np.asarray(x, dtype=np.float64)
    mean_sq = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(mean_sq + eps) * np.asarray(gamma, dtype=np.float64)


def rope3d_transpose(x: np.ndarray, grid, theta: float = 10000.0, token_offset: int = 0) -> np.ndarray:
    """The transpose (inverse) of rope3d: each channel pair rotated by minus its angle, which
    maps the gradient of a rotated tensor to the gradient of its input."""
    x = np.asarray(x, dtype=np.float64)
    coords = token_coords(np.arange(np.shape(x)[-2]) + token_offset, grid)
    out = x.copy()
    for c0, width, axis in ROPE_SECTIONS:
        pos = coords[axis].astype(np.float64)
        for p in range(width // 2):
            phi = pos * theta ** (-2.0 * p / width)
            cos, sin = np.cos(phi), np.sin(phi)
            a = x[..., c0 + 2 * p]
            b = x[..., c0 + 2 * p + 1]
            out[..., c0 + 2 * p] = a * cos + b * sin
            out[..., c0 + 2 * p + 1] = b * cos - a * sin
    return out


def qk_norm_rope_backward(x: np.ndarray, gamma, eps: float, grid, dy: np.ndarray, theta: float = 10000.0,
                          token_offset: int = 0):
    """Gradients of sum(dy * qk_norm_rope(x)) with respect to x and gamma (grid None: the
    RMSNorm alone), by the chain rule: dy_pre = R^T dy, n = x / r with
    r = sqrt(mean(x^2) + eps), dgamma = sum over every row of dy_pre * n,
    dn = dy_pre * gamma, dx = (dn - n * mean(dn * n)) / r.  Returns dx [..., N, 64] and
    dgamma [64] (float64)."""
    x = np.asarray(x, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    dy_pre = np.asarray(dy, dtype=np.float64)
    if grid is not None:
        dy_pre = rope3d_transpose(dy_pre, grid, theta, token_offset)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    n = x / r
    dgamma = np.sum((dy_pre * n).reshape(-1, HEAD_DIM), axis=0)
    dn = dy_pre * gamma
    dx = (dn - n * np.mean(dn * n, axis=-1, keepdims=True)) / r
    return dx, dgamma


def qk_norm_rope(x: np.ndarray, gamma, eps: float, grid, theta: float = 10000.0, token_offset: int = 0) -> np.ndarray:
    """Query/key prologue of the self-attention: RMSNorm of each head's channels, then the
    partitioned 3D-RoPE of the token's position (norm first, rotation second, as the
    rotation acts on the normalised channels)."""
    return rope3d(rmsnorm(x, gamma, eps), grid, theta, token_offset)


# --------------------------------------------------------------------------- layout
def n_blocks_of(n_tokens: int) -> int:
    return -(-n_tokens // BLOCK)


def block_mask(n_blocks: int, local: int, stride: int) -> np.ndarray:
    """Mb[i, j] = |i - j| <= local  or  (stride >= 1 and j % stride == 0)."""
    i = np.arange(n_blocks)[:, None]
    j = np.arange(n_blocks)[None, :]
    mb = np.abs(i - j) <= local
    if stride >= 1:
        mb = mb | (j % stride == 0)
    return mb


def token_mask_rows(rows: np.ndarray, n_tokens: int, cond_len: int, local: int, stride: int) -> np.ndarray:
    """M[q, k] for the query tokens in ``rows`` and every key k < N."""
    return token_mask(rows, np.arange(n_tokens), cond_len, local, stride)


def token_mask(rows: np.ndarray, keys: np.ndarray, cond_len: int, local: int, stride: int) -> np.ndarray:
    """M[q, k] for the query tokens in ``rows`` and the key tokens in ``keys``:
    the block mask of (q // 64, k // 64) and the condition rule (q >= C or k < C)."""
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    qi = rows // BLOCK
    kj = keys // BLOCK
    i = qi[:, None]
    j = kj[None, :]
    mb = np.abs(i - j) <= local
    if stride >= 1:
        mb = mb | (j % stride == 0)
    cond_ok = (rows[:, None] >= cond_len) | (keys[None, :] < cond_len)
    return mb & cond_ok


def block_pairs_attended(n_tokens: int, cond_len: int, local: int, stride: int) -> np.ndarray:
    """Block pairs of the block mask that hold at least one attended token pair.

    For non-empty token sets Qi, Kj:  exists q in Qi, k in Kj with (q >= C or k < C)
    holds iff (some q in Qi has q >= C) or (some k in Kj has k < C)."""
    n = n_blocks_of(n_tokens)
    mb = block_mask(n, local, stride)
    last_row = np.minimum(np.arange(n) * BLOCK + BLOCK, n_tokens) - 1
    first_key = np.arange(n) * BLOCK
    has_noise_row = last_row >= cond_len
    has_cond_key = first_key < cond_len
    return mb & (has_noise_row[:, None] | has_cond_key[None, :])


def csr(n_tokens: int, cond_len: int, local: int, stride: int) -> tuple[np.ndarray, np.ndarray]:
    """row_ptr[n+1], col_idx[nnz] (int32): ascending attended key blocks per query block."""
    pairs = block_pairs_attended(n_tokens, cond_len, local, stride)
    counts = pairs.sum(axis=1)
    row_ptr = np.zeros(pairs.shape[0] + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col_idx = np.nonzero(pairs)[1]          # row-major order -> ascending j per row
    return row_ptr.astype(np.int32), col_idx.astype(np.int32)


def attended_pairs(n_tokens: int, cond_len: int, local: int, stride: int) -> int:
    """Number of (q, k) token pairs with M[q, k] = 1, summed over block pairs of the mask:
    noise rows see every key of the block, condition rows only its condition keys."""
    n = n_blocks_of(n_tokens)
    mb = block_mask(n, local, stride)
    lo = np.arange(n) * BLOCK
    hi = np.minimum(lo + BLOCK, n_tokens)
    size = hi - lo
    n_cond = np.clip(cond_len - lo, 0, size)          # tokens < C in each block
    n_noise = size - n_cond
    per_pair = n_noise[:, None] * size[None, :] + n_cond[:, None] * n_cond[None, :]
    return int((per_pair * mb).sum())


# --------------------------------------------------------------------------- attention
def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray):
    """Softmax attention of q[R,64] over k, v[N,64] with boolean mask[R,N] (fp64).
    Returns out[R,64] and the natural-log LSE[R] of the scaled scores.  Rows whose
    mask is empty give out = 0 and lse = -inf."""
    s = (q @ k.T) * SOFTMAX_SCALE
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, initial=-np.inf)   # no key at all is an empty mask too
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    out = (e @ v) / l_safe[:, None]
    out[empty] = 0.0
    lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return out, lse


def masked_attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray, dout: np.ndarray):
    """Gradients of out = softmax(mask(q k^T / 8)) v with respect to q, k and v for the
    upstream gradient dout[R,64] (fp64), by the chain rule through the softmax:
    P = row softmax, dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dO * O)),
    dQ = dS K / 8, dK = dS^T Q / 8.  Rows with an empty mask contribute nothing."""
    s = (q @ k.T) * SOFTMAX_SCALE
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, initial=-np.inf)   # no key at all is an empty mask too
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    p = e / np.where(empty, 1.0, l)[:, None]
    p[empty] = 0.0
    out = p @ v
    dv = p.T @ dout
    dp = dout @ v.T
    delta = np.sum(dout * out, axis=1)
    ds = p * (dp - delta[:, None])
    dq = (ds @ k) * SOFTMAX_SCALE
    dk = (ds.T @ q) * SOFTMAX_SCALE
    return dq, dk, dv


def bsa_backward(q, k, v, dout, cond_len: int, local: int, stride: int):
    """Gradients dq, dk, dv [B, H, N, 64] of the block-sparse attention (no RoPE: q and k as
    they enter the scores, i.e. already rotated) for the upstream gradient dout."""
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    bsz, heads, n_tokens, _ = q.shape
    mask = token_mask_rows(np.arange(n_tokens), n_tokens, cond_len, local, stride)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(bsz):
        for h in range(heads):
            dq[b, h], dk[b, h], dv[b, h] = masked_attention_backward(q[b, h], k[b, h], v[b, h], mask, dout[b, h])
    return dq, dk, dv


def bsa_backward_rows(q, k, v, dout, cond_len: int, local: int, stride: int, rows):
    """dq [B, H, R, 64] at the query tokens ``rows`` only: a row's dq depends on its own
    softmax row alone, so the chain rule runs on those rows."""
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    rows = np.asarray(rows, dtype=np.int64)
    bsz, heads, n_tokens, _ = q.shape
    mask = token_mask_rows(rows, n_tokens, cond_len, local, stride)
    dq = np.zeros((bsz, heads, rows.size, HEAD_DIM))
    for b in range(bsz):
        for h in range(heads):
            dq[b, h] = masked_attention_backward(q[b, h, rows], k[b, h], v[b, h], mask, dout[b, h, rows])[0]
    return dq


def bsa_backward_keys(q, k, v, dout, cond_len: int, local: int, stride: int, keys, row_chunk: int = 512):
    """dk, dv [B, H, K, 64] at the key tokens ``keys`` only: dk and dv of a key are sums over
    the query rows that attend to it, so the chain rule runs on those rows (in chunks of
    ``row_chunk``, whose contributions add)."""
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    keys = np.asarray(keys, dtype=np.int64)
    bsz, heads, n_tokens, _ = q.shape
    seen = token_mask(np.arange(n_tokens), keys, cond_len, local, stride).any(axis=1)
    rows = np.nonzero(seen)[0]
    dk = np.zeros((bsz, heads, keys.size, HEAD_DIM))
    dv = np.zeros((bsz, heads, keys.size, HEAD_DIM))
    for r0 in range(0, rows.size, row_chunk):
        part = rows[r0:r0 + row_chunk]
        mask = token_mask_rows(part, n_tokens, cond_len, local, stride)
        for b in range(bsz):
            for h in range(heads):
                _, dkp, dvp = masked_attention_backward(q[b, h, part], k[b, h], v[b, h], mask, dout[b, h, part])
                dk[b, h] += dkp[keys]
                dv[b, h] += dvp[keys]
    return dk, dv


def bsa_forward(q, k, v, grid, cond_len: int, local: int, stride: int, theta: float = 10000.0,
                rope_q: bool = True, rope_k: bool = True, rows=None):
    """Block-sparse 3D self-attention of q, k, v [B, H, N, 64] (float64).

    rows: optional query token indices to evaluate (all rows if None).
    Returns out [B, H, R, 64] and lse [B, H, R]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bsz, heads, n_tokens, _ = q.shape
    rows = np.arange(n_tokens) if rows is None else np.asarray(rows, dtype=np.int64)
    mask = token_mask_rows(rows, n_tokens, cond_len, local, stride)
    out = np.zeros((bsz, heads, rows.size, HEAD_DIM))
    lse = np.zeros((bsz, heads, rows.size))
    for b in range(bsz):
        for h in range(heads):
            qb = q[b, h, rows]
            kb = k[b, h]
            if rope_q:
                qb = rope3d_at(qb, rows, grid, theta)
            if rope_k:
                kb = rope3d(kb, grid, theta)
            out[b, h], lse[b, h] = masked_attention(qb, kb, v[b, h], mask)
    return out, lse


def bsa_forward_blocks(q, k, v, grid, cond_len: int, local: int, stride: int, theta: float = 10000.0,
                       q_blocks=None):
    """The same attention as bsa_forward, visiting only the attended key blocks: for each
    query block i, the keys of the blocks that csr lists in row i are gathered and the block's
    query rows attend them under the token mask (the condition rule and k < N).  A CPU
    block-sparse implementation as the pages' Rust one is  [longcat-video-rs page, section
    02 benchmark table: block-sparse self-attention with block=64, local=2, stride=4 on the
    CPU], and the like-for-like CPU figure beside the GPU kernel.

    q_blocks: optional query block indices to evaluate (all if None).
    Returns out [B, H, R, 64] and lse [B, H, R] for the rows of those blocks, in order."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bsz, heads, n_tokens, _ = q.shape
    n = n_blocks_of(n_tokens)
    q_blocks = np.arange(n) if q_blocks is None else np.asarray(q_blocks, dtype=np.int64)
    row_ptr, col_idx = csr(n_tokens, cond_len, local, stride)
    row_sets = [np.arange(i * BLOCK, min(i * BLOCK + BLOCK, n_tokens)) for i in q_blocks]
    key_sets = []
    for i in q_blocks:
        cols = col_idx[row_ptr[i]:row_ptr[i + 1]]
        key_sets.append(np.concatenate([np.arange(j * BLOCK, min(j * BLOCK + BLOCK, n_tokens)) for j in cols]))
    n_rows = sum(r.size for r in row_sets)
    out = np.zeros((bsz, heads, n_rows, HEAD_DIM))
    lse = np.zeros((bsz, heads, n_rows))
    for b in range(bsz):
        for h in range(heads):
            k_rot = rope3d(k[b, h], grid, theta)
            at = 0
            for rows, keys in zip(row_sets, key_sets):
                q_rot = rope3d_at(q[b, h, rows], rows, grid, theta)
                mask = token_mask(rows, keys, cond_len, local, stride)
                o, l = masked_attention(q_rot, k_rot[keys], v[b, h, keys], mask)
                out[b, h, at:at + rows.size] = o
                lse[b, h, at:at + rows.size] = l
                at += rows.size
    return out, lse


def cross_attention(q, k, v, kv_lens=None, rows=None):
    """Cross-attention of the video queries q [B, H, N, 64] over text keys/values
    k, v [B, H, L, 64] (float64): softmax(q k^T / 8) v over the keys k < kv_lens[b] of each
    batch item (all L when kv_lens is None).  rows: optional query indices (all if None).
    Returns out [B, H, R, 64] and lse [B, H, R]; a batch item with no key gives out = 0 and
    lse = -inf."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    bsz, heads, n_q, _ = q.shape
    n_kv = k.shape[2]
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((bsz, heads, rows.size, HEAD_DIM))
    lse = np.zeros((bsz, heads, rows.size))
    for b in range(bsz):
        length = n_kv if kv_lens is None else int(kv_lens[b])
        mask = np.broadcast_to(np.arange(n_kv)[None, :] < length, (rows.size, n_kv))
        for h in range(heads):
            out[b, h], lse[b, h] = masked_attention(q[b, h, rows], k[b, h], v[b, h], mask)
    return out, lse


def cross_attention_backward(q, k, v, dout, kv_lens=None):
    """Gradients dq [B, H, N, 64], dk and dv [B, H, L, 64] of cross_attention for the upstream
    gradient dout, by the chain rule through the row softmax (padded text tokens, k >=
    kv_lens[b], get zero gradients)."""
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    bsz, heads, n_q, _ = q.shape
    n_kv = k.shape[2]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(bsz):
        length = n_kv if kv_lens is None else int(kv_lens[b])
        mask = np.broadcast_to(np.arange(n_kv)[None, :] < length, (n_q, n_kv))
        for h in range(heads):
            dq[b, h], dk[b, h], dv[b, h] = masked_attention_backward(q[b, h], k[b, h], v[b, h], mask, dout[b, h])
    return dq, dk, dv


def merge_partials(outs, lses):
    """Merge attention results over disjoint key sets: outs [P][..., R, 64], lses [P][..., R]
    (float64) -> out [..., R, 64], lse [..., R].  lse = log(sum_i exp(lse_i)) (taken around the
    largest lse_i), out = sum_i exp(lse_i - lse) * out_i; rows where every part is empty
    (all lse_i = -inf) give out = 0, lse = -inf."""
    outs = [np.asarray(o, dtype=np.float64) for o in outs]
    lses = [np.asarray(l, dtype=np.float64) for l in lses]
    m = np.max(np.stack(lses), axis=0)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    weights = [np.exp(l - m_safe) for l in lses]
    total = np.sum(np.stack(weights), axis=0)
    total_safe = np.where(empty, 1.0, total)
    out = np.zeros_like(outs[0])
    for o, wgt in zip(outs, weights):
        out += (wgt / total_safe)[..., None] * o
    out[empty] = 0.0
    lse = np.where(empty, -np.inf, m_safe + np.log(total_safe))
    return out, lse


def bsa_forward_cached(q_noise, k_noise, v_noise, k_cond, v_cond, grid, cond_len: int, local: int,
                       stride: int, theta: float = 10000.0, rope_q: bool = True, rope_k: bool = True,
                       rows=None):
    """Noise-token rows [C, N) of the block-sparse attention whose key/value sequence is
    the cached condition K/V followed by the noise K/V.  q_noise, k_noise, v_noise are
    [B, H, N-C, 64]; k_cond, v_cond are [B, H, C, 64].  ``rows`` (optional) are indices
    into the noise rows.  Returns out [B, H, R, 64] and lse [B, H, R]."""
    q_noise = np.asarray(q_noise, dtype=np.float64)
    k_full = np.concatenate([np.asarray(k_cond, np.float64), np.asarray(k_noise, np.float64)], axis=2)
    v_full = np.concatenate([np.asarray(v_cond, np.float64), np.asarray(v_noise, np.float64)], axis=2)
    bsz, heads, n_tokens, _ = k_full.shape
    local_rows = np.arange(n_tokens - cond_len) if rows is None else np.asarray(rows, dtype=np.int64)
    tokens = local_rows + cond_len
    mask = token_mask_rows(tokens, n_tokens, cond_len, local, stride)
    out = np.zeros((bsz, heads, local_rows.size, HEAD_DIM))
    lse = np.zeros((bsz, heads, local_rows.size))
    for b in range(bsz):
        for h in range(heads):
            qb = q_noise[b, h, local_rows]
            kb = k_full[b, h]
            if rope_q:
                qb = rope3d_at(qb, tokens, grid, theta)
            if rope_k:
                kb = rope3d(kb, grid, theta)
            out[b, h], lse[b, h] = masked_attention(qb, kb, v_full[b, h], mask)
    return out, lse
