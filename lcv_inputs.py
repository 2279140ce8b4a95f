"""Seeded synthetic inputs and workload shapes for LongCat-Video block-sparse attention.

This module is shared by the test-suite, the benchmark and the oracle checks.  It
holds no arithmetic of the method itself: it only names the workloads (latent grid,
heads, condition frames, layout knobs), draws i.i.d. N(0,1) fp32 Q/K/V from a
PCG64 stream, and rounds them to bfloat16 (round-to-nearest-even) so that the GPU
path and the fp64 oracle see exactly the same numbers.

Latent-grid geometry follows the LongCat-Video quickstart (SimpleTuner docs, page
"LongCat-Video Edit (Image-to-Video)", sections 1 and 3): frames satisfy
(frames-1) % 4 == 0 and map to (frames-1)/4+1 latent frames, pixel height and width
are divisible by 16 and map to H/16 x W/16 latent tokens per frame.  Condition frames
come first along time (myzaker article, section on technical principles: condition
and noisy frames are concatenated along the time axis).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 64
BLOCK = 64


def latent_grid(frames: int, height_px: int, width_px: int) -> tuple[int, int, int]:
    """Pixel video shape -> latent token grid (T, H, W)."""
    if (frames - 1) % 4 != 0 or height_px % 16 or width_px % 16:
        raise ValueError("frames must satisfy (frames-1)%4==0 and H, W must be divisible by 16")
    return ((frames - 1) // 4 + 1, height_px // 16, width_px // 16)


@dataclass(frozen=True)
class Workload:
    name: str
    grid: tuple[int, int, int]          # latent (T, H, W)
    heads: int
    cond_frames: int = 0                # condition latent frames at the start of time
    local_blocks: int = 2
    global_stride: int = 4
    seed: int = 0
    batch: int = 1
    theta: float = 10000.0
    cached: bool = False                # a second call reuses the condition K/V
    description: str = ""
    sweep: tuple = field(default_factory=tuple)   # (local, stride) density sweep points

    @property
    def n_tokens(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def cond_len(self) -> int:
        return self.cond_frames * self.grid[1] * self.grid[2]

    @property
    def n_blocks(self) -> int:
        return -(-self.n_tokens // BLOCK)


WORKLOADS = {
    "tiny": Workload("tiny", (4, 8, 16), heads=2, seed=0,
                     description="latent 4x8x16 = 512 tokens, 2 heads, no condition"),
    "t2v480": Workload("t2v480", latent_grid(93, 480, 832), heads=32, seed=1,
                       description="T2V 480x832, 93 frames -> 24x30x52 = 37,440 tokens"),
    "i2v480": Workload("i2v480", latent_grid(93, 480, 832), heads=32, cond_frames=1, seed=2,
                       cached=True,
                       description="I2V 480x832: 1 condition latent frame (1,560 tokens), cached K/V"),
    "t2v720": Workload("t2v720", latent_grid(93, 720, 1280), heads=32, seed=3,
                       description="T2V 720x1280, 93 frames -> 24x45x80 = 86,400 tokens"),
    "vc480": Workload("vc480", (40, 30, 52), heads=32, cond_frames=16, seed=4, cached=True,
                      sweep=((64, 3), (2, 3), (2, 4), (2, 8), (2, 12), (2, 16)),
                      description="video continuation 480x832: 16 condition + 24 noisy latent frames"),
}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bfloat16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u.astype(np.uint64) + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact promotion of bfloat16 bit patterns to float64."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def normal_bf16(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return round_to_bf16_bits(x)


def qkv_bits(seed: int, batch: int, heads: int, n_tokens: int, q_scale: float = 1.0):
    """Q, K, V as bf16 bit patterns [batch, heads, n_tokens, 64], drawn in the order q, k, v."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (batch, heads, n_tokens, HEAD_DIM)
    q = normal_bf16(rng, shape, q_scale)
    k = normal_bf16(rng, shape)
    v = normal_bf16(rng, shape)
    return q, k, v


def grad_bits(seed: int, batch: int, heads: int, n_tokens: int) -> np.ndarray:
    """Upstream gradient dO of the attention output as bf16 bit patterns [batch, heads,
    n_tokens, 64]: i.i.d. N(0,1) from its own PCG64 stream (seed + 10000)."""
    rng = np.random.Generator(np.random.PCG64(seed + 10000))
    return normal_bf16(rng, (batch, heads, n_tokens, HEAD_DIM))


# Text states for the cross-attention: the pages name the text encoder (Qwen-2.5-VL) but no
# prompt length; 512 tokens per prompt is taken as the padded length.
TEXT_LEN = 512


def text_kv_bits(seed: int, batch: int, heads: int, text_len: int = TEXT_LEN):
    """Text keys and values of the cross-attention as bf16 bit patterns [batch, heads,
    text_len, 64]: i.i.d. N(0,1) from their own PCG64 stream (seed + 20000), k then v."""
    rng = np.random.Generator(np.random.PCG64(seed + 20000))
    shape = (batch, heads, text_len, HEAD_DIM)
    k = normal_bf16(rng, shape)
    v = normal_bf16(rng, shape)
    return k, v


def workload_inputs(w: Workload, call: int = 0, q_scale: float = 1.0):
    """Inputs of a workload.  call 0: full Q/K/V over all N tokens.  call 1 (cached
    workloads): fresh noise-token Q/K/V over the N-C noise tokens, seed + 100."""
    if call == 0:
        return qkv_bits(w.seed, w.batch, w.heads, w.n_tokens, q_scale)
    return qkv_bits(w.seed + 100, w.batch, w.heads, w.n_tokens - w.cond_len, q_scale)
