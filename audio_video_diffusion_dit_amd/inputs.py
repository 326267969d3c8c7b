"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module only draws data: it holds none of the block's or the loop's
arithmetic. Every tensor comes from ``numpy.random.Generator(PCG64(seed))`` in a
fixed draw order, and float draws destined for bf16 storage are rounded to the
nearest bfloat16 (ties to even) here, so that the HIP path and the oracle see
identical values.

Workload shapes (the packed joint sequence of [P3] TeleFuser PR #23 "[FEAT] Add
MiniMax H3 joint audio-video generation", "Motivation": video tokens, then audio
tokens, then a zero tail):

  name          D     HxDh    F     video  audio  seq_pad  blocks  intervals
  block_small   256   4x64    683   512    96     640      1       -
  loop_4blk     1024  8x128   2816  4096   512    4608     4       49
  block_h3      3072  24x128  8192  12096  1344   13568    1       -
  attn_ragged   2048  16x128  -     batch of 4, valid {3000, 5100, 7777, 8192} in 8192
  loop_8blk_32k 3072  24x128  8192  30720  2048   32768    8       49

loop_4blk is quoted as "hidden 1024, 16 heads x 128", which cannot hold (16 x 128 = 2048);
the hidden size and FFN width (2816, about 8/3 of 1024) are kept and the head count is read
as 8 heads of 128, the head size every other workload uses.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float -> bfloat16 bit patterns (uint16), round to nearest even."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 values."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    hidden: int
    heads: int
    head_dim: int
    ffn: int
    n_video: int
    n_audio: int
    seq_pad: int
    n_blocks: int = 1
    n_intervals: int = 0
    norm_eps: float = 1e-6
    qk_eps: float = 1e-6
    rope_base: float = 10000.0

    @property
    def n_valid(self) -> int:
        return self.n_video + self.n_audio


def _pad256(n: int) -> int:
    return ((n + 255) // 256) * 256


WORKLOADS = {
    "block_small": Workload("block_small", 256, 4, 64, 683, 512, 96, 640),
    "loop_4blk": Workload("loop_4blk", 1024, 8, 128, 2816, 4096, 512, 4608,
                          n_blocks=4, n_intervals=49),
    "block_h3": Workload("block_h3", 3072, 24, 128, 8192, 12096, 1344,
                         _pad256(12096 + 1344)),
    "loop_8blk_32k": Workload("loop_8blk_32k", 3072, 24, 128, 8192, 30720, 2048, 32768,
                              n_blocks=8, n_intervals=49),
}

ATTN_RAGGED = dict(batch=4, seq_pad=8192, heads=16, head_dim=128,
                   valid=(3000, 5100, 7777, 8192))

# A batch of four ragged requests through one H3-scale block (hidden 3072, 24 x 128 heads, FFN
# 8192), each padded to 8192 rows, with the attention case's length mix: (n_video, n_audio) per
# request, audio about 1/16 of the tokens as in the H3 workload.
BLOCK_RAGGED = dict(hidden=3072, heads=24, head_dim=128, ffn=8192, seq_pad=8192,
                    requests=((2800, 200), (4800, 300), (7277, 500), (7680, 512)))


@dataclass
class BlockParams:
    """One block's parameters: bf16 bit patterns for matrices, fp32 for the rest."""
    w_qkv: np.ndarray      # uint16 [3D, D]
    w_o: np.ndarray        # uint16 [D, D]
    w_gate_up: np.ndarray  # uint16 [2F, D] (gate rows first)
    w_down: np.ndarray     # uint16 [D, F]
    norm1_g: np.ndarray    # f32 [D]
    norm2_g: np.ndarray    # f32 [D]
    q_g: np.ndarray        # f32 [Dh]
    k_g: np.ndarray        # f32 [Dh]
    ada: np.ndarray        # f32 [2, 6, D]

    def as_float(self) -> dict:
        return dict(w_qkv=bf16_to_f32(self.w_qkv), w_o=bf16_to_f32(self.w_o),
                    w_gate_up=bf16_to_f32(self.w_gate_up), w_down=bf16_to_f32(self.w_down),
                    norm1_g=self.norm1_g, norm2_g=self.norm2_g, q_g=self.q_g, k_g=self.k_g,
                    ada=self.ada)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return bf16_bits(a)


def make_block(rng: np.random.Generator, wl: Workload, weight_std: float = 0.02,
               ada_std: float = 0.02) -> BlockParams:
    """Draw order: w_qkv, w_o, w_gate_up, w_down (bf16 N(0, 0.02)), ada (fp32
    N(0, 0.02)); the norm gains are ones."""
    D, F, Dh = wl.hidden, wl.ffn, wl.head_dim
    w_qkv = _normal_bf16(rng, (3 * D, D), weight_std)
    w_o = _normal_bf16(rng, (D, D), weight_std)
    w_gate_up = _normal_bf16(rng, (2 * F, D), weight_std)
    w_down = _normal_bf16(rng, (D, F), weight_std)
    ada = (rng.standard_normal(size=(2, 6, D), dtype=np.float32) * np.float32(ada_std))
    ones_d = np.ones(D, dtype=np.float32)
    ones_h = np.ones(Dh, dtype=np.float32)
    return BlockParams(w_qkv, w_o, w_gate_up, w_down, ones_d.copy(), ones_d.copy(),
                       ones_h.copy(), ones_h.copy(), ada.astype(np.float32))


# Output channels of the velocity head per token (the latent channels of both modalities); the
# pages give no channel count.
HEAD_CHANNELS = 128


@dataclass
class HeadParams:
    """The velocity head: final norm gain and two-row table, per-modality output projection."""
    norm_g: np.ndarray  # f32 [D]
    ada: np.ndarray     # f32 [2, 2, D] (shift, scale)
    w_out: np.ndarray   # uint16 [2, C, D]
    bias: np.ndarray    # f32 [2, C]

    def as_float(self) -> dict:
        return dict(norm_g=self.norm_g, ada=self.ada, w_out=bf16_to_f32(self.w_out), bias=self.bias)


def make_head(rng: np.random.Generator, wl: Workload, channels: int = HEAD_CHANNELS,
              weight_std: float = 0.02) -> HeadParams:
    """Draw order: w_out (bf16 N(0, 0.02)), ada (fp32 N(0, 0.02)), bias (fp32 N(0, 0.02)),
    norm gain (fp32 U(0.5, 1.5))."""
    D = wl.hidden
    w_out = _normal_bf16(rng, (2, channels, D), weight_std)
    ada = rng.standard_normal(size=(2, 2, D), dtype=np.float32) * np.float32(0.02)
    bias = rng.standard_normal(size=(2, channels), dtype=np.float32) * np.float32(0.02)
    g = rng.uniform(0.5, 1.5, size=D).astype(np.float32)
    return HeadParams(g, ada.astype(np.float32), w_out, bias.astype(np.float32))


def make_activation_bf16(rng: np.random.Generator, wl: Workload, std: float = 1.0) -> np.ndarray:
    """x [seq_pad, D] bf16 bits: N(0, std) on the valid rows, zero tail."""
    x = np.zeros((wl.seq_pad, wl.hidden), dtype=np.uint16)
    x[: wl.n_valid] = _normal_bf16(rng, (wl.n_valid, wl.hidden), std)
    return x


def make_latent_f32(rng: np.random.Generator, wl: Workload) -> np.ndarray:
    """x_0 [seq_pad, D] fp32: N(0, 1) on the valid rows, zero tail."""
    x = np.zeros((wl.seq_pad, wl.hidden), dtype=np.float32)
    x[: wl.n_valid] = rng.standard_normal(size=(wl.n_valid, wl.hidden), dtype=np.float32)
    return x


def make_temb(rng: np.random.Generator, wl: Workload) -> np.ndarray:
    """Single-call timestep embedding T [2, 6, D] fp32, N(0, 1)."""
    return rng.standard_normal(size=(2, 6, wl.hidden), dtype=np.float32)


def linear_sigmas(n_intervals: int) -> np.ndarray:
    """sigma_k = 1 - k/N for k = 0..N (computed in float64, stored fp32); sigma_N = 0."""
    k = np.arange(n_intervals + 1, dtype=np.float64)
    s = 1.0 - k / n_intervals
    s[-1] = 0.0
    return s.astype(np.float32)


def shifted_sigmas(n_intervals: int, shift: float) -> np.ndarray:
    """Non-linear schedule: the linear sigmas time-shifted, s' = shift s / (1 + (shift - 1) s)
    (float64, stored fp32); s'_0 = 1, s'_N = 0, and shift = 1 gives the linear schedule."""
    s = linear_sigmas(n_intervals).astype(np.float64)
    out = shift * s / (1.0 + (shift - 1.0) * s)
    out[0], out[-1] = 1.0, 0.0
    return out.astype(np.float32)


def timestep_embeddings(rng: np.random.Generator, wl: Workload, sigmas_video: np.ndarray,
                        sigmas_audio: np.ndarray) -> np.ndarray:
    """Per-interval embeddings T_i [N, 2, 6, D] fp32 that vary smoothly with sigma.

    T_i[m] = reshape(phi(1000 * sigma_m[i]) @ W_t, [6, D]) with phi the 256-wide
    [cos, sin] features of 128 geometric frequencies (max period 1e4) and W_t
    [256, 6D] ~ N(0, 1/128), so each entry has unit variance. Computed in
    float64 and stored fp32; it is harness data, identical for both sides.
    """
    n = len(sigmas_video) - 1
    D = wl.hidden
    w_t = rng.standard_normal(size=(256, 6 * D)).astype(np.float64) / math.sqrt(128.0)
    freqs = np.exp(-math.log(1e4) * np.arange(128, dtype=np.float64) / 128.0)
    out = np.empty((n, 2, 6, D), dtype=np.float32)
    for m, sig in enumerate((sigmas_video, sigmas_audio)):
        t = 1000.0 * np.asarray(sig[:n], dtype=np.float64)
        ang = t[:, None] * freqs[None, :]
        phi = np.concatenate([np.cos(ang), np.sin(ang)], axis=1)   # [N, 256]
        out[:, m] = (phi @ w_t).reshape(n, 6, D).astype(np.float32)
    return out


@dataclass
class BlockCase:
    wl: Workload
    blocks: List[BlockParams]
    x: np.ndarray          # bf16 bits [L, D]
    temb: np.ndarray       # f32 [2, 6, D]


def block_case(wl: Workload, seed: int = 0, n_blocks: Optional[int] = None) -> BlockCase:
    """Draw order: blocks (each per ``make_block``), then x, then T."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nb = wl.n_blocks if n_blocks is None else n_blocks
    blocks = [make_block(rng, wl) for _ in range(nb)]
    x = make_activation_bf16(rng, wl)
    temb = make_temb(rng, wl)
    return BlockCase(wl, blocks, x, temb)


@dataclass
class LoopCase:
    wl: Workload
    blocks: List[BlockParams]
    x0: np.ndarray            # f32 [L, D]
    sigmas_video: np.ndarray  # f32 [N+1]
    sigmas_audio: np.ndarray  # f32 [N+1]
    temb_steps: np.ndarray    # f32 [N, 2, 6, D]


def loop_case(wl: Workload, seed: int = 0, n_blocks: Optional[int] = None,
              n_intervals: Optional[int] = None, shift_video: float = 1.0,
              shift_audio: float = 1.0) -> LoopCase:
    """Draw order: blocks, then x_0, then W_t of the timestep embeddings. Sigmas: linear 1 -> 0
    per modality, or time-shifted (shifted_sigmas) when a shift is not 1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nb = wl.n_blocks if n_blocks is None else n_blocks
    n = wl.n_intervals if n_intervals is None else n_intervals
    blocks = [make_block(rng, wl) for _ in range(nb)]
    x0 = make_latent_f32(rng, wl)
    sv = linear_sigmas(n) if shift_video == 1.0 else shifted_sigmas(n, shift_video)
    sa = linear_sigmas(n) if shift_audio == 1.0 else shifted_sigmas(n, shift_audio)
    temb = timestep_embeddings(rng, wl, sv, sa)
    return LoopCase(wl, blocks, x0, sv, sa, temb)


def attention_case(batch: int, seq_pad: int, heads: int, head_dim: int,
                   valid: Tuple[int, ...], seed: int = 0):
    """q, k, v bf16 bits [batch, seq_pad, heads, head_dim], N(0, 1) on each
    request's valid rows and zero beyond (draw order q, k, v per request)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (batch, seq_pad, heads, head_dim)
    q = np.zeros(shape, dtype=np.uint16)
    k = np.zeros(shape, dtype=np.uint16)
    v = np.zeros(shape, dtype=np.uint16)
    for b, n in enumerate(valid):
        for t in (q, k, v):
            t[b, :n] = _normal_bf16(rng, (n, heads, head_dim), 1.0)
    return q, k, v
