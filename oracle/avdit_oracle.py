"""Float64 CPU oracle of the packed audio-video DiT block and the cached denoise loop.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg, never by the product path.

Pages cited (by title and section):
  [P1] TeleFuser PR #38, "perf(minimax-h3): add conservative DiT velocity reuse"
  [P2] 1Cat-vLLM PR #584, "[Video] Add native H3 request-scoped TeaCache and Cache-DiT"
  [P3] TeleFuser PR #23, "[FEAT] Add MiniMax H3 joint audio-video generation"

The pages name the fused operations (RMSNorm with indexed AdaLN modulation, Q/K
RMSNorm with NeoX RoPE, valid-only attention over a zero tail, SwiGLU) and the
velocity-reuse cache policy, but print no formulas. Each function below is the
plain textbook definition of the named operation; where a choice had to be made
(chunk order, epsilon, which axis QK-norm runs over, the window convention of the
cache) it is stated in the function's docstring.

Pin status: every function is pinned by ``tests/test_oracle_pins.py`` against
closed forms, brute-force scalar loops, special cases or the cache counts the
pages print, except ``block_forward`` as a whole, whose composition is pinned
only through its parts and a brute-force scalar re-derivation on a tiny shape
("parity unpinned" against the pages: they print no numeric example of a block),
``stack_forward``, pinned against those scalar loops chained by hand over two blocks, and
``velocity_head``, pinned by closed forms (one-hot rows, a scale of -1) and scalar loops.

Diagnostics (never the graded reference): ``block_forward_bf16_storage`` and
``attention_bf16_storage`` are the same functions with the intermediates a bf16
implementation stores rounded to bf16 where they are stored; pinned bit for bit
against scalar loops that round each stored element.
"""

from __future__ import annotations

import math
from contextlib import contextmanager
from dataclasses import dataclass
from typing import Callable, Optional, Sequence

import numpy as np

F64 = np.float64

_WORK_DTYPE = [F64]


def work_dtype():
    """Floating type of the block arithmetic: float64, unless a ``precision`` block says
    otherwise."""
    return _WORK_DTYPE[0]


@contextmanager
def precision(dtype):
    """Evaluate the layout, norm, projection, RoPE, attention and SwiGLU functions (and so
    ``block_forward``) in another floating type: the same definitions at that precision. The
    checker is always float64; float32 is used only to time a single-precision evaluation."""
    prev = _WORK_DTYPE[0]
    _WORK_DTYPE[0] = np.dtype(dtype).type
    try:
        yield
    finally:
        _WORK_DTYPE[0] = prev

# Order of the six AdaLN modulation rows of one modality.
SHIFT_MSA, SCALE_MSA, GATE_MSA, SHIFT_MLP, SCALE_MLP, GATE_MLP = range(6)
# Row classes of the packed sequence.
VIDEO, AUDIO, TAIL = 0, 1, -1


@dataclass(frozen=True)
class Dims:
    hidden: int
    heads: int
    head_dim: int
    ffn: int
    norm_eps: float = 1e-6
    qk_eps: float = 1e-6
    rope_base: float = 10000.0


@dataclass(frozen=True)
class Layout:
    n_video: int
    n_audio: int
    seq_pad: int

    @property
    def n_valid(self) -> int:
        return self.n_video + self.n_audio


@dataclass(frozen=True)
class CachePolicy:
    mode: str = "off"  # "off", "velocity" ("conservative" is an alias) or "extrapolate"
    start_ratio: float = 0.2
    end_ratio: float = 0.8
    refresh_interval: int = 2
    max_consecutive_reuse: int = 1
    threshold: Optional[float] = None


# ---------------------------------------------------------------- layout ----

def row_modality(layout: Layout) -> np.ndarray:
    """Modality id of every row of the packed sequence.

    [P3 "Motivation", "Changes Made"]: one packed joint sequence of video and
    audio tokens. [P1 §2]: the padded rows form a zero tail. Rows
    0..n_video-1 are video (0), the next n_audio rows audio (1), the rest tail (-1).
    """
    m = np.full(layout.seq_pad, TAIL, dtype=np.int64)
    m[: layout.n_video] = VIDEO
    m[layout.n_video: layout.n_valid] = AUDIO
    return m


def row_positions(layout: Layout, positions: Optional[np.ndarray] = None) -> np.ndarray:
    """Rotary position of every row: the packed index unless an array is given."""
    if positions is None:
        return np.arange(layout.seq_pad, dtype=work_dtype())
    return np.asarray(positions, dtype=work_dtype())


# --------------------------------------------------------- elementwise ops --

def bf16_round(a) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even), returned as float64 values.

    Used only where the contract itself converts to bf16: the DiT input made from
    the fp32 latent at each refresh of the denoise loop ([P3 "Changes Made"]:
    explicit BF16/FP32 boundaries).
    """
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = rounded.astype(np.uint32).view(np.float32).astype(F64)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = np.nan
    return out


def rms_normalize(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) over the last axis (RMSNorm without its gain)."""
    x = np.asarray(x, dtype=work_dtype())
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps)


def silu(u: np.ndarray) -> np.ndarray:
    """u * sigmoid(u) = u / (1 + exp(-u))."""
    u = np.asarray(u, dtype=work_dtype())
    return u / (1.0 + np.exp(-u))


# --------------------------------------------------------------- AdaLN ------

def modulation_rows(ada: np.ndarray, temb: np.ndarray) -> np.ndarray:
    """Per-modality modulation table E = A + T, shape [n_mod, 6, D].

    [P1 §2] "RMSNorm fused with indexed AdaLN modulation"; [P3 "Changes Made"]
    "indexed modulation" and independent per-modality schedules: each modality
    carries its own timestep, so both the block's learned table A and the
    timestep embedding T have one [6, D] slice per modality, and a row picks its
    slice by modality id.
    """
    return np.asarray(ada, dtype=work_dtype()) + np.asarray(temb, dtype=work_dtype())


def norm_modulate(x, gain, E, modality, shift_chunk: int, scale_chunk: int, eps: float):
    """h = RMSNorm(x) * g * (1 + scale[m]) + shift[m] per valid row; tail rows are 0.

    [P1 §2] fused RMSNorm + indexed AdaLN; [P3 "Changes Made"] indexed modulation.
    """
    x = np.asarray(x, dtype=work_dtype())
    out = np.zeros_like(x)
    valid = modality >= 0
    if not valid.any():
        return out
    xn = rms_normalize(x[valid], eps) * np.asarray(gain, dtype=work_dtype())
    Em = E[modality[valid]]  # [V, 6, D]
    out[valid] = xn * (1.0 + Em[:, scale_chunk]) + Em[:, shift_chunk]
    return out


# ------------------------------------------------------ attention pieces ----

def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """x @ w^T with w in [out, in] layout, no bias."""
    return np.asarray(x, dtype=work_dtype()) @ np.asarray(w, dtype=work_dtype()).T


def qk_rms_norm(t: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """Per-head RMSNorm of q or k over head_dim: t [T, H, Dh], gain [Dh].

    [P1 §2] and [P3 "Changes Made"]: Q/K RMSNorm before RoPE. Read as a per-head
    norm (gain of length head_dim).
    """
    return rms_normalize(t, eps) * np.asarray(gain, dtype=work_dtype())


def rope_inv_freq(head_dim: int, base: float) -> np.ndarray:
    """inv_i = base^(-2i / head_dim), i = 0 .. head_dim/2 - 1."""
    i = np.arange(head_dim // 2, dtype=F64)
    return np.power(F64(base), -2.0 * i / head_dim).astype(work_dtype())


def rope_neox(t: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """NeoX (rotate-half) rotary embedding of t [T, H, Dh] at positions pos [T].

    [P3 "Changes Made"]: "NeoX RoPE". Element i of the first half and element
    i + Dh/2 form one pair, rotated by the angle pos * inv_i:
      out[i]        = t[i] cos - t[i+Dh/2] sin
      out[i+Dh/2]   = t[i+Dh/2] cos + t[i] sin
    """
    t = np.asarray(t, dtype=work_dtype())
    half = t.shape[-1] // 2
    theta = np.asarray(pos, dtype=work_dtype())[:, None] * rope_inv_freq(t.shape[-1], base)[None, :]
    c = np.cos(theta)[:, None, :]
    s = np.sin(theta)[:, None, :]
    a, b = t[..., :half], t[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def attention_valid(q, k, v, n_valid: int, p_store: Optional[Callable] = None) -> np.ndarray:
    """Softmax attention restricted to the valid prefix; q, k, v [L, H, Dh].

    [P1 §2] valid-only attention with zero-tail merge: queries and keys with index
    < n_valid attend to each other bidirectionally (jointly over both
    modalities), with scores q.k / sqrt(Dh); output rows >= n_valid are 0. Rows of
    the inputs at or beyond n_valid are never read.

    p_store (diagnostic only, default none): applied to the unnormalised
    probabilities before they weight the values and are summed, i.e. the form in
    which they are stored as the operand of the P.V product.
    """
    q = np.asarray(q, dtype=work_dtype())
    L, H, Dh = q.shape
    out = np.zeros((L, H, Dh), dtype=work_dtype())
    if n_valid == 0:
        return out
    qv = q[:n_valid].transpose(1, 0, 2)                           # [H, V, Dh]
    kv = np.asarray(k, dtype=work_dtype())[:n_valid].transpose(1, 0, 2)
    vv = np.asarray(v, dtype=work_dtype())[:n_valid].transpose(1, 0, 2)
    s = (qv @ kv.transpose(0, 2, 1)) / math.sqrt(Dh)               # [H, V, V]
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    if p_store is not None:
        p = p_store(p)
    p = p / p.sum(axis=-1, keepdims=True)
    out[:n_valid] = (p @ vv).transpose(1, 0, 2)
    return out


def attention_rows(q_rows, k, v, n_valid: int, p_store: Optional[Callable] = None) -> np.ndarray:
    """Attention output for a subset of query rows q_rows [R, H, Dh] against the
    valid keys k[:n_valid], v[:n_valid] (same definition as ``attention_valid``,
    p_store likewise)."""
    q_rows = np.asarray(q_rows, dtype=work_dtype())
    Dh = q_rows.shape[-1]
    kv = np.asarray(k, dtype=work_dtype())[:n_valid].transpose(1, 0, 2)     # [H, V, Dh]
    vv = np.asarray(v, dtype=work_dtype())[:n_valid].transpose(1, 0, 2)
    qr = q_rows.transpose(1, 0, 2)                                 # [H, R, Dh]
    s = (qr @ kv.transpose(0, 2, 1)) / math.sqrt(Dh)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    if p_store is not None:
        p = p_store(p)
    p = p / p.sum(axis=-1, keepdims=True)
    return (p @ vv).transpose(1, 0, 2)


def swiglu(h, w_gate_up, ffn: int) -> np.ndarray:
    """SwiGLU: silu(h Wg^T) * (h Wu^T), with W_gate_up = [Wg; Wu] of shape [2F, D].

    [P3 "Changes Made"]: fused SwiGLU. Gate rows come first in the packed weight.
    """
    w = np.asarray(w_gate_up, dtype=work_dtype())
    g = linear(h, w[:ffn])
    u = linear(h, w[ffn:2 * ffn])
    return silu(g) * u


# ---------------------------------------------------------------- block -----

def block_forward(x, blk: dict, temb, dims: Dims, layout: Layout,
                  positions: Optional[np.ndarray] = None,
                  rows: Optional[np.ndarray] = None,
                  want_intermediates: bool = False,
                  store: Optional[Callable[[str, np.ndarray], np.ndarray]] = None):
    """One joint audio-video DiT block on the packed sequence x [L, D].

    Composition (the pre-norm AdaLN DiT block that uses every fused operation the
    pages list in [P1 §2] and [P3 "Changes Made"]):
      E   = A + T                                   (per-modality table)
      h   = RMSNorm(x) g1 (1 + E[m,1]) + E[m,0]
      q,k,v = h Wqkv^T, split into heads
      q,k = RoPE(QKNorm(q)), RoPE(QKNorm(k))
      o   = valid-only attention(q, k, v)
      x1  = x + E[m,2] * (o Wo^T)
      h2  = RMSNorm(x1) g2 (1 + E[m,4]) + E[m,3]
      x2  = x1 + E[m,5] * (SwiGLU(h2) Wd^T)
    Tail rows of x2 are 0. With ``rows`` given, only those output rows are
    computed (keys and values still come from every valid row).

    ``store`` (diagnostic only; None for the definition above) is applied to each
    intermediate where a fused implementation writes it out, under these names:
    "h" (norm1 output), "qkv" (the q, k and v projections), "qk" (q and k after
    Q/K norm and RoPE), "p" (the unnormalised attention probabilities as the
    operand of the P.V product; the softmax denominator sums the stored values),
    "o" (attention output), "x1" (mid-block residual), "h2" (norm2 output),
    "act" (SwiGLU output) and "out" (the block output on valid rows).
    """
    st = store if store is not None else (lambda name, a: a)
    D, H, Dh, F = dims.hidden, dims.heads, dims.head_dim, dims.ffn
    x = np.asarray(x, dtype=work_dtype())
    L = layout.seq_pad
    V = layout.n_valid
    mod = row_modality(layout)
    pos = row_positions(layout, positions)
    E = modulation_rows(blk["ada"], temb)

    h = st("h", norm_modulate(x, blk["norm1_g"], E, mod, SHIFT_MSA, SCALE_MSA, dims.norm_eps))
    w_qkv = np.asarray(blk["w_qkv"], dtype=work_dtype())
    kv_rows = slice(0, V)
    k = st("qkv", linear(h[kv_rows], w_qkv[D:2 * D])).reshape(V, H, Dh)
    v = st("qkv", linear(h[kv_rows], w_qkv[2 * D:3 * D])).reshape(V, H, Dh)
    k = st("qk", rope_neox(qk_rms_norm(k, blk["k_g"], dims.qk_eps), pos[:V], dims.rope_base))

    if rows is None:
        rows = np.arange(L)
    rows = np.asarray(rows, dtype=np.int64)
    sel_valid = rows[rows < V]

    q = st("qkv", linear(h[sel_valid], w_qkv[0:D])).reshape(len(sel_valid), H, Dh)
    q = st("qk", rope_neox(qk_rms_norm(q, blk["q_g"], dims.qk_eps), pos[sel_valid], dims.rope_base))
    p_store = None if store is None else (lambda p: st("p", p))
    o = (attention_rows(q, k, v, V, p_store).reshape(len(sel_valid), D) if V > 0
         else np.zeros((0, D)))
    o = st("o", o)

    ms = mod[sel_valid]
    Es = E[ms]                                              # [R, 6, D]
    y = linear(o, blk["w_o"])
    x1 = st("x1", x[sel_valid] + Es[:, GATE_MSA] * y)
    x1n = rms_normalize(x1, dims.norm_eps) * np.asarray(blk["norm2_g"], dtype=work_dtype())
    h2 = st("h2", x1n * (1.0 + Es[:, SCALE_MLP]) + Es[:, SHIFT_MLP])
    a = st("act", swiglu(h2, blk["w_gate_up"], F))
    z = linear(a, blk["w_down"])
    x2_sel = st("out", x1 + Es[:, GATE_MLP] * z)

    out = np.zeros((len(rows), D), dtype=work_dtype())
    idx = np.nonzero(rows < V)[0]
    out[idx] = x2_sel
    if not want_intermediates:
        return out
    inter = dict(h=h[sel_valid], q=q.reshape(len(sel_valid), D), o=o, x1=x1, h2=h2, a=a,
                 k=k.reshape(V, D), v=v.reshape(V, D), rows_valid=sel_valid)
    return out, inter


# Intermediates a bf16 implementation stores as bf16: the operands of every bf16 matrix
# product (h, the q/k/v projections, q and k after norm + RoPE, the attention probabilities, the
# attention output, h2 and the SwiGLU output). The mid-block residual x1 is kept in fp32.
BF16_STORED = ("h", "qkv", "qk", "p", "o", "h2", "act")


def block_forward_bf16_storage(x, blk: dict, temb, dims: Dims, layout: Layout,
                               positions: Optional[np.ndarray] = None,
                               rows: Optional[np.ndarray] = None,
                               out_bf16: bool = True) -> np.ndarray:
    """DIAGNOSTIC, never the graded reference: ``block_forward`` with every intermediate in
    ``BF16_STORED`` (and, when out_bf16, the block output) rounded to bf16 where it is stored,
    all arithmetic between the roundings exact (float64).

    [P3 "Changes Made"]: the H3 DiT runs in BF16 with explicit BF16/FP32 boundaries; the
    matrix products take bf16 operands. The difference between this function and
    ``block_forward`` is the error that bf16 storage alone causes, with no arithmetic error
    of any kernel; it is what a tolerance on a bf16 implementation is derived from.
    """
    names = BF16_STORED + (("out",) if out_bf16 else ())

    def store(name, a):
        return bf16_round(a) if name in names else a

    return block_forward(x, blk, temb, dims, layout, positions, rows, store=store)


def attention_bf16_storage(q, k, v, n_valid: int, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """DIAGNOSTIC, never the graded reference: ``attention_valid`` (or ``attention_rows`` for
    the query rows ``rows``) with the probabilities stored as bf16 before they weight the
    values and are summed, and the output rounded to bf16."""
    if rows is None:
        return bf16_round(attention_valid(q, k, v, n_valid, p_store=bf16_round))
    q = np.asarray(q, dtype=F64)
    return bf16_round(attention_rows(q[rows], k, v, n_valid, p_store=bf16_round))


def stack_forward(x, blocks: Sequence[dict], temb, dims: Dims, layout: Layout,
                  positions: Optional[np.ndarray] = None) -> np.ndarray:
    """B blocks applied in order; the stack output is the velocity prediction."""
    for blk in blocks:
        x = block_forward(x, blk, temb, dims, layout, positions)
    return x


# Order of the two rows of the final AdaLN table of one modality.
HEAD_SHIFT, HEAD_SCALE = range(2)


def velocity_head(x, gain, ada, temb, w_out, bias, layout: Layout, eps: float) -> np.ndarray:
    """Velocity head after the block stack: v [L, C] from the stack output x [L, D].

    [P2 "Test Result"]: the model ends in a final AdaLN layer with a table of its own;
    [P1 §1]: the DiT predicts the flow-matching velocity of the latent. Reading: per modality m
    a two-row table E = A + T ([n_mod, 2, D]; row 0 shift, row 1 scale), the same RMSNorm with
    indexed modulation as the block, h = RMSNorm(x) * g * (1 + scale[m]) + shift[m], then a
    per-modality linear map with bias, v = h W[m]^T + b[m] (W [n_mod, C, D], b [n_mod, C]).
    Tail rows of v are 0.
    """
    mod = row_modality(layout)
    E = modulation_rows(ada, temb)
    h = norm_modulate(x, gain, E, mod, HEAD_SHIFT, HEAD_SCALE, eps)
    w_out = np.asarray(w_out, dtype=F64)
    b = np.zeros(w_out.shape[:2]) if bias is None else np.asarray(bias, dtype=F64)
    v = np.zeros((h.shape[0], w_out.shape[1]), dtype=F64)
    for m in range(w_out.shape[0]):
        sel = mod == m
        v[sel] = linear(h[sel], w_out[m]) + b[m]
    return v


def useful_block_flops(n_valid: int, hidden: int, ffn: int) -> float:
    """Useful matrix/attention FLOPs of one executed block over the valid tokens:
    8VD^2 (QKV + out) + 6VDF (gate/up + down) + 4V^2D (scores + values).

    [P2 "Purpose"]: only executed useful matrix/attention work counts toward
    throughput; padded rows and skipped blocks add nothing.
    """
    V, D, F = float(n_valid), float(hidden), float(ffn)
    return 8 * V * D * D + 6 * V * D * F + 4 * V * V * D


# ------------------------------------------------------------ cache ---------

def _policy_enabled(policy: CachePolicy) -> bool:
    mode = policy.mode.lower()
    if mode in ("conservative", "extrapolate"):
        mode = "velocity"   # the extrapolating mode reuses on exactly the same intervals
    if mode not in ("off", "velocity"):
        raise ValueError(f"unknown cache mode {policy.mode!r}")
    if policy.threshold is not None:
        raise NotImplementedError("threshold-based reuse is not defined on the pages")
    return mode == "velocity"


def cache_schedule(policy: CachePolicy, n_intervals: int) -> list:
    """Hit (True) / refresh (False) flag of every denoise interval.

    [P1 §3] MiniMaxH3DiTCacheConfig: reuse only inside [start_ratio, end_ratio)
    of the denoising progress, a forced refresh every ``refresh_interval`` steps,
    and at most ``max_consecutive_reuse`` reuses in a row. Progress of interval i
    is i / N. A step reuses when a velocity exists, the step is in the window and
    the current run of reuses is below min(max_consecutive_reuse,
    refresh_interval - 1); otherwise it refreshes and the run restarts.
    """
    if not _policy_enabled(policy):
        return [False] * n_intervals
    cap = min(policy.max_consecutive_reuse, policy.refresh_interval - 1)
    have_velocity = False
    run = 0
    flags = []
    for i in range(n_intervals):
        progress = i / n_intervals
        in_window = policy.start_ratio <= progress < policy.end_ratio
        if have_velocity and in_window and run < cap:
            flags.append(True)
            run += 1
        else:
            flags.append(False)
            have_velocity = True
            run = 0
    return flags


# ------------------------------------------------------------ Euler ---------

def euler_step(x, v, modality, dt_video: float, dt_audio: float) -> np.ndarray:
    """Flow-matching Euler update x + dt_m * v, with dt chosen by the row's modality.

    [P3 "Motivation", "Changes Made"]: independent video and audio schedulers,
    so each modality advances by its own sigma interval. Tail rows are left at 0.
    """
    x = np.asarray(x, dtype=F64)
    v = np.asarray(v, dtype=F64)
    out = np.zeros_like(x)
    vid = modality == VIDEO
    aud = modality == AUDIO
    out[vid] = x[vid] + F64(dt_video) * v[vid]
    out[aud] = x[aud] + F64(dt_audio) * v[aud]
    return out


def reused_velocity(i: int, v_last, r_last: int, v_prev, r_prev: Optional[int]) -> np.ndarray:
    """Velocity used on a reused interval i with first-order extrapolation.

    [P2 "Purpose", "Test Result"]: the pages' cache policies include an order-1 TaylorSeer
    predictor. Read at the velocity level: with refreshes r_prev < r_last before i, the
    velocity is continued linearly in the interval index,
    v_last + (i - r_last) / (r_last - r_prev) * (v_last - v_prev);
    with a single refresh so far it is plain reuse of v_last.
    """
    if v_prev is None or r_prev is None:
        return v_last
    lam = F64(i - r_last) / F64(r_last - r_prev)
    return v_last + lam * (v_last - v_prev)


def denoise_loop(x0, velocity: Callable[[int, np.ndarray], np.ndarray],
                 sigmas_video, sigmas_audio, modality, hits: Sequence[bool],
                 input_bf16: bool = True, extrapolate: bool = False):
    """Cached denoise loop over N = len(hits) intervals.

    [P1 §3] on a hit the previous DiT-predicted velocity (both modalities) is
    reused and the DiT call is skipped; on a refresh the DiT runs on the current
    latent, converted to bf16 as the DiT input (input_bf16=False: the latent
    itself, the FP32-residual runs of [P2 "Test Plan", "Test Result"]). Every
    interval then takes one Euler step x_{i+1} = x_i + (sigma_m[i+1] - sigma_m[i]) v
    with each modality on its own sigma schedule [P3 "Motivation"]; with
    extrapolate=True a reused interval takes reused_velocity() instead of the
    last refresh's velocity. Returns the final latent and the list of velocities
    the DiT produced (one per refresh).
    """
    x = np.asarray(x0, dtype=F64).copy()
    v = v_prev = None
    r = r_prev = None
    produced = []
    for i, hit in enumerate(hits):
        if hit:
            if v is None:
                raise ValueError("a hit before any refresh")
            u = reused_velocity(i, v, r, v_prev, r_prev) if extrapolate else v
        else:
            v_prev, r_prev = v, r
            v = np.asarray(velocity(i, bf16_round(x) if input_bf16 else x.copy()), dtype=F64)
            r = i
            produced.append(v)
            u = v
        dt_v = F64(sigmas_video[i + 1]) - F64(sigmas_video[i])
        dt_a = F64(sigmas_audio[i + 1]) - F64(sigmas_audio[i])
        x = euler_step(x, u, modality, dt_v, dt_a)
    return x, produced
