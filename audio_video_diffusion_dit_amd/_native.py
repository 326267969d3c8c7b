"""ctypes binding of ``libavdit.so`` (the C-ABI declared in ``include/avdit.h``).

Argument marshalling only: torch tensors supply device memory and the stream, every step of
the computation runs in the library's HIP kernels. There is no fallback: if the library is
missing or fails to load, importing this module raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_uint8, c_void_p

import torch  # imported before the library so that a single HIP runtime is mapped

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libavdit.so")

DIT_OK, DIT_ERR_INVALID, DIT_ERR_UNSUPPORTED, DIT_ERR_WORKSPACE, DIT_ERR_DEVICE = 0, -1, -2, -3, -4
DIT_ATTN_VALID_ONLY, DIT_ATTN_FIXED_VALID = 0, 1
DIT_CACHE_OFF, DIT_CACHE_VELOCITY, DIT_CACHE_EXTRAPOLATE = 0, 1, 2

EXPORTED = ("dit_last_error", "dit_version", "dit_cache_schedule", "dit_workspace_size",
            "dit_block_forward", "dit_block_forward_f32", "dit_block_forward_batched",
            "dit_workspace_size_batched", "step_update", "denoise_loop", "denoise_loop_f32",
            "dit_attention_forward", "dit_head_workspace_size", "dit_velocity_head",
            "dit_velocity_head_f32", "dit_block_forward_noalloc")

# Bytes of the built-in scratch of dit_block_forward_noalloc (DIT_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 128 << 20


class DitDims(ctypes.Structure):
    _fields_ = [("hidden", c_int32), ("heads", c_int32), ("head_dim", c_int32), ("ffn", c_int32),
                ("n_mod", c_int32), ("norm_eps", c_float), ("qk_eps", c_float),
                ("rope_base", c_float)]


class DitLayout(ctypes.Structure):
    _fields_ = [("n_video", c_int32), ("n_audio", c_int32), ("seq_pad", c_int32),
                ("positions", c_void_p)]


class DitBlockWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("w_qkv", "w_o", "w_gate_up", "w_down", "norm1_g",
                                         "norm2_g", "q_g", "k_g", "ada")]


class DitHeadWeights(ctypes.Structure):
    _fields_ = [("norm_g", c_void_p), ("ada", c_void_p), ("w_out", c_void_p), ("bias", c_void_p),
                ("out_channels", c_int32)]


class DitCachePolicy(ctypes.Structure):
    _fields_ = [("mode", c_int32), ("start_ratio", c_double), ("end_ratio", c_double),
                ("refresh_interval", c_int32), ("max_consecutive_reuse", c_int32),
                ("threshold", c_double)]


class DitLoopStats(ctypes.Structure):
    _fields_ = [("dit_calls", c_int32), ("cache_hits", c_int32), ("executed_blocks", c_int64),
                ("skipped_blocks", c_int64), ("useful_flops", c_double),
                ("step_hit", POINTER(c_uint8))]


class DitWorkspaceMap(ctypes.Structure):
    _fields_ = [(n, c_size_t) for n in ("h", "qkv", "attn_out", "x1", "h2", "act", "x_bf16",
                                         "ping", "pong", "velocity", "velocity_prev", "total")] + \
        [("ffn_ld", c_int64)]


class AvditError(RuntimeError):
    def __init__(self, code: int, fn: str, msg: str):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m audio_video_diffusion_dit_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.dit_last_error.restype = c_char_p
    lib.dit_last_error.argtypes = []
    lib.dit_version.restype = c_char_p
    lib.dit_version.argtypes = []
    lib.dit_cache_schedule.restype = c_int32
    lib.dit_cache_schedule.argtypes = [POINTER(DitCachePolicy), c_int32, POINTER(c_uint8)]
    lib.dit_workspace_size.restype = c_size_t
    lib.dit_workspace_size.argtypes = [POINTER(DitDims), POINTER(DitLayout), c_int32,
                                       POINTER(DitWorkspaceMap)]
    lib.dit_block_forward.restype = c_int32
    lib.dit_block_forward.argtypes = [POINTER(DitDims), POINTER(DitLayout), POINTER(DitBlockWeights),
                                      c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_size_t,
                                      c_void_p]
    lib.dit_workspace_size_batched.restype = c_size_t
    lib.dit_workspace_size_batched.argtypes = [POINTER(DitDims), POINTER(DitLayout), c_int32,
                                               POINTER(DitWorkspaceMap)]
    lib.dit_block_forward_batched.restype = c_int32
    lib.dit_block_forward_batched.argtypes = [POINTER(DitDims), POINTER(DitLayout), c_int32,
                                              POINTER(DitBlockWeights), c_void_p, c_void_p,
                                              c_void_p, c_int32, c_void_p, c_size_t, c_void_p]
    lib.dit_block_forward_noalloc.restype = c_int32
    lib.dit_block_forward_noalloc.argtypes = [POINTER(DitDims), POINTER(DitLayout),
                                              POINTER(DitBlockWeights), c_void_p, c_void_p,
                                              c_void_p, c_int32, c_void_p]
    lib.dit_block_forward_f32.restype = c_int32
    lib.dit_block_forward_f32.argtypes = lib.dit_block_forward.argtypes
    lib.dit_head_workspace_size.restype = c_size_t
    lib.dit_head_workspace_size.argtypes = [POINTER(DitDims), POINTER(DitLayout), c_int32]
    lib.dit_velocity_head.restype = c_int32
    lib.dit_velocity_head.argtypes = [POINTER(DitDims), POINTER(DitLayout), POINTER(DitHeadWeights),
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.dit_velocity_head_f32.restype = c_int32
    lib.dit_velocity_head_f32.argtypes = lib.dit_velocity_head.argtypes
    lib.step_update.restype = c_int32
    lib.step_update.argtypes = [c_void_p, c_void_p, c_void_p, POINTER(DitLayout), c_int32, c_float,
                                c_float, c_void_p]
    lib.denoise_loop.restype = c_int32
    lib.denoise_loop.argtypes = [POINTER(DitDims), POINTER(DitLayout), POINTER(DitBlockWeights),
                                 c_int32, c_int32, POINTER(c_float), POINTER(c_float), c_void_p,
                                 POINTER(DitCachePolicy), c_void_p, c_int32, POINTER(DitLoopStats),
                                 c_void_p, c_size_t, c_void_p]
    lib.denoise_loop_f32.restype = c_int32
    lib.denoise_loop_f32.argtypes = lib.denoise_loop.argtypes
    lib.dit_attention_forward.restype = c_int32
    lib.dit_attention_forward.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                                          c_int32, c_int32, c_int64, c_int64, c_int64, c_int64,
                                          POINTER(c_int32), c_void_p, c_void_p, c_int32, c_void_p]
    return lib


lib = _load()


def last_error() -> str:
    return lib.dit_last_error().decode()


def _check(code: int, fn: str) -> None:
    if code != DIT_OK:
        raise AvditError(code, fn, last_error())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ------------------------------------------------------------------ structs -----------

def make_dims(hidden, heads, head_dim, ffn, norm_eps=1e-6, qk_eps=1e-6, rope_base=10000.0,
              n_mod=2) -> DitDims:
    return DitDims(hidden, heads, head_dim, ffn, n_mod, norm_eps, qk_eps, rope_base)


def make_layout(n_video, n_audio, seq_pad, positions=None) -> DitLayout:
    return DitLayout(n_video, n_audio, seq_pad, _ptr(positions))


def resolve_mode(mode: str = "off", quality: str | None = None) -> int:
    """'off' | 'velocity' | 'conservative' (alias of velocity) | 'extrapolate' (same schedule,
    first-order continued velocity on reused intervals); quality='high' disables the cache
    (1Cat-vLLM PR #584, "Purpose")."""
    if quality is not None and quality.lower() == "high":
        return DIT_CACHE_OFF
    m = mode.lower()
    if m == "off":
        return DIT_CACHE_OFF
    if m in ("velocity", "conservative"):
        return DIT_CACHE_VELOCITY
    if m == "extrapolate":
        return DIT_CACHE_EXTRAPOLATE
    raise ValueError(f"unknown cache mode {mode!r}")


def make_policy(mode="off", start_ratio=0.2, end_ratio=0.8, refresh_interval=2,
                max_consecutive_reuse=1, threshold=None, quality=None) -> DitCachePolicy:
    return DitCachePolicy(resolve_mode(mode, quality), start_ratio, end_ratio, refresh_interval,
                          max_consecutive_reuse, math.nan if threshold is None else float(threshold))


def make_block_weights(t: dict) -> DitBlockWeights:
    """t: dict of device tensors with the names of ``dit_block_weights``."""
    return DitBlockWeights(*[_ptr(t[n]) for n, _ in DitBlockWeights._fields_])


# ---------------------------------------------------------------- entry points --------

def dit_cache_schedule(policy: DitCachePolicy, n_intervals: int) -> list:
    buf = (c_uint8 * max(n_intervals, 1))()
    _check(lib.dit_cache_schedule(ctypes.byref(policy), n_intervals, buf), "dit_cache_schedule")
    return [bool(buf[i]) for i in range(n_intervals)]


def dit_workspace_size(dims: DitDims, layout: DitLayout, n_blocks: int = 0):
    m = DitWorkspaceMap()
    n = lib.dit_workspace_size(ctypes.byref(dims), ctypes.byref(layout), n_blocks, ctypes.byref(m))
    if n == 0:
        raise AvditError(DIT_ERR_INVALID, "dit_workspace_size", last_error())
    return n, m


def dit_block_forward(dims, layout, weights: DitBlockWeights, temb, x_in, x_out,
                      attn_mode=DIT_ATTN_VALID_ONLY, ws=None, ws_bytes=None, stream=None):
    """x_in, x_out: bf16 [seq_pad, hidden] (fp32 for dit_block_forward_f32)."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib.dit_block_forward(ctypes.byref(dims), ctypes.byref(layout), ctypes.byref(weights),
                                 _ptr(temb), _ptr(x_in), _ptr(x_out), attn_mode, _ptr(ws), ws_bytes,
                                 _stream(stream)), "dit_block_forward")


def dit_block_forward_noalloc(dims, layout, weights: DitBlockWeights, temb, x_in, x_out,
                              attn_mode=DIT_ATTN_VALID_ONLY, stream=None):
    """dit_block_forward on the library's built-in scratch: no workspace argument."""
    _check(lib.dit_block_forward_noalloc(ctypes.byref(dims), ctypes.byref(layout),
                                         ctypes.byref(weights), _ptr(temb), _ptr(x_in), _ptr(x_out),
                                         attn_mode, _stream(stream)), "dit_block_forward_noalloc")


def dit_workspace_size_batched(dims: DitDims, layouts):
    """layouts: list of DitLayout (one per request). Returns (bytes, DitWorkspaceMap)."""
    arr = (DitLayout * len(layouts))(*layouts)
    m = DitWorkspaceMap()
    n = lib.dit_workspace_size_batched(ctypes.byref(dims), arr, len(layouts), ctypes.byref(m))
    if n == 0:
        raise AvditError(DIT_ERR_INVALID, "dit_workspace_size_batched", last_error())
    return n, m


def dit_block_forward_batched(dims, layouts, weights: DitBlockWeights, temb, x_in, x_out,
                              attn_mode=DIT_ATTN_VALID_ONLY, ws=None, ws_bytes=None, stream=None):
    """layouts: list of DitLayout sharing seq_pad; temb: [batch, n_mod, 6, D] fp32;
    x_in, x_out: [batch * seq_pad, hidden] bf16."""
    arr = (DitLayout * len(layouts))(*layouts)
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib.dit_block_forward_batched(ctypes.byref(dims), arr, len(layouts), ctypes.byref(weights),
                                         _ptr(temb), _ptr(x_in), _ptr(x_out), attn_mode, _ptr(ws),
                                         ws_bytes, _stream(stream)), "dit_block_forward_batched")


def dit_block_forward_f32(dims, layout, weights: DitBlockWeights, temb, x_in, x_out,
                          attn_mode=DIT_ATTN_VALID_ONLY, ws=None, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(lib.dit_block_forward_f32(ctypes.byref(dims), ctypes.byref(layout), ctypes.byref(weights),
                                     _ptr(temb), _ptr(x_in), _ptr(x_out), attn_mode, _ptr(ws),
                                     ws_bytes, _stream(stream)), "dit_block_forward_f32")


def dit_head_workspace_size(dims, layout, out_channels) -> int:
    n = lib.dit_head_workspace_size(ctypes.byref(dims), ctypes.byref(layout), out_channels)
    if n == 0:
        raise AvditError(DIT_ERR_INVALID, "dit_head_workspace_size", last_error())
    return n


def make_head(norm_g, ada, w_out, bias, out_channels) -> DitHeadWeights:
    return DitHeadWeights(_ptr(norm_g), _ptr(ada), _ptr(w_out), _ptr(bias), out_channels)


def dit_velocity_head(dims, layout, head: DitHeadWeights, temb, x, v, ws=None, ws_bytes=None,
                      stream=None, x_f32=False):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    name = "dit_velocity_head_f32" if x_f32 else "dit_velocity_head"
    _check(getattr(lib, name)(ctypes.byref(dims), ctypes.byref(layout), ctypes.byref(head),
                              _ptr(temb), _ptr(x), _ptr(v), _ptr(ws), ws_bytes, _stream(stream)),
           name)


def step_update(x, v, x_bf16, layout, hidden, dt_video, dt_audio, stream=None):
    _check(lib.step_update(_ptr(x), _ptr(v), _ptr(x_bf16), ctypes.byref(layout), hidden,
                           dt_video, dt_audio, _stream(stream)), "step_update")


def denoise_loop(dims, layout, blocks, n_intervals, sigmas_video, sigmas_audio, temb_steps,
                 policy, x_latent, attn_mode=DIT_ATTN_VALID_ONLY, ws=None, ws_bytes=None,
                 stream=None, want_hits=True, residual_f32=False):
    """blocks: list of DitBlockWeights; sigmas: host float sequences of length N + 1.
    residual_f32 selects denoise_loop_f32 (fp32 residual stream).
    Returns the DitLoopStats and, with want_hits, the per-interval reuse flags."""
    arr = (DitBlockWeights * len(blocks))(*blocks)
    sv = (c_float * (n_intervals + 1))(*[float(s) for s in sigmas_video])
    sa = (c_float * (n_intervals + 1))(*[float(s) for s in sigmas_audio])
    stats = DitLoopStats()
    hit_buf = (c_uint8 * max(n_intervals, 1))() if want_hits else None
    if want_hits:
        stats.step_hit = ctypes.cast(hit_buf, POINTER(c_uint8))
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    fn = lib.denoise_loop_f32 if residual_f32 else lib.denoise_loop
    _check(fn(ctypes.byref(dims), ctypes.byref(layout), arr, len(blocks), n_intervals,
              sv, sa, _ptr(temb_steps), ctypes.byref(policy), _ptr(x_latent),
              attn_mode, ctypes.byref(stats), _ptr(ws), ws_bytes, _stream(stream)),
           "denoise_loop_f32" if residual_f32 else "denoise_loop")
    hits = [bool(hit_buf[i]) for i in range(n_intervals)] if want_hits else None
    return stats, hits


def dit_attention_forward(q, k, v, o, batch, seq_pad, heads, head_dim, batch_stride, row_stride,
                          o_batch_stride, o_row_stride, valid_lens, attn_mode=DIT_ATTN_VALID_ONLY,
                          stream=None, q_gain=None, k_gain=None):
    vl = (c_int32 * len(valid_lens))(*[int(x) for x in valid_lens])
    _check(lib.dit_attention_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), batch, seq_pad, heads,
                                     head_dim, batch_stride, row_stride, o_batch_stride,
                                     o_row_stride, vl, _ptr(q_gain), _ptr(k_gain), attn_mode,
                                     _stream(stream)),
           "dit_attention_forward")
