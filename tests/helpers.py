"""Shared test utilities: tolerance checks and adapters from the seeded workloads to the oracle."""

from __future__ import annotations

import math
import sys

import numpy as np

import oracle as O
from audio_video_diffusion_dit_amd.inputs import Workload, bf16_to_f32

# Floating-point parity bar for bf16 outputs: per-tensor max |err| <= 2e-2 * RMS(reference)
# and cosine similarity >= 0.9995, over the valid rows.
REL_MAX_ERR = 2e-2
MIN_COSINE = 0.9995


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def close_stats(got, ref):
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    rms = float(math.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    den = float(np.linalg.norm(got) * np.linalg.norm(ref))
    cos = float(np.dot(got, ref) / den) if den > 0 else (1.0 if err == 0 else 0.0)
    return err, rms, cos


def bf16_floor(ref) -> float:
    """max |bf16(ref) - ref|: the error of the exact result correctly rounded to bf16 (reported
    only)."""
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(O.bf16_round(ref) - ref))) if ref.size else 0.0


def bf16_ulp(a: float) -> float:
    """Spacing of the bf16 values at magnitude a (8 significant bits): 2^(floor(log2 a) - 7)."""
    if not a > 0:
        return 0.0
    return math.ldexp(1.0, math.frexp(a)[1] - 8)


def assert_close(got, ref, name: str, rel=REL_MAX_ERR, min_cos=MIN_COSINE):
    """The stated floating-point bar, with no allowance: max |err| <= 2e-2 * RMS(ref) and
    cosine >= 0.9995 (loop latents, velocities, any output not judged through the storage
    diagnostic)."""
    err, rms, cos = close_stats(got, ref)
    say(f"  {name}: max|err| {err:.3e}  RMS(ref) {rms:.3e}  ratio {err / max(rms, 1e-30):.2e}  "
        f"bound 2e-2*RMS  cos {cos:.7f}")
    assert np.all(np.isfinite(np.asarray(got))), f"{name}: non-finite values"
    assert err <= rel * rms, f"{name}: max|err| {err:.3e} > 2e-2*RMS {rel * rms:.3e}"
    assert cos >= min_cos, f"{name}: cosine {cos:.7f} < {min_cos}"
    return err / max(rms, 1e-30), cos


def assert_storage_close(got, exact, diag, name: str, rel=REL_MAX_ERR, min_cos=MIN_COSINE):
    """Parity of an output computed through bf16-stored intermediates, judged with the oracle's
    bf16-storage diagnostic ``diag`` (the same function with each stored intermediate rounded to
    bf16 and exact arithmetic in between) beside the exact oracle ``exact``. Rules, fixed before
    any GPU run:

      (a) max |got - diag| <= U, U = one bf16 ulp at max |diag|: the kernels differ from the
          storage model only by fp32 arithmetic, which moves a stored value across a rounding
          midpoint now and then (one ulp of that value) and changes the rest far below an ulp.
      (b) max |got - exact| <= max(2e-2 RMS(exact), E_s + U), E_s = max |diag - exact| (the
          error bf16 storage alone causes, computed by the oracle), and cosine >= 0.9995. When
          (a) holds, (b) follows by the triangle inequality; it is the graded bar, widened only
          by what the storage diagnostic accounts for."""
    got = np.asarray(got, dtype=np.float64)
    exact = np.asarray(exact, dtype=np.float64)
    diag = np.asarray(diag, dtype=np.float64)
    err, rms, cos = close_stats(got, exact)
    e_s = float(np.max(np.abs(diag - exact))) if exact.size else 0.0
    d_gd = float(np.max(np.abs(got - diag))) if exact.size else 0.0
    u = bf16_ulp(float(np.max(np.abs(diag)))) if exact.size else 0.0
    bound = max(rel * rms, e_s + u)
    which = "2e-2*RMS" if bound == rel * rms else "E_s+U"
    r = max(rms, 1e-30)
    same = float(np.mean(got == diag)) if exact.size else 1.0
    say(f"  {name}: max|err| {err / r:.2e}*RMS (RMS {rms:.3e})  storage E_s {e_s / r:.2e}*RMS  "
        f"U {u / r:.2e}*RMS  max|got-diag| {d_gd / max(u, 1e-30):.2f} U  equal to diag {same:.4f}  "
        f"bound {which} {bound / r:.2e}*RMS  bf16 floor {bf16_floor(exact) / r:.2e}*RMS  "
        f"cos {cos:.7f}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert d_gd <= u, f"{name}: max|got - diag| {d_gd:.3e} > one bf16 ulp {u:.3e}"
    assert err <= bound, f"{name}: max|err| {err:.3e} > bound {bound:.3e} ({which})"
    assert cos >= min_cos, f"{name}: cosine {cos:.7f} < {min_cos}"
    return err / r, cos


def check_block(got, x, bp, temb, wl, name: str, rows=None, positions=None, out_bf16=True,
                layout=None):
    """A block output (all rows of the layout, or the rows ``rows``) against the exact oracle
    and the bf16-storage diagnostic, valid rows only; returns the exact reference rows."""
    blk = oracle_block(bp)
    dims = oracle_dims(wl)
    lay = oracle_layout(wl) if layout is None else layout
    x = np.asarray(x, dtype=np.float64)
    exact = O.block_forward(x, blk, temb, dims, lay, positions=positions, rows=rows)
    diag = O.block_forward_bf16_storage(x, blk, temb, dims, lay, positions=positions, rows=rows,
                                        out_bf16=out_bf16)
    sel = np.arange(lay.seq_pad) if rows is None else np.asarray(rows)
    keep = sel < lay.n_valid
    assert_storage_close(np.asarray(got)[keep], exact[keep], diag[keep], name)
    return exact


def check_attention(got, q, k, v, n_valid: int, name: str, rows=None):
    """An attention output (bf16, rows < n_valid, or the query rows ``rows``) against the exact
    oracle and the storage diagnostic (probabilities and output stored as bf16)."""
    if rows is None:
        exact = O.attention_valid(q, k, v, n_valid)[:n_valid]
        diag = O.attention_bf16_storage(q, k, v, n_valid)[:n_valid]
    else:
        exact = O.attention_rows(np.asarray(q, dtype=np.float64)[rows], k, v, n_valid)
        diag = O.attention_bf16_storage(q, k, v, n_valid, rows=rows)
    assert_storage_close(got, exact, diag, name)


# Per-kernel bar for an intermediate stored in bf16 and fed the GPU's own input: a bf16 store
# rounds by at most 2^-8 of the value's magnitude (8 significant bits); a kernel output carries
# at most two such roundings (its bf16 input and its own output) plus fp32 arithmetic, so
# max |err| <= 2^-6 * max |ref| leaves a factor-two margin, and the cosine must be >= 0.9999.
KERNEL_REL_MAX = 2.0 ** -6
KERNEL_MIN_COSINE = 0.9999


def assert_kernel_close(got, ref, name: str):
    ref = np.asarray(ref, dtype=np.float64)
    amax = float(np.max(np.abs(ref))) if ref.size else 0.0
    err, rms, cos = close_stats(got, ref)
    say(f"  {name}: max|err| {err:.3e}  max|ref| {amax:.3e}  ratio {err / max(amax, 1e-30):.2e}  "
        f"err/RMS {err / max(rms, 1e-30):.2e}  cos {cos:.7f}")
    assert np.all(np.isfinite(np.asarray(got))), f"{name}: non-finite values"
    assert err <= KERNEL_REL_MAX * amax, f"{name}: max|err| {err:.3e} > 2^-6 * max|ref| {amax:.3e}"
    assert cos >= KERNEL_MIN_COSINE, f"{name}: cosine {cos:.7f} < {KERNEL_MIN_COSINE}"


def oracle_dims(wl: Workload) -> O.Dims:
    return O.Dims(wl.hidden, wl.heads, wl.head_dim, wl.ffn, wl.norm_eps, wl.qk_eps, wl.rope_base)


def oracle_layout(wl: Workload) -> O.Layout:
    return O.Layout(wl.n_video, wl.n_audio, wl.seq_pad)


def oracle_block(bp) -> dict:
    return {k: np.asarray(v, dtype=np.float64) for k, v in bp.as_float().items()}


def x_values(bits) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)
