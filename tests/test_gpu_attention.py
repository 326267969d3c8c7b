"""GPU parity of the valid-only / fixed-valid attention kernel against the oracle."""

import numpy as np
import pytest

from helpers import assert_close, check_attention, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def N():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from audio_video_diffusion_dit_amd import _native
    return _native


def _run(N, q, k, v, valid, mode, o_fill=None, gains=None):
    import torch
    from audio_video_diffusion_dit_amd.device import to_dev_bf16, to_dev_f32, bf16_bits_of
    B, L, H, Dh = q.shape
    dq, dk, dv = (to_dev_bf16(t) for t in (q, k, v))
    do = torch.empty((B, L, H, Dh), dtype=torch.bfloat16, device="cuda")
    if o_fill is not None:
        do.view(torch.int16).fill_(o_fill)
    gq, gk = (None, None) if gains is None else (to_dev_f32(gains[0]), to_dev_f32(gains[1]))
    N.dit_attention_forward(dq, dk, dv, do, B, L, H, Dh, L * H * Dh, H * Dh, L * H * Dh, H * Dh,
                            valid, mode, q_gain=gq, k_gain=gk)
    torch.cuda.synchronize()
    return bf16_bits_of(do)


def _oracle(q, k, v, valid):
    import oracle as O
    from audio_video_diffusion_dit_amd.inputs import bf16_to_f32
    out = np.zeros(q.shape)
    for b, n in enumerate(valid):
        out[b] = O.attention_valid(bf16_to_f32(q[b]), bf16_to_f32(k[b]), bf16_to_f32(v[b]), n)
    return out


@pytest.mark.parametrize("head_dim", [64, 128])
def test_attention_ragged_small(N, head_dim):
    from audio_video_diffusion_dit_amd.inputs import attention_case, bf16_to_f32
    valid = (1, 63, 130, 300, 0)
    L, H = 300, 2
    say(f"attention ragged small: L={L} H={H} Dh={head_dim} valid={valid}")
    q, k, v = attention_case(len(valid), L, H, head_dim, valid, seed=1)
    got_vo = _run(N, q, k, v, valid, N.DIT_ATTN_VALID_ONLY, o_fill=0x7FC0)
    got_fv = _run(N, q, k, v, valid, N.DIT_ATTN_FIXED_VALID, o_fill=0x7FC0)
    assert np.array_equal(got_vo, got_fv), "fixed-valid and valid-only must agree bit for bit"
    for b, n in enumerate(valid):
        assert np.all(got_vo[b, n:] == 0), f"request {b}: tail rows must be exactly 0"
        if n:
            check_attention(bf16_to_f32(got_vo[b, :n]), bf16_to_f32(q[b]), bf16_to_f32(k[b]),
                            bf16_to_f32(v[b]), n, f"req {b} (valid {n})")


def test_attention_tail_garbage_is_ignored(N):
    from audio_video_diffusion_dit_amd.inputs import attention_case
    valid = (77, 200)
    L, H, Dh = 256, 2, 128
    say(f"attention tail garbage: L={L} valid={valid}")
    q, k, v = attention_case(2, L, H, Dh, valid, seed=2)
    base = _run(N, q, k, v, valid, N.DIT_ATTN_VALID_ONLY)
    qg, kg, vg = q.copy(), k.copy(), v.copy()
    for b, n in enumerate(valid):
        qg[b, n:] = 0x7FC0   # NaN
        kg[b, n:] = 0x7F80   # +inf
        vg[b, n:] = 0xFFC0   # NaN
    for mode in (N.DIT_ATTN_VALID_ONLY, N.DIT_ATTN_FIXED_VALID):
        got = _run(N, qg, kg, vg, valid, mode)
        assert np.array_equal(got, base), f"mode {mode}: tail inputs leaked into the output"


def test_attention_special_cases(N):
    from audio_video_diffusion_dit_amd.inputs import bf16_bits, bf16_to_f32
    L, H, Dh = 128, 1, 128
    rng = np.random.default_rng(3)
    q = bf16_bits(rng.standard_normal((1, L, H, Dh)))
    k = bf16_bits(np.repeat(rng.standard_normal((1, 1, H, Dh)), L, axis=1))
    v = bf16_bits(rng.standard_normal((1, L, H, Dh)))
    say("attention identical keys -> mean of values")
    got = bf16_to_f32(_run(N, q, k, v, (100,), N.DIT_ATTN_VALID_ONLY))
    mean = bf16_to_f32(v)[0, :100].astype(np.float64).mean(axis=0)
    assert_close(got[0, :100], np.broadcast_to(mean, (100, H, Dh)), "identical keys")
    say("attention one valid key -> its value")
    got = _run(N, q, k, v, (1,), N.DIT_ATTN_VALID_ONLY)
    assert np.array_equal(got[0, 0], v[0, 0])


def test_attention_deterministic(N):
    from audio_video_diffusion_dit_amd.inputs import attention_case
    valid = (1000, 517)
    q, k, v = attention_case(2, 1024, 4, 128, valid, seed=4)
    say("attention run-to-run determinism")
    a = _run(N, q, k, v, valid, N.DIT_ATTN_VALID_ONLY)
    b = _run(N, q, k, v, valid, N.DIT_ATTN_VALID_ONLY)
    assert np.array_equal(a, b)


def test_attention_ragged_batch_full_size(N):
    """4 packed requests of 16 heads x 128 in 8192-token buffers with valid lengths
    {3000, 5100, 7777, 8192}: both modes bitwise equal, tails exactly zero, and 24 sampled
    query rows per request (including each request's first and last valid row) against the
    oracle."""
    import oracle as O
    from audio_video_diffusion_dit_amd.inputs import ATTN_RAGGED, attention_case, bf16_to_f32
    cfg = ATTN_RAGGED
    B, L, H, Dh, valid = cfg["batch"], cfg["seq_pad"], cfg["heads"], cfg["head_dim"], cfg["valid"]
    say(f"attention ragged batch: B={B} L={L} H={H}x{Dh} valid={valid}")
    q, k, v = attention_case(B, L, H, Dh, valid, seed=0)
    vo = _run(N, q, k, v, valid, N.DIT_ATTN_VALID_ONLY, o_fill=0x7FC0)
    fv = _run(N, q, k, v, valid, N.DIT_ATTN_FIXED_VALID, o_fill=0x7FC0)
    assert np.array_equal(vo, fv), "fixed-valid and valid-only must agree bit for bit"
    rng = np.random.default_rng(9)
    for b, n in enumerate(valid):
        assert np.all(vo[b, n:] == 0)
        rows = np.sort(np.concatenate([rng.choice(n, 22, replace=False), [0, n - 1]]))
        check_attention(bf16_to_f32(vo[b, rows]), bf16_to_f32(q[b]), bf16_to_f32(k[b]),
                        bf16_to_f32(v[b]), n, f"request {b} (valid {n}), sampled rows", rows=rows)


@pytest.mark.parametrize("head_dim,gain", [(64, 1.0), (128, 1.0), (128, 1.9), (128, 6.0)])
def test_attention_with_qk_norm_gains(N, head_dim, gain):
    """q and k that came out of the per-head Q/K RMSNorm with gains gq, gk have logits bounded by
    max|gq| max|gk| sqrt(Dh). Given the gains, the kernel needs no running row maximum when that
    bound is small: gain 1 (bound 11.7 or 16.6 in log2 units) takes the probabilities unshifted,
    gain 1.9 (bound 59.9) shifts them by the bound, and gain 6 keeps the online maximum. Every
    case matches the oracle; fixed-valid and valid-only still agree bit for bit, and garbage in
    the tail rows still leaves the outputs bitwise unchanged."""
    import oracle as O
    from audio_video_diffusion_dit_amd.inputs import attention_case, bf16_bits, bf16_to_f32
    valid = (1, 77, 300, 513)
    L, H = 520, 3
    say(f"attention with Q/K norm gains: L={L} H={H} Dh={head_dim} gain={gain} valid={valid}")
    q, k, v = attention_case(len(valid), L, H, head_dim, valid, seed=5)
    ramp = np.linspace(0.3, 1.0, head_dim)
    gq = (gain * ramp * np.where(np.arange(head_dim) % 4 == 1, -1.0, 1.0)).astype(np.float32)
    gk = (gain * ramp[::-1]).astype(np.float32)

    def qk_norm(t, g):
        x = bf16_to_f32(t).astype(np.float64)
        y = O.qk_rms_norm(x.reshape(-1, H, head_dim), g.astype(np.float64), 1e-6).reshape(x.shape)
        return bf16_bits(y.astype(np.float32))

    qn, kn = qk_norm(q, gq), qk_norm(k, gk)
    got = _run(N, qn, kn, v, valid, N.DIT_ATTN_VALID_ONLY, o_fill=0x7FC0, gains=(gq, gk))
    got_fv = _run(N, qn, kn, v, valid, N.DIT_ATTN_FIXED_VALID, o_fill=0x7FC0, gains=(gq, gk))
    assert np.array_equal(got, got_fv), "fixed-valid and valid-only must agree bit for bit"
    qg, kg, vg = qn.copy(), kn.copy(), v.copy()
    for b, n in enumerate(valid):
        qg[b, n:], kg[b, n:], vg[b, n:] = 0x7FC0, 0xFF80, 0x7F80  # NaN, -inf, +inf in the tail
    got_g = _run(N, qg, kg, vg, valid, N.DIT_ATTN_VALID_ONLY, gains=(gq, gk))
    assert np.array_equal(got, got_g), "tail contents must not change the outputs"
    for b, n in enumerate(valid):
        assert np.all(got[b, n:] == 0)
        check_attention(bf16_to_f32(got[b, :n]), bf16_to_f32(qn[b]), bf16_to_f32(kn[b]),
                        bf16_to_f32(v[b]), n, f"req {b} (valid {n}, gain {gain})")
