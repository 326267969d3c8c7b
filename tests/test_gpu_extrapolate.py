"""GPU parity of the extrapolating velocity-reuse mode (DIT_CACHE_EXTRAPOLATE) of denoise_loop and
denoise_loop_f32 against the oracle."""

import numpy as np
import pytest

from helpers import assert_close, oracle_block, oracle_dims, oracle_layout, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from audio_video_diffusion_dit_amd import _native, device
    return _native, device


def _loop(env, case, policy, residual_f32):
    import torch
    N, dev = env
    wl = case.wl
    dims, lay = dev.dims_of(wl), dev.layout_of(wl)
    blocks = dev.upload_blocks(case.blocks)
    x = dev.to_dev_f32(case.x0)
    ws, _ = dev.workspace(dims, lay, len(blocks))
    n = len(case.sigmas_video) - 1
    stats, hits = N.denoise_loop(dims, lay, [b.weights for b in blocks], n, case.sigmas_video,
                                 case.sigmas_audio, dev.to_dev_f32(case.temb_steps), policy, x, 0,
                                 ws, residual_f32=residual_f32)
    torch.cuda.synchronize()
    return x.cpu().numpy(), stats, hits


@pytest.mark.parametrize("residual_f32", [False, True])
def test_loop_extrapolate_matches_oracle(env, residual_f32):
    """2 blocks, 24 intervals, reuse window [0, 1) with refresh every 3rd interval and up to 2
    reuses in a row: the reused intervals continue the velocity with lambda = 1/3 and 2/3 from
    the last two refreshes. Schedule bit-exact; final latent within the floating-point bar of
    the float64 oracle; the result differs from plain reuse."""
    import oracle as O
    from audio_video_diffusion_dit_amd import inputs as I
    N, _ = env
    case = I.loop_case(I.WORKLOADS["block_small"], seed=8, n_blocks=2, n_intervals=24,
                       shift_video=2.0)
    wl = case.wl
    say(f"extrapolating loop, residual {'fp32' if residual_f32 else 'bf16'}: 2 blocks, 24 intervals")
    pol = N.make_policy("extrapolate", 0.0, 1.0, 3, 2)
    got, stats, hits = _loop(env, case, pol, residual_f32)
    ref_hits = O.cache_schedule(O.CachePolicy("extrapolate", 0.0, 1.0, 3, 2), 24)
    assert hits == ref_hits and stats.cache_hits == sum(ref_hits) == 16
    blocks = [oracle_block(b) for b in case.blocks]
    dims, lay = oracle_dims(wl), oracle_layout(wl)
    vel = lambda i, xb: O.stack_forward(xb, blocks, case.temb_steps[i], dims, lay)
    ref, _ = O.denoise_loop(case.x0, vel, case.sigmas_video, case.sigmas_audio, O.row_modality(lay),
                            ref_hits, input_bf16=not residual_f32, extrapolate=True)
    V = wl.n_valid
    assert np.all(got[V:] == 0)
    assert_close(got[:V], ref[:V], "final latent (extrapolated reuse)")
    plain, _, _ = _loop(env, case, N.make_policy("velocity", 0.0, 1.0, 3, 2), residual_f32)
    assert not np.array_equal(plain, got)


def test_extrapolate_without_reuse_is_the_uncached_loop(env):
    """With an empty reuse window the extrapolating mode runs every interval and equals the
    cache-off loop bit for bit."""
    from audio_video_diffusion_dit_amd import inputs as I
    N, _ = env
    case = I.loop_case(I.WORKLOADS["block_small"], seed=9, n_blocks=1, n_intervals=10)
    a, sa, _ = _loop(env, case, N.make_policy("extrapolate", 0.5, 0.5, 2, 1), False)
    b, sb, _ = _loop(env, case, N.make_policy("off"), False)
    assert sa.cache_hits == 0 and sb.cache_hits == 0
    assert np.array_equal(a, b)
