"""GPU parity of step_update and the cached denoise_loop against the oracle."""

import numpy as np
import pytest

from helpers import assert_close, check_block, oracle_block, oracle_dims, oracle_layout, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from audio_video_diffusion_dit_amd import _native, device
    return _native, device


def test_step_update_matches_oracle(env):
    import torch
    import oracle as O
    from audio_video_diffusion_dit_amd import inputs as I
    N, dev = env
    rng = np.random.default_rng(21)
    nv, na, L, D = 300, 77, 400, 256
    x = np.zeros((L, D), np.float32)
    x[: nv + na] = rng.standard_normal((nv + na, D), dtype=np.float32)
    x[nv + na:] = 5.0   # garbage in the tail is cleared
    v = I.bf16_bits(rng.standard_normal((L, D)))
    lay = N.make_layout(nv, na, L)
    say("step_update: 300 video + 77 audio rows of 400")
    dx, dv = dev.to_dev_f32(x), dev.to_dev_bf16(v)
    dxb = torch.empty((L, D), dtype=torch.bfloat16, device="cuda")
    N.step_update(dx, dv, dxb, lay, D, -0.125, -0.03125)
    torch.cuda.synchronize()
    got = dx.cpu().numpy()
    mod = O.row_modality(O.Layout(nv, na, L))
    ref = O.euler_step(np.where(mod[:, None] >= 0, x, 0), I.bf16_to_f32(v), mod, -0.125, -0.03125)
    # one fp32 fused multiply-add per element: within 1 ulp of the float64 result
    assert np.allclose(got, ref, rtol=2 ** -23, atol=0)
    assert np.all(got[nv + na:] == 0)
    assert np.array_equal(dev.bf16_bits_of(dxb), I.bf16_bits(got))


def _gpu_loop(env, case, mode, attn_mode=0):
    import torch
    N, dev = env
    wl = case.wl
    dims, lay = dev.dims_of(wl), dev.layout_of(wl)
    blocks = dev.upload_blocks(case.blocks)
    temb = dev.to_dev_f32(case.temb_steps)
    x = dev.to_dev_f32(case.x0)
    ws, _ = dev.workspace(dims, lay, len(blocks))
    pol = N.make_policy(mode)
    n = len(case.sigmas_video) - 1
    stats, hits = N.denoise_loop(dims, lay, [b.weights for b in blocks], n, case.sigmas_video,
                                 case.sigmas_audio, temb, pol, x, attn_mode, ws)
    torch.cuda.synchronize()
    return x.cpu().numpy(), stats, hits


def _small_loop_case(n_blocks=2, seed=0):
    from audio_video_diffusion_dit_amd import inputs as I
    return I.loop_case(I.WORKLOADS["block_small"], seed=seed, n_blocks=n_blocks, n_intervals=49)


@pytest.mark.parametrize("mode", ["off", "conservative"])
def test_loop_small_free_running(env, mode):
    """block_small dims, 2 blocks, 49 intervals: schedule bit-exact, final latent within the
    floating-point bar of the float64 oracle run."""
    import oracle as O
    N, dev = env
    case = _small_loop_case()
    wl = case.wl
    say(f"loop small ({mode}): 2 blocks, 49 intervals, V={wl.n_valid} L={wl.seq_pad}")
    got, stats, hits = _gpu_loop(env, case, mode)
    ref_hits = O.cache_schedule(O.CachePolicy(mode=mode), 49)
    assert hits == ref_hits
    assert stats.cache_hits == sum(ref_hits) and stats.dit_calls == 49 - sum(ref_hits)
    assert stats.executed_blocks == 2 * stats.dit_calls and stats.skipped_blocks == 2 * stats.cache_hits
    assert stats.useful_flops == stats.executed_blocks * O.useful_block_flops(wl.n_valid, wl.hidden, wl.ffn)
    if mode == "conservative":
        assert (stats.dit_calls, stats.cache_hits) == (34, 15)
    blocks = [oracle_block(b) for b in case.blocks]
    dims, lay = oracle_dims(wl), oracle_layout(wl)
    vel = lambda i, xb: O.stack_forward(xb, blocks, case.temb_steps[i], dims, lay)
    ref, _ = O.denoise_loop(case.x0, vel, case.sigmas_video, case.sigmas_audio,
                            O.row_modality(lay), ref_hits)
    V = wl.n_valid
    assert np.all(got[V:] == 0)
    assert_close(got[:V], ref[:V], f"final latent ({mode})")


def _composed(env, case, hits, check_steps=(), rows=None):
    """Re-run the loop from Python as dit_block_forward + step_update calls. At the intervals
    in check_steps every block is compared (sampled rows) with the oracle block fed the GPU's
    own block input."""
    import torch
    from audio_video_diffusion_dit_amd import inputs as I
    N, dev = env
    wl = case.wl
    dims, lay = dev.dims_of(wl), dev.layout_of(wl)
    blocks = dev.upload_blocks(case.blocks)
    ws, _ = dev.workspace(dims, lay, 0)
    temb = dev.to_dev_f32(case.temb_steps)
    L, D = wl.seq_pad, wl.hidden
    x = dev.to_dev_f32(case.x0)
    xb = dev.to_dev_bf16(I.bf16_bits(case.x0))
    bufs = [torch.empty_like(xb), torch.empty_like(xb)]
    v = torch.empty_like(xb)
    sv, sa = case.sigmas_video, case.sigmas_audio
    nb = len(blocks)
    for i, hit in enumerate(hits):
        if not hit:
            cur = xb
            for b in range(nb):
                out = v if b == nb - 1 else bufs[b & 1]
                N.dit_block_forward(dims, lay, blocks[b].weights, temb[i], cur, out, 0, ws)
                if i in check_steps:
                    torch.cuda.synchronize()
                    check_block(dev.bf16_values_of(out)[rows], dev.bf16_values_of(cur),
                                case.blocks[b], case.temb_steps[i], wl,
                                f"interval {i} block {b} (sampled rows, teacher-forced)", rows=rows)
                cur = out
        N.step_update(x, v, xb, lay, D, float(np.float32(sv[i + 1]) - np.float32(sv[i])),
                      float(np.float32(sa[i + 1]) - np.float32(sa[i])))
    torch.cuda.synchronize()
    return x.cpu().numpy()


def test_loop_equals_composed_calls_and_isolation(env):
    """The loop is bitwise the composition of dit_block_forward and step_update calls with
    the schedule's reuse; cached -> off -> cached runs repeat bitwise."""
    N, dev = env
    case = _small_loop_case(n_blocks=2, seed=3)
    say("loop small: loop vs composed calls, cached/off/cached isolation")
    a, _, hits = _gpu_loop(env, case, "conservative")
    off, _, _ = _gpu_loop(env, case, "off")
    c, _, _ = _gpu_loop(env, case, "conservative")
    assert np.array_equal(a, c), "repeated cached runs differ"
    assert not np.array_equal(a, off)
    comp = _composed(env, case, hits)
    assert np.array_equal(comp, a), "loop != composed block/step calls"


def test_loop_4blk_schedule_and_teacher_forced_blocks(env):
    """Full 4-block loop shape (D=1024, 4608 tokens, 49 intervals): 34 calls / 15 hits, the
    loop equals its composed calls bitwise, and at two refreshes each block matches the
    oracle on sampled rows when fed the GPU's own block input."""
    import oracle as O
    from audio_video_diffusion_dit_amd import inputs as I
    N, dev = env
    wl = I.WORKLOADS["loop_4blk"]
    case = I.loop_case(wl, seed=0)
    say(f"loop_4blk: conservative, V={wl.n_valid}, 4 blocks, 49 intervals")
    got, stats, hits = _gpu_loop(env, case, "conservative")
    assert (stats.dit_calls, stats.cache_hits) == (34, 15)
    assert hits == O.cache_schedule(O.CachePolicy(mode="conservative"), 49)
    assert np.all(np.isfinite(got)) and np.all(got[wl.n_valid:] == 0)
    V = wl.n_valid
    rng = np.random.default_rng(5)
    rows = np.sort(np.concatenate([rng.choice(V, 28, replace=False),
                                   [0, wl.n_video - 1, wl.n_video, V - 1]]))
    comp = _composed(env, case, hits, check_steps=(0, 11), rows=rows)
    assert np.array_equal(comp, got), "loop != composed block/step calls"


def _latent_compare(a, ref):
    a = np.asarray(a, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    d = a - ref
    mse = float(np.mean(d * d))
    peak = float(np.max(np.abs(ref)))
    return dict(cosine=float(a @ ref / (np.linalg.norm(a) * np.linalg.norm(ref))),
                rel_l2=float(np.linalg.norm(d) / np.linalg.norm(ref)),
                psnr_db=float(10.0 * np.log10(peak * peak / mse)) if mse > 0 else float("inf"))


def test_loop_4blk_free_running_vs_golden(env):
    """The 4-block, 4,608-token, 49-interval loop run free on the GPU, cache off and
    conservative, against the float64 oracle's final latents (sampled rows written by
    tests/golden/make_loop_4blk_golden.py, oracle only): the stated bar on the fp32 latent, the
    hit flags bit for bit. The conservative-vs-off comparison of the GPU's own final latents is
    reported beside the oracle's (report only)."""
    import json
    import os
    import oracle as O
    from audio_video_diffusion_dit_amd import inputs as I
    with open(os.path.join(os.path.dirname(__file__), "golden", "loop_4blk_final_rows.json")) as f:
        gold = json.load(f)
    wl = I.WORKLOADS["loop_4blk"]
    g = gold["workload"]
    assert (g["hidden"], g["heads"], g["ffn"], g["n_video"], g["n_audio"], g["n_blocks"],
            g["n_intervals"]) == (wl.hidden, wl.heads, wl.ffn, wl.n_video, wl.n_audio,
                                  wl.n_blocks, wl.n_intervals)
    case = I.loop_case(wl, seed=g["seed"])
    rows = np.asarray(gold["rows"])
    V = wl.n_valid
    finals = {}
    for mode, key in (("off", "final_off"), ("conservative", "final_conservative")):
        say(f"loop_4blk free running ({mode}): 4 blocks, 49 intervals, V={V}")
        got, stats, hits = _gpu_loop(env, case, mode)
        want_hits = gold["hits_conservative"] if mode == "conservative" else gold["hits_off"]
        assert [int(h) for h in hits] == want_hits
        assert hits == O.cache_schedule(O.CachePolicy(mode=mode), 49)
        assert np.all(got[V:] == 0)
        assert_close(got[rows], np.asarray(gold[key]), f"final latent, sampled rows ({mode})")
        finals[mode] = got[:V]
    gpu_q = _latent_compare(finals["conservative"], finals["off"])
    ref_q = gold["conservative_vs_off_all_valid_rows"]
    say(f"  conservative vs off, all valid rows: GPU cos {gpu_q['cosine']:.6f} rel-L2 "
        f"{gpu_q['rel_l2']:.4e} PSNR {gpu_q['psnr_db']:.2f} dB; oracle cos {ref_q['cosine']:.6f} "
        f"rel-L2 {ref_q['rel_l2']:.4e} PSNR {ref_q['psnr_db']:.2f} dB")
    assert np.isfinite(gpu_q["rel_l2"])
