"""GPU parity of the fp32 residual-stream block and loop (dit_block_forward_f32,
denoise_loop_f32) and of loops on non-linear per-modality sigma schedules, against the oracle."""

import dataclasses

import numpy as np
import pytest

from helpers import assert_close, assert_kernel_close, check_block, oracle_block, oracle_dims, oracle_layout, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from audio_video_diffusion_dit_amd import _native, device
    return _native, device


ODD = dict(name="block_odd", hidden=256, heads=2, head_dim=128, ffn=300, n_video=100,
           n_audio=37, seq_pad=200)


def _case(name, seed=0):
    from audio_video_diffusion_dit_amd import inputs as I
    wl = I.Workload(**ODD) if name == "block_odd" else I.WORKLOADS[name]
    return I.block_case(wl, seed=seed, n_blocks=1)


def _x_f32(wl, seed):
    """fp32 residual-stream input: N(0, 1) fp32 on the valid rows (not bf16 values), garbage in
    the tail."""
    rng = np.random.default_rng(seed)
    x = np.full((wl.seq_pad, wl.hidden), 7.5, np.float32)
    x[: wl.n_valid] = rng.standard_normal((wl.n_valid, wl.hidden), dtype=np.float32)
    return x


def _gpu_block_f32(env, case, x, attn_mode=0, blk_params=None):
    import torch
    N, dev = env
    wl = case.wl
    dims, lay = dev.dims_of(wl), dev.layout_of(wl)
    blk = dev.upload_block(blk_params or case.blocks[0])
    dx = dev.to_dev_f32(x)
    out = torch.full_like(dx, float("nan"))
    ws, m = dev.workspace(dims, lay, 0)
    N.dit_block_forward_f32(dims, lay, blk.weights, dev.to_dev_f32(case.temb), dx, out, attn_mode, ws)
    torch.cuda.synchronize()
    x1 = ws[m.x1:m.x1 + wl.seq_pad * wl.hidden * 4].view(torch.float32).view(wl.seq_pad, wl.hidden)
    return out.cpu().numpy(), x1.cpu().numpy()


@pytest.mark.parametrize("name", ["block_small", "block_odd"])
def test_block_f32_end_to_end(env, name):
    """fp32 in, fp32 out: within the floating-point bar of the float64 block on the same fp32
    input; exact zero tail whatever the input tail holds; the mid-block residual x1 matches the
    oracle's; fixed-valid and valid-only agree bit for bit."""
    import oracle as O
    case = _case(name)
    wl = case.wl
    V = wl.n_valid
    x = _x_f32(wl, 11)
    say(f"fp32-residual block {name}: D={wl.hidden} H={wl.heads}x{wl.head_dim} F={wl.ffn} V={V} L={wl.seq_pad}")
    got, x1 = _gpu_block_f32(env, case, x)
    blk = oracle_block(case.blocks[0])
    dims, lay = oracle_dims(wl), oracle_layout(wl)
    xv = np.where(np.arange(wl.seq_pad)[:, None] < V, x, 0).astype(np.float64)
    ref = O.block_forward(xv, blk, case.temb, dims, lay)
    assert np.all(got[V:] == 0) and np.all(x1[V:] == 0)
    check_block(got, xv, case.blocks[0], case.temb, wl, f"{name} fp32-residual block output",
                out_bf16=False)
    # x1 = x + gate_msa * (o Wo^T) from the oracle's own attention output: compare loosely (the
    # GPU's o carries bf16 roundings), as a per-kernel intermediate
    mod = O.row_modality(lay)
    E = O.modulation_rows(blk["ada"], case.temb)
    h = O.norm_modulate(xv, blk["norm1_g"], E, mod, O.SHIFT_MSA, O.SCALE_MSA, dims.norm_eps)
    qkv = O.linear(h[:V], blk["w_qkv"])
    D, H, Dh = wl.hidden, wl.heads, wl.head_dim
    pos = np.arange(V, dtype=np.float64)
    q = O.rope_neox(O.qk_rms_norm(qkv[:, :D].reshape(V, H, Dh), blk["q_g"], dims.qk_eps), pos, dims.rope_base)
    k = O.rope_neox(O.qk_rms_norm(qkv[:, D:2 * D].reshape(V, H, Dh), blk["k_g"], dims.qk_eps), pos, dims.rope_base)
    o = O.attention_valid(q, k, qkv[:, 2 * D:].reshape(V, H, Dh), V).reshape(V, D)
    x1_ref = xv[:V] + E[mod[:V], O.GATE_MSA] * O.linear(o, blk["w_o"])
    assert_kernel_close(x1[:V], x1_ref, "fp32-residual mid-block x1")
    got_fv, _ = _gpu_block_f32(env, case, x, attn_mode=1)
    assert np.array_equal(got, got_fv), "fixed-valid and valid-only must agree bit for bit"


def test_block_f32_zero_gates_identity(env):
    """With gate_msa = gate_mlp = 0 the fp32 block passes its input through bit for bit."""
    case = _case("block_small", seed=2)
    wl = case.wl
    bp = case.blocks[0]
    ada = bp.ada.copy()
    ada[:, 2] = 0.0
    ada[:, 5] = 0.0
    temb = case.temb.copy()
    temb[:, 2] = 0.0
    temb[:, 5] = 0.0
    case = dataclasses.replace(case, temb=temb)
    x = _x_f32(wl, 3)
    got, _ = _gpu_block_f32(env, case, x, blk_params=dataclasses.replace(bp, ada=ada))
    V = wl.n_valid
    assert np.array_equal(got[:V], x[:V]) and np.all(got[V:] == 0)


def test_block_f32_h3_sampled_rows(env):
    """H3-scale fp32-residual block (the large-tile GEMM path's fp32-in / fp32-out epilogue):
    sampled rows against the float64 oracle (keys/values for every row)."""
    import oracle as O
    case = _case("block_h3")
    wl = case.wl
    V = wl.n_valid
    x = _x_f32(wl, 5)
    say(f"fp32-residual block_h3: V={V} L={wl.seq_pad}")
    got, _ = _gpu_block_f32(env, case, x)
    rows = np.sort(np.concatenate([np.random.default_rng(4).choice(V, 40, replace=False),
                                   [0, wl.n_video - 1, wl.n_video, V - 1]]))
    xv = np.where(np.arange(wl.seq_pad)[:, None] < V, x, 0).astype(np.float64)
    assert np.all(got[V:] == 0)
    check_block(got[rows], xv, case.blocks[0], case.temb, wl,
                "block_h3 fp32-residual output (sampled rows)", rows=rows, out_bf16=False)


def _loop(env, case, mode, residual_f32):
    import torch
    N, dev = env
    wl = case.wl
    dims, lay = dev.dims_of(wl), dev.layout_of(wl)
    blocks = dev.upload_blocks(case.blocks)
    x = dev.to_dev_f32(case.x0)
    ws, _ = dev.workspace(dims, lay, len(blocks))
    n = len(case.sigmas_video) - 1
    stats, hits = N.denoise_loop(dims, lay, [b.weights for b in blocks], n, case.sigmas_video,
                                 case.sigmas_audio, dev.to_dev_f32(case.temb_steps),
                                 N.make_policy(mode), x, 0, ws, residual_f32=residual_f32)
    torch.cuda.synchronize()
    return x.cpu().numpy(), stats, hits


@pytest.mark.parametrize("residual_f32", [False, True])
def test_loop_nonlinear_per_modality_schedules(env, residual_f32):
    """2 blocks, 24 intervals, conservative reuse, video on a time-shifted schedule (shift 3) and
    audio on another (shift 0.5): the bf16-residual loop and the fp32-residual loop each match
    the float64 oracle loop (DiT input rounded to bf16, or the latent itself)."""
    import oracle as O
    from audio_video_diffusion_dit_amd import inputs as I
    case = I.loop_case(I.WORKLOADS["block_small"], seed=4, n_blocks=2, n_intervals=24,
                       shift_video=3.0, shift_audio=0.5)
    wl = case.wl
    assert not np.allclose(case.sigmas_video, case.sigmas_audio)
    say(f"loop, shifted schedules, residual {'fp32' if residual_f32 else 'bf16'}: 2 blocks, 24 intervals")
    got, stats, hits = _loop(env, case, "conservative", residual_f32)
    ref_hits = O.cache_schedule(O.CachePolicy(mode="conservative"), 24)
    assert hits == ref_hits and stats.cache_hits == sum(ref_hits)
    blocks = [oracle_block(b) for b in case.blocks]
    dims, lay = oracle_dims(wl), oracle_layout(wl)
    vel = lambda i, xb: O.stack_forward(xb, blocks, case.temb_steps[i], dims, lay)
    ref, _ = O.denoise_loop(case.x0, vel, case.sigmas_video, case.sigmas_audio,
                            O.row_modality(lay), ref_hits, input_bf16=not residual_f32)
    V = wl.n_valid
    assert np.all(got[V:] == 0)
    assert_close(got[:V], ref[:V], "final latent")


def test_loop_f32_is_closer_to_the_unrounded_oracle(env):
    """The fp32-residual loop tracks the unrounded float64 loop more closely than the bf16 loop
    does (the point of the fp32 residual stream)."""
    import oracle as O
    from audio_video_diffusion_dit_amd import inputs as I
    from helpers import close_stats
    case = I.loop_case(I.WORKLOADS["block_small"], seed=6, n_blocks=2, n_intervals=12)
    wl = case.wl
    blocks = [oracle_block(b) for b in case.blocks]
    dims, lay = oracle_dims(wl), oracle_layout(wl)
    hits = O.cache_schedule(O.CachePolicy(mode="off"), 12)
    vel = lambda i, xb: O.stack_forward(xb, blocks, case.temb_steps[i], dims, lay)
    ref, _ = O.denoise_loop(case.x0, vel, case.sigmas_video, case.sigmas_audio,
                            O.row_modality(lay), hits, input_bf16=False)
    V = wl.n_valid
    e32 = close_stats(_loop(env, case, "off", True)[0][:V], ref[:V])[0]
    e16 = close_stats(_loop(env, case, "off", False)[0][:V], ref[:V])[0]
    say(f"  max|err| vs unrounded oracle: fp32 residual {e32:.3e}, bf16 residual {e16:.3e}")
    assert e32 < e16
