"""GPU parity of dit_block_forward (and each of its kernels) against the oracle."""

import dataclasses

import numpy as np
import pytest

from helpers import (assert_kernel_close, check_block, oracle_block, oracle_dims, oracle_layout,
                     say, x_values)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from audio_video_diffusion_dit_amd import _native, device
    return _native, device


def _gpu_block(env, case, attn_mode=0, x_bits=None, ws_fill=None):
    import torch
    N, dev = env
    wl = case.wl
    dims, lay = dev.dims_of(wl), dev.layout_of(wl)
    blk = dev.upload_block(case.blocks[0])
    temb = dev.to_dev_f32(case.temb)
    x = dev.to_dev_bf16(case.x if x_bits is None else x_bits)
    out = torch.empty_like(x)
    out.view(torch.int16).fill_(0x7FC0)
    ws, m = dev.workspace(dims, lay, 0)
    if ws_fill is not None:
        ws.fill_(ws_fill)
    N.dit_block_forward(dims, lay, blk.weights, temb, x, out, attn_mode, ws)
    torch.cuda.synchronize()
    return out, ws, m


def _inter(dev, ws, m, wl):
    import torch
    L, D = wl.seq_pad, wl.hidden
    g = lambda off, cols: dev.bf16_values_of(dev.ws_view_bf16(ws, off, L, cols)).astype(np.float64)
    act = g(m.act, int(m.ffn_ld))[:, : wl.ffn]
    x1 = ws[m.x1:m.x1 + L * D * 4].view(torch.float32).view(L, D).cpu().numpy().astype(np.float64)
    return dict(h=g(m.h, D), qkv=g(m.qkv, 3 * D), o=g(m.attn_out, D), x1=x1,
                h2=g(m.h2, D), act=act)


ODD = dict(name="block_odd", hidden=256, heads=2, head_dim=128, ffn=300, n_video=100,
           n_audio=37, seq_pad=200)
# Large enough for the 256 x 256 direct-to-LDS tiles on the QKV and gate/up projections, with a
# partial last feature tile in each (QKV: 3 x 1088 = 12.75 tiles of 256; SwiGLU: 2880 outputs =
# 22.5 tiles of 128) and in the out- and down-projections on the 128 x 128 tiles (1088 = 8.5 x 128).
TILES = dict(name="block_tiles", hidden=1088, heads=17, head_dim=64, ffn=2880, n_video=3000,
             n_audio=1000, seq_pad=4096)
# A reduction that is not a multiple of 64 (FFN 2856) over enough rows that the down projection
# runs the 128 x 128 register-staged tiles in more than one round (59 x 9 = 531 tiles for 512
# slots); the other projections take the 256 x 256 direct-to-LDS tiles.
KPAD = dict(name="block_kpad", hidden=1088, heads=17, head_dim=64, ffn=2856, n_video=6000,
            n_audio=1500, seq_pad=8192)
# The widest hidden sizes the boundary accepts, on short sequences: the norm kernels' 8-, 12- and
# 16-chunk-per-lane instantiations (hidden 4096, 6144, 8192) and the GEMMs at those reductions.
WIDE = {f"block_wide{d}": dict(name=f"block_wide{d}", hidden=d, heads=d // 128, head_dim=128,
                               ffn=ffn, n_video=200, n_audio=56, seq_pad=320)
        for d, ffn in ((4096, 1000), (6144, 1536), (8192, 2048))}
EXTRA = {"block_odd": ODD, "block_tiles": TILES, "block_kpad": KPAD, **WIDE}


def _case(name, seed=0):
    from audio_video_diffusion_dit_amd import inputs as I
    wl = I.Workload(**EXTRA[name]) if name in EXTRA else I.WORKLOADS[name]
    return I.block_case(wl, seed=seed, n_blocks=1)


@pytest.mark.parametrize("name", ["block_small", "block_odd", "block_tiles"])
def test_block_end_to_end_and_per_kernel(env, name):
    import oracle as O
    N, dev = env
    case = _case(name)
    wl = case.wl
    V, D, H, Dh = wl.n_valid, wl.hidden, wl.heads, wl.head_dim
    say(f"block {name}: D={D} H={H}x{Dh} F={wl.ffn} video={wl.n_video} audio={wl.n_audio} L={wl.seq_pad}")
    out, ws, m = _gpu_block(env, case)
    got = dev.bf16_values_of(out).astype(np.float64)
    blk = oracle_block(case.blocks[0])
    dims, lay = oracle_dims(wl), oracle_layout(wl)
    x = x_values(case.x)
    assert np.all(got[V:] == 0), "tail rows of the block output must be exactly 0"
    check_block(got, x, case.blocks[0], case.temb, wl, f"{name} block output (end to end)")

    # teacher-forced per-kernel checks: each kernel against the oracle step fed with the GPU's
    # own input to that step
    it = _inter(dev, ws, m, wl)
    mod = O.row_modality(lay)
    E = O.modulation_rows(blk["ada"], case.temb)
    h_ref = O.norm_modulate(x, blk["norm1_g"], E, mod, O.SHIFT_MSA, O.SCALE_MSA, dims.norm_eps)
    assert_kernel_close(it["h"][:V], h_ref[:V], "norm1+mod")
    assert np.all(it["h"][V:] == 0)
    qkv_ref = O.linear(it["h"][:V], blk["w_qkv"])
    pos = np.arange(V, dtype=np.float64)
    q_ref = O.rope_neox(O.qk_rms_norm(qkv_ref[:, :D].reshape(V, H, Dh), blk["q_g"], dims.qk_eps), pos, dims.rope_base)
    k_ref = O.rope_neox(O.qk_rms_norm(qkv_ref[:, D:2 * D].reshape(V, H, Dh), blk["k_g"], dims.qk_eps), pos, dims.rope_base)
    assert_kernel_close(it["qkv"][:V, :D], q_ref.reshape(V, D), "qkv GEMM + q norm/rope")
    assert_kernel_close(it["qkv"][:V, D:2 * D], k_ref.reshape(V, D), "qkv GEMM + k norm/rope")
    assert_kernel_close(it["qkv"][:V, 2 * D:], qkv_ref[:, 2 * D:], "qkv GEMM (v)")
    q_g = it["qkv"][:V, :D].reshape(V, H, Dh)
    k_g = it["qkv"][:V, D:2 * D].reshape(V, H, Dh)
    v_g = it["qkv"][:V, 2 * D:].reshape(V, H, Dh)
    o_ref = O.attention_valid(q_g, k_g, v_g, V).reshape(V, D)
    assert_kernel_close(it["o"][:V], o_ref, "attention")
    gate = lambda c: E[mod[:V], c]
    x1_ref = x[:V] + gate(O.GATE_MSA) * O.linear(it["o"][:V], blk["w_o"])
    assert_kernel_close(it["x1"][:V], x1_ref, "out-proj + gated residual")
    assert np.all(it["x1"][V:] == 0)
    h2_ref = O.norm_modulate(it["x1"], blk["norm2_g"], E, mod, O.SHIFT_MLP, O.SCALE_MLP, dims.norm_eps)
    assert_kernel_close(it["h2"][:V], h2_ref[:V], "norm2+mod")
    a_ref = O.swiglu(it["h2"][:V], blk["w_gate_up"], wl.ffn)
    assert_kernel_close(it["act"][:V], a_ref, "gate/up GEMM + SwiGLU")
    x2_ref = it["x1"][:V] + gate(O.GATE_MLP) * O.linear(it["act"][:V], blk["w_down"])
    assert_kernel_close(got[:V], x2_ref, "down GEMM + gated residual")


@pytest.mark.parametrize("name", ["block_small", "block_odd", "block_tiles"])
def test_block_modes_bitwise_and_deterministic(env, name):
    N, dev = env
    case = _case(name, seed=5)
    say(f"block {name}: valid-only vs fixed-valid, twice")
    a, _, _ = _gpu_block(env, case, attn_mode=N.DIT_ATTN_VALID_ONLY, ws_fill=0xFF)
    b, _, _ = _gpu_block(env, case, attn_mode=N.DIT_ATTN_FIXED_VALID, ws_fill=0x00)
    c, _, _ = _gpu_block(env, case, attn_mode=N.DIT_ATTN_VALID_ONLY, ws_fill=0x7F)
    ab, bb, cb = (dev.bf16_bits_of(t) for t in (a, b, c))
    assert np.array_equal(ab, bb), "fixed-valid and valid-only differ"
    assert np.array_equal(ab, cb), "two runs differ (nondeterminism or workspace dependence)"


def test_block_tail_input_garbage(env):
    N, dev = env
    case = _case("block_odd", seed=6)
    wl = case.wl
    say("block: garbage in the input tail")
    a, _, _ = _gpu_block(env, case)
    xg = case.x.copy()
    xg[wl.n_valid:] = 0x7FC0
    b, _, _ = _gpu_block(env, case, x_bits=xg)
    assert np.array_equal(dev.bf16_bits_of(a), dev.bf16_bits_of(b))


def test_block_zero_gates_identity(env):
    N, dev = env
    case = _case("block_odd", seed=7)
    wl = case.wl
    for bp in case.blocks:
        bp.ada[:, 2] = 0.0
        bp.ada[:, 5] = 0.0
    case.temb[:, 2] = 0.0
    case.temb[:, 5] = 0.0
    say("block: zero gates give the input back")
    out, _, _ = _gpu_block(env, case)
    bits = dev.bf16_bits_of(out)
    assert np.array_equal(bits[: wl.n_valid], case.x[: wl.n_valid])
    assert np.all(bits[wl.n_valid:] == 0)


def test_block_h3_sampled_rows(env):
    """Full H3-scale shape (13440 valid of 13568 rows, D=3072, F=8192): 48 sampled output rows
    against the oracle, which computes keys and values for every valid row."""
    import oracle as O
    N, dev = env
    case = _case("block_h3")
    wl = case.wl
    V = wl.n_valid
    say(f"block_h3 sampled rows: V={V} L={wl.seq_pad}")
    out, _, _ = _gpu_block(env, case)
    got = dev.bf16_values_of(out).astype(np.float64)
    assert np.all(got[V:] == 0)
    rng = np.random.default_rng(11)
    rows = np.sort(np.concatenate([rng.choice(V, 44, replace=False), [0, wl.n_video - 1, wl.n_video, V - 1]]))
    check_block(got[rows], x_values(case.x), case.blocks[0], case.temb, wl, "block_h3 sampled rows",
                rows=rows)


def test_block_kpad_sampled_rows(env):
    """Hidden 1088, FFN 2856 (not a multiple of 64), 7500 valid of 8192 rows: 48 sampled output
    rows against the oracle, which computes keys and values for every valid row."""
    N, dev = env
    case = _case("block_kpad")
    wl = case.wl
    V = wl.n_valid
    say(f"block_kpad sampled rows: V={V} L={wl.seq_pad} F={wl.ffn}")
    out, _, _ = _gpu_block(env, case)
    got = dev.bf16_values_of(out).astype(np.float64)
    assert np.all(got[V:] == 0)
    rng = np.random.default_rng(12)
    rows = np.sort(np.concatenate([rng.choice(V, 44, replace=False), [0, wl.n_video - 1, wl.n_video, V - 1]]))
    check_block(got[rows], x_values(case.x), case.blocks[0], case.temb, wl, "block_kpad sampled rows",
                rows=rows)


@pytest.mark.parametrize("name", sorted(WIDE))
def test_block_wide_hidden(env, name):
    """Hidden 4096, 6144 and 8192 (32, 48 and 64 heads of 128) on 256 valid of 320 rows: the whole
    block output against the oracle."""
    N, dev = env
    case = _case(name, seed=4)
    wl = case.wl
    V = wl.n_valid
    say(f"block {name}: D={wl.hidden} H={wl.heads}x{wl.head_dim} F={wl.ffn} L={wl.seq_pad}")
    out, _, _ = _gpu_block(env, case)
    got = dev.bf16_values_of(out).astype(np.float64)
    assert np.all(got[V:] == 0)
    check_block(got, x_values(case.x), case.blocks[0], case.temb, wl, f"{name} block output")


@pytest.mark.parametrize("name", ["block_small", "block_odd"])
def test_block_unaligned_gemm_weights_bitwise(env, name):
    """Projection weights that start 2 bytes past a 16-byte boundary take the GEMMs' element-wise
    operand path (128 x 128 tiles instead of the aligned 64 x 128 ones). The block output equals
    the aligned call's bit for bit: every output sums the same products in the same order."""
    import torch
    N, dev = env
    case = _case(name, seed=5)
    wl = case.wl
    out_a, _, _ = _gpu_block(env, case)
    bp = case.blocks[0]

    def off_by_one(bits):  # bf16 bits placed one element past a 16-byte-aligned start
        flat = np.concatenate([np.zeros(1, np.uint16), np.ascontiguousarray(bits).reshape(-1)])
        t = dev.to_dev_bf16(flat)
        assert t.data_ptr() % 16 == 0
        return t[1:]

    t = dict(w_qkv=off_by_one(bp.w_qkv), w_o=off_by_one(bp.w_o), w_gate_up=off_by_one(bp.w_gate_up),
             w_down=off_by_one(bp.w_down), norm1_g=dev.to_dev_f32(bp.norm1_g),
             norm2_g=dev.to_dev_f32(bp.norm2_g), q_g=dev.to_dev_f32(bp.q_g), k_g=dev.to_dev_f32(bp.k_g),
             ada=dev.to_dev_f32(bp.ada))
    assert all(t[k].data_ptr() % 16 == 2 for k in ("w_qkv", "w_o", "w_gate_up", "w_down"))
    dims, lay = dev.dims_of(wl), dev.layout_of(wl)
    x = dev.to_dev_bf16(case.x)
    out_u = torch.empty_like(x)
    out_u.view(torch.int16).fill_(0x7FC0)
    ws, m = dev.workspace(dims, lay, 0)
    N.dit_block_forward(dims, lay, N.make_block_weights(t), dev.to_dev_f32(case.temb), x, out_u, 0, ws)
    torch.cuda.synchronize()
    a, u = dev.bf16_bits_of(out_a), dev.bf16_bits_of(out_u)
    say(f"block {name}: unaligned weights, {np.count_nonzero(a != u)} of {a.size} output values differ")
    assert np.array_equal(a, u)


@pytest.mark.parametrize("name,gain,path", [("block_small", 1.2, "shift-free"),
                                            ("block_odd", 1.3, "shift-free"),
                                            ("block_small", -2.0, "bound shift"),
                                            ("block_small", 3.0, "online"),
                                            ("block_odd", 1.8, "bound shift"),
                                            ("block_odd", 4.0, "online")])
def test_block_attention_softmax_paths(env, name, gain, path):
    """The Q/K RMSNorm gains bound every attention logit by max|gq| max|gk| sqrt(Dh). With that
    bound B in log2 units (1 + 2^-6 margin) the kernel takes the probabilities as exp2(s) without
    any shift for B <= 30, as exp2(s - B) for B <= 60, and keeps the online maximum otherwise.
    Every path matches the oracle, per kernel and end to end, with gains that vary across the
    head dimension and change sign."""
    import oracle as O
    N, dev = env
    case = _case(name, seed=3)
    wl = case.wl
    V, D, H, Dh = wl.n_valid, wl.hidden, wl.heads, wl.head_dim
    ramp = np.linspace(0.25, 1.0, Dh, dtype=np.float32)
    sign = np.where(np.arange(Dh) % 3 == 0, -1.0, 1.0).astype(np.float32)
    blk_p = dataclasses.replace(case.blocks[0], q_g=(gain * ramp * sign).astype(np.float32),
                                k_g=(gain * ramp[::-1] * sign).astype(np.float32))
    case = dataclasses.replace(case, blocks=[blk_p])
    bound = gain * gain * Dh * (np.log2(np.e) / np.sqrt(Dh)) * (1 + 2 ** -6)
    want = "shift-free" if bound <= 30 else ("bound shift" if bound <= 60 else "online")
    assert want == path, bound
    say(f"block {name}: gains up to |{gain}|, logit bound {bound:.1f} (log2 units) -> {path} path")
    out, ws, m = _gpu_block(env, case)
    got = dev.bf16_values_of(out).astype(np.float64)
    blk = oracle_block(blk_p)
    dims, lay = oracle_dims(wl), oracle_layout(wl)
    assert np.all(got[V:] == 0)
    check_block(got, x_values(case.x), blk_p, case.temb, wl, f"{name} block output ({path} softmax path)")
    it = _inter(dev, ws, m, wl)
    q_g = it["qkv"][:V, :D].reshape(V, H, Dh)
    k_g = it["qkv"][:V, D:2 * D].reshape(V, H, Dh)
    v_g = it["qkv"][:V, 2 * D:].reshape(V, H, Dh)
    o_ref = O.attention_valid(q_g, k_g, v_g, V).reshape(V, D)
    assert_kernel_close(it["o"][:V], o_ref, f"attention ({path} softmax path)")
    assert np.all(it["o"][V:] == 0)


def test_block_32k_sampled_rows(env):
    """One block at the benchmarked 32,768-token shape (30,720 video + 2,048 audio, no tail;
    D=3072, 24 x 128 heads, F=8192): rows 0, 30719, 30720, 32767 (both ends of both modalities,
    the largest rotary positions) and 60 drawn rows against the oracle, which computes keys and
    values for all 32,768 rows; fixed-valid equals valid-only bit for bit."""
    N, dev = env
    from audio_video_diffusion_dit_amd import inputs as I
    wl = I.WORKLOADS["loop_8blk_32k"]
    case = I.block_case(wl, seed=0, n_blocks=1)
    V = wl.n_valid
    say(f"block 32k sampled rows: V={V} L={wl.seq_pad} D={wl.hidden} F={wl.ffn}")
    out, _, _ = _gpu_block(env, case)
    bits = dev.bf16_bits_of(out)
    fv, _, _ = _gpu_block(env, case, attn_mode=N.DIT_ATTN_FIXED_VALID)
    assert np.array_equal(bits, dev.bf16_bits_of(fv)), "fixed-valid and valid-only differ"
    got = dev.bf16_values_of(out).astype(np.float64)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(32)
    edges = [0, wl.n_video - 1, wl.n_video, V - 1]
    rows = np.sort(np.concatenate([rng.choice(np.setdiff1d(np.arange(V), edges), 60, replace=False),
                                   edges]))
    check_block(got[rows], x_values(case.x), case.blocks[0], case.temb, wl,
                "32k block sampled rows", rows=rows)


@pytest.mark.parametrize("nv,na,L", [(0, 0, 256), (0, 300, 320), (250, 0, 256)])
def test_block_degenerate_layouts(env, nv, na, L):
    """No valid row (the output is all zero), audio rows only, video rows only: against the
    oracle and its storage diagnostic; fixed-valid equals valid-only bit for bit."""
    N, dev = env
    from audio_video_diffusion_dit_amd import inputs as I
    wl = I.Workload("block_degenerate", 256, 2, 128, 300, nv, na, L)
    case = I.block_case(wl, seed=nv + 3 * na + L, n_blocks=1)
    say(f"block degenerate layout: video {nv} audio {na} seq_pad {L}")
    out, _, _ = _gpu_block(env, case)
    fv, _, _ = _gpu_block(env, case, attn_mode=N.DIT_ATTN_FIXED_VALID)
    assert np.array_equal(dev.bf16_bits_of(out), dev.bf16_bits_of(fv))
    got = dev.bf16_values_of(out).astype(np.float64)
    V = wl.n_valid
    assert np.all(got[V:] == 0)
    if V == 0:
        return
    check_block(got, x_values(case.x), case.blocks[0], case.temb, wl,
                f"block, video {nv} audio {na}")


def test_block_largest_sequence_at_hidden_3072(env):
    """The longest sequence the library takes at hidden 3072: 116,508 rows, whose q/k/v rows
    [seq_pad, 3D] span 2,147,475,456 bytes, just under the 2 GiB the kernels' 32-bit buffer
    offsets address (one row more is rejected during validation). Sampled rows, including the
    last ones, against the oracle with keys and values for every row."""
    N, dev = env
    from audio_video_diffusion_dit_amd import inputs as I
    wl = I.Workload("block_max", 3072, 24, 128, 8192, 110000, 6508, 116508)
    assert wl.seq_pad * 3 * wl.hidden * 2 < 2 ** 31 <= (wl.seq_pad + 1) * 3 * wl.hidden * 2
    case = I.block_case(wl, seed=8, n_blocks=1)
    V = wl.n_valid
    say(f"block at the largest sequence: V={V} L={wl.seq_pad}")
    out, _, _ = _gpu_block(env, case)
    got = dev.bf16_values_of(out).astype(np.float64)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(116)
    edges = [0, 65535, 65536, wl.n_video - 1, wl.n_video, V - 2, V - 1]
    rows = np.sort(np.concatenate([rng.choice(np.setdiff1d(np.arange(V), edges), 25, replace=False),
                                   edges]))
    check_block(got[rows], x_values(case.x), case.blocks[0], case.temb, wl,
                "largest-sequence block sampled rows", rows=rows)
