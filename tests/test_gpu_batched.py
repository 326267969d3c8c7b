"""GPU checks of dit_block_forward_batched: a batch of ragged requests in one call equals the
requests' own dit_block_forward calls bit for bit, and matches the oracle."""

import numpy as np
import pytest

from helpers import check_block, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from audio_video_diffusion_dit_amd import _native, device
    return _native, device


def _run(env, wl_dims, reqs, seq_pad, seed, attn_mode=0):
    """reqs: list of (n_video, n_audio, positions or None). Returns batched and single outputs."""
    import torch
    import oracle as O
    from audio_video_diffusion_dit_amd import inputs as I
    N, dev = env
    wl = I.Workload("batch", *wl_dims, reqs[0][0], reqs[0][1], seq_pad)
    rng = np.random.Generator(np.random.PCG64(seed))
    blk_p = I.make_block(rng, wl)
    B, L, D = len(reqs), seq_pad, wl.hidden
    x = np.zeros((B * L, D), np.uint16)
    for b, (nv, na, _) in enumerate(reqs):
        x[b * L: b * L + nv + na] = I.bf16_bits(rng.standard_normal((nv + na, D), dtype=np.float32))
        x[b * L + nv + na: (b + 1) * L] = 0x7FC0      # NaN in every tail: must not leak
    temb = rng.standard_normal((B, 2, 6, D), dtype=np.float32)
    dims = dev.dims_of(wl)
    blk = dev.upload_block(blk_p)
    pos_dev = [None if p is None else torch.from_numpy(p.astype(np.int32)).cuda() for *_, p in reqs]
    lays = [N.make_layout(nv, na, L, pos_dev[b]) for b, (nv, na, _) in enumerate(reqs)]
    dx, dt = dev.to_dev_bf16(x), dev.to_dev_f32(temb)
    out = torch.empty_like(dx)
    out.view(torch.int16).fill_(0x7FC0)
    nbytes, _ = N.dit_workspace_size_batched(dims, lays)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    N.dit_block_forward_batched(dims, lays, blk.weights, dt, dx, out, attn_mode, ws)
    torch.cuda.synchronize()
    got = dev.bf16_bits_of(out)
    singles = []
    for b in range(B):
        o = torch.empty((L, D), dtype=torch.bfloat16, device="cuda")
        ws1, _ = dev.workspace(dims, lays[b], 0)
        N.dit_block_forward(dims, lays[b], blk.weights, dt[b], dx[b * L:(b + 1) * L], o, 0, ws1)
        torch.cuda.synchronize()
        singles.append(dev.bf16_bits_of(o))
    return wl, blk_p, x, temb, got, singles


def test_batched_small_ragged_equals_single_requests(env):
    """Four requests of 768 rows at hidden 256 (4 x 64, FFN 683): valid 608, 300 (video only),
    350 (100 video + 250 audio, rotary positions offset by 1000) and 0 (all tail)."""
    import oracle as O
    reqs = [(512, 96, None), (300, 0, None), (100, 250, np.arange(768) + 1000), (0, 0, None)]
    say("batched block: 4 requests x 768 rows, valid 608 / 300 / 350 / 0")
    wl, blk_p, x, temb, got, singles = _run(env, (256, 4, 64, 683), reqs, 768, seed=12)
    L = 768
    for b, (nv, na, pos) in enumerate(reqs):
        assert np.array_equal(got[b * L:(b + 1) * L], singles[b]), f"request {b} differs from its single call"
        assert np.all(got[b * L + nv + na:(b + 1) * L] == 0)
    # one request against the oracle (independence of the requests in the batch)
    from audio_video_diffusion_dit_amd.inputs import bf16_to_f32
    b, (nv, na, pos) = 2, reqs[2]
    lay = O.Layout(nv, na, L)
    xs = bf16_to_f32(x[b * L:(b + 1) * L]).astype(np.float64)
    xs[nv + na:] = 0
    check_block(bf16_to_f32(got[b * L:(b + 1) * L]), xs, blk_p, temb[b], wl, "request 2 vs oracle",
                positions=pos, layout=lay)


def test_batched_h3_scale_equals_single_requests(env):
    """Two requests of 4096 rows at hidden 3072 (24 x 128, FFN 8192), valid 4096 and 2500: the
    batched GEMMs take the large-tile path where the single calls may not."""
    reqs = [(3584, 512, None), (2000, 500, None)]
    say("batched block, H3 dims: 2 requests x 4096 rows, valid 4096 / 2500")
    _, _, _, _, got, singles = _run(env, (3072, 24, 128, 8192), reqs, 4096, seed=13)
    L = 4096
    for b, (nv, na, _) in enumerate(reqs):
        assert np.array_equal(got[b * L:(b + 1) * L], singles[b]), f"request {b} differs from its single call"


def test_batched_block_ragged_full_size(env):
    """The measured batch: four requests of 8192 rows through one H3-scale block, valid
    3000 / 5100 / 7777 / 8192. Each request equals its own single call bit for bit, tails are
    exactly 0, and 24 sampled rows of requests 0 and 3 match the oracle."""
    import oracle as O
    from audio_video_diffusion_dit_amd import inputs as I
    cfg = I.BLOCK_RAGGED
    reqs = [(nv, na, None) for nv, na in cfg["requests"]]
    L = cfg["seq_pad"]
    say(f"batched block, H3 dims: {len(reqs)} requests x {L} rows, valid "
        f"{[nv + na for nv, na, _ in reqs]}")
    wl, blk_p, x, temb, got, singles = _run(
        env, (cfg["hidden"], cfg["heads"], cfg["head_dim"], cfg["ffn"]), reqs, L, seed=14)
    rng = np.random.default_rng(15)
    for b, (nv, na, _) in enumerate(reqs):
        V = nv + na
        assert np.array_equal(got[b * L:(b + 1) * L], singles[b]), f"request {b} differs from its single call"
        assert np.all(got[b * L + V:(b + 1) * L] == 0)
        if b not in (0, 3):
            continue
        rows = np.sort(np.concatenate([rng.choice(V, 20, replace=False), [0, nv - 1, nv, V - 1]]))
        xs = I.bf16_to_f32(x[b * L:(b + 1) * L]).astype(np.float64)
        xs[V:] = 0
        check_block(I.bf16_to_f32(got[b * L + rows]), xs, blk_p, temb[b], wl,
                    f"request {b} sampled rows vs oracle", rows=rows, layout=O.Layout(nv, na, L))


def test_batched_fixed_valid_equals_valid_only(env):
    """Fixed-valid attention inside the batched block (every key tile of each request swept with
    a mask) gives the valid-only result bit for bit."""
    N, _ = env
    reqs = [(400, 100, None), (0, 0, None), (700, 60, None)]
    say("batched block: fixed-valid vs valid-only, 3 requests x 768 rows")
    *_, vo, _ = _run(env, (256, 4, 64, 683), reqs, 768, seed=16, attn_mode=N.DIT_ATTN_VALID_ONLY)
    *_, fv, _ = _run(env, (256, 4, 64, 683), reqs, 768, seed=16, attn_mode=N.DIT_ATTN_FIXED_VALID)
    assert np.array_equal(vo, fv)


def test_batched_maximum_batch(env):
    """The largest batch the entry point takes: 64 requests of 256 rows at hidden 256, valid
    lengths drawn in [0, 256] (video and audio split at random); every request equals its own
    single-request call bit for bit."""
    rng = np.random.default_rng(17)
    reqs = []
    for _ in range(64):
        n = int(rng.integers(0, 257))
        nv = int(rng.integers(0, n + 1))
        reqs.append((nv, n - nv, None))
    reqs[0] = (200, 56, None)        # one full request; make_block takes its layout
    say(f"batched block: 64 requests x 256 rows, valid {min(a + b for a, b, _ in reqs)}.."
        f"{max(a + b for a, b, _ in reqs)}")
    _, _, _, _, got, singles = _run(env, (256, 4, 64, 683), reqs, 256, seed=18)
    for b, (nv, na, _) in enumerate(reqs):
        assert np.array_equal(got[b * 256:(b + 1) * 256], singles[b]), f"request {b} differs"
        assert np.all(got[b * 256 + nv + na:(b + 1) * 256] == 0)
