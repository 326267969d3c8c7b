"""dit_block_forward_noalloc (the block on the library's built-in scratch, no workspace
argument) against dit_block_forward with a caller workspace: bit for bit, on two calls in a row,
the second with a smaller input, each compared with its own workspace call."""

import numpy as np
import pytest

from helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from audio_video_diffusion_dit_amd import _native, device
    return _native, device


def _both(env, wl, seed, attn_mode=0):
    import torch
    from audio_video_diffusion_dit_amd import inputs as I
    N, dev = env
    case = I.block_case(wl, seed=seed, n_blocks=1)
    dims, lay = dev.dims_of(wl), dev.layout_of(wl)
    need, _ = N.dit_workspace_size(dims, lay, 0)
    assert need <= N.NOALLOC_SCRATCH_BYTES
    blk = dev.upload_block(case.blocks[0])
    temb = dev.to_dev_f32(case.temb)
    x = dev.to_dev_bf16(case.x)
    ref = torch.empty_like(x)
    ref.view(torch.int16).fill_(0x7FC0)
    ws, _ = dev.workspace(dims, lay, 0)
    N.dit_block_forward(dims, lay, blk.weights, temb, x, ref, attn_mode, ws)
    got = torch.empty_like(x)
    got.view(torch.int16).fill_(0x7FC0)
    N.dit_block_forward_noalloc(dims, lay, blk.weights, temb, x, got, attn_mode)
    torch.cuda.synchronize()
    return dev.bf16_bits_of(got), dev.bf16_bits_of(ref), wl.n_valid


def test_noalloc_equals_workspace_call_twice_second_smaller(env):
    from audio_video_diffusion_dit_amd import inputs as I
    odd = I.Workload("block_odd", 256, 2, 128, 300, 100, 37, 200)
    for wl, seed in ((I.WORKLOADS["loop_4blk"], 3), (odd, 4)):
        say(f"noalloc block: {wl.name} V={wl.n_valid} L={wl.seq_pad} D={wl.hidden}")
        got, ref, V = _both(env, wl, seed)
        assert np.array_equal(got, ref), f"{wl.name}: noalloc output differs from the workspace call"
        assert np.all(got[V:] == 0)
    # fixed-valid attention through the scratch too, after the two calls above
    got, ref, _ = _both(env, I.WORKLOADS["block_small"], 5, attn_mode=1)
    assert np.array_equal(got, ref)
