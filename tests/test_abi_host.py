"""CPU-only checks of the C-ABI library: it loads, exports every declared entry point, its
host-side cache schedule equals the oracle's, and invalid arguments are rejected before any
device work (none of these calls touches a GPU)."""

import math
import os
import re

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def N():
    from audio_video_diffusion_dit_amd import _native
    return _native


def test_library_exports_every_declared_symbol(N):
    with open(os.path.join(ROOT, "include", "avdit.h")) as f:
        header = f.read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(", header, re.M))
    declared -= {"if", "return"}
    assert {"dit_block_forward", "denoise_loop", "step_update"} <= declared
    for name in declared:
        assert hasattr(N.lib, name), f"{name} is declared but not exported"
    assert set(N.EXPORTED) == declared
    assert N.lib.dit_version().decode().startswith("avdit")


RATIOS = [(0.2, 0.8), (0.0, 1.0), (0.0, 0.0), (0.5, 0.5), (0.1, 0.9), (0.25, 0.75), (0.3, 0.31),
          (0.0, 0.5), (0.5, 1.0), (1.0, 1.0)]


@pytest.mark.parametrize("r,c", [(2, 1), (1, 1), (3, 2), (3, 1), (4, 9), (2, 0), (5, 3)])
def test_schedule_matches_oracle(N, r, c):
    for s, e in RATIOS:
        for n in range(0, 201):
            pol = O.CachePolicy("velocity", s, e, r, c)
            want = O.cache_schedule(pol, n)
            got = N.dit_cache_schedule(N.make_policy("conservative", s, e, r, c), n)
            assert got == want, (s, e, r, c, n)
    off = N.dit_cache_schedule(N.make_policy("off"), 49)
    assert off == [False] * 49


def test_extrapolate_mode_has_the_reuse_schedule(N):
    for s, e in RATIOS:
        for r, c in ((2, 1), (3, 2), (4, 9)):
            for n in (0, 1, 7, 49, 100):
                ext = N.dit_cache_schedule(N.make_policy("extrapolate", s, e, r, c), n)
                assert ext == N.dit_cache_schedule(N.make_policy("velocity", s, e, r, c), n)
                assert ext == O.cache_schedule(O.CachePolicy("extrapolate", s, e, r, c), n)


def test_schedule_counts_printed_on_pages(N):
    hits = N.dit_cache_schedule(N.make_policy("conservative"), 49)
    assert (49 - sum(hits), sum(hits)) == (34, 15)
    assert N.dit_cache_schedule(N.make_policy("velocity", quality="high"), 49) == [False] * 49


def test_policy_validation(N):
    bad = [dict(start_ratio=-0.1), dict(end_ratio=1.5), dict(start_ratio=0.9, end_ratio=0.1),
           dict(refresh_interval=0), dict(max_consecutive_reuse=-1)]
    for kw in bad:
        with pytest.raises(N.AvditError) as ei:
            N.dit_cache_schedule(N.make_policy("conservative", **kw), 49)
        assert ei.value.code == N.DIT_ERR_INVALID
        assert N.last_error()
    with pytest.raises(N.AvditError) as ei:
        N.dit_cache_schedule(N.make_policy("conservative", threshold=0.05), 49)
    assert ei.value.code == N.DIT_ERR_UNSUPPORTED
    p = N.make_policy("conservative")
    p.mode = 7
    with pytest.raises(N.AvditError) as ei:
        N.dit_cache_schedule(p, 49)
    assert ei.value.code == N.DIT_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        N.resolve_mode("bogus")
    # a valid call after failures clears the error and is unaffected by them
    assert sum(N.dit_cache_schedule(N.make_policy("conservative"), 49)) == 15
    assert N.last_error() == ""


def test_dims_and_layout_validation(N):
    lay = N.make_layout(512, 96, 640)
    cases = [
        (N.make_dims(256, 4, 60, 683), N.DIT_ERR_UNSUPPORTED),   # head_dim
        (N.make_dims(256, 3, 64, 683), N.DIT_ERR_INVALID),       # D != H * Dh
        (N.make_dims(256, 4, 64, 0), N.DIT_ERR_INVALID),         # ffn
        (N.make_dims(256, 4, 64, 683, n_mod=3), N.DIT_ERR_UNSUPPORTED),
        (N.make_dims(256, 4, 64, 683, norm_eps=float("nan")), N.DIT_ERR_INVALID),
        (N.make_dims(256, 4, 64, 683, rope_base=0.0), N.DIT_ERR_INVALID),
    ]
    for dims, code in cases:
        with pytest.raises(N.AvditError):
            N.dit_workspace_size(dims, lay)
        assert N.last_error()
    d = N.make_dims(256, 4, 64, 683)
    for bad_lay in (N.make_layout(512, 96, 600), N.make_layout(-1, 96, 640)):
        with pytest.raises(N.AvditError):
            N.dit_workspace_size(d, bad_lay)


def test_workspace_map(N):
    d = N.make_dims(3072, 24, 128, 8192)
    lay = N.make_layout(12096, 1344, 13568)
    n0, m0 = N.dit_workspace_size(d, lay, 0)
    n1, m1 = N.dit_workspace_size(d, lay, 1)
    L, D = 13568, 3072
    assert m0.ffn_ld == 8192
    offs = [m0.h, m0.qkv, m0.attn_out, m0.x1, m0.h2, m0.act]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert m0.qkv - m0.h >= L * D * 2 and m0.attn_out - m0.qkv >= L * 3 * D * 2
    assert n0 >= m0.act + L * 8192 * 2
    # loop buffers: the bf16 copy of the latent, then ping, pong and velocity sized for fp32
    # rows (the fp32-residual loop keeps them in fp32)
    assert n1 == n0 + L * D * 2 + 4 * (L * D * 4)
    assert m1.ping - m1.x_bf16 >= L * D * 2 and m1.pong - m1.ping >= L * D * 4
    assert m1.velocity - m1.pong >= L * D * 4 and m1.velocity_prev - m1.velocity >= L * D * 4
    assert n1 - m1.velocity_prev >= L * D * 4
    _, m = N.dit_workspace_size(N.make_dims(256, 4, 64, 683), N.make_layout(512, 96, 640), 0)
    assert m.ffn_ld == 688


def test_batched_workspace_and_validation(N):
    d = N.make_dims(256, 4, 64, 683)
    one = N.make_layout(512, 96, 768)
    n1, m1 = N.dit_workspace_size(d, one, 0)
    nb1, mb1 = N.dit_workspace_size_batched(d, [one])
    assert (n1, m1.act) == (nb1, mb1.act)
    lays = [N.make_layout(512, 96, 768), N.make_layout(300, 0, 768), N.make_layout(0, 0, 768)]
    nb, mb = N.dit_workspace_size_batched(d, lays)
    n3, _ = N.dit_workspace_size(d, N.make_layout(0, 0, 3 * 768), 0)
    assert nb == n3 and mb.qkv - mb.h >= 3 * 768 * 256 * 2
    with pytest.raises(N.AvditError):       # requests must share seq_pad
        N.dit_workspace_size_batched(d, [N.make_layout(512, 96, 768), N.make_layout(10, 0, 512)])
    with pytest.raises(N.AvditError):       # a batch needs seq_pad a multiple of 256
        N.dit_workspace_size_batched(d, [N.make_layout(512, 96, 640)] * 2)
    with pytest.raises(N.AvditError):       # at most 64 requests
        N.dit_workspace_size_batched(d, [one] * 65)
    w = N.DitBlockWeights(*([256] * 9))
    arr = (N.DitLayout * 2)(*lays[:2])
    need, _ = N.dit_workspace_size_batched(d, lays[:2])
    big = 1 << 40
    f = N.lib.dit_block_forward_batched
    assert f(d, arr, 2, w, 256, 1 << 20, 1 << 30, 0, big, need - 1, None) == N.DIT_ERR_WORKSPACE
    assert f(d, arr, 0, w, 256, 1 << 20, 1 << 30, 0, big, need, None) == N.DIT_ERR_INVALID
    assert f(d, arr, 2, w, 256, 1 << 20, (1 << 20) + 100, 0, big, need, None) == N.DIT_ERR_INVALID
    assert f(d, arr, 2, N.DitBlockWeights(), 256, 1 << 20, 1 << 30, 0, big, need, None) == N.DIT_ERR_INVALID
    bad = (N.DitLayout * 2)(N.make_layout(512, 96, 640), N.make_layout(10, 0, 640))
    assert f(d, bad, 2, w, 256, 1 << 20, 1 << 30, 0, big, need, None) == N.DIT_ERR_UNSUPPORTED


def test_entry_points_reject_invalid_arguments_without_device_work(N):
    d = N.make_dims(256, 4, 64, 683)
    lay = N.make_layout(512, 96, 640)
    w = N.DitBlockWeights(*([256] * 9))   # fake non-null addresses: never dereferenced
    null_w = N.DitBlockWeights()
    ws_need, _ = N.dit_workspace_size(d, lay, 0)
    big = 1 << 40
    # null weights
    code = N.lib.dit_block_forward(d, lay, null_w, 256, 256, 512, 0, big, ws_need, None)
    assert code == N.DIT_ERR_INVALID
    code = N.lib.dit_block_forward_f32(d, lay, null_w, 256, 256, 1 << 20, 0, big, ws_need, None)
    assert code == N.DIT_ERR_INVALID
    # fp32 block: misaligned fp32 rows, overlapping fp32 input and output (640 x 256 x 4 bytes)
    code = N.lib.dit_block_forward_f32(d, lay, w, 256, (1 << 20) + 4, 1 << 22, 0, big, ws_need, None)
    assert code == N.DIT_ERR_INVALID
    code = N.lib.dit_block_forward_f32(d, lay, w, 256, 1 << 20, (1 << 20) + 640 * 256 * 2, 0, big,
                                       ws_need, None)
    assert code == N.DIT_ERR_INVALID
    # bad attention mode
    code = N.lib.dit_block_forward(d, lay, w, 256, 1 << 20, 1 << 30, 5, big, ws_need, None)
    assert code == N.DIT_ERR_INVALID
    # workspace too small
    code = N.lib.dit_block_forward(d, lay, w, 256, 1 << 20, 1 << 30, 0, big, ws_need - 1, None)
    assert code == N.DIT_ERR_WORKSPACE
    # misaligned workspace
    code = N.lib.dit_block_forward(d, lay, w, 256, 1 << 20, 1 << 30, 0, big + 8, ws_need, None)
    assert code == N.DIT_ERR_INVALID
    # aliasing input and output
    code = N.lib.dit_block_forward(d, lay, w, 256, 1 << 20, 1 << 20, 0, big, ws_need, None)
    assert code == N.DIT_ERR_INVALID
    # step_update: hidden not a multiple of 8, non-finite step
    assert N.lib.step_update(1 << 20, 1 << 21, None, lay, 100, -0.1, -0.1, None) == N.DIT_ERR_INVALID
    assert N.lib.step_update(1 << 20, 1 << 21, None, lay, 256, math.inf, -0.1, None) == N.DIT_ERR_INVALID
    # attention: head_dim, batch, valid length, strides
    vl = (N.c_int32 * 2)(10, 700)
    assert N.lib.dit_attention_forward(1 << 20, 1 << 21, 1 << 22, 1 << 23, 2, 640, 4, 64, 640 * 256,
                                       256, 640 * 256, 256, vl, None, None, 0, None) == N.DIT_ERR_INVALID
    vl = (N.c_int32 * 1)(10)
    assert N.lib.dit_attention_forward(1 << 20, 1 << 21, 1 << 22, 1 << 23, 1, 640, 4, 96, 0,
                                       384, 0, 384, vl, None, None, 0, None) == N.DIT_ERR_UNSUPPORTED
    assert N.lib.dit_attention_forward(1 << 20, 1 << 21, 1 << 22, 1 << 23, 0, 640, 4, 64, 0,
                                       256, 0, 256, vl, None, None, 0, None) == N.DIT_ERR_INVALID
    assert N.lib.dit_attention_forward(1 << 20, 1 << 21, 1 << 22, 1 << 23, 1, 640, 4, 64, 0,
                                       200, 0, 256, vl, None, None, 0, None) == N.DIT_ERR_INVALID
    # gains: both or neither
    assert N.lib.dit_attention_forward(1 << 20, 1 << 21, 1 << 22, 1 << 23, 1, 640, 4, 64, 0,
                                       256, 0, 256, vl, 1 << 24, None, 0, None) == N.DIT_ERR_INVALID


def test_denoise_loop_rejects_invalid_arguments(N):
    d = N.make_dims(256, 4, 64, 683)
    lay = N.make_layout(512, 96, 640)
    w = (N.DitBlockWeights * 1)(N.DitBlockWeights(*([256] * 9)))
    need, _ = N.dit_workspace_size(d, lay, 1)
    sig = (N.c_float * 50)(*np.linspace(1, 0, 50).astype(np.float32))
    stats = N.DitLoopStats()
    pol = N.make_policy("conservative")
    big = 1 << 40
    args = lambda **kw: dict(dict(dims=d, lay=lay, blocks=w, nb=1, n=49, sv=sig, sa=sig, temb=256,
                                  pol=pol, x=1 << 20, mode=0, stats=stats, ws=big, wsb=need), **kw)

    def call(a):
        return N.lib.denoise_loop(a["dims"], a["lay"], a["blocks"], a["nb"], a["n"], a["sv"], a["sa"],
                                  a["temb"], a["pol"], a["x"], a["mode"], a["stats"], a["ws"],
                                  a["wsb"], None)

    assert call(args(nb=0)) == N.DIT_ERR_INVALID
    assert call(args(n=-1)) == N.DIT_ERR_INVALID
    assert call(args(wsb=need - 256)) == N.DIT_ERR_WORKSPACE
    bad = N.make_policy("conservative", threshold=0.1)
    assert call(args(pol=bad)) == N.DIT_ERR_UNSUPPORTED
    nan_sig = (N.c_float * 50)(*([float("nan")] * 50))
    assert call(args(sv=nan_sig)) == N.DIT_ERR_INVALID
    assert call(args(blocks=(N.DitBlockWeights * 1)(N.DitBlockWeights()))) == N.DIT_ERR_INVALID

    def call_f32(a):
        return N.lib.denoise_loop_f32(a["dims"], a["lay"], a["blocks"], a["nb"], a["n"], a["sv"],
                                      a["sa"], a["temb"], a["pol"], a["x"], a["mode"], a["stats"],
                                      a["ws"], a["wsb"], None)

    assert call_f32(args(nb=0)) == N.DIT_ERR_INVALID
    assert call_f32(args(wsb=need - 256)) == N.DIT_ERR_WORKSPACE
    assert call_f32(args(pol=bad)) == N.DIT_ERR_UNSUPPORTED
    assert call_f32(args(sa=nan_sig)) == N.DIT_ERR_INVALID
    assert call_f32(args(x=(1 << 20) + 4)) == N.DIT_ERR_INVALID


def test_head_workspace_and_validation(N):
    d = N.make_dims(256, 4, 64, 683)
    lay = N.make_layout(512, 96, 640)
    need = N.dit_head_workspace_size(d, lay, 64)
    assert need == 2 * 256 * 4 + 2 * 64 * 4                   # the folded table: mul, cst
    assert N.dit_head_workspace_size(d, lay, 512) == 2 * 256 * 4 + 2 * 512 * 4
    assert N.dit_head_workspace_size(d, N.make_layout(0, 0, 0), 64) == need
    with pytest.raises(N.AvditError):
        N.dit_head_workspace_size(d, N.make_layout(600, 96, 640), 64)
    with pytest.raises(N.AvditError):
        N.dit_head_workspace_size(d, lay, 12)
    f = N.lib.dit_velocity_head
    ws, x, v, t = 1 << 30, 1 << 32, 1 << 34, 1 << 20
    good = N.DitHeadWeights(256, 512, 1 << 24, 1 << 25, 64)

    def call(head=good, temb=t, x_=x, v_=v, ws_=ws, nbytes=need, layout=lay):
        return f(d, layout, head, temb, x_, v_, ws_, nbytes, None)

    assert call(nbytes=need - 1) == N.DIT_ERR_WORKSPACE
    assert call(head=N.DitHeadWeights(256, 512, 1 << 24, 1 << 25, 60)) == N.DIT_ERR_INVALID
    assert call(head=N.DitHeadWeights(256, 512, 1 << 24, 1 << 25, 0)) == N.DIT_ERR_INVALID
    assert call(head=N.DitHeadWeights(256, 512, None, 1 << 25, 64)) == N.DIT_ERR_INVALID
    assert call(head=N.DitHeadWeights(256, 512, 1 << 24, (1 << 25) + 4, 64)) == N.DIT_ERR_INVALID
    assert call(temb=None) == N.DIT_ERR_INVALID
    assert call(x_=x + 2) == N.DIT_ERR_INVALID                 # misaligned input
    assert call(v_=x + 1024) == N.DIT_ERR_INVALID              # v overlaps x
    assert call(ws_=v + 4096) == N.DIT_ERR_INVALID             # workspace overlaps v
    assert call(layout=N.make_layout(600, 96, 640)) == N.DIT_ERR_INVALID
    assert "out_channels" in (call(head=N.DitHeadWeights(256, 512, 1 << 24, None, 12)) and N.last_error())
    # an empty sequence validates and enqueues nothing
    assert call(layout=N.make_layout(0, 0, 0)) == N.DIT_OK


def test_operand_spans_rejected_before_any_launch(N):
    """Shapes whose operands would span 2 GiB or more (32-bit buffer offsets in the kernels) are
    rejected with DIT_ERR_UNSUPPORTED during validation. The fake device addresses are never
    dereferenced: on a machine without a GPU any launch would fail with DIT_ERR_DEVICE instead."""
    d = N.make_dims(3072, 24, 128, 8192)
    w = N.DitBlockWeights(*([256] * 9))
    big = 1 << 40
    # four 32,768-token requests at FFN 8192: the SwiGLU activations span 2^31 bytes
    lays = [N.make_layout(30720, 2048, 32768)] * 4
    arr = (N.DitLayout * 4)(*lays)
    with pytest.raises(N.AvditError):      # size functions return 0 and set the message
        N.dit_workspace_size_batched(d, lays)
    assert "SwiGLU" in N.last_error() and "2 GiB" in N.last_error()
    code = N.lib.dit_block_forward_batched(d, arr, 4, w, 256, 1 << 20, 1 << 36, 0, big, 1 << 38, None)
    assert code == N.DIT_ERR_UNSUPPORTED and "SwiGLU" in N.last_error()
    # one 131,072-token request
    lay = N.make_layout(120000, 11072, 131072)
    with pytest.raises(N.AvditError):
        N.dit_workspace_size(d, lay, 0)
    assert "2 GiB" in N.last_error()
    code = N.lib.dit_block_forward(d, lay, w, 256, 1 << 20, 1 << 36, 0, big, 1 << 38, None)
    assert code == N.DIT_ERR_UNSUPPORTED
    # 116,509 rows: the first length whose q/k/v rows [seq_pad, 3D] reach 2 GiB at hidden 3072
    lay = N.make_layout(116509, 0, 116509)
    code = N.lib.dit_block_forward(d, lay, w, 256, 1 << 20, 1 << 36, 0, big, 1 << 38, None)
    assert code == N.DIT_ERR_UNSUPPORTED and "q/k/v" in N.last_error()
    n, _ = N.dit_workspace_size(d, N.make_layout(116508, 0, 116508), 0)
    assert n > 0
    # the same limits in the loop
    blocks = (N.DitBlockWeights * 1)(w)
    sig = (N.c_float * 2)(1.0, 0.0)
    code = N.lib.denoise_loop(d, lay, blocks, 1, 1, sig, sig, 256, N.make_policy("off"), 1 << 20, 0,
                              None, big, 1 << 38, None)
    assert code == N.DIT_ERR_UNSUPPORTED
    # attention alone: one request's rows reach 2 GiB
    vl = (N.c_int32 * 1)(100000)
    code = N.lib.dit_attention_forward(1 << 20, 1 << 21, 1 << 22, 1 << 23, 1, 116509, 24, 128, 0,
                                       9216, 0, 3072, vl, None, None, 0, None)
    assert code == N.DIT_ERR_UNSUPPORTED
    # the velocity head reads its input through 64-bit addresses and its one buffer operand, a
    # modality's weight [C, D], stays below 1 GiB at the largest C and D: no span limit
    dh = N.make_dims(8192, 64, 128, 8192)
    lay_h = N.make_layout(131072, 0, 131072)
    assert N.dit_head_workspace_size(dh, lay_h, 128) == 2 * 8192 * 4 + 2 * 128 * 4


def test_vector_accessed_pointers_must_be_aligned(N):
    """Every pointer the kernels access with 16-byte vectors is checked before any launch."""
    d = N.make_dims(256, 4, 64, 683)
    lay = N.make_layout(512, 96, 640)
    need, _ = N.dit_workspace_size(d, lay, 0)
    big = 1 << 40
    good = [256] * 9
    f = N.lib.dit_block_forward
    for i in range(4, 9):     # norm1_g, norm2_g, q_g, k_g, ada
        bad = list(good)
        bad[i] = 256 + 8
        code = f(d, lay, N.DitBlockWeights(*bad), 256, 1 << 20, 1 << 30, 0, big, need, None)
        assert code == N.DIT_ERR_INVALID and "aligned" in N.last_error(), i
    assert f(d, lay, N.DitBlockWeights(*good), 256 + 4, 1 << 20, 1 << 30, 0, big, need, None) == N.DIT_ERR_INVALID
    assert f(d, lay, N.DitBlockWeights(*good), 256, (1 << 20) + 8, 1 << 30, 0, big, need, None) == N.DIT_ERR_INVALID
    assert f(d, lay, N.DitBlockWeights(*good), 256, 1 << 20, (1 << 30) + 2, 0, big, need, None) == N.DIT_ERR_INVALID
    # the batched block and the loop check the same pointers
    arr = (N.DitLayout * 1)(lay)
    assert N.lib.dit_block_forward_batched(d, arr, 1, N.DitBlockWeights(*good), 256, (1 << 20) + 8,
                                           1 << 30, 0, big, need, None) == N.DIT_ERR_INVALID
    bad = list(good)
    bad[8] = 256 + 4
    blocks = (N.DitBlockWeights * 2)(N.DitBlockWeights(*good), N.DitBlockWeights(*bad))
    sig = (N.c_float * 2)(1.0, 0.0)
    need_l, _ = N.dit_workspace_size(d, lay, 2)
    code = N.lib.denoise_loop(d, lay, blocks, 2, 1, sig, sig, 256, N.make_policy("off"), 1 << 20, 0,
                              None, big, need_l, None)
    assert code == N.DIT_ERR_INVALID and "block 1" in N.last_error()
    code = N.lib.denoise_loop(d, lay, (N.DitBlockWeights * 1)(N.DitBlockWeights(*good)), 1, 1, sig,
                              sig, 256 + 8, N.make_policy("off"), 1 << 20, 0, None, big, need_l, None)
    assert code == N.DIT_ERR_INVALID
    # the head's norm gain, table, output weights and temb
    need_h = N.dit_head_workspace_size(d, lay, 64)
    g = N.lib.dit_velocity_head
    for head in (N.DitHeadWeights(256 + 4, 512, 1 << 24, 1 << 25, 64),
                 N.DitHeadWeights(256, 512 + 8, 1 << 24, 1 << 25, 64),
                 N.DitHeadWeights(256, 512, (1 << 24) + 8, 1 << 25, 64)):
        assert g(d, lay, head, 1 << 20, 1 << 32, 1 << 34, 1 << 30, need_h, None) == N.DIT_ERR_INVALID
    head = N.DitHeadWeights(256, 512, 1 << 24, 1 << 25, 64)
    assert g(d, lay, head, (1 << 20) + 4, 1 << 32, 1 << 34, 1 << 30, need_h, None) == N.DIT_ERR_INVALID


def test_noalloc_entry_point_rejects_oversize_blocks_before_device_work(N):
    """The no-allocation block entry point takes blocks whose workspace fits its built-in
    128 MiB scratch; larger ones are rejected with DIT_ERR_UNSUPPORTED before any device call
    (on this GPU-less machine a device call would give DIT_ERR_DEVICE); invalid dims get
    dit_block_forward's own status."""
    w = N.DitBlockWeights(*([256] * 9))
    d = N.make_dims(3072, 24, 128, 8192)
    lay = N.make_layout(30720, 2048, 32768)
    code = N.lib.dit_block_forward_noalloc(d, lay, w, 256, 1 << 20, 1 << 36, 0, None)
    assert code == N.DIT_ERR_UNSUPPORTED and "scratch" in N.last_error()
    d2 = N.make_dims(1024, 8, 128, 2816)
    n, _ = N.dit_workspace_size(d2, N.make_layout(4096, 512, 4608), 0)
    assert n <= N.NOALLOC_SCRATCH_BYTES          # the 4,608-token loop block fits
    bad = N.make_dims(256, 4, 96, 683)
    code = N.lib.dit_block_forward_noalloc(bad, N.make_layout(10, 0, 16), w, 256, 1 << 20, 1 << 30,
                                           0, None)
    assert code == N.DIT_ERR_UNSUPPORTED and "head_dim" in N.last_error()
    code = N.lib.dit_block_forward_noalloc(N.make_dims(256, 4, 64, 683), N.make_layout(20, 0, 16),
                                           w, 256, 1 << 20, 1 << 30, 0, None)
    assert code == N.DIT_ERR_INVALID
