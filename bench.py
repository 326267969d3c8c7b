#!/usr/bin/env python3
"""Benchmark of the cached joint audio-video DiT denoise loop on one MI355X.

A step is one full 49-interval denoise loop (conservative velocity reuse: 34 DiT calls and
15 reuses) of the 8-block stack at hidden 3072, 24 heads x 128, FFN 8192, over 32,768 packed
tokens (30,720 video + 2,048 audio), with seeded synthetic bf16 weights and inputs already
resident in device memory. ``value`` is the useful TFLOP/s of that loop: the matrix and
attention FLOPs of the executed blocks over the valid tokens (8VD^2 + 6VDF + 4V^2D per block;
reused intervals add nothing) divided by the wall time of the loop. The cache-off loop is
timed too, for steps/sec off vs conservative.

roofline: the attention kernel (the largest FLOP share of the block at this length), timed
with HIP events on the stream it runs on over repeated launches on the block's own q/k/v
layout; useful FLOPs 4 V^2 D per launch against the 2.5 PFLOP/s dense bf16 MFMA peak.
cpu_baseline: the float64 oracle on the host cores, one block of the same workload with a
sample of output rows (keys/values for every valid row), in the same useful-FLOP unit.
roofline.traffic: HBM bytes per attention launch from the committed counter summary
profiles/k_attn_traffic.json (FETCH_SIZE and WRITE_SIZE, scaled by the same counters on a
1 GiB device copy), reported only while that summary's recorded source hash matches the
current attention kernel source; otherwise null.

Prints ONE JSON line. --roofline-only runs just one block, the attention timing and the copy
used to calibrate the traffic counters (the command the counter runs profile).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "useful DiT TFLOP/s on 1 MI355X; denoise steps/sec (cache off vs conservative)"
BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--workload", default="loop_8blk_32k")
    p.add_argument("--attn-reps", type=int, default=10)
    p.add_argument("--cpu-rows", type=int, default=1024)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-off", action="store_true", help="skip the cache-off loop")
    p.add_argument("--roofline-only", action="store_true",
                   help="one block, the attention timing and the counter-calibration copy only")
    return p.parse_args()


ATTN_SRC = os.path.join(ROOT, "audio_video_diffusion_dit_amd", "csrc", "k_attention.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_attn_traffic.json")


def stored_traffic():
    """Bytes per attention launch from the committed counter summary, if it was taken on the
    current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        with open(ATTN_SRC, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != sha:
        return None
    return t.get("bytes_per_launch")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(case, rows_n):
    """Float64 oracle on the host cores: one block of the workload, rows_n sampled output rows."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    wl = case.wl
    V, D, F = wl.n_valid, wl.hidden, wl.ffn
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(V, rows_n, replace=False))
    blk = {k: np.asarray(v, dtype=np.float64) for k, v in case.blocks[0].as_float().items()}
    from audio_video_diffusion_dit_amd.inputs import bf16_bits, bf16_to_f32
    x = bf16_to_f32(bf16_bits(case.x0)).astype(np.float64)
    dims = O.Dims(D, wl.heads, wl.head_dim, F)
    lay = O.Layout(wl.n_video, wl.n_audio, wl.seq_pad)
    t0 = time.perf_counter()
    O.block_forward(x, blk, case.temb_steps[0], dims, lay, rows=rows)
    dt = time.perf_counter() - t0
    R = float(rows_n)
    flops = 4.0 * V * D * D + R * (4.0 * D * D + 6.0 * D * F + 4.0 * V * D)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"one block of {wl.name} (float64 NumPy): keys/values for all {V} valid rows, "
                      f"{rows_n} sampled output rows; {flops:.3e} useful FLOPs"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from audio_video_diffusion_dit_amd import _native as N
    from audio_video_diffusion_dit_amd import device as dev
    from audio_video_diffusion_dit_amd import inputs as I

    torch.cuda.set_device(0)
    wl = I.WORKLOADS[args.workload]
    log(f"[bench] generating {wl.name} inputs")
    if args.roofline_only:
        case = I.loop_case(wl, seed=0, n_blocks=1, n_intervals=2)
    else:
        case = I.loop_case(wl, seed=0)
    dims, lay = dev.dims_of(wl), dev.layout_of(wl)
    blocks = dev.upload_blocks(case.blocks)
    bw = [b.weights for b in blocks]
    temb = dev.to_dev_f32(case.temb_steps)
    x0 = dev.to_dev_f32(case.x0)
    x = torch.empty_like(x0)
    n = wl.n_intervals
    stream = torch.cuda.current_stream()
    per_block = 8.0 * wl.n_valid * wl.hidden ** 2 + 6.0 * wl.n_valid * wl.hidden * wl.ffn + \
        4.0 * float(wl.n_valid) ** 2 * wl.hidden

    t_c = t_o = flops_c = flops_o = None
    calls = hits = None
    if not args.roofline_only:
        ws, _ = dev.workspace(dims, lay, len(blocks))
        pol_c = N.make_policy("conservative")
        pol_o = N.make_policy("off")

        def run(pol):
            x.copy_(x0)
            return N.denoise_loop(dims, lay, bw, n, case.sigmas_video, case.sigmas_audio, temb,
                                  pol, x, N.DIT_ATTN_VALID_ONLY, ws, stream=stream,
                                  want_hits=False)[0]

        log(f"[bench] warmup x{args.warmup}")
        for _ in range(args.warmup):
            run(pol_c)
        torch.cuda.synchronize()
        log(f"[bench] timing {args.steps} conservative loops")
        t0 = time.perf_counter()
        for _ in range(args.steps):
            st = run(pol_c)
        torch.cuda.synchronize()
        t_c = (time.perf_counter() - t0) / args.steps
        flops_c = st.useful_flops
        assert abs(flops_c - st.executed_blocks * per_block) <= 1e-6 * flops_c
        calls, hits = st.dit_calls, st.cache_hits
        log(f"[bench] conservative: {t_c:.3f} s/loop, {flops_c / t_c / 1e12:.1f} TFLOP/s")
        if not args.no_off:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            so = run(pol_o)
            torch.cuda.synchronize()
            t_o = time.perf_counter() - t0
            flops_o = so.useful_flops
            log(f"[bench] off: {t_o:.3f} s/loop, {flops_o / t_o / 1e12:.1f} TFLOP/s")
        del ws

    # roofline: the attention kernel on the block's own qkv layout (filled by one block call)
    D, L, H, Dh = wl.hidden, wl.seq_pad, wl.heads, wl.head_dim
    xin = x0.to(torch.bfloat16)
    xout = torch.empty_like(xin)
    ws0, m0 = dev.workspace(dims, lay, 0)
    N.dit_block_forward(dims, lay, bw[0], temb[0], xin, xout, N.DIT_ATTN_VALID_ONLY, ws0, stream=stream)
    qkv = ws0.data_ptr() + m0.qkv
    att = ws0.data_ptr() + m0.attn_out

    def attn():
        N.dit_attention_forward(qkv, qkv + 2 * D, qkv + 4 * D, att, 1, L, H, Dh, L * 3 * D, 3 * D,
                                L * D, D, [wl.n_valid], N.DIT_ATTN_VALID_ONLY, stream=stream,
                                q_gain=bw[0].q_g, k_gain=bw[0].k_g)

    attn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.attn_reps):
        attn()
    e1.record(stream)
    torch.cuda.synchronize()
    t_attn = e0.elapsed_time(e1) / 1e3 / args.attn_reps
    attn_flops = 4.0 * float(wl.n_valid) ** 2 * D
    achieved = attn_flops / t_attn / 1e12
    log(f"[bench] attention kernel: {t_attn * 1e3:.3f} ms, {achieved:.1f} TFLOP/s")
    if args.roofline_only:
        # plain device copy of 1 GiB: calibrates FETCH_SIZE / WRITE_SIZE for the traffic figure
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline and not args.roofline_only:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(case, args.cpu_rows)

    out = {
        "metric": METRIC,
        "value": round(flops_c / t_c / 1e12, 2) if t_c else None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_c * 1e3, 2) if t_c else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, N(0,1) latent; no checkpoint)",
        "config": {"workload": wl.name, "hidden": D, "heads": H, "head_dim": Dh, "ffn": wl.ffn,
                   "n_video": wl.n_video, "n_audio": wl.n_audio, "seq_pad": L,
                   "blocks": wl.n_blocks, "intervals": n, "cache": "conservative",
                   "global_batch": 1, "seq_len": wl.n_valid, "parallelism": "single GPU"},
        "steps_per_sec_conservative": round(n / t_c, 3) if t_c else None,
        "steps_per_sec_off": round(n / t_o, 3) if t_o else None,
        "tflops_off": round(flops_o / t_o / 1e12, 2) if t_o else None,
        "dit_calls": calls,
        "cache_hits": hits,
        "roofline": {"kernel": "avdit::k_attn<128> (valid-only attention, 4 V^2 D flop/launch)",
                     "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": stored_traffic(),
                     "launch_ms": round(t_attn * 1e3, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
