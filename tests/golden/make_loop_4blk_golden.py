"""Writes ``loop_4blk_final_rows.json``: sampled rows of the final latent of the 4-block,
4,608-token, 49-interval denoise loop (hidden 1024, 8 x 128 heads, FFN 2816, seed 0), with the
cache off and with the conservative policy, computed by the float64 oracle only.

The conservative run is TeleFuser PR #38's policy (section 3: start 0.2, end 0.8, refresh every
2nd interval, at most one reuse in a row; section 1: 34 DiT calls and 15 reuses over 49
intervals). The file also holds the oracle's conservative-vs-off comparison of the two final
latents over all valid rows (cosine, relative L2 and PSNR, defined below), the latent-level
stand-in for the media comparison of section 5, which is made on decoded videos and audio and
cannot be reproduced here.

Run from the repository root: ``python tests/golden/make_loop_4blk_golden.py`` (about 15 minutes
on 8 cores). It imports only ``oracle`` and the seeded input generators.
"""

from __future__ import annotations

import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle as O  # noqa: E402
from audio_video_diffusion_dit_amd import inputs as I  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "loop_4blk_final_rows.json")
SEED = 0


def sampled_rows(wl) -> list:
    """First and last row of each modality, plus eight rows drawn with seed 23."""
    V = wl.n_valid
    fixed = [0, wl.n_video - 1, wl.n_video, V - 1]
    rng = np.random.default_rng(23)
    extra = rng.choice(np.setdiff1d(np.arange(V), fixed), 8, replace=False)
    return sorted(int(r) for r in np.concatenate([fixed, extra]))


def compare(a: np.ndarray, ref: np.ndarray) -> dict:
    """cosine, relative L2 = |a - ref| / |ref|, and PSNR = 10 log10(peak^2 / MSE) with the
    peak max |ref| (all over the given rows)."""
    a = np.asarray(a, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    d = a - ref
    mse = float(np.mean(d * d))
    peak = float(np.max(np.abs(ref)))
    return dict(cosine=float(a @ ref / (np.linalg.norm(a) * np.linalg.norm(ref))),
                rel_l2=float(np.linalg.norm(d) / np.linalg.norm(ref)),
                psnr_db=float(10.0 * math.log10(peak * peak / mse)) if mse > 0 else float("inf"))


def run(case, mode: str):
    wl = case.wl
    dims = O.Dims(wl.hidden, wl.heads, wl.head_dim, wl.ffn, wl.norm_eps, wl.qk_eps, wl.rope_base)
    lay = O.Layout(wl.n_video, wl.n_audio, wl.seq_pad)
    blocks = [{k: np.asarray(v, dtype=np.float64) for k, v in b.as_float().items()}
              for b in case.blocks]
    hits = O.cache_schedule(O.CachePolicy(mode=mode), wl.n_intervals)
    t0 = time.time()

    def velocity(i, xb):
        print(f"  {mode}: interval {i} (DiT call), {time.time() - t0:.0f} s", flush=True)
        return O.stack_forward(xb, blocks, case.temb_steps[i], dims, lay)

    x, _ = O.denoise_loop(case.x0, velocity, case.sigmas_video, case.sigmas_audio,
                          O.row_modality(lay), hits)
    return x, hits


def main() -> None:
    wl = I.WORKLOADS["loop_4blk"]
    case = I.loop_case(wl, seed=SEED)
    rows = sampled_rows(wl)
    x_off, h_off = run(case, "off")
    x_con, h_con = run(case, "conservative")
    V = wl.n_valid
    doc = {
        "workload": dict(name=wl.name, hidden=wl.hidden, heads=wl.heads, head_dim=wl.head_dim,
                         ffn=wl.ffn, n_video=wl.n_video, n_audio=wl.n_audio,
                         seq_pad=wl.seq_pad, n_blocks=wl.n_blocks,
                         n_intervals=wl.n_intervals, seed=SEED),
        "written_by": "tests/golden/make_loop_4blk_golden.py (float64 oracle only)",
        "rows": rows,
        "hits_conservative": [int(h) for h in h_con],
        "hits_off": [int(h) for h in h_off],
        "final_off": [[float(f"{v:.8e}") for v in x_off[r]] for r in rows],
        "final_conservative": [[float(f"{v:.8e}") for v in x_con[r]] for r in rows],
        "conservative_vs_off_all_valid_rows": compare(x_con[:V], x_off[:V]),
    }
    with open(OUT, "w") as f:
        json.dump(doc, f, separators=(",", ":"))
        f.write("\n")
    print(f"wrote {OUT}: {doc['conservative_vs_off_all_valid_rows']}", flush=True)


if __name__ == "__main__":
    main()
