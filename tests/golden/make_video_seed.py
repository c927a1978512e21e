"""Pick the seed of the video workload and store the float64 decisions for it.

Rule (fixed before any GPU result exists): the first seed 1400, 1401, ... whose
float64 oracle run keeps every similarity that decides a step more than
MARGIN away from gamma, so that no per-head reuse decision sits on a near-tie
that rounding in a bf16 pipeline could flip.  Writes ``video_seed.json`` next
to this file: the seed, the decision array [steps, batch, heads], the
similarities and the smallest margin.  Calls only the oracle and the seeded
input generator.

    python tests/golden/make_video_seed.py
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from cached_attention_fb_amd import workload as wl  # noqa: E402

MARGIN = 1e-3


def oracle_run(w, seed):
    inp = wl.generate(w, seed=seed)
    steps = [oracle.StepData(wl.to_f64(s.q), wl.to_f64(s.k), wl.to_f64(s.v), s.n_updated)
             for s in inp.blocks[0].steps]
    return oracle.run_block(wl.to_f64(inp.k_prefix), wl.to_f64(inp.v_prefix), w.prefix, steps,
                            oracle.GAMMA, gamma=w.gamma), inp.blocks[0].sigma


def deciding_margins(res, gamma):
    """|sim - gamma| for every similarity that decides a later step."""
    margins = []
    n_steps = res.reuse.shape[0]
    for s in range(1, n_steps - 1):
        sims = res.sim[s]
        margins.extend(np.abs(sims[~np.isnan(sims)] - gamma).tolist())
    return margins


def main():
    w = wl.WORKLOADS["video-1560x15600"]
    for seed in range(1400, 1500):
        t0 = time.time()
        res, sigma = oracle_run(w, seed)
        margins = deciding_margins(res, w.gamma)
        ok = min(margins) > MARGIN
        print(f"seed {seed}: min margin {min(margins):.3e} ({time.time() - t0:.1f}s) {'ok' if ok else 'rejected'}",
              flush=True)
        if ok:
            out = {
                "rule": "first seed >= 1400 whose float64 run keeps every deciding similarity "
                        f"more than {MARGIN} from gamma",
                "workload": w.name, "gamma": w.gamma, "seed": seed,
                "min_margin": min(margins),
                "sigma": sigma.tolist(),
                "reuse": res.reuse.astype(int).tolist(),
                "sim": [[[None if np.isnan(x) else float(x) for x in row] for row in st] for st in res.sim],
            }
            with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "video_seed.json"), "w") as f:
                json.dump(out, f, indent=1)
            return
    raise SystemExit("no seed passed the margin rule")


if __name__ == "__main__":
    main()
