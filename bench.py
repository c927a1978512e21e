"""Benchmark of the FlashBlock denoising-step attention on one MI355X.

A bench step is one denoising step of the attention path (reuse decision,
block-external attention for the heads that recompute, block-internal
attention with the log-space merge) for every layer of a stack of
independent attention layers of the workload's shape.  The timed steps walk
through the workload's seeded block of steps in order; every ``steps per
block`` steps the caches are reset and the block starts again on the same
prefix.  The stack holds enough layers that their prefix K/V exceed the
256 MB MALL, as the layers of a model do, so every step streams its K/V from
HBM without a cache flush in the timed region.

Printed: one JSON line.  ``value`` is the effective KV bandwidth: the prefix
K/V bytes a recompute-every-step (ALWAYS) run would read, divided by the time
taken under the workload's reuse policy.  ``roofline`` reports the external
attention kernel's algorithmic bytes per launch over its average launch
duration (HIP events around each launch on its stream, in a profiled pass of
the same steps under ALWAYS).  ``cpu_baseline`` times the float64 oracle on
a bounded sample on the host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dllm-8k]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "denoise-step attention µs & effective KV GB/s (% of HBM roofline), reuse vs full"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
FP32_PEAK_TFLOPS = 157.3
MALL_BYTES = 256 << 20


def kernel_source_hash() -> str:
    """Hash of the kernel sources: stored traffic counters apply only to the
    kernels they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "cached_attention_fb_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def algorithmic(w, n_prefix):
    """Algorithmic work of one full external attention: K+V read once per
    (sequence, kv head), Q read, A_out (fp32) and L_out (fp32) written."""
    e = w.elem_bytes
    kv = 2 * w.batch * w.n_kv_heads * n_prefix * w.head_dim * e
    q = w.batch * w.n_q_heads * w.block * w.head_dim * e
    out = w.batch * w.n_q_heads * w.block * (w.head_dim + 1) * 4
    flops = 4.0 * w.batch * w.n_q_heads * w.block * n_prefix * w.head_dim
    return kv, kv + q + out, flops


def run(args):
    import torch
    from cached_attention_fb_amd import fb
    from cached_attention_fb_amd import workload as wl

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    w = wl.workload(args.workload)
    inp = wl.generate(w)
    blk = inp.blocks[0]
    S = len(blk.steps)
    n = w.prefix
    kv_bytes, alg_bytes, alg_flops = algorithmic(w, n)
    layers = args.layers or max(1, math.ceil(2.5 * MALL_BYTES / kv_bytes))
    dev = "cuda"
    dt = w.torch_dtype
    policy = {"tau": fb.POLICY_TAU, "gamma": fb.POLICY_GAMMA, "always": fb.POLICY_ALWAYS}[args.policy or w.policy]

    # device inputs: per-layer prefix K/V and caches; step inputs shared by the layers
    kp0 = inp.k_prefix.to(dev)
    vp0 = inp.v_prefix.to(dev)
    prefixes = [(kp0, vp0)] + [(kp0.clone(), vp0.clone()) for _ in range(layers - 1)]
    del inp
    caches = [fb.Cache(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block, n, dt, kv_splits=args.splits)
              for _ in range(layers)]
    qs = [st.q.to(dev) for st in blk.steps]
    ks = [st.k.to(dev) for st in blk.steps]
    vs = [st.v.to(dev) for st in blk.steps]
    ms = [np.ascontiguousarray(st.n_updated, dtype=np.int32) for st in blk.steps]
    outs = [torch.empty_like(qs[0]) for _ in range(layers)]
    # buffers checked once; each call then marshals only scalars
    prepared = [[c.prepare(qs[s], ks[s], vs[s], prefixes[li][0], prefixes[li][1], outs[li]) for s in range(S)]
                for li, c in enumerate(caches)]
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()

    state = {"s": 0}

    def step(pol):
        s = state["s"]
        m = ms[s]
        for li, c in enumerate(caches):
            if s == 0:
                c.reset(stream)
            prepared[li][s](pol, n, m, w.tau, w.gamma, stream)
        state["s"] = (s + 1) % S

    def timed(pol, k_steps):
        state["s"] = 0
        for _ in range(args.warmup):
            step(pol)
        state["s"] = 0
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(k_steps):
            step(pol)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall, e0.elapsed_time(e1) / 1e3

    wall, gpu_s = timed(policy, args.steps)
    wall_always, gpu_always = timed(fb.POLICY_ALWAYS, args.steps)

    # decisions of one block under the policy (from the caches' own record)
    state["s"] = 0
    reuse_counts = []
    for s in range(S):
        step(policy)
        reuse_counts.append(int(caches[0].read(fb.FIELD_REUSE).sum()))

    # profiled pass: HIP events around every launch, ALWAYS policy (every step launches the external kernel)
    for c in caches:
        c.profile_enable(True)
    state["s"] = 0
    for _ in range(args.steps):
        step(fb.POLICY_ALWAYS)
    torch.cuda.synchronize()
    prof = {}
    for c in caches:
        for kname, (cnt, tms) in c.profile_read().items():
            a, b = prof.get(kname, (0, 0.0))
            prof[kname] = (a + cnt, b + tms)
        c.profile_enable(False)
    ext_n, ext_ms = prof["external"]
    ext_us = 1e3 * ext_ms / max(1, ext_n)
    kernel_us = {k: round(1e3 * v[1] / v[0], 3) for k, v in prof.items() if v[0]}

    bound_flops = alg_flops / (BF16_PEAK_TFLOPS * 1e12 if w.dtype == "bf16" else FP32_PEAK_TFLOPS * 1e12)
    bound_bytes = alg_bytes / (HBM_PEAK_GBS * 1e9)
    if bound_flops > bound_bytes:
        peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
        achieved = alg_flops / (ext_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s"}
    else:
        achieved = alg_bytes / (ext_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = "attn_kernel (external, split-KV partials)"
    roof["avg_launch_us"] = round(ext_us, 3)
    roof["algorithmic_bytes_per_launch"] = alg_bytes
    roof["traffic"] = None
    pmc = os.path.join(ROOT, "profiles", f"pmc_{w.name}.json")
    if os.path.exists(pmc):
        with open(pmc) as f:
            rec = json.load(f)
        if rec.get("kernel_source_hash") == kernel_source_hash():
            roof["traffic"] = rec.get("hbm_bytes_per_launch")

    per_step_s = gpu_s / args.steps
    per_layer_step_us = 1e6 * per_step_s / layers
    always_layer_step_us = 1e6 * gpu_always / args.steps / layers
    eff_gbs = kv_bytes * layers * args.steps / gpu_s / 1e9

    result = {
        "metric": METRIC,
        "value": round(eff_gbs, 1),
        "unit": "GB/s (effective prefix-KV bandwidth under the reuse policy)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * per_step_s, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; random values of the workload's distributions)",
        "config": {"workload": w.name, "shape": w.description, "policy": args.policy or w.policy,
                   "tau": w.tau, "gamma": w.gamma, "layers": layers,
                   "kv_bytes_per_layer": kv_bytes, "prefix": n},
        "us_per_layer_step": round(per_layer_step_us, 3),
        "always_us_per_layer_step": round(always_layer_step_us, 3),
        "reuse_vs_full_speedup": round(always_layer_step_us / per_layer_step_us, 3),
        "reused_heads_per_step": reuse_counts,
        "wall_s": round(wall, 4),
        "kernel_avg_us_always": kernel_us,
        "roofline": roof,
    }
    for c in caches:
        c.close()
    return result, w


def cpu_baseline(w, budget_s: float):
    """The float64 oracle on the host cores, on one block of the same workload
    over a sample of heads; scaled to all heads."""
    import oracle
    from threadpoolctl import threadpool_info
    from cached_attention_fb_amd import workload as wl

    inp = wl.generate(w)
    blk = inp.blocks[0]
    kv_bytes, _, _ = algorithmic(w, w.prefix)
    heads = [(b, h) for b in range(w.batch) for h in range(w.n_q_heads)]
    done, t_total = 0, 0.0
    for (b, h) in heads:
        g = h // w.group
        steps = [oracle.StepData(wl.to_f64(s.q[b:b + 1, h:h + 1]), wl.to_f64(s.k[b:b + 1, g:g + 1]),
                                 wl.to_f64(s.v[b:b + 1, g:g + 1]), np.asarray(s.n_updated)[b:b + 1])
                 for s in blk.steps]
        kp = wl.to_f64(inp.k_prefix[b:b + 1, g:g + 1])
        vp = wl.to_f64(inp.v_prefix[b:b + 1, g:g + 1])
        t0 = time.perf_counter()
        oracle.run_block(kp, vp, w.prefix, steps, w.policy, tau=w.tau, gamma=w.gamma)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total > budget_s:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    block_s = t_total * len(heads) / done
    gbs = kv_bytes * len(blk.steps) / block_s / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s (effective prefix-KV bandwidth under the reuse policy)",
            "cores": threads, "kind": "oracle",
            "sample": f"one block of {len(blk.steps)} steps for {done} of {len(heads)} heads "
                      f"({t_total:.1f} s), scaled to all heads; os.cpu_count()={os.cpu_count()}, "
                      f"affinity={len(os.sched_getaffinity(0))}",
            "us_per_layer_step": round(1e6 * block_s / len(blk.steps), 1)}


def calibrate():
    """A plain elementwise kernel of known traffic (reads 256 MiB, writes
    256 MiB), run under the same counters as the attention kernels to scale
    FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch
    x = torch.ones(128 << 20, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        torch.mul(x, 2.0, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "torch.mul bf16, 256 MiB read + 256 MiB written per launch", "launches": 3}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="dllm-8k")
    ap.add_argument("--policy", default=None, choices=[None, "tau", "gamma", "always"])
    ap.add_argument("--layers", type=int, default=0, help="0: enough layers to exceed 2.5x the MALL")
    ap.add_argument("--splits", type=int, default=0, help="0: automatic split-KV count")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate", action="store_true", help="only run the known-traffic reference kernel")
    args = ap.parse_args()
    if args.calibrate:
        calibrate()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus above 1 is not supported "
                                   "(the path would shard by (sequence, kv head) or by prefix chunk)"}))
        raise SystemExit(2)
    result, w = run(args)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
