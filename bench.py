"""Benchmark of the FlashBlock denoising-step attention on one MI355X.

A bench step is one denoising step of the attention path (reuse decision,
block-external attention for the heads that recompute, split combine,
block-internal attention with the log-space merge) for every layer of a stack
of independent attention layers of the workload's shape.  The timed steps walk
through the workload's seeded block of steps in order; every ``steps per
block`` steps the caches are reset and the block starts again on the same
prefix.  The stack holds enough layers that their prefix K/V exceed the
256 MB MALL, as the layers of a model do, so every step streams its K/V from
HBM without a cache flush in the timed region.

Printed: one JSON line for the headline workload, the largest single-GPU
one (max-128k: batch 1, 32/8 heads, D=128, prefix 131072, block 64).
``value`` is the effective KV bandwidth: the prefix K/V bytes a
recompute-every-step (ALWAYS) run would read, divided by the time taken under
the workload's reuse policy (it counts the bytes a reuse step does not read,
so it can exceed the HBM peak).  ``roofline`` reports the recompute step's
attention launch (block-external split-KV items plus the block-internal items
it carries): algorithmic bytes per launch over its average launch duration
(HIP events around each launch on its stream, in a profiled pass of the same
steps under ALWAYS); its ``frac`` is the share of the HBM (or MFMA) roofline.
``step_us`` gives median, p10 and p90 of at least 50 timed steps per kind.
``cpu_baseline`` times the float64 oracle on the host cores.  ``workloads``
holds the same step and kernel figures, from fewer steps, for the other
workloads.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload max-128k] [--no-extra]
    python bench.py --always-only --workload NAME --steps K   (recompute steps only, for rocprofv3)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "denoise-step attention µs & effective KV GB/s (% of HBM roofline), reuse vs full"
UNIT = "GB/s (effective prefix-KV bandwidth under the reuse policy)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
FP32_PEAK_TFLOPS = 157.3
MALL_BYTES = 256 << 20
EXTRA = ["long-32k-b4", "dllm-8k", "video-1560x15600", "tiny-fp32"]
HEADLINE = "max-128k"
PERCENTILE_REPS = 50


def _code_text(src: str) -> str:
    """Source text without comments and with whitespace collapsed: what the
    compiler sees (no string literal in the kernel sources holds // or /*)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code (comments and layout ignored): stored
    traffic counters apply only to the kernels they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "cached_attention_fb_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), encoding="utf-8") as f:
                h.update(name.encode() + _code_text(f.read()).encode())
    return h.hexdigest()[:16]


def algorithmic(w, n_prefix):
    """Algorithmic work of one recompute-step attention launch, which holds
    the block-external attention of every head and (fused step) its
    block-internal attention: prefix K+V read once per (sequence, kv head),
    block K+V and Q read, and the two results (A, L in fp32) written.
    Returns (prefix K/V bytes, bytes of the launch, flops of the launch)."""
    e = w.elem_bytes
    kv = 2 * w.batch * w.n_kv_heads * n_prefix * w.head_dim * e
    kv_blk = 2 * w.batch * w.n_kv_heads * w.block * w.head_dim * e
    q = w.batch * w.n_q_heads * w.block * w.head_dim * e
    out = 2 * w.batch * w.n_q_heads * w.block * (w.head_dim + 1) * 4
    flops = 4.0 * w.batch * w.n_q_heads * w.block * (n_prefix + w.block) * w.head_dim
    return kv, kv + kv_blk + q + out, flops


def roofline(w, ext_us, alg_bytes, alg_flops):
    """Roofline entry of the external kernel: the bound is whichever of HBM
    bytes or MFMA flops takes longer at the published peaks."""
    peak_f = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    if alg_flops / (peak_f * 1e12) > alg_bytes / (HBM_PEAK_GBS * 1e9):
        achieved = alg_flops / (ext_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_f, "unit": "TFLOP/s"}
    else:
        achieved = alg_bytes / (ext_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    return roof


def measure(name, steps, warmup, policy_name=None, layers=0, splits=0, decisions=True):
    """Time `steps` bench steps of workload `name` under its policy and under
    ALWAYS, then a profiled ALWAYS pass (HIP events around every launch)."""
    import torch
    from cached_attention_fb_amd import fb
    from cached_attention_fb_amd import workload as wl

    w = wl.workload(name)
    inp = wl.generate(w)
    blk = inp.blocks[0]
    S = len(blk.steps)
    n = w.prefix
    kv_bytes, alg_bytes, alg_flops = algorithmic(w, n)
    layers = layers or max(1, math.ceil(2.5 * MALL_BYTES / kv_bytes))
    dev = "cuda"
    policy_name = policy_name or w.policy
    policy = {"tau": fb.POLICY_TAU, "gamma": fb.POLICY_GAMMA, "always": fb.POLICY_ALWAYS,
              "tau_cum": fb.POLICY_TAU_CUM, "gamma_group": fb.POLICY_GAMMA_GROUP}[policy_name]

    # device inputs: per-layer prefix K/V and caches; step inputs shared by the layers
    kp0 = inp.k_prefix.to(dev)
    vp0 = inp.v_prefix.to(dev)
    prefixes = [(kp0, vp0)] + [(kp0.clone(), vp0.clone()) for _ in range(layers - 1)]
    caches = [fb.Cache(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block, n, w.torch_dtype,
                       kv_splits=splits) for _ in range(layers)]
    qs = [st.q.to(dev) for st in blk.steps]
    ks = [st.k.to(dev) for st in blk.steps]
    vs = [st.v.to(dev) for st in blk.steps]
    ms = [np.ascontiguousarray(st.n_updated, dtype=np.int32) for st in blk.steps]
    del inp, blk
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

    def timed(pol):
        state["s"] = 0
        for _ in range(warmup):
            step(pol)
        state["s"] = 0
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            step(pol)
        e1.record()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, e0.elapsed_time(e1) / 1e3

    def profiled(pol):
        """One more pass like the timed one with HIP events around every
        launch: per profile kind, (launches, ms)."""
        for c in caches:
            c.profile_enable(True)
        state["s"] = 0
        for _ in range(steps):
            step(pol)
        torch.cuda.synchronize()
        prof = {}
        for c in caches:
            for kname, (cnt, tms) in c.profile_read().items():
                a, b = prof.get(kname, (0, 0.0))
                prof[kname] = (a + cnt, b + tms)
            c.profile_enable(False)
        return prof

    wall, gpu_s = timed(policy)
    # the timed region's own recompute launches, in its own mix of steps (a
    # repeat of it, profiled): the roofline's launch duration
    prof_pol = profiled(policy)
    _, gpu_always = timed(fb.POLICY_ALWAYS)

    reuse_counts = []
    step_stats = None
    if decisions:   # decisions of one block under the policy (the caches' own record)
        state["s"] = 0
        for _ in range(S):
            step(policy)
            reuse_counts.append(int(caches[0].read(fb.FIELD_REUSE).sum()))
        # per-step times (HIP events around each step of all layers), split into
        # steps where some head recomputes ("full") and steps where all reuse,
        # whole blocks at a time until each kind has PERCENTILE_REPS samples
        # (or the block has none of that kind); then always-recompute steps
        nh = w.batch * w.n_q_heads
        n_full_blk = sum(1 for c in reuse_counts if c != nh)
        n_reuse_blk = S - n_full_blk
        need = max(math.ceil(PERCENTILE_REPS / max(1, n)) for n in
                   ([n_full_blk] if n_full_blk else []) + ([n_reuse_blk] if n_reuse_blk else []))
        reps = S * min(need, 64)

        def per_step(pol, count):
            state["s"] = 0
            for _ in range(S):
                step(pol)
            state["s"] = 0
            torch.cuda.synchronize()
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(count + 1)]
            evs[0].record()
            for i in range(count):
                step(pol)
                evs[i + 1].record()
            torch.cuda.synchronize()
            return [1e3 * evs[i].elapsed_time(evs[i + 1]) / layers for i in range(count)]

        times = per_step(policy, reps)
        full = [t for i, t in enumerate(times) if reuse_counts[i % S] != nh]
        reuse = [t for i, t in enumerate(times) if reuse_counts[i % S] == nh]
        always = per_step(fb.POLICY_ALWAYS, max(PERCENTILE_REPS, S))

        def pct(xs):
            if not xs:
                return None
            return {"median": round(float(np.median(xs)), 3), "p10": round(float(np.percentile(xs, 10)), 3),
                    "p90": round(float(np.percentile(xs, 90)), 3), "n": len(xs)}

        step_stats = {"full": pct(full), "all_reuse": pct(reuse), "always": pct(always)}

    # profiled pass under ALWAYS: every step launches the external kernel
    # (sustained recompute: the chip runs hotter and clocks lower than in the
    # policy's mix)
    prof = profiled(fb.POLICY_ALWAYS)
    ext_us_always = 1e3 * prof["external"][1] / max(1, prof["external"][0])
    kernel_us = {k: round(1e3 * v[1] / v[0], 3) for k, v in prof.items() if v[0]}
    kernel_us_pol = {k: round(1e3 * v[1] / v[0], 3) for k, v in prof_pol.items() if v[0]}
    # The policy pass's launches are whole recompute launches (the algorithmic
    # work per launch) when decisions are per sequence and there is one
    # sequence; otherwise (several sequences, or per-head decisions) a launch
    # may cover only some heads, and the always pass stands in, as it does
    # when the policy's pass recomputes nowhere.
    whole = w.batch == 1 and policy_name in ("tau", "tau_cum", "always") and "external" in kernel_us_pol
    ext_us = kernel_us_pol["external"] if whole else ext_us_always
    for c in caches:
        c.close()
    del prepared, caches, prefixes, kp0, vp0, qs, ks, vs, outs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    roof = roofline(w, ext_us, alg_bytes, alg_flops)
    roof["kernel"] = ("attn_bf16_kernel" if w.dtype == "bf16" else "attn_f32_kernel") + \
        " (recompute step: block-external split-KV partials + block-internal items)"
    roof["avg_launch_us"] = round(ext_us, 3)
    roof["launches"] = prof_pol["external"][0] if whole else prof["external"][0]
    roof["pass"] = policy_name if whole else "always"
    roof["algorithmic_bytes_per_launch"] = alg_bytes
    roof["algorithmic_flops_per_launch"] = alg_flops
    roof_always = roofline(w, ext_us_always, alg_bytes, alg_flops)
    roof_always["avg_launch_us"] = round(ext_us_always, 3)
    return {
        "w": w, "layers": layers, "kv_bytes": kv_bytes, "gpu_s": gpu_s, "wall_s": wall,
        "per_layer_step_us": 1e6 * gpu_s / steps / layers,
        "always_layer_step_us": 1e6 * gpu_always / steps / layers,
        "eff_gbs": kv_bytes * layers * steps / gpu_s / 1e9, "reuse_counts": reuse_counts,
        "kernel_us": kernel_us, "kernel_us_policy": kernel_us_pol, "roofline": roof,
        "roofline_always": roof_always, "policy": policy_name, "step_stats": step_stats,
    }


def graph_bench(name, blocks=8, warmup=2):
    """Threshold decisions made on the device (counts in device memory), run
    eagerly and as one HIP graph per block (reset + every step of every layer,
    recorded by stream capture), beside host decisions run eagerly: µs per
    layer-step under the workload's threshold and under always-recompute, and
    the host's time per fb_step call while enqueueing."""
    import torch
    from cached_attention_fb_amd import fb
    from cached_attention_fb_amd import workload as wl

    w = wl.workload(name)
    inp = wl.generate(w)
    blk = inp.blocks[0]
    S = len(blk.steps)
    n = w.prefix
    kv_bytes, _, _ = algorithmic(w, n)
    layers = max(1, math.ceil(2.5 * MALL_BYTES / kv_bytes))
    pol = {"tau": fb.POLICY_TAU, "tau_cum": fb.POLICY_TAU_CUM}[w.policy]
    dev = "cuda"
    kp0 = inp.k_prefix.to(dev)
    vp0 = inp.v_prefix.to(dev)
    prefixes = [(kp0, vp0)] + [(kp0.clone(), vp0.clone()) for _ in range(layers - 1)]
    caches = [fb.Cache(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block, n, w.torch_dtype)
              for _ in range(layers)]
    qs = [st.q.to(dev) for st in blk.steps]
    ks = [st.k.to(dev) for st in blk.steps]
    vs = [st.v.to(dev) for st in blk.steps]
    ms_host = [np.ascontiguousarray(st.n_updated, dtype=np.int32) for st in blk.steps]
    ms_dev = [torch.as_tensor(m).to(dev) for m in ms_host]
    ms_ptr = [m.data_ptr() for m in ms_dev]
    del inp, blk
    outs = [torch.empty_like(qs[0]) for _ in range(layers)]
    prepared = [[c.prepare(qs[s], ks[s], vs[s], prefixes[li][0], prefixes[li][1], outs[li]) for s in range(S)]
                for li, c in enumerate(caches)]

    def block(mode, stream):
        for s in range(S):
            for li in range(layers):
                if s == 0:
                    caches[li].reset(stream)
                if mode == "host":
                    prepared[li][s](pol, n, ms_host[s], w.tau, 0.0, stream)
                elif mode == "device":
                    prepared[li][s](pol, n, None, w.tau, 0.0, stream, n_updated_dev=ms_ptr[s])
                else:
                    prepared[li][s](fb.POLICY_ALWAYS, n, None, 0, 0.0, stream)

    cur = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        t0 = time.perf_counter()
        for _ in range(blocks):
            fn()
        t1 = time.perf_counter()
        e1.record()
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / (blocks * S * layers), 1e6 * (t1 - t0) / (blocks * S * layers)

    res = {"workload": name, "layers": layers, "steps_per_block": S, "blocks": blocks}
    for mode in ("host", "device", "always"):
        us, enq = timed(lambda: block(mode, cur.cuda_stream))
        res[f"eager_{mode}_us_per_layer_step"] = round(us, 3)
        res[f"eager_{mode}_enqueue_us_per_call"] = round(enq, 3)
    side = torch.cuda.Stream()
    for mode in ("device", "always"):
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            block(mode, side.cuda_stream)
        torch.cuda.synchronize()
        us, enq = timed(g.replay)
        res[f"graph_{mode}_us_per_layer_step"] = round(us, 3)
        del g
    res["graph_reuse_vs_full_speedup"] = round(res["graph_always_us_per_layer_step"] /
                                               res["graph_device_us_per_layer_step"], 3)
    for c in caches:
        c.close()
    del prepared, caches, prefixes, kp0, vp0, qs, ks, vs, outs, ms_dev
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def sparse_bench(name, densities=(0.2, 0.3, 0.4), blocks=4, warmup=1):
    """FlashBlock over a sparse attention (fb_step_sparse): synthetic tile
    selections at several densities, every layer its own.  Per density: µs
    per layer-step under the workload's threshold and under always-recompute,
    and the kept-tile attention kernel (HIP events, profiled threshold pass)
    against the HBM roofline of its kept K/V; beside them the dense path
    under the same threshold."""
    import torch
    from cached_attention_fb_amd import fb
    from cached_attention_fb_amd import workload as wl

    w = wl.workload(name)
    inp = wl.generate(w)
    blk = inp.blocks[0]
    S = len(blk.steps)
    n = w.prefix
    kv_bytes, _, _ = algorithmic(w, n)
    layers = max(1, math.ceil(2.5 * MALL_BYTES / kv_bytes))
    pol = {"tau": fb.POLICY_TAU, "tau_cum": fb.POLICY_TAU_CUM}[w.policy]
    dev = "cuda"
    kp0 = inp.k_prefix.to(dev)
    vp0 = inp.v_prefix.to(dev)
    prefixes = [(kp0, vp0)] + [(kp0.clone(), vp0.clone()) for _ in range(layers - 1)]
    caches = [fb.Cache(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block, n, w.torch_dtype)
              for _ in range(layers)]
    qs = [st.q.to(dev) for st in blk.steps]
    ks = [st.k.to(dev) for st in blk.steps]
    vs = [st.v.to(dev) for st in blk.steps]
    ms = [np.ascontiguousarray(st.n_updated, dtype=np.int32) for st in blk.steps]
    del inp, blk
    outs = [torch.empty_like(qs[0]) for _ in range(layers)]

    def run(prepared, policy, n_blocks):
        for _ in range(n_blocks):
            for s in range(S):
                for li in range(layers):
                    if s == 0:
                        caches[li].reset()
                    prepared[li][s](policy, n, ms[s], w.tau, 0.0)

    def timed(prepared, policy):
        run(prepared, policy, warmup)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run(prepared, policy, blocks)
        e1.record()
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / (blocks * S * layers)

    dense = [[c.prepare(qs[s], ks[s], vs[s], prefixes[li][0], prefixes[li][1], outs[li]) for s in range(S)]
             for li, c in enumerate(caches)]
    res = {"workload": name, "layers": layers, "policy": w.policy, "tau": w.tau,
           "dense_tau_us_per_layer_step": round(timed(dense, pol), 3),
           "dense_always_us_per_layer_step": round(timed(dense, fb.POLICY_ALWAYS), 3), "densities": {}}
    del dense
    for dens in densities:
        sels = [torch.as_tensor(wl.sparse_selection(w, n, dens, seed=w.seed + li)).to(dev).contiguous()
                for li in range(layers)]
        n_sel = int(sels[0].shape[2])
        prep = [[c.prepare(qs[s], ks[s], vs[s], prefixes[li][0], prefixes[li][1], outs[li], sel_tiles=sels[li])
                 for s in range(S)] for li, c in enumerate(caches)]
        tau_us = timed(prep, pol)
        always_us = timed(prep, fb.POLICY_ALWAYS)
        for c in caches:
            c.profile_enable(True)
        run(prep, pol, 1)
        torch.cuda.synchronize()
        prof = {}
        for c in caches:
            for kname, (cnt, tms) in c.profile_read().items():
                a, b = prof.get(kname, (0, 0.0))
                prof[kname] = (a + cnt, b + tms)
            c.profile_enable(False)
        kern = {k: round(1e3 * v[1] / v[0], 3) for k, v in prof.items() if v[0]}
        kept_rows = min(n, n_sel * 64)
        kept_roof = None
        if "sparse_kept" in kern:   # the kept tiles' launch also carries the block-internal items
            _, kept_bytes, kept_flops = algorithmic(w, kept_rows)
            kept_roof = roofline(w, kern["sparse_kept"], kept_bytes, kept_flops)
        res["densities"][str(dens)] = {
            "kept_tiles": n_sel, "kept_fraction": round(n_sel * 64 / n, 4),
            "tau_us_per_layer_step": round(tau_us, 3), "always_us_per_layer_step": round(always_us, 3),
            "reuse_vs_full_speedup": round(always_us / tau_us, 3), "kernel_avg_us_tau": kern,
            "kept_attention_roofline": kept_roof}
        del prep, sels
    for c in caches:
        c.close()
    del caches, prefixes, kp0, vp0, qs, ks, vs, outs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def staleness(name, policies):
    """Output error of each reuse policy against always-recompute on the same
    seeded block (one layer): max |out - out_always| / max |out_always| and the
    RMS error over the RMS of out_always, over the block's steps, and the
    fraction of (step, head) pairs that reused."""
    import torch
    from cached_attention_fb_amd import fb
    from cached_attention_fb_amd import workload as wl

    codes = {"always": fb.POLICY_ALWAYS, "tau": fb.POLICY_TAU, "gamma": fb.POLICY_GAMMA,
             "tau_cum": fb.POLICY_TAU_CUM, "gamma_group": fb.POLICY_GAMMA_GROUP}
    w = wl.workload(name)
    inp = wl.generate(w)
    blk = inp.blocks[0]
    kp, vp = inp.k_prefix.cuda(), inp.v_prefix.cuda()
    cache = fb.Cache(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block, w.prefix, w.torch_dtype)
    outs = {}
    reuse = {}
    for pol in ("always",) + tuple(policies):
        cache.reset()
        o, r = [], []
        for st in blk.steps:
            out = torch.empty_like(st.q, device="cuda")
            cache.step(codes[pol], st.q.cuda(), st.k.cuda(), st.v.cuda(), kp, vp, w.prefix, out,
                       tau=w.tau, gamma=w.gamma, n_updated=st.n_updated)
            o.append(out.float().cpu())
            r.append(cache.read(fb.FIELD_REUSE).astype(np.int64))
        outs[pol], reuse[pol] = torch.stack(o), np.stack(r)
    cache.close()
    ref = outs["always"]
    scale = float(ref.abs().max())
    rms = float(ref.pow(2).mean().sqrt())
    return {pol: {"max_rel_err_vs_always": round(float((outs[pol] - ref).abs().max()) / scale, 6),
                  "rms_rel_err_vs_always": round(float((outs[pol] - ref).pow(2).mean().sqrt()) / rms, 6),
                  "reused_fraction": round(float(reuse[pol].mean()), 4)} for pol in policies}


def counters_for(name):
    """Stored counters of the recompute-step attention launch (HBM bytes per
    launch, MFMA busy share), while the kernel sources are the ones they were
    taken on (else None)."""
    pmc = os.path.join(ROOT, "profiles", f"pmc_{name}.json")
    if not os.path.exists(pmc):
        return None
    with open(pmc) as f:
        rec = json.load(f)
    return rec if rec.get("kernel_source_hash") == kernel_source_hash() else None


def cpu_baseline(name, budget_s: float, threads=None):
    """The float64 oracle on the host cores, on the same workload's block:
    single-head runs in head order (starting over when every head is done)
    until about budget_s seconds of work, scaled to all heads.  threads: cap
    the BLAS pool (None: every core it has)."""
    import contextlib
    from threadpoolctl import threadpool_info, threadpool_limits
    from cached_attention_fb_amd import workload as wl
    with (threadpool_limits(threads) if threads else contextlib.nullcontext()):
        return _cpu_baseline(name, budget_s, wl, threadpool_info)


def _cpu_baseline(name, budget_s, wl, threadpool_info):
    import oracle

    w = wl.workload(name)
    inp = wl.generate(w)
    blk = inp.blocks[0]
    kv_bytes, _, _ = algorithmic(w, w.prefix)
    heads = [(b, h) for b in range(w.batch) for h in range(w.n_q_heads)]
    done, t_total = 0, 0.0
    while t_total < budget_s:
        b, h = heads[done % len(heads)]
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
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    block_s = t_total * len(heads) / done
    return {"value": round(kv_bytes * len(blk.steps) / block_s / 1e9, 4), "unit": UNIT,
            "cores": threads, "kind": "oracle",
            "sample": f"{done} single-head runs of one {len(blk.steps)}-step block of {name} "
                      f"({len(heads)} heads per block, {t_total:.1f} s of oracle time), scaled to all heads; "
                      f"os.cpu_count()={os.cpu_count()}, affinity={len(os.sched_getaffinity(0))}",
            "us_per_layer_step": round(1e6 * block_s / len(blk.steps), 1)}


SWEEP_PREFIXES = (100_000, 200_000, 400_000, 800_000)


def sweep(prefixes=SWEEP_PREFIXES, n_blocks=3):
    """Multi-block long-context sweep on the dLLM layer shape (batch 1, 32/8
    heads, D=128, block 32, bf16): from each starting prefix, n_blocks
    consecutive blocks of 8 steps, the block's final K/V appended to the
    prefix at block end (a device copy on the stream) and the cache reset;
    the workload's threshold policy and always-recompute run on the same
    inputs.  The prefix K/V are seeded device draws of the workload's
    distribution (one layer; at 100k tokens its K/V are already 1.6x the
    MALL)."""
    import torch
    from cached_attention_fb_amd import fb
    from cached_attention_fb_amd import workload as wl

    w = wl.workload("dllm-8k").with_(blocks=n_blocks)
    inp = wl.generate(w, prefix=0)
    B, Hkv, D, Bs = w.batch, w.n_kv_heads, w.head_dim, w.block
    max_prefix = max(prefixes) + n_blocks * Bs
    gen = torch.Generator(device="cuda").manual_seed(w.seed)
    kp = torch.empty((B, Hkv, max_prefix, D), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    for t in (kp, vp):
        for c0 in range(0, max_prefix, 65536):
            c1 = min(max_prefix, c0 + 65536)
            t[:, :, c0:c1].copy_(torch.randn((B, Hkv, c1 - c0, D), generator=gen, device="cuda") * w.value_std)
    cache = fb.Cache(B, w.n_q_heads, Hkv, D, Bs, max_prefix, torch.bfloat16)
    dev_steps = [[(st.q.cuda(), st.k.cuda(), st.v.cuda(), np.asarray(st.n_updated, dtype=np.int32)) for st in blk.steps]
                 for blk in inp.blocks]
    out = torch.empty_like(dev_steps[0][0][0])
    stream = torch.cuda.current_stream().cuda_stream
    pols = {"tau": fb.POLICY_TAU, "always": fb.POLICY_ALWAYS}

    def run(P, pol, evs=None):
        n = P
        i = 0
        for blk in dev_steps:
            cache.reset(stream)
            for (q, k, v, m) in blk:
                cache.step(pols[pol], q, k, v, kp, vp, n, out, tau=w.tau, n_updated=m, stream=stream)
                if evs is not None:
                    evs[i].record()
                i += 1
            last_k, last_v = blk[-1][1], blk[-1][2]   # block end: its final K/V join the prefix
            kp[:, :, n:n + Bs].copy_(last_k)
            vp[:, :, n:n + Bs].copy_(last_v)
            n += Bs

    rows = []
    n_steps = n_blocks * w.steps
    for P in prefixes:
        rec = {"prefix": P}
        for pol in ("tau", "always"):
            run(P, pol)   # warm-up (also writes the same appended rows)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps)]
            e0.record()
            run(P, pol, evs)
            torch.cuda.synchronize()
            times = [1e3 * e0.elapsed_time(evs[0])] + [1e3 * evs[i - 1].elapsed_time(evs[i]) for i in range(1, n_steps)]
            rec[f"{pol}_block_us"] = round(sum(times) / n_blocks, 2)
            if pol == "tau":   # the host's decision: a step after the first reuses when M < tau
                ms = [int(st[3][0]) for blk in dev_steps for st in blk]
                full = [t for i, t in enumerate(times) if i % w.steps == 0 or ms[i] >= w.tau]
                reuse = [t for i, t in enumerate(times) if not (i % w.steps == 0 or ms[i] >= w.tau)]
                rec["tau_full_step_us"] = round(float(np.median(full)), 2)
                rec["tau_reuse_step_us"] = round(float(np.median(reuse)), 2) if reuse else None
            else:
                rec["always_step_us"] = round(float(np.median(times)), 2)
        rec["reuse_vs_full"] = round(rec["always_block_us"] / rec["tau_block_us"], 3)
        # external attention alone at this prefix (events around each launch)
        cache.profile_enable(True)
        run(P, "always")
        torch.cuda.synchronize()
        prof = cache.profile_read()
        cache.profile_enable(False)
        ext_us = 1e3 * prof["external"][1] / max(1, prof["external"][0])
        _, alg_bytes, _ = algorithmic(w, P + Bs)
        rec["external_us"] = round(ext_us, 2)
        rec["external_frac_hbm"] = round(alg_bytes / (ext_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
        rows.append(rec)
        print(json.dumps({"sweep_row": rec}), flush=True)
    cache.close()
    return {"metric": "multi-block long-context sweep: step time vs prefix length, threshold policy vs always-recompute",
            "unit": "us", "higher_is_better": False, "data": "synthetic (seeded device draws; dLLM layer shape)",
            "config": {"workload": "dllm-8k layer shape, batch 1, 32/8 heads, D=128, block 32, bf16",
                       "blocks_per_prefix": n_blocks, "steps_per_block": w.steps, "tau": w.tau},
            "rows": rows}


def always_only(name, steps, warmup, policy_name="always"):
    """Passes of one policy over a workload's block, for profiler runs: under
    ALWAYS every head recomputes at every step, so every dispatch of the
    attention kernel is a full recompute launch; under the workload's own
    policy (`policy_name` "policy") they are the recompute launches of the
    benchmark's timed region, in its own mix of steps.  `warmup` untimed
    steps, then `steps` timed ones over the same layer stack as the
    benchmark."""
    import torch
    from cached_attention_fb_amd import fb
    from cached_attention_fb_amd import workload as wl

    w = wl.workload(name)
    inp = wl.generate(w)
    blk = inp.blocks[0]
    S = len(blk.steps)
    n = w.prefix
    kv_bytes, _, _ = algorithmic(w, n)
    layers = max(1, math.ceil(2.5 * MALL_BYTES / kv_bytes))
    kp0, vp0 = inp.k_prefix.cuda(), inp.v_prefix.cuda()
    prefixes = [(kp0, vp0)] + [(kp0.clone(), vp0.clone()) for _ in range(layers - 1)]
    caches = [fb.Cache(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block, n, w.torch_dtype)
              for _ in range(layers)]
    qs = [st.q.cuda() for st in blk.steps]
    ks = [st.k.cuda() for st in blk.steps]
    vs = [st.v.cuda() for st in blk.steps]
    outs = [torch.empty_like(qs[0]) for _ in range(layers)]
    ms = [np.ascontiguousarray(st.n_updated, dtype=np.int32) for st in blk.steps]
    del inp, blk
    prepared = [[c.prepare(qs[s], ks[s], vs[s], prefixes[li][0], prefixes[li][1], outs[li]) for s in range(S)]
                for li, c in enumerate(caches)]
    stream = torch.cuda.current_stream().cuda_stream
    pname = w.policy if policy_name == "policy" else policy_name
    pol = {"tau": fb.POLICY_TAU, "gamma": fb.POLICY_GAMMA, "always": fb.POLICY_ALWAYS,
           "tau_cum": fb.POLICY_TAU_CUM, "gamma_group": fb.POLICY_GAMMA_GROUP}[pname]

    def run(count):
        for i in range(count):
            s = i % S
            for li, c in enumerate(caches):
                if s == 0:
                    c.reset(stream)
                prepared[li][s](pol, n, ms[s], w.tau, w.gamma, stream)

    run(warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run(steps)
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / (steps * layers)
    for c in caches:
        c.close()
    return {"profiled_pass": name, "policy": pname, "layers": layers, "steps": steps, "us_per_layer_step": round(us, 3)}


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
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--policy", default=None, choices=[None, "tau", "gamma", "always", "tau_cum", "gamma_group"])
    ap.add_argument("--layers", type=int, default=0, help="0: enough layers to exceed 2.5x the MALL")
    ap.add_argument("--splits", type=int, default=0, help="0: automatic split-KV count")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--calibrate", action="store_true", help="only run the known-traffic reference kernel")
    ap.add_argument("--sweep", action="store_true", help="only run the multi-block long-context prefix sweep")
    ap.add_argument("--sparse", action="store_true",
                    help="only run FlashBlock over a sparse attention at densities 0.2/0.3/0.4")
    ap.add_argument("--graph", action="store_true",
                    help="only run device-side threshold decisions, eager and as HIP graphs")
    ap.add_argument("--always-only", action="store_true",
                    help="only time recompute-every-step passes of --workload (profiling runs)")
    ap.add_argument("--policy-only", action="store_true",
                    help="only time passes of --workload under its own policy, as in the timed region "
                         "(profiling runs)")
    args = ap.parse_args()
    if args.calibrate:
        calibrate()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus above 1 is not supported "
                                   "(the path would shard by (sequence, kv head) or by prefix chunk)"}))
        raise SystemExit(2)
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    if args.sweep:
        print(json.dumps(sweep()), flush=True)
        return
    if args.graph:
        print(json.dumps(graph_bench(args.workload)), flush=True)
        return
    if args.sparse:
        print(json.dumps(sparse_bench(args.workload)), flush=True)
        return
    if args.always_only or args.policy_only:
        print(json.dumps(always_only(args.workload, args.steps, args.warmup,
                                     "always" if args.always_only else "policy")), flush=True)
        return

    # the largest prefix one layer's K/V can take in the free device memory
    from cached_attention_fb_amd import workload as wl
    w0 = wl.workload(args.workload)
    capacity = int(torch.cuda.mem_get_info()[0] // (2 * w0.batch * w0.n_kv_heads * w0.head_dim * w0.elem_bytes))
    r = measure(args.workload, args.steps, args.warmup, args.policy, args.layers, args.splits)
    w = r["w"]
    roof = dict(r["roofline"])
    ctr = counters_for(w.name)
    roof["traffic"] = None if ctr is None else ctr.get("hbm_bytes_per_launch")
    if ctr is not None and ctr.get("mfma_busy_frac") is not None:
        roof["mfma_busy_frac"] = ctr["mfma_busy_frac"]   # SQ_VALU_MFMA_BUSY_CYCLES share, stored counters
    result = {
        "metric": METRIC,
        "value": round(r["eff_gbs"], 1),
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * r["gpu_s"] / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; random values of the workload's distributions)",
        "config": {"workload": w.name, "shape": w.description, "policy": r["policy"], "tau": w.tau,
                   "gamma": w.gamma, "layers": r["layers"], "kv_bytes_per_layer": r["kv_bytes"],
                   "prefix": w.prefix},
        "us_per_layer_step": round(r["per_layer_step_us"], 3),
        "always_us_per_layer_step": round(r["always_layer_step_us"], 3),
        "reuse_vs_full_speedup": round(r["always_layer_step_us"] / r["per_layer_step_us"], 3),
        "reused_heads_per_step": r["reuse_counts"],
        "step_us": r["step_stats"],
        "ext_plus_combine_us": round(r["kernel_us"].get("external", 0.0) + r["kernel_us"].get("combine", 0.0), 3),
        "capacity_prefix_tokens_per_layer": capacity,
        "wall_s": round(r["wall_s"], 4),
        "kernel_avg_us_always": r["kernel_us"],
        "kernel_avg_us_policy": r["kernel_us_policy"],
        "roofline": roof,
        # the same kernel in the always-recompute pass (every step a recompute
        # launch: sustained load, lower clocks)
        "roofline_always": {**r["roofline_always"], "traffic": roof["traffic"]},
    }
    if not args.no_extra:
        extra = {}
        for name in EXTRA:
            if name == args.workload:
                continue
            S = wl.workload(name).steps
            e = measure(name, 2 * S, S, decisions=False)
            rf = e["roofline"]
            rc = counters_for(name)
            extra[name] = {"policy": e["policy"], "layers": e["layers"], "steps": 2 * S,
                           "us_per_layer_step": round(e["per_layer_step_us"], 2),
                           "always_us_per_layer_step": round(e["always_layer_step_us"], 2),
                           "reuse_vs_full_speedup": round(e["always_layer_step_us"] / e["per_layer_step_us"], 3),
                           "effective_kv_gbs": round(e["eff_gbs"], 1),
                           "external": {**{k: rf[k] for k in ("bound", "achieved", "peak", "unit", "frac",
                                                              "avg_launch_us", "pass")},
                                        "frac_always": e["roofline_always"]["frac"],
                                        "traffic": None if rc is None else rc.get("hbm_bytes_per_launch"),
                                        "mfma_busy_frac": None if rc is None else rc.get("mfma_busy_frac")},
                           "kernel_avg_us_always": e["kernel_us"]}
        result["workloads"] = extra
        # threshold variants (per-step vs cumulative M): step time, reuse and
        # output error against always-recompute on the same block
        variants = {}
        for name, pols in (("dllm-8k", ("tau", "tau_cum")), ("long-32k-b4", ("tau", "tau_cum"))):
            S = wl.workload(name).steps
            err = staleness(name, pols)
            variants[name] = {}
            for pol in pols:
                e = measure(name, 2 * S, S, policy_name=pol, decisions=False)
                variants[name][pol] = {"us_per_layer_step": round(e["per_layer_step_us"], 2),
                                       "reuse_vs_full_speedup": round(e["always_layer_step_us"] / e["per_layer_step_us"], 3),
                                       **err[pol]}
        result["policy_variants"] = variants
        # threshold decisions on the device, eager and replayed as HIP graphs
        result["device_decisions"] = graph_bench("dllm-8k")
        # FlashBlock over a sparse attention (left-out tiles cached, kept tiles fresh)
        result["sparse"] = {nm: sparse_bench(nm) for nm in ("dllm-8k", "long-32k-b4")}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w.name, args.cpu_budget)
        if not args.no_extra:   # the small workloads' oracle on one thread
            result["cpu_oracle_1thread"] = {nm: cpu_baseline(nm, 4.0, threads=1) for nm in ("tiny-fp32", "dllm-8k")}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
