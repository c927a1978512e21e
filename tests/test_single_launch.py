"""The single-launch fused step (opt-in with FB_FIN=1: split attention,
block-internal attention and split combine in one grid, roles by workgroup
index; host decisions, and threshold decisions made on the device after a
block's first step) against the two-launch form of the same step (FB_FIN=0): the combine is the same code over the same
partials, so caches, decisions and the outputs of recomputed heads are
bitwise equal; a group in which every head reuses is finished by its
block-internal items (the merge launch's epilogue), whose outputs agree to
one rounding.  Also: the counters return
to zero within a launch (steps and blocks in a row, and graph replays, keep
working), and the wait never runs out."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from cached_attention_fb_amd import fb
from cached_attention_fb_amd import workload as wl
from tests import harness as H

pytestmark = pytest.mark.gpu


def same_step(x, y, label):
    """One step of the single launch (x) against the two launches (y): the
    decisions and the cache bitwise; the output bitwise for a head that
    recomputed (the same combine over the same partials), and within one
    rounding of the output for a head that reused, whose output the single
    launch takes from its block-internal items' merge epilogue (the
    block-internal part in fp32) where the two launches fold that part's
    bf16 partial in the combine."""
    out_x, out_y = x[0].float(), y[0].float()
    for i, what in ((1, "A_out"), (2, "L_out"), (3, "reuse")):
        assert np.array_equal(x[i], y[i]), f"{label} {what}"
    reused = torch.from_numpy(y[3].astype(bool))
    assert torch.equal(out_x[~reused], out_y[~reused]), f"{label} out of recomputed heads"
    if bool(reused.any()):
        scale = float(out_y.abs().max())
        diff = float((out_x[reused] - out_y[reused]).abs().max())
        assert diff <= 2.0 ** -7 * scale, f"{label} out of reused heads: {diff} (scale {scale})"


def run(inp, policy, fin: bool, monkeypatch, steps=None):
    """Every step of the first block; returns per-step outputs, caches and the
    profile (kind -> launches)."""
    monkeypatch.setenv("FB_FIN", "1" if fin else "0")
    w = inp.workload
    n = inp.k_prefix.shape[2]
    cache = H.make_cache(w, n)
    monkeypatch.delenv("FB_FIN", raising=False)
    kp, vp = H.device_prefix(inp, n)
    blk = inp.blocks[0]
    q = blk.steps[0].q.cuda()
    out = torch.empty_like(q)
    cache.profile_enable(True)
    res = []
    for st in blk.steps[:steps]:
        q.copy_(st.q)
        cache.step(H.POLICY_CODE[policy], q, st.k.cuda(), st.v.cuda(), kp, vp, n, out, tau=w.tau, gamma=w.gamma,
                   n_updated=st.n_updated)
        res.append((out.cpu().clone(), cache.read(fb.FIELD_A_OUT), cache.read(fb.FIELD_L_OUT),
                    cache.read(fb.FIELD_REUSE)))
    prof = {k: v[0] for k, v in cache.profile_read().items()}
    err = int(cache.read(fb.FIELD_WAIT_ERR)[0])
    cache.close()
    return res, prof, err


@pytest.mark.parametrize("name,prefix", [("dllm-8k", 8192), ("dllm-8k", 1000), ("long-32k-b4", 4160),
                                         ("max-128k", 6000)])
@pytest.mark.parametrize("policy", ["always", "tau"])
def test_single_launch_equals_two_launches(name, prefix, policy, monkeypatch):
    w = wl.WORKLOADS[name]
    if os.environ.get("FB_ATTN_R64") == "1" and w.n_q_heads // w.n_kv_heads * w.block > 128:
        pytest.skip("FB_ATTN_R64=1: the two launches take these groups to the 64-row kernel, the single "
                    "launch keeps the 32-row one, so their partials are not bitwise comparable")
    inp = wl.generate(w, prefix=prefix)
    print(f"[single launch] {name} prefix {prefix} {policy}", flush=True)
    a, pa, ea = run(inp, policy, True, monkeypatch)
    b, pb, eb = run(inp, policy, False, monkeypatch)
    assert ea == 0 and eb == 0
    assert pb["combine"] == pb["external"] > 0, pb           # two launches per recompute step
    assert pa["external"] == pb["external"], pa
    # one launch per recompute step, also where a threshold step recomputes
    # some sequences only and enumerates just their groups (a device plan)
    assert pa["combine"] == 0, pa
    for s, (x, y) in enumerate(zip(a, b)):
        same_step(x, y, f"step {s}")


def test_single_launch_many_splits(monkeypatch):
    """Two kv heads over a 64k-token prefix: each group's keys go to more
    than 32 ranges (the planner fills the chip with two groups), which the
    combine folds in several rounds; the single launch still matches the two
    launches."""
    w = wl.workload("dllm-8k").with_(n_q_heads=8, n_kv_heads=2, blocks=1, steps=3)
    inp = wl.generate(w, prefix=65536)
    print("[single launch] 8/2 heads, prefix 65536", flush=True)
    a, pa, ea = run(inp, "always", True, monkeypatch)
    b, pb, eb = run(inp, "always", False, monkeypatch)
    assert ea == 0 and eb == 0
    assert pa["combine"] == 0 and pb["combine"] == pb["external"] == 3, (pa, pb)
    for s, (x, y) in enumerate(zip(a, b)):
        same_step(x, y, f"step {s}")


def test_single_launch_graph_replays(monkeypatch):
    """A recompute step captured in a HIP graph and replayed several times with
    eager work between the replays: every replay equals the eager step (the
    counters are back at zero after each launch)."""
    monkeypatch.setenv("FB_FIN", "1")
    w = wl.WORKLOADS["dllm-8k"]
    inp = wl.generate(w, prefix=2048)
    n = inp.k_prefix.shape[2]
    cache = H.make_cache(w, n)
    monkeypatch.delenv("FB_FIN", raising=False)
    kp, vp = H.device_prefix(inp, n)
    st = inp.blocks[0].steps[0]
    q, kb, vb = st.q.cuda(), st.k.cuda(), st.v.cuda()
    out = torch.empty_like(q)
    cache.reset()
    cache.step(fb.POLICY_ALWAYS, q, kb, vb, kp, vp, n, out)
    ref = out.clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        cache.reset(stream=s)
        with torch.cuda.graph(g, stream=s):
            cache.step(fb.POLICY_ALWAYS, q, kb, vb, kp, vp, n, out, stream=s)
    torch.cuda.synchronize()
    for r in range(4):
        out.zero_()
        cache.reset()
        cache.step(fb.POLICY_ALWAYS, q, kb, vb, kp, vp, n, out)   # eager, between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"eager step before replay {r}"
        out.zero_()
        cache.reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r}"
    assert int(cache.read(fb.FIELD_WAIT_ERR)[0]) == 0
    cache.close()


def run_dev(inp, counts, fin_env, monkeypatch):
    """Every step of the first block under the threshold rule with the counts
    in device memory (`counts[s]` per sequence); FB_FIN as given at
    allocation."""
    monkeypatch.setenv("FB_FIN", fin_env)
    w = inp.workload
    n = inp.k_prefix.shape[2]
    cache = H.make_cache(w, n)
    monkeypatch.delenv("FB_FIN", raising=False)
    kp, vp = H.device_prefix(inp, n)
    blk = inp.blocks[0]
    q = blk.steps[0].q.cuda()
    out = torch.empty_like(q)
    m = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    cache.profile_enable(True)
    res = []
    for s, st in enumerate(blk.steps):
        q.copy_(st.q)
        m.copy_(torch.as_tensor(np.asarray(counts[s], dtype=np.int32)))
        cache.step(fb.POLICY_TAU, q, st.k.cuda(), st.v.cuda(), kp, vp, n, out, tau=w.tau, n_updated_dev=m)
        res.append((out.cpu().clone(), cache.read(fb.FIELD_A_OUT), cache.read(fb.FIELD_L_OUT),
                    cache.read(fb.FIELD_REUSE)))
    prof = {k: v[0] for k, v in cache.profile_read().items()}
    err = int(cache.read(fb.FIELD_WAIT_ERR)[0])
    cache.close()
    return res, prof, err


@pytest.mark.parametrize("name,prefix", [("dllm-8k", 8192), ("dllm-8k", 1000), ("long-32k-b4", 4160)])
def test_device_decided_steps_single_launch(name, prefix, monkeypatch):
    """Threshold steps decided on the device take the single launch after the
    block's first step: the two-launch form's results (see same_step), on the
    workload's counts and on seeded counts that make some sequences reuse
    while others recompute."""
    w = wl.WORKLOADS[name]
    inp = wl.generate(w, prefix=prefix)
    steps = inp.blocks[0].steps
    rng = np.random.default_rng(11)
    patterns = {"workload": [np.asarray(st.n_updated) for st in steps],
                "mixed": [rng.integers(0, 2 * max(1, w.tau), w.batch) for _ in steps]}
    for label, counts in patterns.items():
        print(f"[single launch, device decisions] {name} prefix {prefix} {label} counts", flush=True)
        a, pa, ea = run_dev(inp, counts, "1", monkeypatch)
        b, pb, eb = run_dev(inp, counts, "0", monkeypatch)
        assert ea == 0 and eb == 0
        assert pb["combine"] == pb["external"] == len(steps), pb   # two launches every step
        assert pa["external"] == len(steps) and pa["combine"] == 1, pa   # the block's first step only
        reused = 0
        for s, (x, y) in enumerate(zip(a, b)):
            same_step(x, y, f"{label} step {s}")
            reused += int(y[3].sum())
        assert reused > 0, "no step reused: the pattern tests nothing"
