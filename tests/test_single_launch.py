"""The single-launch fused step (opt-in with FB_FIN=1: split attention,
block-internal attention and split combine in one grid, roles by workgroup
index) against the two-launch form of the same step: the combine is the same code over the same
partials, so outputs and caches are bitwise equal.  Also: the counters return
to zero within a launch (steps and blocks in a row, and graph replays, keep
working), and the wait never runs out."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from cached_attention_fb_amd import fb
from cached_attention_fb_amd import workload as wl
from tests import harness as H

pytestmark = pytest.mark.gpu


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
    inp = wl.generate(w, prefix=prefix)
    print(f"[single launch] {name} prefix {prefix} {policy}", flush=True)
    a, pa, ea = run(inp, policy, True, monkeypatch)
    b, pb, eb = run(inp, policy, False, monkeypatch)
    assert ea == 0 and eb == 0
    assert pb["combine"] == pb["external"] > 0, pb           # two launches per recompute step
    assert pa["external"] == pb["external"], pa
    if policy == "always" or w.batch == 1:
        assert pa["combine"] == 0, pa                        # one
    else:
        # a threshold step that recomputes some sequences only enumerates
        # their groups (a device plan): those keep the two launches
        assert pa["combine"] < pb["combine"], pa
    for s, (x, y) in enumerate(zip(a, b)):
        for i, what in enumerate(("out", "A_out", "L_out", "reuse")):
            assert torch.equal(x[i], y[i]) if i == 0 else np.array_equal(x[i], y[i]), f"step {s} {what}"


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
