"""Threshold decisions made on the device, and whole blocks recorded as HIP
graphs.

With the updated-token counts in device memory (fb_policy_args.n_updated_dev)
the external-attention launch decides per head and records the decisions for
the launches after it.  These must equal the host's decisions bit for bit,
and since the same kernels then refresh the cache on the same split plan, so
must the cached parts; the outputs of steps where every head reuses may come
from another kernel on the host path (one launch when the host knows it), so
they agree to rounding; the oracle checks both.  A block recorded by stream capture (reset + every
step) and replayed with other counts and with other work between the replays
must reproduce, replay after replay, what the same steps give eagerly.
"""
import numpy as np
import pytest
import torch

import harness as H
import oracle
from cached_attention_fb_amd import fb
from cached_attention_fb_amd import workload as wl

pytestmark = pytest.mark.gpu


def _workload(name):
    w = wl.workload(name)
    return w.with_(steps=6) if name == "long-32k-b4" else w


@pytest.mark.parametrize("name,prefix,policy", [
    ("tiny-fp32", None, "tau"),
    ("tiny-fp32", None, "tau_cum"),
    ("dllm-8k", 1000, "tau"),
    ("dllm-8k", 1000, "tau_cum"),
    ("dllm-8k", None, "tau"),         # the full 8192-token prefix
    ("long-32k-b4", 700, "tau"),      # four sequences, each deciding on its own count
])
def test_device_counts_match_host_and_oracle(name, prefix, policy):
    w = _workload(name)
    inp = wl.generate(w, prefix=prefix)
    print(f"[device-decisions] {name} prefix={inp.k_prefix.shape[2]} {policy}", flush=True)
    dev = H.run_gpu(inp, policy=policy, device_counts=True)
    host = H.run_gpu(inp, policy=policy)
    ref = H.run_oracle(inp, policy=policy)
    for i, (d, h, r) in enumerate(zip(dev, host, ref)):
        np.testing.assert_array_equal(d.reuse, h.reuse)
        scale = float(np.max(np.abs(h.out)))
        ulp = 2.0 ** -7 if w.dtype == "bf16" else 2.0 ** -20   # one rounding of the output
        assert float(np.max(np.abs(d.out - h.out))) <= ulp * scale
        np.testing.assert_array_equal(d.a_out, h.a_out)
        np.testing.assert_array_equal(d.l_out, h.l_out)
        errs = H.compare_block(d, r, w.dtype, what=f"{name} {policy} device block {i}")
        print(f"[device-decisions] block {i} errs {errs} reused {int(d.reuse.sum())}", flush=True)
    assert 0 < int(ref[0].reuse.sum()) < ref[0].reuse.size


def test_device_counts_arguments():
    w = _workload("tiny-fp32")
    c = H.make_cache(w, w.prefix)
    q = torch.zeros((w.batch, w.n_q_heads, w.block, w.head_dim), device="cuda")
    kb = torch.zeros((w.batch, w.n_kv_heads, w.block, w.head_dim), device="cuda")
    kp = torch.zeros((w.batch, w.n_kv_heads, w.prefix, w.head_dim), device="cuda")
    m = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    with pytest.raises(fb.FBError) as e:     # both count sources
        c.step(fb.POLICY_TAU, q, kb, kb, kp, kp, w.prefix, q, tau=4, n_updated=[0] * w.batch, n_updated_dev=m)
    assert e.value.code == fb.FB_E_ARG
    c.step(fb.POLICY_TAU, q, kb, kb, kp, kp, w.prefix, q, tau=4, n_updated_dev=m)
    with pytest.raises(fb.FBError) as e:     # host counts inside a block decided on the device
        c.step(fb.POLICY_TAU, q, kb, kb, kp, kp, w.prefix, q, tau=4, n_updated=[0] * w.batch)
    assert e.value.code == fb.FB_E_STATE
    c.reset()
    c.step(fb.POLICY_TAU, q, kb, kb, kp, kp, w.prefix, q, tau=4, n_updated=[0] * w.batch)
    torch.cuda.synchronize()
    c.close()


class _Block:
    """Every step's inputs in buffers of their own (a graph keeps addresses)."""

    def __init__(self, inp, policy):
        w = inp.workload
        self.w, self.policy = w, policy
        blk = inp.blocks[0]
        self.S = len(blk.steps)
        self.n = inp.k_prefix.shape[2]
        self.kp, self.vp = H.device_prefix(inp, self.n)
        self.q = [st.q.cuda() for st in blk.steps]
        self.k = [st.k.cuda() for st in blk.steps]
        self.v = [st.v.cuda() for st in blk.steps]
        self.m = [torch.zeros(w.batch, dtype=torch.int32, device="cuda") for _ in blk.steps]
        self.m_host = [np.asarray(st.n_updated, dtype=np.int32) for st in blk.steps]
        self.inp = inp

    def set_counts(self, counts):
        for s in range(self.S):
            self.m[s].copy_(torch.as_tensor(counts[s]))

    def run(self, cache, outs, stream):
        cache.reset(stream)
        w = self.w
        dev_counts = self.policy in ("tau", "tau_cum")
        for s in range(self.S):
            cache.step(H.POLICY_CODE[self.policy], self.q[s], self.k[s], self.v[s], self.kp, self.vp,
                       self.n, outs[s], tau=w.tau, gamma=w.gamma,
                       n_updated_dev=self.m[s] if dev_counts else None, stream=stream)

    def oracle(self, counts):
        steps = [oracle.StepData(wl.to_f64(st.q), wl.to_f64(st.k), wl.to_f64(st.v), np.asarray(counts[s]))
                 for s, st in enumerate(self.inp.blocks[0].steps)]
        w = self.w
        return oracle.run_block(wl.to_f64(self.inp.k_prefix), wl.to_f64(self.inp.v_prefix), self.n, steps,
                                self.policy, tau=w.tau, gamma=w.gamma)


@pytest.mark.parametrize("name,prefix,policy", [
    ("dllm-8k", 1000, "tau"),
    ("long-32k-b4", 700, "tau_cum"),
    ("tiny-fp32", None, "gamma"),
])
def test_graph_replay_matches_eager(name, prefix, policy):
    w = _workload(name)
    if policy == "gamma":
        w = w.with_(policy="gamma", gamma=0.9)
    inp = wl.generate(w, prefix=prefix)
    blk = _Block(inp, policy)
    print(f"[graph] {name} prefix={blk.n} {policy} steps={blk.S}", flush=True)
    cg = H.make_cache(w, blk.n)
    ce = H.make_cache(w, blk.n)
    outs_g = [torch.empty_like(blk.q[0]) for _ in range(blk.S)]
    outs_e = [torch.empty_like(blk.q[0]) for _ in range(blk.S)]
    # count patterns: the workload's own, none updated, all updated, mixed per sequence
    rng = np.random.default_rng(7)
    patterns = [blk.m_host,
                [np.zeros(w.batch, np.int32)] * blk.S,
                [np.full(w.batch, w.block, np.int32)] * blk.S,
                [rng.integers(0, 2 * max(1, w.tau), w.batch).astype(np.int32) for _ in range(blk.S)],
                blk.m_host]
    blk.set_counts(patterns[0])
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        blk.run(cg, outs_g, side.cuda_stream)
    torch.cuda.synchronize()
    for i, counts in enumerate(patterns):
        blk.set_counts(counts)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        reuse_g = cg.read(fb.FIELD_REUSE)
        a_g = cg.read(fb.FIELD_A_OUT)
        got = [o.clone() for o in outs_g]
        # eager run of the same steps on another cache, then unrelated work
        blk.run(ce, outs_e, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for s in range(blk.S):
            assert torch.equal(got[s], outs_e[s]), f"replay {i} step {s}: output differs from eager"
        np.testing.assert_array_equal(reuse_g, ce.read(fb.FIELD_REUSE))
        np.testing.assert_array_equal(a_g, ce.read(fb.FIELD_A_OUT))
        junk = torch.randn(1 << 20, device="cuda")
        (junk * 2).sum().item()
        if policy != "gamma":   # the oracle on the replay (threshold decisions are exact)
            ref = blk.oracle(counts)
            for s in range(blk.S):
                H.tolerance_check(got[s].double().cpu().numpy(), ref.out[s], w.dtype, f"replay {i} step {s}")
            np.testing.assert_array_equal(reuse_g, ref.reuse[-1].astype(np.uint8))
        print(f"[graph] replay {i} ok, last-step reuse {int(reuse_g.sum())}", flush=True)
    cg.close()
    ce.close()


def test_profiling_refused_under_capture():
    w = _workload("tiny-fp32")
    c = H.make_cache(w, w.prefix)
    c.profile_enable(True)
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    err = None
    torch.cuda.synchronize()
    try:
        with torch.cuda.graph(graph, stream=side):
            try:
                c.reset(side.cuda_stream)
            except fb.FBError as e:
                err = e
    finally:
        torch.cuda.synchronize()
    assert err is not None and err.code == fb.FB_E_STATE
    c.profile_enable(False)
    c.close()
