"""Parity of fb_step_sparse (FlashBlock over a sparse attention) with the
float64 oracle.

A seeded synthetic selection keeps some 64-key tiles of the prefix per
(sequence, kv head); the tiles it leaves out are the cached external set, the
kept ones are attended afresh at every step.  Decisions must be bit-exact and
outputs, cached parts and their L within the usual tolerances; with every
head recomputing the result is exact attention over the prefix and block.
"""
import numpy as np
import pytest
import torch

import harness as H
import oracle
from cached_attention_fb_amd import fb
from cached_attention_fb_amd import workload as wl

pytestmark = pytest.mark.gpu


def run_gpu_sparse(inp, density, policy=None, device_counts=False, n_sel=None, kv_splits=0, prof=None):
    """Every block of ``inp`` through fb_step_sparse; a fresh selection per
    block (its prefix grows by the block).  Returns (GpuBlocks, selections);
    with a dict `prof`, fills it with the launches per profile kind."""
    w = inp.workload
    policy = policy or w.policy
    n0 = inp.k_prefix.shape[2]
    max_prefix = n0 + w.block * (len(inp.blocks) - 1)
    cache = H.make_cache(w, max_prefix, kv_splits=kv_splits)
    cache.profile_enable(prof is not None)
    kp, vp = H.device_prefix(inp, max_prefix)
    q = torch.empty((w.batch, w.n_q_heads, w.block, w.head_dim), dtype=w.torch_dtype, device="cuda")
    kb = torch.empty((w.batch, w.n_kv_heads, w.block, w.head_dim), dtype=w.torch_dtype, device="cuda")
    vb = torch.empty_like(kb)
    out = torch.empty_like(q)
    m_dev = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    n = n0
    res, sels = [], []
    for bi, blk in enumerate(inp.blocks):
        sel = wl.sparse_selection(w, n, density, seed=w.seed + bi)
        if n_sel is not None:   # a given count: the first n_sel tiles of a random order
            tiles = (n + 63) // 64
            rng = np.random.default_rng(bi)
            sel = np.stack([np.stack([np.sort(rng.permutation(tiles)[:n_sel]) for _ in range(w.n_kv_heads)])
                            for _ in range(w.batch)]).astype(np.int32)
        sels.append(sel)
        sel_dev = torch.as_tensor(sel).cuda().contiguous()
        cache.reset()
        S = len(blk.steps)
        g = H.GpuBlock(np.zeros((S,) + tuple(q.shape)), np.zeros((S,) + tuple(q.shape), np.float32),
                       np.zeros((S,) + tuple(q.shape[:3]), np.float32),
                       np.zeros((S, w.batch, w.n_q_heads), np.uint8),
                       np.zeros((S, w.batch, w.n_q_heads), np.float32))
        for s, st in enumerate(blk.steps):
            q.copy_(st.q)
            kb.copy_(st.k)
            vb.copy_(st.v)
            kw = dict(tau=w.tau, gamma=w.gamma, sel_tiles=sel_dev)
            if device_counts:
                m_dev.copy_(torch.as_tensor(np.asarray(st.n_updated, dtype=np.int32)))
                kw["n_updated_dev"] = m_dev
            else:
                kw["n_updated"] = st.n_updated
            cache.step(H.POLICY_CODE[policy], q, kb, vb, kp, vp, n, out, **kw)
            g.out[s] = out.to(torch.float64).cpu().numpy()
            g.reuse[s] = cache.read(fb.FIELD_REUSE)
            g.a_out[s] = cache.read(fb.FIELD_A_OUT)
            g.l_out[s] = cache.read(fb.FIELD_L_OUT)
            g.sim[s] = cache.read(fb.FIELD_SIM)
        res.append(g)
        last = blk.steps[-1]
        if n + w.block <= max_prefix:
            kp[:, :, n:n + w.block].copy_(last.k)
            vp[:, :, n:n + w.block].copy_(last.v)
        n += w.block
    torch.cuda.synchronize()
    if prof is not None:
        prof.update({k: v[0] for k, v in cache.profile_read().items()})
    cache.close()
    return res, sels


def run_oracle_sparse(inp, sels, policy=None):
    w = inp.workload
    policy = policy or w.policy
    kp, vp = wl.to_f64(inp.k_prefix), wl.to_f64(inp.v_prefix)
    out = []
    for blk, sel in zip(inp.blocks, sels):
        steps = H.oracle_steps(blk)
        out.append(oracle.run_block_sparse(kp, vp, kp.shape[2], steps, sel, policy, tau=w.tau, gamma=w.gamma))
        kp = np.concatenate([kp, steps[-1].k], axis=2)
        vp = np.concatenate([vp, steps[-1].v], axis=2)
    return out


def _check(w, prefix, density, policy=None, device_counts=False, n_sel=None, min_reuse=True):
    inp = wl.generate(w, prefix=prefix)
    print(f"[sparse] {w.name} prefix={inp.k_prefix.shape[2]} density={density} n_sel={n_sel} "
          f"policy={policy or w.policy} device_counts={device_counts}", flush=True)
    gpu, sels = run_gpu_sparse(inp, density, policy, device_counts, n_sel)
    ref = run_oracle_sparse(inp, sels, policy)
    for i, (g, r) in enumerate(zip(gpu, ref)):
        errs = H.compare_block(g, r, w.dtype, what=f"{w.name} sparse block {i}")
        print(f"[sparse] block {i} kept {sels[i].shape[2]} tiles, errs {errs}, reused {int(g.reuse.sum())}",
              flush=True)
    if min_reuse and (policy or w.policy) != "always":
        assert int(ref[0].reuse.sum()) > 0
    return gpu, ref


def test_sparse_tiny_fp32_two_blocks():
    _check(wl.workload("tiny-fp32"), None, 0.3)


def test_sparse_tiny_fp32_ragged_prefix_gamma():
    w = wl.workload("tiny-fp32").with_(policy="gamma", gamma=0.913, blocks=1)   # mixed decisions, margin 2e-3
    inp = wl.generate(w, prefix=500)
    gpu, sels = run_gpu_sparse(inp, 0.4)
    ref = run_oracle_sparse(inp, sels)
    sims = ref[0].sim[1:]
    margin = np.nanmin(np.abs(sims - w.gamma))
    assert margin > 1e-3, margin
    H.compare_block(gpu[0], ref[0], "f32", what="tiny gamma sparse")
    fin = ~np.isnan(ref[0].sim)
    assert np.max(np.abs(gpu[0].sim[fin] - ref[0].sim[fin])) <= 1e-5


def test_sparse_dllm_small_prefix():
    _check(wl.workload("dllm-8k"), 1000, 0.2)


def test_sparse_dllm_device_counts():
    _check(wl.workload("dllm-8k"), 3000, 0.3, device_counts=True)


def test_sparse_long_batch4_cumulative():
    _check(wl.workload("long-32k-b4").with_(steps=6), 700, 0.3, policy="tau_cum")


def test_sparse_always_is_exact_attention():
    """Every head recomputing: exact attention over prefix + block, which the
    dense oracle gives too (any selection)."""
    w = wl.workload("dllm-8k").with_(steps=3)
    gpu, ref = _check(w, 2000, 0.2, policy="always")
    inp = wl.generate(w, prefix=2000)
    dense = H.run_oracle(inp, policy="always")
    for s in range(3):
        H.tolerance_check(gpu[0].out[s], dense[0].out[s], "bf16", f"sparse always vs dense step {s}")


@pytest.mark.parametrize("name,density,steps", [("dllm-8k", 0.3, None), ("long-32k-b4", 0.2, 4)])
def test_sparse_full_size(name, density, steps):
    """The bench's sparse configurations at their full prefix (8192 and 32768
    tokens) under the workload's threshold: recompute steps take both tile
    sets in one launch (one sequence, or four deciding on their own counts),
    reuse steps the kept set alone."""
    w = wl.workload(name).with_(blocks=1)
    if steps:
        w = w.with_(steps=steps)
    _check(w, None, density)


@pytest.mark.parametrize("kv_splits", [0, 64])
def test_sparse_recompute_launches(kv_splits):
    """A step in which some head recomputes attends the left-out and the kept
    tiles in one launch with one combine when both sets' chunks fit the
    partial buffer together (here with the planner's own split counts),
    and in two launches each where they do not (here forced: 64 of the 128
    tiles kept, and the other 64 cut into 64 chunks that fill the buffer);
    both agree with the oracle."""
    w = wl.workload("dllm-8k").with_(steps=3, blocks=1)
    inp = wl.generate(w, prefix=8192)
    print(f"[sparse] recompute launches kv_splits={kv_splits}", flush=True)
    prof = {}
    gpu, sels = run_gpu_sparse(inp, 0.0, "always", n_sel=64, kv_splits=kv_splits, prof=prof)
    ref = run_oracle_sparse(inp, sels, "always")
    H.compare_block(gpu[0], ref[0], w.dtype, what=f"sparse always kv_splits={kv_splits}")
    assert prof["external"] == prof["combine"] == 3, prof
    assert prof["sparse_kept"] == prof["sparse_total"] == (0 if kv_splits == 0 else 3), prof


@pytest.mark.parametrize("n_sel", [0, 1, 16])
def test_sparse_edge_counts(n_sel):
    """Nothing kept (the method is FlashBlock itself), one tile, every tile
    (the cached part is empty)."""
    _check(wl.workload("dllm-8k").with_(steps=4), 1000, 0.0, n_sel=n_sel)


def test_sparse_video_small_always():
    """Frame-sized block (1560 queries per head) over a 49-tile prefix."""
    w = wl.workload("video-1560x15600").with_(steps=2)
    _check(w, 3120, 0.3, policy="always")


def test_sparse_graph_replay():
    """A sparse block recorded by stream capture replays like the eager steps."""
    w = wl.workload("dllm-8k").with_(steps=4)
    inp = wl.generate(w, prefix=1500)
    blk = inp.blocks[0]
    n = 1500
    kp, vp = H.device_prefix(inp, n)
    sel = torch.as_tensor(wl.sparse_selection(w, n, 0.3)).cuda().contiguous()
    qs = [st.q.cuda() for st in blk.steps]
    ks = [st.k.cuda() for st in blk.steps]
    vs = [st.v.cuda() for st in blk.steps]
    ms = [torch.as_tensor(np.asarray(st.n_updated, np.int32)).cuda() for st in blk.steps]
    outs_g = [torch.empty_like(qs[0]) for _ in qs]
    outs_e = [torch.empty_like(qs[0]) for _ in qs]
    cg, ce = H.make_cache(w, n), H.make_cache(w, n)

    def run(cache, outs, stream):
        cache.reset(stream)
        for s in range(len(qs)):
            cache.step(fb.POLICY_TAU, qs[s], ks[s], vs[s], kp, vp, n, outs[s], tau=w.tau, n_updated_dev=ms[s],
                       sel_tiles=sel, stream=stream)

    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        run(cg, outs_g, side.cuda_stream)
    torch.cuda.synchronize()
    for i in range(3):
        if i == 1:
            for m in ms:
                m.fill_(w.block)   # every step recomputes
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs_g]
        run(ce, outs_e, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for s in range(len(qs)):
            assert torch.equal(got[s], outs_e[s]), f"replay {i} step {s}"
        np.testing.assert_array_equal(cg.read(fb.FIELD_REUSE), ce.read(fb.FIELD_REUSE))
    cg.close()
    ce.close()


def test_sparse_arguments():
    w = wl.workload("tiny-fp32")
    c = H.make_cache(w, w.prefix)
    q = torch.zeros((w.batch, w.n_q_heads, w.block, w.head_dim), device="cuda")
    kb = torch.zeros((w.batch, w.n_kv_heads, w.block, w.head_dim), device="cuda")
    kp = torch.zeros((w.batch, w.n_kv_heads, w.prefix, w.head_dim), device="cuda")
    tiles = w.prefix // 64
    too_many = torch.zeros((w.batch, w.n_kv_heads, tiles + 1), dtype=torch.int32, device="cuda")
    with pytest.raises(fb.FBError) as e:
        c.step(fb.POLICY_TAU, q, kb, kb, kp, kp, w.prefix, q, tau=4, n_updated=[0], sel_tiles=too_many)
    assert e.value.code == fb.FB_E_SHAPE
    sel2 = torch.arange(2, dtype=torch.int32, device="cuda").repeat(w.batch, w.n_kv_heads, 1).contiguous()
    sel3 = torch.arange(3, dtype=torch.int32, device="cuda").repeat(w.batch, w.n_kv_heads, 1).contiguous()
    c.step(fb.POLICY_TAU, q, kb, kb, kp, kp, w.prefix, q, tau=4, n_updated=[0], sel_tiles=sel2)
    with pytest.raises(fb.FBError) as e:     # another count inside the block
        c.step(fb.POLICY_TAU, q, kb, kb, kp, kp, w.prefix, q, tau=4, n_updated=[0], sel_tiles=sel3)
    assert e.value.code == fb.FB_E_STATE
    with pytest.raises(fb.FBError) as e:     # a dense step inside a sparse block
        c.step(fb.POLICY_TAU, q, kb, kb, kp, kp, w.prefix, q, tau=4, n_updated=[0])
    assert e.value.code == fb.FB_E_STATE
    c.reset()
    c.step(fb.POLICY_TAU, q, kb, kb, kp, kp, w.prefix, q, tau=4, n_updated=[0])
    torch.cuda.synchronize()
    c.close()
