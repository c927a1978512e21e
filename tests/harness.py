"""Helpers shared by the parity tests: run a workload through the HIP library
(via the Python binding) and through the float64 oracle on the same seeded
inputs, and compare them.  Test infrastructure; imports the oracle."""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

import oracle
from cached_attention_fb_amd import fb
from cached_attention_fb_amd import workload as wl

POLICY_CODE = {"always": fb.POLICY_ALWAYS, "tau": fb.POLICY_TAU, "gamma": fb.POLICY_GAMMA,
               "tau_cum": fb.POLICY_TAU_CUM, "gamma_group": fb.POLICY_GAMMA_GROUP}


@dataclass
class GpuBlock:
    out: np.ndarray      # [S, B, Hq, Bs, D] float64 (from the working dtype)
    a_out: np.ndarray    # [S, B, Hq, Bs, D] float32 cached A_out after each step
    l_out: np.ndarray    # [S, B, Hq, Bs]
    reuse: np.ndarray    # [S, B, Hq] uint8
    sim: np.ndarray      # [S, B, Hq]
    wait_err: int = 0    # the single-launch step's wait error flag at block end


def tolerance_check(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str, rel: bool = True) -> float:
    """Max-abs 1e-5 for fp32; for bf16 max-abs 2e-2 and, since bf16 workloads
    may have tiny outputs, also 2e-2 of the reference's largest magnitude."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(gpu)), f"{what}: non-finite pattern differs"
    err = float(np.max(np.abs(gpu[fin] - ref[fin]))) if fin.any() else 0.0
    if dtype == "f32":
        assert err <= 1e-5, f"{what}: max abs err {err:.3e} > 1e-5"
    else:
        scale = float(np.max(np.abs(ref[fin]))) if fin.any() else 0.0
        assert err <= 2e-2, f"{what}: max abs err {err:.3e} > 2e-2"
        if rel:
            assert err <= 2e-2 * scale + 1e-30, f"{what}: err {err:.3e} > 2e-2 * max|ref| ({scale:.3e})"
    return err


def l_check(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.array_equal(np.isneginf(gpu), np.isneginf(ref)), f"{what}: -inf pattern differs"
    fin = np.isfinite(ref)
    err = float(np.max(np.abs(gpu[fin] - ref[fin]))) if fin.any() else 0.0
    assert err <= (1e-5 if dtype == "f32" else 1e-3), f"{what}: max abs err {err:.3e}"
    return err


def make_cache(w: wl.Workload, max_prefix: int, kv_splits: int = 0) -> fb.Cache:
    return fb.Cache(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block, max_prefix,
                    w.torch_dtype, kv_splits=kv_splits)


def device_prefix(inp: wl.Inputs, max_prefix: int, dev="cuda") -> Tuple[torch.Tensor, torch.Tensor]:
    w = inp.workload
    shape = (w.batch, w.n_kv_heads, max_prefix, w.head_dim)
    k = torch.zeros(shape, dtype=w.torch_dtype, device=dev)
    v = torch.zeros(shape, dtype=w.torch_dtype, device=dev)
    n = inp.k_prefix.shape[2]
    k[:, :, :n].copy_(inp.k_prefix)
    v[:, :, :n].copy_(inp.v_prefix)
    return k, v


def run_gpu(inp: wl.Inputs, policy: Optional[str] = None, kv_splits: int = 0,
            record_cache: bool = True, device_counts: bool = False) -> List[GpuBlock]:
    """All blocks of ``inp`` through fb_step, block K/V appended at block end.
    device_counts: the threshold counts are passed in device memory (the
    decisions are then made by the kernels)."""
    w = inp.workload
    policy = policy or w.policy
    n0 = inp.k_prefix.shape[2]
    max_prefix = n0 + w.block * (len(inp.blocks) - 1)
    cache = make_cache(w, max_prefix, kv_splits)
    kp, vp = device_prefix(inp, max_prefix)
    dt = w.torch_dtype
    q = torch.empty((w.batch, w.n_q_heads, w.block, w.head_dim), dtype=dt, device="cuda")
    kb = torch.empty((w.batch, w.n_kv_heads, w.block, w.head_dim), dtype=dt, device="cuda")
    vb = torch.empty_like(kb)
    out = torch.empty_like(q)
    m_dev = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    n = n0
    res = []
    for blk in inp.blocks:
        cache.reset()
        S = len(blk.steps)
        g = GpuBlock(np.zeros((S,) + tuple(q.shape)), np.zeros((S,) + tuple(q.shape), np.float32),
                     np.zeros((S,) + tuple(q.shape[:3]), np.float32),
                     np.zeros((S, w.batch, w.n_q_heads), np.uint8),
                     np.zeros((S, w.batch, w.n_q_heads), np.float32))
        for s, st in enumerate(blk.steps):
            q.copy_(st.q)
            kb.copy_(st.k)
            vb.copy_(st.v)
            if device_counts:
                m_dev.copy_(torch.as_tensor(np.asarray(st.n_updated, dtype=np.int32)))
                cache.step(POLICY_CODE[policy], q, kb, vb, kp, vp, n, out, tau=w.tau, gamma=w.gamma,
                           n_updated_dev=m_dev)
            else:
                cache.step(POLICY_CODE[policy], q, kb, vb, kp, vp, n, out, tau=w.tau, gamma=w.gamma,
                           n_updated=st.n_updated)
            g.out[s] = out.to(torch.float64).cpu().numpy()
            g.reuse[s] = cache.read(fb.FIELD_REUSE)
            if record_cache:
                g.a_out[s] = cache.read(fb.FIELD_A_OUT)
                g.l_out[s] = cache.read(fb.FIELD_L_OUT)
                g.sim[s] = cache.read(fb.FIELD_SIM)
        g.wait_err = int(cache.read(fb.FIELD_WAIT_ERR)[0])
        res.append(g)
        # block end: the final block K/V join the prefix
        last = blk.steps[-1]
        if n + w.block <= max_prefix:
            kp[:, :, n:n + w.block].copy_(last.k)
            vp[:, :, n:n + w.block].copy_(last.v)
        n += w.block
    torch.cuda.synchronize()
    cache.close()
    return res


def oracle_steps(blk: wl.BlockInputs, bsel=slice(None), hsel=slice(None), gsel=slice(None)):
    return [oracle.StepData(wl.to_f64(s.q[bsel, hsel]), wl.to_f64(s.k[bsel, gsel]),
                            wl.to_f64(s.v[bsel, gsel]), np.asarray(s.n_updated)[bsel])
            for s in blk.steps]


def run_oracle(inp: wl.Inputs, policy: Optional[str] = None) -> List[oracle.BlockResult]:
    w = inp.workload
    policy = policy or w.policy
    blocks = [oracle_steps(b) for b in inp.blocks]
    return oracle.run_blocks(wl.to_f64(inp.k_prefix), wl.to_f64(inp.v_prefix), blocks, policy,
                             tau=w.tau, gamma=w.gamma)


def compare_block(gpu: GpuBlock, ref: oracle.BlockResult, dtype: str, pairs=None, what="") -> dict:
    """Decisions bit-exact; outputs and cached A_out/L_out within tolerance.

    ``pairs`` maps GPU heads to oracle heads as ((b_gpu, h_gpu), (b_ref, h_ref));
    by default every head maps to itself.  Per-step outputs are also checked
    relative to the largest reference magnitude of the compared heads."""
    errs = {"out": 0.0, "a_out": 0.0, "l_out": 0.0}
    assert gpu.wait_err == 0, f"{what} a single-launch step gave up waiting for its attention items"
    S = ref.reuse.shape[0]
    if pairs is None:
        pairs = [((b, h), (b, h)) for b in range(ref.reuse.shape[1]) for h in range(ref.reuse.shape[2])]
    for (bg, hg), (br, hr) in pairs:
        np.testing.assert_array_equal(gpu.reuse[:, bg, hg], ref.reuse[:, br, hr].astype(np.uint8),
                                      err_msg=f"{what} decisions differ at head ({bg},{hg})")
    for s in range(S):
        g_out = np.stack([gpu.out[s, bg, hg] for (bg, hg), _ in pairs])
        r_out = np.stack([ref.out[s, br, hr] for _, (br, hr) in pairs])
        errs["out"] = max(errs["out"], tolerance_check(g_out, r_out, dtype, f"{what} step {s} out"))
        g_a = np.stack([gpu.a_out[s, bg, hg] for (bg, hg), _ in pairs])
        r_a = np.stack([ref.a_out[s, br, hr] for _, (br, hr) in pairs])
        errs["a_out"] = max(errs["a_out"], tolerance_check(g_a, r_a, dtype, f"{what} step {s} A_out"))
        g_l = np.stack([gpu.l_out[s, bg, hg] for (bg, hg), _ in pairs])
        r_l = np.stack([ref.l_out[s, br, hr] for _, (br, hr) in pairs])
        errs["l_out"] = max(errs["l_out"], l_check(g_l, r_l, dtype, f"{what} step {s} L_out"))
    return errs
