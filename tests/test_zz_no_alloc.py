"""fb_step_noalloc, the entry point that allocates nothing (its scratch is a
static device array), against the existing entry point it varies: fb_step
under FB_POLICY_ALWAYS on a cache.  Two calls in a row, the second with a
smaller input (the scratch keeps the first call's contents), each compared
with fb_step's output, A_out and L_out (to the bf16 / fp32 tolerances) and
with the float64 oracle; and a shape whose partials exceed the scratch is
rejected before anything runs."""
import numpy as np
import pytest
import torch

import harness as H
import oracle
from cached_attention_fb_amd import fb
from cached_attention_fb_amd import workload as wl

pytestmark = pytest.mark.gpu


def _inputs(w, prefix):
    inp = wl.generate(w, prefix=prefix)
    st = inp.blocks[0].steps[0]
    dev = [t.cuda().contiguous() for t in (st.q, st.k, st.v, inp.k_prefix, inp.v_prefix)]
    return inp, st, dev


def _via_cache(w, dev, prefix):
    q, kb, vb, kp, vp = dev
    cache = fb.Cache(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block, prefix, w.torch_dtype)
    out = torch.empty_like(q)
    cache.reset()
    cache.step(fb.POLICY_ALWAYS, q, kb, vb, kp, vp, prefix, out)
    torch.cuda.synchronize()
    res = out.to(torch.float64).cpu().numpy(), cache.read(fb.FIELD_A_OUT), cache.read(fb.FIELD_L_OUT)
    cache.close()
    return res


def _via_noalloc(w, dev, prefix):
    q, kb, vb, kp, vp = dev
    out = torch.empty_like(q)
    a_out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    l_out = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    fb.step_noalloc(q, kb, vb, kp, vp, prefix, a_out, l_out, out)
    torch.cuda.synchronize()
    return out.to(torch.float64).cpu().numpy(), a_out.cpu().numpy(), l_out.cpu().numpy()


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_fb_step_on_two_calls(order):
    cases = [
        (wl.workload("dllm-8k"), 3000),                                                  # 32/8 heads, bf16
        (wl.workload("dllm-8k").with_(n_q_heads=8, n_kv_heads=2, block=16), 500),       # smaller, bf16
    ]
    for w, prefix in cases:
        print(f"[noalloc] {w.n_q_heads}/{w.n_kv_heads} heads block {w.block} prefix {prefix}", flush=True)
        inp, st, dev = _inputs(w, prefix)
        got = _via_noalloc(w, dev, prefix)
        ref_step = _via_cache(w, dev, prefix)
        for g, r, what in zip(got, ref_step, ("out", "A_out", "L_out")):
            if what == "L_out":
                H.l_check(g, r, w.dtype, f"noalloc vs fb_step {what}")
            else:
                H.tolerance_check(g, r, w.dtype, f"noalloc vs fb_step {what}")
        # and against the float64 oracle
        q64, kb64, vb64 = wl.to_f64(st.q), wl.to_f64(st.k), wl.to_f64(st.v)
        a_ref, l_ref = oracle.external(q64, wl.to_f64(inp.k_prefix), wl.to_f64(inp.v_prefix), prefix)
        out_ref = oracle.internal_merge(q64, kb64, vb64, a_ref, l_ref)
        H.tolerance_check(got[0], out_ref, w.dtype, "noalloc out vs oracle")
        H.tolerance_check(got[1], a_ref, w.dtype, "noalloc A_out vs oracle")
        H.l_check(got[2], l_ref, w.dtype, "noalloc L_out vs oracle")
        print(f"[noalloc] bitwise equal to fb_step: out {np.array_equal(got[0], ref_step[0])} "
              f"A_out {np.array_equal(got[1], ref_step[1])}", flush=True)


def test_noalloc_fp32_and_empty_prefix():
    w = wl.workload("tiny-fp32").with_(blocks=1)
    for prefix in (512, 0):
        inp, st, dev = _inputs(w, prefix)
        if prefix == 0:   # prefix buffers of one (unused) row
            dev[3] = torch.zeros((w.batch, w.n_kv_heads, 1, w.head_dim), device="cuda")
            dev[4] = dev[3].clone()
        got = _via_noalloc(w, dev, prefix)
        q64, kb64, vb64 = wl.to_f64(st.q), wl.to_f64(st.k), wl.to_f64(st.v)
        kp64 = wl.to_f64(inp.k_prefix) if prefix else np.zeros((w.batch, w.n_kv_heads, 0, w.head_dim))
        a_ref, l_ref = oracle.external(q64, kp64, kp64, prefix) if prefix == 0 else \
            oracle.external(q64, wl.to_f64(inp.k_prefix), wl.to_f64(inp.v_prefix), prefix)
        out_ref = oracle.internal_merge(q64, kb64, vb64, a_ref, l_ref)
        H.tolerance_check(got[0], out_ref, "f32", f"noalloc fp32 prefix {prefix} out")
        H.l_check(got[2], l_ref, "f32", f"noalloc fp32 prefix {prefix} L_out")


def test_noalloc_rejects_shapes_beyond_the_scratch():
    q = torch.zeros((1, 256, 1024, 128), dtype=torch.bfloat16, device="cuda")   # 64 MiB of partials per chunk
    kb = torch.zeros((1, 1, 1024, 128), dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    a_out = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    l_out = torch.zeros(q.shape[:3], dtype=torch.float32, device="cuda")
    with pytest.raises(fb.FBError) as e:
        fb.step_noalloc(q, kb, kb, kp, kp, 64, a_out, l_out, q.clone())
    assert e.value.code == fb.FB_E_SHAPE
    assert "scratch" in str(e.value)
