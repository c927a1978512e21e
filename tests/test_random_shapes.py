"""Seeded random shapes through fb_step against the float64 oracle.

The configurations straddle the launch-shape boundaries of the bf16 kernels:
packed rows per kv head up to 32 (one wave), up to 128 (key-half 4x2, or four
whole-tile waves for short key ranges), up to 511 (eight row-waves) and 512 or
more (block-internal attention on the split-key shape); blocks of at most one
key tile (the one-tile block-internal launch) and longer ones; prefixes from
empty to many tiles, with automatic or forced split counts; D = 64 and 128;
several sequences; and a few fp32 caches.  Each runs one short block under the
threshold policy (some steps reuse, some recompute) and is compared with the
oracle on outputs, decisions and the cached parts.
"""
import numpy as np
import pytest

import harness as H
from cached_attention_fb_amd import workload as wl

N_CASES = 48
ROW_TARGETS = (20, 32, 100, 128, 200, 511, 600)   # packed rows per kv head, around each shape limit
BUDGET = 3.0e6                                      # B * Hq * Bs * (prefix + Bs): the oracle's work


def draw(i):
    rng = np.random.default_rng(9000 + i)
    fp32 = i % 8 == 7
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4]))
    grp = int(rng.choice([1, 2, 4, 8]))
    rows = int(ROW_TARGETS[i % len(ROW_TARGETS)]) + int(rng.integers(-3, 4))
    bs = max(1, rows // grp)
    batch = int(rng.choice([1, 1, 2, 3]))
    hq = hkv * grp
    cap = int(BUDGET / (batch * hq * bs)) - bs
    prefix = int(rng.integers(0, max(1, min(cap, 5000)) + 1))
    splits = int(rng.choice([0, 0, 1, 2, 5]))
    base = wl.workload("tiny-fp32" if fp32 else "dllm-8k")
    # the updated-token count is drawn over the block's own tokens
    upd = bs if base.update == "binomial" else min(int(base.update_a), bs)
    w = base.with_(batch=batch, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, block=bs, steps=3, blocks=1,
                   update_a=upd, tau=max(1, bs // 4), seed=7000 + i)
    return w, prefix, splits


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    w, prefix, splits = draw(i)
    print(f"[random {i}] {w.dtype} B={w.batch} Hq/Hkv={w.n_q_heads}/{w.n_kv_heads} D={w.head_dim} "
          f"Bs={w.block} rows={w.block * w.n_q_heads // w.n_kv_heads} prefix={prefix} splits={splits}", flush=True)
    inp = wl.generate(w, prefix=prefix)
    gpu = H.run_gpu(inp, kv_splits=splits)
    ref = H.run_oracle(inp)
    for b, (g, r) in enumerate(zip(gpu, ref)):
        errs = H.compare_block(g, r, w.dtype, what=f"random {i} block {b}")
        print(f"[random {i}] errs {errs} reused {int(g.reuse.sum())}", flush=True)


def test_draws_cover_the_shapes():
    """The draws reach every row range, both block kinds and both head sizes
    (a property of the seeded draws, checked without a GPU)."""
    seen = set()
    for i in range(N_CASES):
        w, prefix, _ = draw(i)
        rows = w.block * w.n_q_heads // w.n_kv_heads
        seen.add(("rows", 0 if rows <= 32 else 1 if rows <= 128 else 2 if rows < 512 else 3))
        seen.add(("one_tile", w.block <= 64))
        seen.add(("d", w.head_dim))
        seen.add(("empty", prefix == 0))
    for key in [("rows", k) for k in range(4)] + [("one_tile", True), ("one_tile", False), ("d", 64), ("d", 128)]:
        assert key in seen, key


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(0, N_CASES, 3))
def test_random_shape_device_counts(i):
    """The same shapes with the threshold counts in device memory: decisions
    made by the kernels, compared with the oracle's."""
    w, prefix, splits = draw(i)
    print(f"[random-dev {i}] {w.dtype} B={w.batch} Hq/Hkv={w.n_q_heads}/{w.n_kv_heads} D={w.head_dim} "
          f"Bs={w.block} prefix={prefix} splits={splits}", flush=True)
    inp = wl.generate(w, prefix=prefix)
    gpu = H.run_gpu(inp, kv_splits=splits, device_counts=True)
    ref = H.run_oracle(inp)
    for b, (g, r) in enumerate(zip(gpu, ref)):
        H.compare_block(g, r, w.dtype, what=f"random-dev {i} block {b}")


@pytest.mark.gpu
@pytest.mark.parametrize("i", [i for i in range(1, N_CASES, 2) if i % 8 != 7])
def test_random_shape_sparse(i):
    """The bf16 shapes through fb_step_sparse with a seeded selection of
    20-60 % of the prefix tiles (tile-list attention in every launch shape),
    with the draw's split count (automatic or forced: the two tile sets of a
    recompute step planned together, or the kept set cut to the left-out
    set's range length) and, for every other case, the threshold counts in
    device memory (the split plan chosen on the device)."""
    from test_sparse_parity import run_gpu_sparse, run_oracle_sparse
    w, prefix, splits = draw(i)
    density = 0.2 + 0.4 * ((i * 37) % 11) / 10
    dev = i % 4 == 3
    print(f"[random-sparse {i}] B={w.batch} Hq/Hkv={w.n_q_heads}/{w.n_kv_heads} D={w.head_dim} "
          f"Bs={w.block} prefix={prefix} density={density:.2f} splits={splits} device_counts={dev}", flush=True)
    inp = wl.generate(w, prefix=prefix)
    gpu, sels = run_gpu_sparse(inp, density, device_counts=dev, kv_splits=splits)
    ref = run_oracle_sparse(inp, sels)
    for b, (g, r) in enumerate(zip(gpu, ref)):
        H.compare_block(g, r, w.dtype, what=f"random-sparse {i} block {b}")


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(0, N_CASES, 4))
def test_random_shape_single_launch(i, monkeypatch):
    """The same shapes with the opt-in single-launch step (FB_FIN=1 at cache
    allocation), with host decisions and, for every other case, device-made
    ones: where the kernels allow it a recompute step is one launch, else it
    keeps the two; either way the oracle's results."""
    w, prefix, splits = draw(i)
    dev = i % 8 == 4
    print(f"[random-fin {i}] {w.dtype} B={w.batch} Hq/Hkv={w.n_q_heads}/{w.n_kv_heads} D={w.head_dim} "
          f"Bs={w.block} prefix={prefix} splits={splits} device_counts={dev}", flush=True)
    inp = wl.generate(w, prefix=prefix)
    monkeypatch.setenv("FB_FIN", "1")
    gpu = H.run_gpu(inp, kv_splits=splits, device_counts=dev)
    monkeypatch.delenv("FB_FIN", raising=False)
    ref = H.run_oracle(inp)
    for b, (g, r) in enumerate(zip(gpu, ref)):
        H.compare_block(g, r, w.dtype, what=f"random-fin {i} block {b}")
