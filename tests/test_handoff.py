"""What the bf16 hand-off of the split partials costs, on its own.

In the bf16 path the attention launch splits the prefix keys of a group into
chunks, normalises each chunk's partial A and hands it to the fp32 combine
rounded once to bf16 (its L stays fp32); the combine folds the chunks in log
space (§2 "Mécanisme Central", the A_full equation, chained over the chunks).
Everything else here is exact (float64), so the differences below are the
hand-off's alone: the elementwise error against the unsplit external part,
and the change it makes to the per-head similarity that the gamma rule reads
(§2 "Sélection par tête"), whose GPU-vs-oracle budget in the parity tests is
5e-4.  CPU only."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from cached_attention_fb_amd import workload as wl

TILE = 64


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (nearest, ties to even) through float32, as the
    kernels store a float32 value; returned as float64."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def split_external(q, kp, vp, n, splits):
    """External part of every head with the keys cut into `splits` tile-aligned
    chunks, each chunk's A rounded to bf16 before the log-space fold; also the
    largest |A| of any chunk per row (the scale of the rounding)."""
    bsz, hq, bs, d = q.shape
    group = hq // kp.shape[1]
    scale = oracle.default_scale(d)
    per = -(-(-(-n // TILE)) // splits) * TILE
    a = np.empty((bsz, hq, bs, d))
    amax = np.zeros((bsz, hq, bs))
    for b in range(bsz):
        for h in range(hq):
            acc_a, acc_l = np.zeros((bs, d)), np.full(bs, -np.inf)
            for k0 in range(0, n, per):
                k1 = min(n, k0 + per)
                ca, cl = oracle.attend(q[b, h], kp[b, h // group, k0:k1], vp[b, h // group, k0:k1], scale)
                amax[b, h] = np.maximum(amax[b, h], np.abs(ca).max(axis=1))
                acc_a, acc_l = oracle.merge(acc_a, acc_l, to_bf16(ca), cl)
            a[b, h] = acc_a
    return a, amax


def test_to_bf16_rounding():
    """Nearest-even rounding at the bf16 grid: 1 + 2^-8 is a tie (to 1), 1 + 3*2^-8
    a tie to the even neighbour above, values on the grid stay."""
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -7, -2.5, 0.0])
    assert np.array_equal(to_bf16(x), [1.0, 1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -2.5, 0.0])


@pytest.mark.parametrize("name,prefix,splits", [("dllm-8k", 8192, 32), ("video-1560x15600", 3120, 8)])
def test_bf16_handoff_error(name, prefix, splits):
    w = wl.WORKLOADS[name]
    inp = wl.generate(w, prefix=prefix)
    kp, vp = wl.to_f64(inp.k_prefix), wl.to_f64(inp.v_prefix)
    steps = inp.blocks[0].steps[:2]
    exact, hand = [], []
    for st in steps:
        q = wl.to_f64(st.q)
        a_ref, _ = oracle.external(q, kp, vp, prefix)
        a_bf, amax = split_external(q, kp, vp, prefix, splits)
        # the fold is a convex combination of the chunks: its error is at most
        # the largest rounding of a chunk, half a bf16 ulp (2^-9 relative)
        bound = 2.0 ** -9 * amax[..., None] * (1 + 1e-9) + 1e-15
        assert np.all(np.abs(a_bf - a_ref) <= bound)
        exact.append(a_ref)
        hand.append(a_bf)
    bsz, hq = exact[0].shape[:2]
    worst = 0.0
    for b in range(bsz):
        for h in range(hq):
            s_ref = oracle.cosine(exact[1][b, h], exact[0][b, h])
            s_bf = oracle.cosine(hand[1][b, h], hand[0][b, h])
            worst = max(worst, abs(s_bf - s_ref))
    # a tenth of the similarity budget of the parity tests at most
    assert worst <= 5e-5, worst
