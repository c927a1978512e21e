"""Pins of the float64 oracle to things other than itself.

Each ``pin_*`` function checks one fact that the page or plain mathematics
fixes: a scalar brute force on tiny inputs, an independent library routine
(torch's float64 scaled_dot_product_attention and logsumexp, scipy's cosine
distance), closed forms, invariants, and the policy's special cases.  The pins
look the oracle's functions up on the module at call time, so
``test_planted_mistakes`` can swap a function for a plausibly wrong one and
show that some pin fails.  Everything here runs on the CPU.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.spatial.distance
import torch

import oracle.flashblock as fb

TOL = 1e-12


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- attend

def pin_attend_bruteforce():
    """Scalar triple loop on tiny inputs: softmax written out term by term."""
    rng = _rng(1)
    for (r, n, d) in [(3, 5, 4), (1, 1, 2), (2, 7, 3)]:
        q, k, v = rng.standard_normal((r, d)), rng.standard_normal((n, d)), rng.standard_normal((n, d))
        scale = 0.37
        a, lse = fb.attend(q, k, v, scale)
        for i in range(r):
            scores = [scale * sum(q[i][t] * k[j][t] for t in range(d)) for j in range(n)]
            z = sum(math.exp(sc) for sc in scores)
            assert abs(lse[i] - math.log(z)) <= TOL
            for t in range(d):
                ref = sum(math.exp(scores[j]) * v[j][t] for j in range(n)) / z
                assert abs(a[i][t] - ref) <= TOL


def pin_attend_vs_torch():
    """torch float64 SDPA (default scale 1/sqrt(D)) and logsumexp."""
    rng = _rng(2)
    for (r, n, d) in [(32, 512, 64), (5, 1, 128), (1, 65, 16), (64, 300, 128)]:
        q, k, v = (rng.standard_normal((r, d)), rng.standard_normal((n, d)),
                   rng.standard_normal((n, d)))
        a, lse = fb.attend(q, k, v, fb.default_scale(d))
        tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, 0].numpy()
        assert np.max(np.abs(a - ref)) <= TOL
        ref_l = torch.logsumexp(torch.from_numpy(q @ k.T) / math.sqrt(d), dim=-1).numpy()
        assert np.max(np.abs(lse - ref_l)) <= 1e-10


def pin_external_gqa_vs_torch():
    """Query head h reads key/value head h // G: torch's enable_gqa mapping."""
    rng = _rng(3)
    b, hq, hkv, bs, n, d = 2, 8, 2, 6, 40, 16
    q = rng.standard_normal((b, hq, bs, d))
    kp = rng.standard_normal((b, hkv, n + 5, d)) * 2.0
    vp = rng.standard_normal((b, hkv, n + 5, d))
    a, lse = fb.external(q, kp, vp, n)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(kp[:, :, :n]).contiguous(),
        torch.from_numpy(vp[:, :, :n]).contiguous(), enable_gqa=True).numpy()
    assert np.max(np.abs(a - ref)) <= TOL
    kr = np.repeat(kp[:, :, :n], hq // hkv, axis=1)
    ref_l = torch.logsumexp(torch.from_numpy(np.einsum("bhrd,bhnd->bhrn", q, kr)) / math.sqrt(d), -1)
    assert np.max(np.abs(lse - ref_l.numpy())) <= 1e-10


def pin_attend_closed_forms():
    rng = _rng(4)
    d = 8
    # a single key: A = v, L = its score
    q, k, v = rng.standard_normal((3, d)), rng.standard_normal((1, d)), rng.standard_normal((1, d))
    a, lse = fb.attend(q, k, v, 0.5)
    assert np.max(np.abs(a - v[0])) <= TOL
    assert np.max(np.abs(lse - 0.5 * (q @ k[0]))) <= TOL
    # constant values: A = that constant whatever the weights
    k = rng.standard_normal((9, d))
    v = np.tile(rng.standard_normal(d), (9, 1))
    a, _ = fb.attend(q, k, v, 0.5)
    assert np.max(np.abs(a - v[0])) <= TOL
    # all keys equal: uniform weights, A = mean(V), L = s + ln N
    k = np.tile(rng.standard_normal(d), (9, 1))
    v = rng.standard_normal((9, d))
    a, lse = fb.attend(q, k, v, 0.5)
    assert np.max(np.abs(a - v.mean(0))) <= TOL
    assert np.max(np.abs(lse - (0.5 * (q @ k[0]) + math.log(9)))) <= TOL
    # zero queries: L = ln N exactly, A = mean(V)
    a, lse = fb.attend(np.zeros((2, d)), rng.standard_normal((9, d)), v, 0.5)
    assert np.max(np.abs(lse - math.log(9))) <= TOL
    assert np.max(np.abs(a - v.mean(0))) <= TOL
    # worked two-key case: scores 0 and ln 3 -> weights 1/4, 3/4, L = ln 4
    a, lse = fb.attend(np.array([[1.0]]), np.array([[0.0], [math.log(3.0)]]),
                       np.array([[2.0, -1.0], [6.0, 3.0]]), 1.0)
    assert np.max(np.abs(a[0] - np.array([5.0, 2.0]))) <= TOL
    assert abs(lse[0] - math.log(4.0)) <= TOL
    # huge logits stay finite: the max key dominates, L = its score
    q = np.array([[30.0] * d])
    k = np.array([[1.0] * d, [0.5] * d, [-1.0] * d])
    v = rng.standard_normal((3, d))
    a, lse = fb.attend(q, k, v, 1.0)
    assert np.all(np.isfinite(a)) and np.isfinite(lse[0])
    assert np.max(np.abs(a[0] - v[0])) <= TOL
    assert abs(lse[0] - 240.0) <= 1e-9
    # empty key set: no mass
    a, lse = fb.attend(q, np.zeros((0, d)), np.zeros((0, d)), 1.0)
    assert np.all(a == 0) and np.all(np.isneginf(lse))


def pin_attend_permutation_invariance():
    rng = _rng(5)
    q, k, v = rng.standard_normal((4, 16)), rng.standard_normal((33, 16)), rng.standard_normal((33, 16))
    perm = rng.permutation(33)
    a1, l1 = fb.attend(q, k, v, 0.25)
    a2, l2 = fb.attend(q, k[perm], v[perm], 0.25)
    assert np.max(np.abs(a1 - a2)) <= TOL and np.max(np.abs(l1 - l2)) <= TOL


# ---------------------------------------------------------------- merge

def pin_merge_equals_full_attention():
    """Merging fresh external and internal parts is attention over J_out u J_in."""
    rng = _rng(6)
    for (r, n_out, n_in, d, sd) in [(32, 512, 32, 64, 1.0), (16, 1, 16, 128, 3.0),
                                    (8, 100, 1, 32, 0.1), (5, 2000, 64, 16, 2.0)]:
        q = rng.standard_normal((r, d)) * sd
        ko, vo = rng.standard_normal((n_out, d)) * sd, rng.standard_normal((n_out, d))
        ki, vi = rng.standard_normal((n_in, d)) * sd, rng.standard_normal((n_in, d))
        scale = fb.default_scale(d)
        a_o, l_o = fb.attend(q, ko, vo, scale)
        a_i, l_i = fb.attend(q, ki, vi, scale)
        a_m, l_m = fb.merge(a_o, l_o, a_i, l_i)
        a_f, l_f = fb.attend(q, np.concatenate([ko, ki]), np.concatenate([vo, vi]), scale)
        assert np.max(np.abs(a_m - a_f)) <= TOL
        assert np.max(np.abs(l_m - l_f)) <= 1e-10
        assert np.max(np.abs(l_m - np.logaddexp(l_o, l_i))) <= 1e-10


def pin_merge_special_cases():
    rng = _rng(7)
    q = rng.standard_normal((6, 16))
    ki, vi = rng.standard_normal((10, 16)), rng.standard_normal((10, 16))
    a_i, l_i = fb.attend(q, ki, vi, 0.25)
    a_o, l_o = fb.attend(q, np.zeros((0, 16)), np.zeros((0, 16)), 0.25)
    a_m, l_m = fb.merge(a_o, l_o, a_i, l_i)      # empty prefix: output = internal part
    assert np.max(np.abs(a_m - a_i)) <= TOL and np.max(np.abs(l_m - l_i)) <= TOL
    ko, vo = rng.standard_normal((20, 16)), rng.standard_normal((20, 16))
    a_o, l_o = fb.attend(q, ko, vo, 0.25)
    a1, l1 = fb.merge(a_o, l_o, a_i, l_i)
    a2, l2 = fb.merge(a_i, l_i, a_o, l_o)        # the roles are symmetric
    assert np.max(np.abs(a1 - a2)) <= TOL and np.max(np.abs(l1 - l2)) <= TOL
    # equal normalisers: plain average of the two parts
    a_m, _ = fb.merge(a_o, np.zeros(6), a_i, np.zeros(6))
    assert np.max(np.abs(a_m - 0.5 * (a_o + a_i))) <= TOL
    # a part with e^{L} twice the other weighs 2/3
    a_m, l_m = fb.merge(a_o, np.full(6, math.log(2.0)), a_i, np.zeros(6))
    assert np.max(np.abs(a_m - (2 * a_o + a_i) / 3)) <= TOL
    assert np.max(np.abs(l_m - math.log(3.0))) <= TOL


def pin_split_associativity():
    """Splitting J_out into k chunks and merging them in any order gives the unsplit result."""
    rng = _rng(8)
    n, d = 97, 32
    q = rng.standard_normal((7, d))
    k, v = rng.standard_normal((n, d)) * 1.5, rng.standard_normal((n, d))
    a_ref, l_ref = fb.attend(q, k, v, 0.2)
    for chunks in (1, 2, 7, n):
        bounds = np.linspace(0, n, chunks + 1).astype(int)
        parts = [fb.attend(q, k[s:e], v[s:e], 0.2) for s, e in zip(bounds[:-1], bounds[1:])]
        for order in (list(range(chunks)), list(reversed(range(chunks))), list(rng.permutation(chunks))):
            a, lse = parts[order[0]]
            for i in order[1:]:
                a, lse = fb.merge(a, lse, *parts[i])
            assert np.max(np.abs(a - a_ref)) <= TOL and np.max(np.abs(lse - l_ref)) <= 1e-10
        # pairwise tree
        level = list(parts)
        while len(level) > 1:
            nxt = [fb.merge(*level[i], *level[i + 1]) for i in range(0, len(level) - 1, 2)]
            if len(level) % 2:
                nxt.append(level[-1])
            level = nxt
        assert np.max(np.abs(level[0][0] - a_ref)) <= TOL


# ---------------------------------------------------------------- cosine

def pin_cosine():
    rng = _rng(9)
    for _ in range(5):
        a, o = rng.standard_normal((4, 8)), rng.standard_normal((4, 8))
        ref = 1.0 - scipy.spatial.distance.cosine(a.ravel(), o.ravel())
        assert abs(fb.cosine(a, o) - ref) <= 1e-12
    a = rng.standard_normal(50)
    assert abs(fb.cosine(a, 3.0 * a) - 1.0) <= 1e-12
    assert abs(fb.cosine(a, -a) + 1.0) <= 1e-12
    assert fb.cosine(a, a) <= 1.0
    x, y = np.zeros(4), np.zeros(4)
    x[0], y[1] = 2.0, 5.0
    assert abs(fb.cosine(x, y)) <= 1e-15
    assert fb.cosine(np.zeros(3), np.zeros(3)) == 1.0
    assert fb.cosine(np.zeros(3), np.ones(3)) == 0.0
    # a vector and a small perturbation of it: 1 - cos ~ |e|^2 sin^2 / 2 > 0
    e = rng.standard_normal(50) * 1e-3
    assert 0.0 < 1.0 - fb.cosine(a, a + e) < 1e-5


# ---------------------------------------------------------------- policy

def _steps(rng, b, hq, hkv, bs, d, m_list, redraw=True, sd=1.0):
    """Block inputs where the M rows of each step are redrawn (or kept when redraw=False)."""
    q = rng.standard_normal((b, hq, bs, d)) * sd
    k = rng.standard_normal((b, hkv, bs, d)) * sd
    v = rng.standard_normal((b, hkv, bs, d))
    steps = []
    for s, m in enumerate(m_list):
        m = np.asarray(m)
        if s > 0 and redraw:
            for bi in range(b):
                pos = rng.choice(bs, int(m[bi]), replace=False)
                q[bi][:, pos] = rng.standard_normal((hq, len(pos), d)) * sd
                k[bi][:, pos] = rng.standard_normal((hkv, len(pos), d)) * sd
                v[bi][:, pos] = rng.standard_normal((hkv, len(pos), d))
        steps.append(fb.StepData(q.copy(), k.copy(), v.copy(), m.astype(np.int32)))
    return steps


def _exact(kp, vp, n, step, b, h, group):
    g = h // group
    return fb.attend(step.q[b, h], np.concatenate([kp[b, g, :n], step.k[b, g]]),
                     np.concatenate([vp[b, g, :n], step.v[b, g]]), fb.default_scale(step.q.shape[-1]))[0]


def pin_tau_policy():
    rng = _rng(10)
    b, hq, hkv, bs, d, n = 2, 4, 2, 8, 16, 40
    kp, vp = rng.standard_normal((b, hkv, n, d)), rng.standard_normal((b, hkv, n, d))
    m_list = [[0, 0], [3, 0], [4, 1], [5, 4], [0, 8], [4, 3], [2, 4]]
    steps = _steps(rng, b, hq, hkv, bs, d, m_list)
    tau = 4
    res = fb.run_block(kp, vp, n, steps, fb.TAU, tau=tau)
    for s, m in enumerate(m_list):
        for bi in range(b):
            expect = 0 if s == 0 else int(m[bi] < tau)     # strict: M == tau recomputes
            assert np.all(res.reuse[s, bi] == expect), (s, bi)
    # number of reuse steps = sum over s >= 1 of [M_s < tau]
    for bi in range(b):
        assert int(res.reuse[:, bi, 0].sum()) == sum(int(m[bi] < tau) for m in m_list[1:])
    # tau = 0: never reuse, every output is exact attention over J_out u J_in
    res0 = fb.run_block(kp, vp, n, steps, fb.TAU, tau=0)
    assert np.all(res0.reuse == 0)
    for s, st in enumerate(steps):
        for bi, h in itertools.product(range(b), range(hq)):
            assert np.max(np.abs(res0.out[s, bi, h] - _exact(kp, vp, n, st, bi, h, hq // hkv))) <= TOL
    # always: never reuse either
    assert np.all(fb.run_block(kp, vp, n, steps, fb.ALWAYS).reuse == 0)
    # tau > Bs: every step after the first reuses, and the cache keeps step 0's A_out
    resb = fb.run_block(kp, vp, n, steps, fb.TAU, tau=bs + 1)
    assert np.all(resb.reuse[0] == 0) and np.all(resb.reuse[1:] == 1)
    for s in range(1, len(steps)):
        assert np.array_equal(resb.a_out[s], resb.a_out[0])
        assert np.array_equal(resb.l_out[s], resb.l_out[0])
    # a reuse step with changed queries is not exact attention (the cache is stale)
    assert np.max(np.abs(resb.out[1, 0] - res0.out[1, 0])) > 1e-6
    # M = 0 at every step: nothing changes, every step after 0 reuses and stays exact
    steps0 = _steps(rng, b, hq, hkv, bs, d, [[0, 0]] * 5)
    resz = fb.run_block(kp, vp, n, steps0, fb.TAU, tau=1)
    assert np.all(resz.reuse[1:] == 1)
    for s, st in enumerate(steps0):
        for bi, h in itertools.product(range(b), range(hq)):
            assert np.max(np.abs(resz.out[s, bi, h] - _exact(kp, vp, n, st, bi, h, hq // hkv))) <= TOL


def _video_steps(rng, hq, bs, d, sigma, n_steps):
    qb = rng.standard_normal((1, hq, bs, d))
    k = rng.standard_normal((1, hq, bs, d))
    v = rng.standard_normal((1, hq, bs, d))
    steps = []
    for _ in range(n_steps):
        q = qb + sigma[None, :, None, None] * rng.standard_normal(qb.shape)
        steps.append(fb.StepData(q, k, v, np.full(1, bs, dtype=np.int32)))
    return steps


def pin_gamma_policy():
    rng = _rng(11)
    hq, bs, d, n = 3, 6, 8, 30
    kp, vp = rng.standard_normal((1, hq, n, d)), rng.standard_normal((1, hq, n, d))
    # sigma = 0: the queries never change, sim = 1 > gamma, the head reuses from step 2 on
    steps = _video_steps(rng, hq, bs, d, np.zeros(hq), 5)
    res = fb.run_block(kp, vp, n, steps, fb.GAMMA, gamma=0.95)
    assert np.all(res.reuse[:2] == 0) and np.all(res.reuse[2:] == 1)
    assert np.all(np.abs(res.sim[1:] - 1.0) <= 1e-12) and np.all(np.isnan(res.sim[0]))
    # gamma = 1 never reuses (strict, cosine <= 1)
    assert np.all(fb.run_block(kp, vp, n, steps, fb.GAMMA, gamma=1.0).reuse == 0)
    # gamma = -1: every head reuses from step 2 whatever its queries do
    steps = _video_steps(rng, hq, bs, d, np.array([0.05, 1.0, 5.0]), 5)
    res = fb.run_block(kp, vp, n, steps, fb.GAMMA, gamma=-1.0)
    assert np.all(res.reuse[:2] == 0) and np.all(res.reuse[2:] == 1)
    # mixed: a quiet head reuses, a loud one keeps recomputing, sims match scipy
    res = fb.run_block(kp, vp, n, steps, fb.GAMMA, gamma=0.95)
    assert res.reuse[2, 0, 0] == 1 and np.all(res.reuse[:, 0, 2] == 0)
    for s in range(1, 5):
        if res.reuse[s, 0, 2] == 0:
            ref = fb.attend(steps[s - 1].q[0, 2], kp[0, 2], vp[0, 2], fb.default_scale(d))[0]
            new = fb.attend(steps[s].q[0, 2], kp[0, 2], vp[0, 2], fb.default_scale(d))[0]
            assert abs(res.sim[s, 0, 2] - (1 - scipy.spatial.distance.cosine(new.ravel(), ref.ravel()))) < 1e-12


def pin_multi_block_append():
    """Block end: the block's final K/V join the prefix and the caches restart."""
    rng = _rng(12)
    b, hq, hkv, bs, d, n = 1, 2, 1, 4, 8, 10
    kp, vp = rng.standard_normal((b, hkv, n, d)), rng.standard_normal((b, hkv, n, d))
    blk1 = _steps(rng, b, hq, hkv, bs, d, [[0], [1], [4]])
    blk2 = _steps(rng, b, hq, hkv, bs, d, [[0], [0], [2]])
    r1, r2 = fb.run_blocks(kp, vp, [blk1, blk2], fb.TAU, tau=3)
    assert np.all(r2.reuse[0] == 0)                    # fresh block: no reuse at its first step
    kp2 = np.concatenate([kp, blk1[-1].k], axis=2)
    vp2 = np.concatenate([vp, blk1[-1].v], axis=2)
    for h in range(hq):
        assert np.max(np.abs(r2.out[0, 0, h] - _exact(kp2, vp2, n + bs, blk2[0], 0, h, hq))) <= TOL


def pin_tau_cum_policy():
    """Cumulative variant: the updated tokens are summed since the cache was
    computed; a worked sequence, and its special cases."""
    rng = _rng(13)
    b, hq, hkv, bs, d, n = 1, 2, 1, 8, 8, 20
    kp, vp = rng.standard_normal((b, hkv, n, d)), rng.standard_normal((b, hkv, n, d))
    m_list = [[0], [3], [3], [3], [0], [5], [1]]
    steps = _steps(rng, b, hq, hkv, bs, d, m_list)
    res = fb.run_block(kp, vp, n, steps, fb.TAU_CUM, tau=5)
    # sums since the last computation: 3 (reuse), 6 (compute), 3, 3, 8 (compute), 1
    assert [int(res.reuse[s, 0, 0]) for s in range(len(m_list))] == [0, 1, 0, 1, 1, 0, 1]
    for s in (0, 2, 5):   # computed steps are exact attention
        for h in range(hq):
            assert np.max(np.abs(res.out[s, 0, h] - _exact(kp, vp, n, steps[s], 0, h, hq))) <= TOL
    assert np.array_equal(res.a_out[4], res.a_out[2]) and np.array_equal(res.a_out[6], res.a_out[5])
    # the per-step rule on the same inputs reuses at every step with M < 5
    res_tau = fb.run_block(kp, vp, n, steps, fb.TAU, tau=5)
    assert [int(res_tau.reuse[s, 0, 0]) for s in range(len(m_list))] == [0, 1, 1, 1, 1, 0, 1]
    # tau = 0 never reuses; M = 0 throughout reuses from step 1 and stays exact
    assert np.all(fb.run_block(kp, vp, n, steps, fb.TAU_CUM, tau=0).reuse == 0)
    steps0 = _steps(rng, b, hq, hkv, bs, d, [[0]] * 4)
    r0 = fb.run_block(kp, vp, n, steps0, fb.TAU_CUM, tau=1)
    assert np.all(r0.reuse[1:] == 1)
    for s, st in enumerate(steps0):
        for h in range(hq):
            assert np.max(np.abs(r0.out[s, 0, h] - _exact(kp, vp, n, st, 0, h, hq))) <= TOL


def pin_gamma_group_policy():
    """Group variant: one similarity per group of query heads sharing a kv
    head, the cosine of their A_out taken as one vector."""
    rng = _rng(14)
    hq, hkv, bs, d, n = 4, 2, 6, 8, 30
    kp, vp = rng.standard_normal((1, hkv, n, d)), rng.standard_normal((1, hkv, n, d))
    sigma = np.array([0.02, 0.6, 0.05, 0.04])
    qb = rng.standard_normal((1, hq, bs, d))
    k = rng.standard_normal((1, hkv, bs, d))
    v = rng.standard_normal((1, hkv, bs, d))
    steps = [fb.StepData(qb + sigma[None, :, None, None] * rng.standard_normal(qb.shape), k, v,
                         np.full(1, bs, dtype=np.int32)) for _ in range(5)]
    res = fb.run_block(kp, vp, n, steps, fb.GAMMA_GROUP, gamma=2.0)   # never reuses: every sim defined
    sc = fb.default_scale(d)
    for s in range(1, 5):
        for g in range(hkv):
            new = np.concatenate([fb.attend(steps[s].q[0, h], kp[0, g], vp[0, g], sc)[0].ravel()
                                  for h in (2 * g, 2 * g + 1)])
            old = np.concatenate([fb.attend(steps[s - 1].q[0, h], kp[0, g], vp[0, g], sc)[0].ravel()
                                  for h in (2 * g, 2 * g + 1)])
            ref = 1.0 - scipy.spatial.distance.cosine(new, old)
            assert abs(res.sim[s, 0, 2 * g] - ref) <= 1e-12 and res.sim[s, 0, 2 * g + 1] == res.sim[s, 0, 2 * g]
    # the decision is shared by the group: the loud head 1 keeps group 0 recomputing
    resg = fb.run_block(kp, vp, n, steps, fb.GAMMA_GROUP, gamma=0.97)
    assert np.all(resg.reuse[:, 0, 0] == resg.reuse[:, 0, 1]) and np.all(resg.reuse[:, 0, 2] == resg.reuse[:, 0, 3])
    assert np.all(resg.reuse[:, 0, 0] == 0) and np.all(resg.reuse[2:, 0, 2] == 1)
    resh = fb.run_block(kp, vp, n, steps, fb.GAMMA, gamma=0.97)
    assert np.all(resh.reuse[2:, 0, 0] == 1)      # per head, the quiet head 0 would reuse
    # groups of one head: identical to the per-head rule
    kp1, vp1 = rng.standard_normal((1, hq, n, d)), rng.standard_normal((1, hq, n, d))
    steps1 = _video_steps(rng, hq, bs, d, np.array([0.02, 0.3, 0.05, 1.0]), 5)
    a = fb.run_block(kp1, vp1, n, steps1, fb.GAMMA_GROUP, gamma=0.95)
    bres = fb.run_block(kp1, vp1, n, steps1, fb.GAMMA, gamma=0.95)
    assert np.array_equal(a.reuse, bres.reuse) and np.array_equal(a.out, bres.out)
    assert np.array_equal(np.nan_to_num(a.sim, nan=-9), np.nan_to_num(bres.sim, nan=-9))


# ---------------------------------------------------------------- sparse residual reuse

def _sdpa_rows(q, k, v):
    """torch's float64 scaled-dot-product attention of rows q over keys k."""
    t = lambda x: torch.as_tensor(np.asarray(x, np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))[0, 0].numpy()


def _sparse_setup(seed, n=150, b=2, hq=4, hkv=2, bs=8, d=16, m_list=None):
    rng = _rng(seed)
    kp, vp = rng.standard_normal((b, hkv, n, d)), rng.standard_normal((b, hkv, n, d))
    m_list = m_list or [[0] * b, [2] * b, [8] * b, [1] * b]
    steps = _steps(rng, b, hq, hkv, bs, d, m_list)
    return rng, kp, vp, steps


def pin_sparse_always_is_exact():
    """Recomputing the residual every step gives exact attention over the whole
    prefix and the block, whatever the selection (kept + left = prefix)."""
    rng, kp, vp, steps = _sparse_setup(30)
    n, tiles = kp.shape[2], 3                      # tiles 0, 1 and a ragged tile 2 (22 rows)
    for sel in (np.array([[[2], [0]], [[1], [2]]]), np.array([[[0, 2], [1, 2]], [[0, 1], [0, 2]]])):
        res = fb.run_block_sparse(kp, vp, n, steps, sel, fb.ALWAYS)
        for s, st in enumerate(steps):
            for bi in range(2):
                for h in range(4):
                    g = h // 2
                    ref = _sdpa_rows(st.q[bi, h], np.concatenate([kp[bi, g], st.k[bi, g]]),
                                     np.concatenate([vp[bi, g], st.v[bi, g]]))
                    assert np.max(np.abs(res.out[s, bi, h] - ref)) < 1e-12
        assert np.all(res.reuse == 0)


def pin_sparse_all_kept_is_exact():
    """With every tile kept the residual is empty (L = -inf), so even steps
    that reuse it are exact attention."""
    rng, kp, vp, steps = _sparse_setup(31)
    sel = np.tile(np.arange(3), (2, 2, 1))
    res = fb.run_block_sparse(kp, vp, kp.shape[2], steps, sel, fb.TAU, tau=4)
    assert res.reuse[1:].any()
    assert np.all(np.isneginf(res.l_out))
    for s, st in enumerate(steps):
        for bi in range(2):
            for h in range(4):
                g = h // 2
                ref = _sdpa_rows(st.q[bi, h], np.concatenate([kp[bi, g], st.k[bi, g]]),
                                 np.concatenate([vp[bi, g], st.v[bi, g]]))
                assert np.max(np.abs(res.out[s, bi, h] - ref)) < 1e-12


def pin_sparse_none_kept_is_flashblock():
    """With no tile kept the method is FlashBlock itself: every record equals
    run_block's bit for bit (merging an empty part changes nothing)."""
    rng, kp, vp, steps = _sparse_setup(32)
    sel = np.zeros((2, 2, 0), np.int64)
    for pol, kw in ((fb.TAU, {"tau": 4}), (fb.GAMMA, {"gamma": 0.5})):
        a = fb.run_block_sparse(kp, vp, kp.shape[2], steps, sel, pol, **kw)
        r = fb.run_block(kp, vp, kp.shape[2], steps, pol, **kw)
        for f in ("out", "a_out", "l_out", "reuse"):
            assert np.array_equal(getattr(a, f), getattr(r, f)), f
        assert np.array_equal(np.nan_to_num(a.sim, nan=-9), np.nan_to_num(r.sim, nan=-9))


def pin_sparse_stale_residual_bruteforce():
    """A reused residual is the left-out keys' contribution for the query of
    the step that computed it: scalar brute force over two steps (the second
    reuses), with the kept tile the ragged last one."""
    rng = _rng(33)
    n, bs, d = 70, 3, 4
    kp, vp = rng.standard_normal((1, 1, n, d)), rng.standard_normal((1, 1, n, d))
    steps = _steps(rng, 1, 1, 1, bs, d, [[0], [3]])
    sel = np.array([[[1]]])                       # keeps rows 64..69, leaves 0..63
    res = fb.run_block_sparse(kp, vp, n, steps, sel, fb.TAU, tau=100)
    assert list(res.reuse[:, 0, 0]) == [0, 1]
    c = 1.0 / math.sqrt(d)
    q1, st2 = steps[0].q[0, 0], steps[1]
    for i in range(bs):
        num, den = [0.0] * d, 0.0
        terms = [(st2.q[0, 0, i], kp[0, 0, j], vp[0, 0, j]) for j in range(64, n)]
        terms += [(st2.q[0, 0, i], st2.k[0, 0, j], st2.v[0, 0, j]) for j in range(bs)]
        terms += [(q1[i], kp[0, 0, j], vp[0, 0, j]) for j in range(64)]   # stale: the first step's query
        for qi, kj, vj in terms:
            w = math.exp(c * sum(float(qi[t]) * float(kj[t]) for t in range(d)))
            den += w
            num = [num[t] + w * float(vj[t]) for t in range(d)]
        assert np.max(np.abs(res.out[1, 0, 0, i] - np.array(num) / den)) < 1e-12


def pin_sparse_gamma_on_residual():
    """Under gamma the similarity is that of the residual part: scipy's cosine
    of torch's attention over the left-out rows for two consecutive queries."""
    rng, kp, vp, steps = _sparse_setup(34, m_list=[[0] * 2, [3] * 2, [3] * 2])
    sel = np.array([[[1], [0, 2]], [[2], [1]]], dtype=object)
    sel = [[np.array(x) for x in row] for row in sel]
    sel_arr = np.empty((2, 2), dtype=object)
    for i in range(2):
        for j in range(2):
            sel_arr[i, j] = sel[i][j]
    res = fb.run_block_sparse(kp, vp, kp.shape[2], steps, sel_arr, fb.GAMMA, gamma=0.99)
    for bi in range(2):
        for h in range(4):
            g = h // 2
            kept = {r for t in sel_arr[bi, g] for r in range(64 * t, min(64 * t + 64, kp.shape[2]))}
            left = [r for r in range(kp.shape[2]) if r not in kept]
            a1 = _sdpa_rows(steps[0].q[bi, h], kp[bi, g, left], vp[bi, g, left])
            a2 = _sdpa_rows(steps[1].q[bi, h], kp[bi, g, left], vp[bi, g, left])
            ref = 1.0 - scipy.spatial.distance.cosine(a2.ravel(), a1.ravel())
            assert abs(res.sim[1, bi, h] - ref) < 1e-12


# ---------------------------------------------------------------- internal_merge

def pin_internal_merge_fresh_is_full_attention():
    """Block-internal attention merged with a freshly computed external part
    is attention over the prefix and the block together (the identity the A_full
    equation implies), for every query head with its grouped key/value head:
    torch's float64 SDPA with its own GQA mapping over the concatenated keys."""
    rng = _rng(40)
    for (b, hq, hkv, bs, n, d) in [(2, 8, 2, 5, 37, 16), (1, 6, 3, 1, 1, 8), (1, 4, 4, 9, 64, 32)]:
        q = rng.standard_normal((b, hq, bs, d)) * 1.5
        kp, vp = rng.standard_normal((b, hkv, n + 3, d)) * 1.5, rng.standard_normal((b, hkv, n + 3, d))
        kb, vb = rng.standard_normal((b, hkv, bs, d)) * 1.5, rng.standard_normal((b, hkv, bs, d))
        a_out, l_out = fb.external(q, kp, vp, n)
        out = fb.internal_merge(q, kb, vb, a_out, l_out)
        kc = torch.from_numpy(np.concatenate([kp[:, :, :n], kb], axis=2)).contiguous()
        vc = torch.from_numpy(np.concatenate([vp[:, :, :n], vb], axis=2)).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), kc, vc, enable_gqa=True).numpy()
        assert np.max(np.abs(out - ref)) <= TOL


def pin_internal_merge_stale_bruteforce():
    """With a stale external part (computed for other queries), the output
    weighs the prefix keys by those queries' scores and the block keys by the
    current ones: scalar brute force per (sequence, query head), key/value head
    h // G, on tiny inputs."""
    rng = _rng(41)
    b, hq, hkv, bs, n, d = 2, 4, 2, 3, 6, 4
    q_old = rng.standard_normal((b, hq, bs, d))
    q = rng.standard_normal((b, hq, bs, d))
    kp, vp = rng.standard_normal((b, hkv, n, d)), rng.standard_normal((b, hkv, n, d))
    kb, vb = rng.standard_normal((b, hkv, bs, d)), rng.standard_normal((b, hkv, bs, d))
    a_old, l_old = fb.external(q_old, kp, vp, n)
    out = fb.internal_merge(q, kb, vb, a_old, l_old)
    c = 1.0 / math.sqrt(d)
    for bi in range(b):
        for h in range(hq):
            g = h // (hq // hkv)
            for i in range(bs):
                terms = [(q_old[bi, h, i], kp[bi, g, j], vp[bi, g, j]) for j in range(n)]
                terms += [(q[bi, h, i], kb[bi, g, j], vb[bi, g, j]) for j in range(bs)]
                num, den = [0.0] * d, 0.0
                for qi, kj, vj in terms:
                    w = math.exp(c * sum(float(qi[t]) * float(kj[t]) for t in range(d)))
                    den += w
                    num = [num[t] + w * float(vj[t]) for t in range(d)]
                assert np.max(np.abs(out[bi, h, i] - np.array(num) / den)) < 1e-12


def pin_internal_merge_empty_external():
    """An empty external part (no prefix: A = 0, L = -inf) leaves the block's
    own attention: torch SDPA over the block keys alone."""
    rng = _rng(42)
    b, hq, hkv, bs, d = 1, 6, 2, 7, 16
    q = rng.standard_normal((b, hq, bs, d))
    kb, vb = rng.standard_normal((b, hkv, bs, d)), rng.standard_normal((b, hkv, bs, d))
    out = fb.internal_merge(q, kb, vb, np.zeros((b, hq, bs, d)), np.full((b, hq, bs), -np.inf))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(kb), torch.from_numpy(vb), enable_gqa=True).numpy()
    assert np.max(np.abs(out - ref)) <= TOL


PINS = [pin_attend_bruteforce, pin_attend_vs_torch, pin_external_gqa_vs_torch, pin_attend_closed_forms,
        pin_attend_permutation_invariance, pin_merge_equals_full_attention, pin_merge_special_cases,
        pin_split_associativity, pin_cosine, pin_tau_policy, pin_gamma_policy, pin_multi_block_append,
        pin_tau_cum_policy, pin_gamma_group_policy, pin_sparse_always_is_exact, pin_sparse_all_kept_is_exact,
        pin_sparse_none_kept_is_flashblock, pin_sparse_stale_residual_bruteforce, pin_sparse_gamma_on_residual,
        pin_internal_merge_fresh_is_full_attention, pin_internal_merge_stale_bruteforce,
        pin_internal_merge_empty_external]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ---------------------------------------------------------------- planted mistakes

_real_attend, _real_merge, _real_cosine, _real_decide = fb.attend, fb.merge, fb.cosine, fb.decide


def _attend_no_max_shift(q, k, v, scale):
    s = scale * (q @ k.T)
    with np.errstate(over="ignore", invalid="ignore"):
        p = np.exp(s)
        z = p.sum(1)
        return (p @ v) / z[:, None], np.log(z)


def _attend_log2(q, k, v, scale):
    a, lse = _real_attend(q, k, v, scale)
    return a, lse / math.log(2.0)


def _attend_no_scale(q, k, v, scale):
    return _real_attend(q, k, v, 1.0)


def _attend_kv_swapped(q, k, v, scale):
    return _real_attend(q, v, k, scale)


def _attend_unnormalised(q, k, v, scale):
    a, lse = _real_attend(q, k, v, scale)
    return a * np.exp(lse)[:, None] if k.shape[0] else a, lse


def _merge_sign(a_out, l_out, a_in, l_in):
    m = np.maximum(l_out, l_in)
    w_o, w_i = np.exp(m - l_out), np.exp(m - l_in)
    return (w_o[:, None] * a_out + w_i[:, None] * a_in) / (w_o + w_i)[:, None], m + np.log(w_o + w_i)


def _merge_no_denominator(a_out, l_out, a_in, l_in):
    m = np.maximum(l_out, l_in)
    w_o, w_i = np.exp(l_out - m), np.exp(l_in - m)
    return w_o[:, None] * a_out + w_i[:, None] * a_in, m + np.log(w_o + w_i)


def _merge_drop_in(a_out, l_out, a_in, l_in):
    return _real_merge(a_out, l_out, np.zeros_like(a_in), l_in)


def _decide_le(policy, st, n_updated, tau, gamma):
    if policy == fb.TAU and st.valid:
        return n_updated <= tau
    return _real_decide(policy, st, n_updated, tau, gamma)


def _decide_ge(policy, st, n_updated, tau, gamma):
    if policy == fb.GAMMA and st.valid:
        return st.sim is not None and st.sim >= gamma
    return _real_decide(policy, st, n_updated, tau, gamma)


def _decide_ignore_valid(policy, st, n_updated, tau, gamma):
    if policy == fb.TAU:
        return n_updated < tau
    return _real_decide(policy, st, n_updated, tau, gamma)


def _decide_cum_le(policy, st, n_updated, tau, gamma):
    if policy == fb.TAU_CUM and st.valid:
        return st.cum + n_updated <= tau
    return _real_decide(policy, st, n_updated, tau, gamma)


def _decide_cum_per_step(policy, st, n_updated, tau, gamma):
    if policy == fb.TAU_CUM and st.valid:
        return n_updated < tau   # forgets the sum since the last computation
    return _real_decide(policy, st, n_updated, tau, gamma)


def _cosine_mean_of_rows(a, o):
    # averages the similarity of the stacked parts instead of one cosine over all of them
    a, o = np.atleast_2d(np.asarray(a, dtype=np.float64).reshape(len(a), -1)), np.atleast_2d(np.asarray(o).reshape(len(o), -1))
    return float(np.mean([_real_cosine(x, y) for x, y in zip(a, o)]))


def _cosine_unclamped_l1(a, o):
    a, o = np.ravel(a), np.ravel(o)
    na, no = np.abs(a).sum(), np.abs(o).sum()
    return float(np.dot(a, o) / (na * no)) if na and no else 1.0


def _cosine_no_abs(a, o):
    return abs(_real_cosine(a, o))


def _external_mod_group(q, k_prefix, v_prefix, n_prefix, scale=None):
    bsz, hq, bs, d = q.shape
    hkv = k_prefix.shape[1]
    a, lse = np.empty((bsz, hq, bs, d)), np.empty((bsz, hq, bs))
    for b in range(bsz):
        for h in range(hq):
            a[b, h], lse[b, h] = _real_attend(q[b, h], k_prefix[b, h % hkv, :n_prefix],
                                              v_prefix[b, h % hkv, :n_prefix], fb.default_scale(d))
    return a, lse


def _sparse_sets_shifted(tiles, n_prefix):
    kept = np.array([r for t in sorted(set(int(t) for t in tiles)) for r in range(64 * t + 1, 64 * t + 65)
                     if r < n_prefix], dtype=np.int64)
    return kept, np.setdiff1d(np.arange(n_prefix), kept)


def _sparse_sets_no_residual(tiles, n_prefix):
    return fb.tile_rows(tiles, n_prefix), np.zeros(0, np.int64)


def _sparse_sets_whole_prefix_left(tiles, n_prefix):
    return fb.tile_rows(tiles, n_prefix), np.arange(n_prefix)


def _internal_merge_mod_group(q, k_blk, v_blk, a_out, l_out, scale=None):
    # query head h reads block key/value head h % Hkv instead of h // G
    bsz, hq, bs, d = q.shape
    hkv = k_blk.shape[1]
    out = np.empty((bsz, hq, bs, d))
    for b in range(bsz):
        for h in range(hq):
            a_in, l_in = _real_attend(q[b, h], k_blk[b, h % hkv], v_blk[b, h % hkv], fb.default_scale(d))
            out[b, h], _ = _real_merge(a_out[b, h], l_out[b, h], a_in, l_in)
    return out


def _internal_merge_swapped_l(q, k_blk, v_blk, a_out, l_out, scale=None):
    # each part weighted with the other part's normaliser
    bsz, hq, bs, d = q.shape
    group = hq // k_blk.shape[1]
    out = np.empty((bsz, hq, bs, d))
    for b in range(bsz):
        for h in range(hq):
            a_in, l_in = _real_attend(q[b, h], k_blk[b, h // group], v_blk[b, h // group], fb.default_scale(d))
            out[b, h], _ = _real_merge(a_out[b, h], l_in, a_in, l_out[b, h])
    return out


MUTANTS = [
    ("attend", _attend_no_max_shift), ("attend", _attend_log2), ("attend", _attend_no_scale),
    ("attend", _attend_kv_swapped), ("attend", _attend_unnormalised),
    ("merge", _merge_sign), ("merge", _merge_no_denominator), ("merge", _merge_drop_in),
    ("decide", _decide_le), ("decide", _decide_ge), ("decide", _decide_ignore_valid),
    ("cosine", _cosine_unclamped_l1), ("cosine", _cosine_no_abs), ("cosine", _cosine_mean_of_rows),
    ("decide", _decide_cum_le), ("decide", _decide_cum_per_step),
    ("external", _external_mod_group),
    ("sparse_key_sets", _sparse_sets_shifted), ("sparse_key_sets", _sparse_sets_no_residual),
    ("sparse_key_sets", _sparse_sets_whole_prefix_left),
    ("internal_merge", _internal_merge_mod_group), ("internal_merge", _internal_merge_swapped_l),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_planted_mistakes(monkeypatch, name, mutant):
    """Every plausible mistake planted in the oracle makes at least one pin fail."""
    monkeypatch.setattr(fb, name, mutant)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, FloatingPointError, ValueError, IndexError, TypeError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {mutant.__name__}"


def test_sparse_residual_recovers_dropped_keys():
    """The pages' claim for sparse attention, on synthetic dLLM-shaped data:
    caching the left-out keys' part (refreshed under the threshold policy)
    brings the output far closer to exact attention than dropping those keys.
    Sparse-only = attention over the kept tiles and the block alone."""
    from cached_attention_fb_amd import workload as wl
    w = wl.workload("dllm-8k").with_(n_q_heads=4, n_kv_heads=1, head_dim=32, steps=6)
    inp = wl.generate(w, prefix=1024)
    steps = [fb.StepData(wl.to_f64(st.q), wl.to_f64(st.k), wl.to_f64(st.v), np.asarray(st.n_updated))
             for st in inp.blocks[0].steps]
    kp, vp = wl.to_f64(inp.k_prefix), wl.to_f64(inp.v_prefix)
    sel = wl.sparse_selection(w, 1024, 0.2)
    exact = fb.run_block_sparse(kp, vp, 1024, steps, sel, fb.ALWAYS)
    reuse = fb.run_block_sparse(kp, vp, 1024, steps, sel, fb.TAU, tau=w.tau)
    assert reuse.reuse.sum() > 0
    kept, _ = fb.sparse_key_sets(sel[0, 0], 1024)
    scale = fb.default_scale(w.head_dim)
    err_sparse = err_reuse = 0.0
    for s, st in enumerate(steps):
        for h in range(4):
            a, l = fb.attend(st.q[0, h], kp[0, 0, kept], vp[0, 0, kept], scale)
            a_in, l_in = fb.attend(st.q[0, h], st.k[0, 0], st.v[0, 0], scale)
            only, _ = fb.merge(a, l, a_in, l_in)
            err_sparse = max(err_sparse, np.max(np.abs(only - exact.out[s, 0, h])))
            err_reuse = max(err_reuse, np.max(np.abs(reuse.out[s, 0, h] - exact.out[s, 0, h])))
    assert err_reuse < 0.25 * err_sparse, (err_reuse, err_sparse)
