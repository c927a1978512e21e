"""Plain float64 CPU oracle for FlashBlock's block-diffusion attention step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
HIP library and its Python binding never do, and nothing here imports them.

Source: the page "Résumé Technique : FlashBlock" (gist.science, paper
2602.05305) §2 "Mécanisme Central" and "Stratégies de Réutilisation
Adaptatives", and the English abstract on the paper's fugumt.com page.

What is computed, step by step, for every (sequence b, query head h):

* ``attend`` — softmax attention of the block's query rows over one key set,
  and the natural-log normaliser L = log Z (§2 "Mécanisme Central": A_in over
  the block's own tokens J_in, A_out over the tokens outside the block J_out,
  cached together with L_out = log Z_out).
* ``merge`` — the log-space composition of the two parts (§2, the A_full
  equation with m = max(L_out, L_in)).
* ``cosine`` — per-head similarity of two A_out tensors (§2 "Sélection par
  tête"; the measure itself is not named on the page, cosine is the reading
  taken here).
* ``run_block_sparse`` — the same policy over a sparse attention (§2
  "Compatibilité avec l'attention parcimonieuse"): the prefix keys a
  selection leaves out form the cached external set, the kept ones are
  attended afresh at every step.
* ``decide`` / ``run_block`` — the reuse policy (§2 "Réutilisation basée sur
  un seuil": reuse when M^{s+1} < tau, else recompute; "Sélection par tête":
  only heads whose similarity exceeds gamma reuse) driving one block of
  denoising steps.

Readings taken where the page is silent (all listed in the design notes):
scale 1/sqrt(D); L in natural log; A_out and A_in each normalised over its
own key set; J_out = whole committed prefix, J_in = whole block, no mask;
M counts tokens changed since the previous step, compared strictly; the cache
holds the most recent *computed* A_out/L_out; the first step of a block always
computes, and under gamma the second one too; similarity = cosine of the head's
A_out flattened over (block rows x head_dim), compared strictly.

Pins (tests/test_oracle.py): ``attend`` against a scalar brute force, torch's
float64 scaled_dot_product_attention (with its GQA head mapping) and
logsumexp, and closed forms (single key, constant V, equal keys, a worked
two-key case); ``merge`` against full attention over the concatenated keys
(the exact identity the equation implies), the empty-prefix case and split
associativity; ``internal_merge`` against torch's SDPA over the prefix and
the block together (fresh external part), a scalar brute force with a stale
external part, and the empty-prefix case; ``cosine`` against scipy and its
special values; ``decide`` /
``run_block`` through the policy closed forms (tau=0, M=0, tau>Bs, gamma>=1,
gamma=-1, sigma=0).  Parity unpinned: the composition of a whole policy run
beyond those special cases has no printed values to compare with.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

ALWAYS = "always"
TAU = "tau"
GAMMA = "gamma"
# Variants at the edges of the two rules (the same passages; not the pages'
# own choices): M summed since the head's last computation, and one similarity
# per group of query heads that share a key/value head.
TAU_CUM = "tau_cum"
GAMMA_GROUP = "gamma_group"


def default_scale(head_dim: int) -> float:
    """Softmax scale 1/sqrt(D): the page gives none; this is the usual
    scaled-dot-product choice of the FlashAttention family it refers to."""
    return 1.0 / np.sqrt(head_dim)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of rows ``q`` [R, D] over keys ``k`` [N, D] with values
    ``v`` [N, D]; returns (A [R, D], L [R]) with L = log Z in natural log.

    §2 "Mécanisme Central": each part of the output is attention over its own
    token set, and its log-normaliser L = log Z is kept beside it.  The row max
    is subtracted before exponentiating and added back into L, which leaves
    both results unchanged mathematically.  An empty key set gives A = 0 and
    L = -inf (no mass), the neutral element of ``merge``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = q.shape[0]
    if k.shape[0] == 0:
        return np.zeros((rows, v.shape[1])), np.full(rows, -np.inf)
    s = scale * (q @ k.T)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    z = p.sum(axis=1)
    a = (p @ v) / z[:, None]
    lse = m[:, 0] + np.log(z)
    return a, lse


def merge(a_out: np.ndarray, l_out: np.ndarray, a_in: np.ndarray, l_in: np.ndarray
          ) -> Tuple[np.ndarray, np.ndarray]:
    """Log-space composition of two attention parts (§2, A_full equation):
    m = max(L_out, L_in); A_full = (e^{L_out-m} A_out + e^{L_in-m} A_in) /
    (e^{L_out-m} + e^{L_in-m}).  Also returns the merged normaliser
    m + log(e^{L_out-m} + e^{L_in-m}) so that merges can be chained.
    Rows where both parts are empty stay empty (A = 0, L = -inf)."""
    l_out = np.asarray(l_out, dtype=np.float64)
    l_in = np.asarray(l_in, dtype=np.float64)
    m = np.maximum(l_out, l_in)
    both_empty = np.isneginf(m)
    m_safe = np.where(both_empty, 0.0, m)
    w_out = np.exp(l_out - m_safe)
    w_in = np.exp(l_in - m_safe)
    den = w_out + w_in
    den_safe = np.where(both_empty, 1.0, den)
    a = (w_out[:, None] * a_out + w_in[:, None] * a_in) / den_safe[:, None]
    lse = np.where(both_empty, -np.inf, m_safe + np.log(den_safe))
    return a, lse


def cosine(a: np.ndarray, o: np.ndarray) -> float:
    """Cosine similarity of two tensors flattened to vectors: <a,o>/(|a||o|).
    §2 "Sélection par tête" estimates a per-head similarity without naming
    it; cosine is the reading taken.  Zero norms: 1 when both are zero (the
    tensors are equal), else 0.  The value is clamped to [-1, 1], the range of
    the exact quantity, so that rounding cannot carry it past gamma = 1."""
    a = np.asarray(a, dtype=np.float64).ravel()
    o = np.asarray(o, dtype=np.float64).ravel()
    na = np.sqrt(np.dot(a, a))
    no = np.sqrt(np.dot(o, o))
    if na == 0.0 or no == 0.0:
        return 1.0 if (na == 0.0 and no == 0.0) else 0.0
    return float(min(1.0, max(-1.0, np.dot(a, o) / (na * no))))


@dataclass
class HeadState:
    """Cache of one (sequence, query head) inside a block: the most recently
    computed A_out/L_out (§2: cached from the previous diffusion step), whether
    it holds anything yet, and the last similarity measured for the head."""

    valid: bool = False
    sim: Optional[float] = None
    a_out: Optional[np.ndarray] = None
    l_out: Optional[np.ndarray] = None
    cum: int = 0   # tau_cum: updated tokens summed since the last computation


def decide(policy: str, st: HeadState, n_updated: int, tau: int, gamma: float) -> bool:
    """Reuse decision for one head at one step.

    * always: never reuse (plain block diffusion, recompute every step);
    * tau (§2 "Réutilisation basée sur un seuil"): reuse when the cache holds
      something and the number of updated tokens M is strictly below tau;
    * gamma (§2 "Sélection par tête"): reuse when the cache holds something and
      the head's last measured similarity strictly exceeds gamma;
    * tau_cum (variant of tau): the updated tokens are summed over the steps
      since the cache was computed, this step's included, and compared
      strictly with tau;
    * gamma_group (variant of gamma): the similarity is that of the head's
      group (see run_block).
    """
    if policy == ALWAYS or not st.valid:
        return False
    if policy == TAU:
        return n_updated < tau
    if policy == TAU_CUM:
        return st.cum + n_updated < tau
    if policy in (GAMMA, GAMMA_GROUP):
        return st.sim is not None and st.sim > gamma
    raise ValueError(f"unknown policy {policy!r}")


@dataclass
class StepData:
    q: np.ndarray        # [B, Hq, Bs, D] float64
    k: np.ndarray        # [B, Hkv, Bs, D]
    v: np.ndarray        # [B, Hkv, Bs, D]
    n_updated: np.ndarray  # [B] int


@dataclass
class BlockResult:
    out: np.ndarray      # [S, B, Hq, Bs, D]  merged attention output per step
    a_out: np.ndarray    # [S, B, Hq, Bs, D]  cached A_out after the step
    l_out: np.ndarray    # [S, B, Hq, Bs]     cached L_out after the step
    reuse: np.ndarray    # [S, B, Hq] int8: 1 reused, 0 computed, -1 head not evaluated
    sim: np.ndarray      # [S, B, Hq] similarity held after the step (NaN: none)


def run_block(k_prefix: np.ndarray, v_prefix: np.ndarray, n_prefix: int,
              steps: Sequence[StepData], policy: str, tau: int = 0, gamma: float = 0.0,
              scale: Optional[float] = None,
              heads: Optional[Iterable[Tuple[int, int]]] = None) -> BlockResult:
    """One block of denoising steps for every (b, h) in ``heads`` (all by default).

    Per step s and head: decide reuse; if not reused, compute A_out/L_out over
    the prefix J_out (rows 0..n_prefix-1), measure the similarity with the
    previous cached A_out when the gamma policy holds one, and refresh the
    cache; always compute A_in/L_in over the block J_in; output = merge of the
    cached external part with the fresh internal part (§2 "Mécanisme
    Central").  Query head h reads key/value head h // (Hq/Hkv).  Heads are
    independent of one another, so any subset can be evaluated alone; under
    gamma_group the heads of a group decide together (one similarity, the
    cosine of the group's A_out tensors taken as one vector), so the group of
    every requested head is evaluated."""
    s0 = steps[0]
    n_steps = len(steps)
    bsz, hq, bs, d = s0.q.shape
    hkv = s0.k.shape[1]
    group = hq // hkv
    scale = default_scale(d) if scale is None else scale
    heads = [(b, h) for b in range(bsz) for h in range(hq)] if heads is None else list(heads)
    out = np.full((n_steps, bsz, hq, bs, d), np.nan)
    a_rec = np.full((n_steps, bsz, hq, bs, d), np.nan)
    l_rec = np.full((n_steps, bsz, hq, bs), np.nan)
    reuse = np.full((n_steps, bsz, hq), -1, dtype=np.int8)
    sim = np.full((n_steps, bsz, hq), np.nan)
    if policy == GAMMA_GROUP:
        units = [[(b, g * group + i) for i in range(group)] for b, g in sorted({(b, h // group) for b, h in heads})]
    else:
        units = [[bh] for bh in heads]
    for unit in units:
        b, g = unit[0][0], unit[0][1] // group
        kp = k_prefix[b, g, :n_prefix]
        vp = v_prefix[b, g, :n_prefix]
        sts = [HeadState() for _ in unit]   # heads of a unit decide together (one head unless gamma_group)
        for s, step in enumerate(steps):
            m = int(step.n_updated[b])
            r = decide(policy, sts[0], m, tau, gamma)
            if not r:
                news = [attend(step.q[b, h], kp, vp, scale) for _, h in unit]
                if policy in (GAMMA, GAMMA_GROUP) and sts[0].valid:
                    sim_u = cosine(np.stack([a for a, _ in news]), np.stack([st.a_out for st in sts]))
                    for st in sts:
                        st.sim = sim_u
                for st, (a_new, l_new) in zip(sts, news):
                    st.a_out, st.l_out, st.valid, st.cum = a_new, l_new, True, 0
            else:
                for st in sts:
                    st.cum += m
            for st, (_, h) in zip(sts, unit):
                a_in, l_in = attend(step.q[b, h], step.k[b, g], step.v[b, g], scale)
                out[s, b, h], _ = merge(st.a_out, st.l_out, a_in, l_in)
                a_rec[s, b, h] = st.a_out
                l_rec[s, b, h] = st.l_out
                reuse[s, b, h] = 1 if r else 0
                sim[s, b, h] = np.nan if st.sim is None else st.sim
    return BlockResult(out, a_rec, l_rec, reuse, sim)


SPARSE_TILE = 64   # prefix keys per selectable tile (the selection's granularity)


def tile_rows(tiles: Sequence[int], n_prefix: int, tile: int = SPARSE_TILE) -> np.ndarray:
    """Prefix rows of the listed key tiles (tile t holds rows tile*t ..
    tile*t + tile - 1, cut at n_prefix), ascending."""
    tiles = [int(t) for t in tiles]
    n_tiles = (n_prefix + tile - 1) // tile
    if len(set(tiles)) != len(tiles) or any(t < 0 or t >= n_tiles for t in tiles):
        raise ValueError("a selection lists distinct tiles of the prefix")
    rows = [np.arange(t * tile, min((t + 1) * tile, n_prefix)) for t in sorted(tiles)]
    return np.concatenate(rows).astype(np.int64) if rows else np.zeros(0, np.int64)


def sparse_key_sets(tiles: Sequence[int], n_prefix: int) -> Tuple[np.ndarray, np.ndarray]:
    """Prefix rows kept by a selection of tiles, and the rows it leaves out
    (the rest of 0..n_prefix-1); together they cover the prefix once."""
    kept = tile_rows(tiles, n_prefix)
    return kept, np.setdiff1d(np.arange(n_prefix), kept)


def run_block_sparse(k_prefix: np.ndarray, v_prefix: np.ndarray, n_prefix: int,
                     steps: Sequence[StepData], sel_tiles: np.ndarray, policy: str, tau: int = 0,
                     gamma: float = 0.0, scale: Optional[float] = None,
                     heads: Optional[Iterable[Tuple[int, int]]] = None) -> BlockResult:
    """FlashBlock over a sparse attention (§2 "Compatibilité avec l'attention
    parcimonieuse", §3 item 3): the prefix keys a sparse selection keeps are
    attended afresh at every step; the keys it leaves out play the role of the
    block-external set, whose part (A_res, L_res) is cached and reused under
    the policy exactly as A_out/L_out are in ``run_block``.

    ``sel_tiles`` [B, Hkv, n_sel]: the kept prefix tiles of each (sequence,
    key/value head), shared by the query heads that read that key/value head,
    and fixed for the block.  Per step and head: decide reuse of the residual;
    if not reused, A_res, L_res = attend over the left-out rows (similarity
    under gamma measured on A_res); A_sel, L_sel = attend over the kept rows;
    A_in, L_in = attend over the block; output = merge(merge(residual, kept),
    internal).  With no kept tile this is ``run_block``; with every tile kept
    the residual is empty and every step is exact attention.  Records: out,
    the cached residual (a_out, l_out), reuse, sim."""
    s0 = steps[0]
    n_steps = len(steps)
    bsz, hq, bs, d = s0.q.shape
    hkv = s0.k.shape[1]
    group = hq // hkv
    scale = default_scale(d) if scale is None else scale
    heads = [(b, h) for b in range(bsz) for h in range(hq)] if heads is None else list(heads)
    out = np.full((n_steps, bsz, hq, bs, d), np.nan)
    a_rec = np.full((n_steps, bsz, hq, bs, d), np.nan)
    l_rec = np.full((n_steps, bsz, hq, bs), np.nan)
    reuse = np.full((n_steps, bsz, hq), -1, dtype=np.int8)
    sim = np.full((n_steps, bsz, hq), np.nan)
    if policy == GAMMA_GROUP:
        units = [[(b, g * group + i) for i in range(group)] for b, g in sorted({(b, h // group) for b, h in heads})]
    else:
        units = [[bh] for bh in heads]
    for unit in units:
        b, g = unit[0][0], unit[0][1] // group
        kept, left = sparse_key_sets(sel_tiles[b, g], n_prefix)
        k_kept, v_kept = k_prefix[b, g, kept], v_prefix[b, g, kept]
        k_left, v_left = k_prefix[b, g, left], v_prefix[b, g, left]
        sts = [HeadState() for _ in unit]
        for s, step in enumerate(steps):
            m = int(step.n_updated[b])
            r = decide(policy, sts[0], m, tau, gamma)
            if not r:
                news = [attend(step.q[b, h], k_left, v_left, scale) for _, h in unit]
                if policy in (GAMMA, GAMMA_GROUP) and sts[0].valid:
                    sim_u = cosine(np.stack([a for a, _ in news]), np.stack([st.a_out for st in sts]))
                    for st in sts:
                        st.sim = sim_u
                for st, (a_new, l_new) in zip(sts, news):
                    st.a_out, st.l_out, st.valid, st.cum = a_new, l_new, True, 0
            else:
                for st in sts:
                    st.cum += m
            for st, (_, h) in zip(sts, unit):
                a_sel, l_sel = attend(step.q[b, h], k_kept, v_kept, scale)
                a_ext, l_ext = merge(st.a_out, st.l_out, a_sel, l_sel)
                a_in, l_in = attend(step.q[b, h], step.k[b, g], step.v[b, g], scale)
                out[s, b, h], _ = merge(a_ext, l_ext, a_in, l_in)
                a_rec[s, b, h] = st.a_out
                l_rec[s, b, h] = st.l_out
                reuse[s, b, h] = 1 if r else 0
                sim[s, b, h] = np.nan if st.sim is None else st.sim
    return BlockResult(out, a_rec, l_rec, reuse, sim)


def run_blocks(k_prefix: np.ndarray, v_prefix: np.ndarray, blocks: Sequence[Sequence[StepData]],
               policy: str, tau: int = 0, gamma: float = 0.0, scale: Optional[float] = None,
               heads=None) -> List[BlockResult]:
    """Several blocks in a row.  At the end of a block its final K/V join the
    prefix (block-causal generation with a KV cache, page §1 and the
    abstract), and every head's cache starts empty in the next block."""
    results = []
    kp, vp = k_prefix, v_prefix
    for steps in blocks:
        results.append(run_block(kp, vp, kp.shape[2], steps, policy, tau, gamma, scale, heads))
        kp = np.concatenate([kp, steps[-1].k], axis=2)
        vp = np.concatenate([vp, steps[-1].v], axis=2)
    return results


def external(q: np.ndarray, k_prefix: np.ndarray, v_prefix: np.ndarray, n_prefix: int,
             scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Fresh block-external part for every head: (A_out [B,Hq,Bs,D], L_out [B,Hq,Bs])."""
    bsz, hq, bs, d = q.shape
    group = hq // k_prefix.shape[1]
    scale = default_scale(d) if scale is None else scale
    a = np.empty((bsz, hq, bs, d))
    lse = np.empty((bsz, hq, bs))
    for b in range(bsz):
        for h in range(hq):
            a[b, h], lse[b, h] = attend(q[b, h], k_prefix[b, h // group, :n_prefix],
                                        v_prefix[b, h // group, :n_prefix], scale)
    return a, lse


def internal_merge(q: np.ndarray, k_blk: np.ndarray, v_blk: np.ndarray, a_out: np.ndarray,
                   l_out: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
    """Block-internal part for every head (§2 "Mécanisme Central": A_in over
    the block's own tokens J_in, key/value head h // G), merged with a given
    external part (A_out, L_out) by the A_full equation; the external part may
    be stale, i.e. computed at an earlier step for other queries."""
    bsz, hq, bs, d = q.shape
    group = hq // k_blk.shape[1]
    scale = default_scale(d) if scale is None else scale
    out = np.empty((bsz, hq, bs, d))
    for b in range(bsz):
        for h in range(hq):
            a_in, l_in = attend(q[b, h], k_blk[b, h // group], v_blk[b, h // group], scale)
            out[b, h], _ = merge(a_out[b, h], l_out[b, h], a_in, l_in)
    return out
