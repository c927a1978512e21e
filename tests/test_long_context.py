"""Multi-block parity at long context: a 262144-token starting prefix, three
blocks in a row, each appending its final K/V to the prefix (and resetting
the cache) before the next (page "Résumé Technique : FlashBlock", §4: the
latency gap at 100k-800k tokens; §1: block-causal generation with a KV
cache).  The GPU runs every head; the float64 oracle evaluates one query
head of each kv group (heads are independent), whose decisions must be
bit-exact and outputs, A_out and L_out within tolerance at every step."""
import numpy as np
import pytest

import harness as H
import oracle
from cached_attention_fb_amd import workload as wl

pytestmark = pytest.mark.gpu


def test_three_blocks_at_256k_prefix():
    prefix = 262144
    w = wl.workload("dllm-8k").with_(n_q_heads=8, n_kv_heads=2, blocks=3, steps=4)
    inp = wl.generate(w, prefix=prefix)
    print(f"[long] dLLM layer, 8/2 heads, prefix {prefix}, 3 blocks x 4 steps", flush=True)
    gpu = H.run_gpu(inp)
    heads = [(0, 1), (0, 6)]   # one query head of each kv group
    blocks = [H.oracle_steps(b) for b in inp.blocks]
    ref = oracle.run_blocks(wl.to_f64(inp.k_prefix), wl.to_f64(inp.v_prefix), blocks, w.policy,
                            tau=w.tau, gamma=w.gamma, heads=heads)
    pairs = [(bh, bh) for bh in heads]
    for i, (g, r) in enumerate(zip(gpu, ref)):
        errs = H.compare_block(g, r, w.dtype, pairs=pairs, what=f"256k block {i}")
        print(f"[long] block {i} prefix {prefix + i * w.block} errs {errs} reuse {g.reuse[:, 0, 1].tolist()}",
              flush=True)
    assert len(gpu) == 3
    # every head of a sequence follows the same threshold decision
    for g in gpu:
        assert np.all(g.reuse == g.reuse[:, :, :1])
