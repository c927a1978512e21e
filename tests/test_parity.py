"""Kernel-level parity of the HIP library with the float64 oracle.

fb_external_attn (A_out, L_out read back from the cache) and
fb_internal_attn_merge, on seeded inputs whose sizes span several 128-row and
64-key tiles with ragged tails, GQA groups, both head sizes and dtypes, empty
and one-key prefixes, forced split counts, and head masks.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from cached_attention_fb_amd import fb
from harness import l_check, tolerance_check

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def draw(rng, shape, dtype, std):
    x = rng.standard_normal(shape) * std
    t = torch.from_numpy(x).to(DT[dtype])
    return t, t.to(torch.float64).numpy()


class Case:
    def __init__(self, dtype, d, hq, hkv, bs, n, std=1.0, b=1, splits=0, max_prefix=None, seed=0):
        self.dtype, self.d, self.hq, self.hkv, self.bs, self.n, self.std, self.b = dtype, d, hq, hkv, bs, n, std, b
        self.splits = splits
        self.max_prefix = n + 7 if max_prefix is None else max_prefix
        self.seed = seed
        self.built = False

    def build(self):
        """Draw the inputs (at test time, not at collection)."""
        if self.built:
            return self
        b, hq, hkv, bs, d, dtype, std = self.b, self.hq, self.hkv, self.bs, self.d, self.dtype, self.std
        rng = np.random.default_rng(self.seed + 17 * self.n + bs)
        self.q, self.q64 = draw(rng, (b, hq, bs, d), dtype, std)
        self.kp, self.kp64 = draw(rng, (b, hkv, self.max_prefix, d), dtype, std)
        self.vp, self.vp64 = draw(rng, (b, hkv, self.max_prefix, d), dtype, 1.0)
        self.kb, self.kb64 = draw(rng, (b, hkv, bs, d), dtype, std)
        self.vb, self.vb64 = draw(rng, (b, hkv, bs, d), dtype, 1.0)
        self.built = True
        return self

    def __repr__(self):
        return f"{self.dtype}-D{self.d}-h{self.hq}/{self.hkv}-b{self.b}-Bs{self.bs}-N{self.n}-s{self.splits}-std{self.std:.3g}"

    def cache(self):
        return fb.Cache(self.b, self.hq, self.hkv, self.d, self.bs, self.max_prefix, DT[self.dtype],
                        kv_splits=self.splits)

    def dev(self):
        self.build()
        return [t.cuda() for t in (self.q, self.kp, self.vp, self.kb, self.vb)]


S128 = 1 / math.sqrt(128)
CASES = [
    Case("f32", 64, 4, 4, 32, 512),
    Case("f32", 64, 4, 4, 32, 544),
    Case("f32", 128, 8, 2, 5, 65),
    Case("f32", 64, 4, 4, 32, 0),
    Case("f32", 64, 2, 1, 70, 1, b=2),
    Case("bf16", 128, 32, 8, 32, 8192, std=S128),
    Case("bf16", 128, 32, 8, 32, 8192, std=1.0),
    Case("bf16", 128, 8, 2, 100, 1000),
    Case("bf16", 64, 4, 1, 33, 63),
    Case("bf16", 128, 4, 4, 1, 1),
    Case("bf16", 128, 4, 1, 64, 64),
    Case("bf16", 128, 4, 1, 64, 65),
    Case("bf16", 128, 2, 2, 200, 3000, b=3),
    Case("bf16", 128, 4, 2, 32, 0),
    Case("bf16", 128, 32, 8, 32, 8192, std=S128, splits=1),
    Case("bf16", 128, 32, 8, 32, 4000, std=1.0, splits=7),
    Case("f32", 64, 4, 4, 32, 512, splits=3),
    Case("bf16", 128, 12, 12, 300, 2000, splits=2),
    Case("bf16", 64, 8, 2, 32, 1000),        # D=64, 128 packed rows, short items: one wave per SIMD
    Case("bf16", 64, 8, 2, 32, 1000, splits=2),   # D=64, 128 packed rows, 8-tile items: the 4x2 shape
    Case("bf16", 128, 8, 2, 32, 300),        # 128 rows, short items with a ragged last tile
    Case("bf16", 64, 4, 4, 16, 700),         # D=64 in the one-wave shape
    Case("bf16", 64, 4, 1, 200, 900),        # D=64, 8-row-wave shape, 4 row tiles
    Case("bf16", 128, 16, 2, 40, 2000),      # GQA 8, 2 row tiles
    # the two forms of the K/V/Q DMA addressing: whole tiles and a full
    # 32-row Q block (uniform base + lane offsets) vs ragged ones (clamped)
    Case("bf16", 128, 4, 1, 8, 4096, splits=4),   # 32 packed rows, every tile whole
    Case("bf16", 128, 1, 1, 31, 4095, splits=3),  # 31 rows, ragged last tile
    Case("bf16", 64, 4, 1, 8, 2048, splits=4),    # D=64, 32 rows, every tile whole
]


@pytest.mark.parametrize("case", CASES, ids=repr)
def test_external_attn(case):
    case.build()
    c = case.cache()
    q, kp, vp, kb, vb = case.dev()
    c.external_attn(q, kp, vp, case.n)
    a = c.read(fb.FIELD_A_OUT)
    lse = c.read(fb.FIELD_L_OUT)
    a_ref, l_ref = oracle.external(case.q64, case.kp64, case.vp64, case.n)
    tolerance_check(a, a_ref, case.dtype, f"{case} A_out")
    l_check(lse, l_ref, case.dtype, f"{case} L_out")
    assert np.all(c.read(fb.FIELD_VALID) == 1)


@pytest.mark.parametrize("case", CASES, ids=repr)
def test_internal_merge(case):
    case.build()
    c = case.cache()
    q, kp, vp, kb, vb = case.dev()
    out = torch.empty_like(q)
    c.external_attn(q, kp, vp, case.n)
    c.internal_attn_merge(q, kb, vb, out)
    a_ref, l_ref = oracle.external(case.q64, case.kp64, case.vp64, case.n)
    ref = oracle.internal_merge(case.q64, case.kb64, case.vb64, a_ref, l_ref)
    got = out.to(torch.float64).cpu().numpy()
    tolerance_check(got, ref, case.dtype, f"{case} out")
    # closed form: fresh external merged with internal = attention over prefix + block
    g = case.hq // case.hkv
    full = np.empty_like(ref)
    for b in range(case.b):
        for h in range(case.hq):
            kk = np.concatenate([case.kp64[b, h // g, :case.n], case.kb64[b, h // g]])
            vv = np.concatenate([case.vp64[b, h // g, :case.n], case.vb64[b, h // g]])
            full[b, h] = oracle.attend(case.q64[b, h], kk, vv, 1 / math.sqrt(case.d))[0]
    tolerance_check(got, full, case.dtype, f"{case} out vs full attention")


def test_merge_without_cached_part_is_internal_attention():
    case = Case("bf16", 128, 8, 2, 40, 300)
    case.build()
    c = case.cache()
    q, kp, vp, kb, vb = case.dev()
    out = torch.empty_like(q)
    c.internal_attn_merge(q, kb, vb, out)        # right after allocation: nothing cached
    ref = np.empty((1, 8, 40, 128))
    for h in range(8):
        ref[0, h] = oracle.attend(case.q64[0, h], case.kb64[0, h // 4], case.vb64[0, h // 4], 1 / math.sqrt(128))[0]
    tolerance_check(out.to(torch.float64).cpu().numpy(), ref, "bf16", "no cached part")


def test_head_mask_updates_only_selected_heads():
    case = Case("f32", 64, 4, 2, 16, 200, b=2)
    case.build()
    c = case.cache()
    q, kp, vp, kb, vb = case.dev()
    c.external_attn(q, kp, vp, 100)                     # every head over 100 keys
    a100 = c.read(fb.FIELD_A_OUT)
    mask = torch.tensor([[1, 0, 0, 1], [0, 1, 0, 0]], dtype=torch.uint8, device="cuda")
    c.external_attn(q, kp, vp, 200, head_mask=mask)     # selected heads over 200 keys
    a = c.read(fb.FIELD_A_OUT)
    a200, _ = oracle.external(case.q64, case.kp64, case.vp64, 200)
    for b in range(2):
        for h in range(4):
            ref = a200[b, h] if mask[b, h] else a100[b, h]
            tolerance_check(a[b, h], ref, "f32", f"head ({b},{h})")


def test_bad_arguments_enqueue_nothing():
    case = Case("bf16", 128, 4, 2, 16, 100)
    case.build()
    c = case.cache()
    q, kp, vp, kb, vb = case.dev()
    code = c.lib.fb_external_attn(c.h, q.data_ptr(), kp.data_ptr(), vp.data_ptr(), case.max_prefix + 1, None, None)
    assert code == fb.FB_E_SHAPE and b"prefix_len" in c.lib.fb_last_error()
    assert np.all(c.read(fb.FIELD_VALID) == 0)
