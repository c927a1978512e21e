"""Python binding of libfb.so (include/fb.h): argument marshalling only.

Every step of the attention path runs in the library's HIP kernels; this
module checks tensor dtypes, shapes, devices and contiguity, then passes raw
device pointers and the current HIP stream through ctypes.  It raises
``ImportError`` when the library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfb.so")

FB_OK, FB_E_ARG, FB_E_SHAPE, FB_E_DTYPE, FB_E_STATE, FB_E_NOMEM, FB_E_HIP, FB_E_UNSUPPORTED = range(8)
FB_F32, FB_BF16 = 0, 1
POLICY_ALWAYS, POLICY_TAU, POLICY_GAMMA, POLICY_TAU_CUM, POLICY_GAMMA_GROUP = 0, 1, 2, 3, 4
FIELD_A_OUT, FIELD_L_OUT, FIELD_SIM, FIELD_REUSE, FIELD_VALID, FIELD_WAIT_ERR = range(6)
PROFILE_KINDS = 8
KIND_NAMES = ["external", "combine", "internal_merge", "decide", "reset", "sparse_kept", "sparse_total",
              "sparse_complement"]

STATUS_NAMES = {0: "FB_OK", 1: "FB_E_ARG", 2: "FB_E_SHAPE", 3: "FB_E_DTYPE", 4: "FB_E_STATE",
                5: "FB_E_NOMEM", 6: "FB_E_HIP", 7: "FB_E_UNSUPPORTED"}

EXPORTED = ["fb_cache_alloc", "fb_cache_alloc_ex", "fb_cache_free", "fb_cache_reset", "fb_external_attn",
            "fb_internal_attn_merge", "fb_step", "fb_step_ex", "fb_step_sparse", "fb_cache_read",
            "fb_cache_info", "fb_profile_enable", "fb_profile_read", "fb_step_noalloc", "fb_last_error"]


class FBConfig(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32), ("max_prefix", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


class FBCacheOpts(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("kv_splits", ctypes.c_int32)]


class FBPolicyArgs(ctypes.Structure):
    _fields_ = [("policy", ctypes.c_int32), ("tau", ctypes.c_int32), ("gamma", ctypes.c_float),
                ("n_updated", ctypes.POINTER(ctypes.c_int32))]


class FBStepOpts(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("n_updated_dev", ctypes.c_void_p)]


def step_opts(n_updated_dev: Optional[int]) -> FBStepOpts:
    return FBStepOpts(ctypes.sizeof(FBStepOpts), n_updated_dev)


class FBProfileStats(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64 * PROFILE_KINDS), ("ms", ctypes.c_double * PROFILE_KINDS)]


class FBError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    """Load libfb.so (once).  Raises ImportError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m cached_attention_fb_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32
    lib.fb_cache_alloc.argtypes = [ctypes.POINTER(FBConfig), ctypes.POINTER(vp)]
    lib.fb_cache_alloc_ex.argtypes = [ctypes.POINTER(FBConfig), ctypes.POINTER(FBCacheOpts), ctypes.POINTER(vp)]
    lib.fb_cache_free.argtypes = [vp]
    lib.fb_cache_reset.argtypes = [vp, vp]
    lib.fb_external_attn.argtypes = [vp, vp, vp, vp, i32, vp, vp]
    lib.fb_internal_attn_merge.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.fb_step.argtypes = [vp, ctypes.POINTER(FBPolicyArgs), vp, vp, vp, vp, vp, i32, vp, vp]
    lib.fb_step_ex.argtypes = [vp, ctypes.POINTER(FBPolicyArgs), ctypes.POINTER(FBStepOpts), vp, vp, vp, vp, vp, i32,
                               vp, vp]
    lib.fb_step_sparse.argtypes = [vp, ctypes.POINTER(FBPolicyArgs), ctypes.POINTER(FBStepOpts), vp, vp, vp, vp, vp,
                                   i32, vp, i32, vp, vp]
    lib.fb_cache_read.argtypes = [vp, i32, vp, ctypes.c_size_t, vp]
    lib.fb_cache_info.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(i32)]
    lib.fb_profile_enable.argtypes = [vp, i32]
    lib.fb_profile_read.argtypes = [vp, ctypes.POINTER(FBProfileStats)]
    lib.fb_step_noalloc.argtypes = [ctypes.POINTER(FBConfig), vp, vp, vp, vp, vp, i32, vp, vp, vp, vp]
    for name in EXPORTED[:-1]:
        getattr(lib, name).restype = st
    lib.fb_last_error.argtypes = []
    lib.fb_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(code: int) -> None:
    if code != FB_OK:
        raise FBError(code, load().fb_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


class Cache:
    """One FlashBlock cache (fb_cache) and the entry points that use it."""

    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, block_size: int,
                 max_prefix: int, dtype: torch.dtype, softmax_scale: float = 0.0, kv_splits: int = 0):
        self.lib = load()
        self.dtype = dtype
        self.cfg = FBConfig(batch, n_q_heads, n_kv_heads, head_dim, block_size, max_prefix,
                            FB_F32 if dtype == torch.float32 else FB_BF16 if dtype == torch.bfloat16 else -1,
                            softmax_scale)
        h = ctypes.c_void_p()
        if kv_splits:
            opts = FBCacheOpts(ctypes.sizeof(FBCacheOpts), kv_splits)
            _check(self.lib.fb_cache_alloc_ex(ctypes.byref(self.cfg), ctypes.byref(opts), ctypes.byref(h)))
        else:
            _check(self.lib.fb_cache_alloc(ctypes.byref(self.cfg), ctypes.byref(h)))
        self.h = h

    # -- shape checks (marshalling only) --------------------------------
    def _t(self, t: torch.Tensor, shape: Sequence[int], name: str) -> int:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if t.dtype != self.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, the cache uses {self.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return t.data_ptr()

    def _q(self, q, name="q_blk"):
        c = self.cfg
        return self._t(q, (c.batch, c.n_q_heads, c.block_size, c.head_dim), name)

    def _kv_blk(self, t, name):
        c = self.cfg
        return self._t(t, (c.batch, c.n_kv_heads, c.block_size, c.head_dim), name)

    def _kv_pre(self, t, name):
        c = self.cfg
        return self._t(t, (c.batch, c.n_kv_heads, c.max_prefix, c.head_dim), name)

    # -- entry points ----------------------------------------------------
    def reset(self, stream=None) -> None:
        _check(self.lib.fb_cache_reset(self.h, _stream(stream)))

    def external_attn(self, q, k_prefix, v_prefix, prefix_len: int, head_mask=None, stream=None) -> None:
        mask = None
        if head_mask is not None:
            if head_mask.dtype != torch.uint8 or not head_mask.is_cuda or head_mask.numel() != self.cfg.batch * self.cfg.n_q_heads:
                raise ValueError("head_mask must be a device uint8 tensor of B*Hq elements")
            mask = head_mask.contiguous().data_ptr()
        _check(self.lib.fb_external_attn(self.h, self._q(q), self._kv_pre(k_prefix, "k_prefix"),
                                         self._kv_pre(v_prefix, "v_prefix"), int(prefix_len), mask,
                                         _stream(stream)))

    def internal_attn_merge(self, q, k_blk, v_blk, out, stream=None) -> None:
        _check(self.lib.fb_internal_attn_merge(self.h, self._q(q), self._kv_blk(k_blk, "k_blk"),
                                               self._kv_blk(v_blk, "v_blk"), self._q(out, "out"),
                                               _stream(stream)))

    def step(self, policy: int, q, k_blk, v_blk, k_prefix, v_prefix, prefix_len: int, out,
             tau: int = 0, gamma: float = 0.0, n_updated=None, n_updated_dev=None, stream=None,
             sel_tiles=None) -> None:
        """One denoising step.  Threshold counts come either from the host
        (`n_updated`, B ints) or from device memory (`n_updated_dev`, an int32
        tensor of B entries on the cache's device), in which case the
        decisions are made on the device.  `sel_tiles` (int32 device tensor
        [B, Hkv, n_sel]): a sparse attention's kept prefix tiles
        (fb_step_sparse)."""
        args = FBPolicyArgs(policy, tau, gamma, None)
        opts = None
        keep = None
        if n_updated_dev is not None:
            if (not isinstance(n_updated_dev, torch.Tensor) or n_updated_dev.dtype != torch.int32
                    or not n_updated_dev.is_cuda or n_updated_dev.numel() != self.cfg.batch
                    or not n_updated_dev.is_contiguous()):
                raise ValueError(f"n_updated_dev must be a contiguous int32 device tensor of {self.cfg.batch} entries")
            opts = step_opts(n_updated_dev.data_ptr())
        if n_updated is not None:
            keep = np.ascontiguousarray(np.asarray(n_updated, dtype=np.int32).reshape(-1))
            if keep.size != self.cfg.batch:
                raise ValueError(f"n_updated needs {self.cfg.batch} entries")
            args.n_updated = keep.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        if sel_tiles is not None:
            sel_ptr, n_sel = self._sel(sel_tiles)
            _check(self.lib.fb_step_sparse(self.h, ctypes.byref(args), None if opts is None else ctypes.byref(opts),
                                           self._q(q), self._kv_blk(k_blk, "k_blk"),
                                           self._kv_blk(v_blk, "v_blk"), self._kv_pre(k_prefix, "k_prefix"),
                                           self._kv_pre(v_prefix, "v_prefix"), int(prefix_len), sel_ptr, n_sel,
                                           self._q(out, "out"), _stream(stream)))
            return
        ptrs = (self._q(q), self._kv_blk(k_blk, "k_blk"), self._kv_blk(v_blk, "v_blk"),
                self._kv_pre(k_prefix, "k_prefix"), self._kv_pre(v_prefix, "v_prefix"), int(prefix_len),
                self._q(out, "out"), _stream(stream))
        if opts is not None:
            _check(self.lib.fb_step_ex(self.h, ctypes.byref(args), ctypes.byref(opts), *ptrs))
        else:
            _check(self.lib.fb_step(self.h, ctypes.byref(args), *ptrs))

    def _sel(self, t: torch.Tensor):
        c = self.cfg
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or not t.is_cuda or t.dim() != 3
                or tuple(t.shape[:2]) != (c.batch, c.n_kv_heads) or not t.is_contiguous()):
            raise ValueError(f"sel_tiles must be a contiguous int32 device tensor [{c.batch}, {c.n_kv_heads}, n_sel]")
        return (t.data_ptr() if t.numel() else None), int(t.shape[2])

    def prepare(self, q, k_blk, v_blk, k_prefix, v_prefix, out, sel_tiles=None) -> "PreparedStep":
        """Check a set of step buffers once; the returned object calls fb_step
        (fb_step_sparse with sel_tiles) on them with only scalar marshalling
        (for loops over many steps)."""
        sel = self._sel(sel_tiles) if sel_tiles is not None else None
        return PreparedStep(self, self._q(q), self._kv_blk(k_blk, "k_blk"), self._kv_blk(v_blk, "v_blk"),
                            self._kv_pre(k_prefix, "k_prefix"), self._kv_pre(v_prefix, "v_prefix"),
                            self._q(out, "out"), (q, k_blk, v_blk, k_prefix, v_prefix, out, sel_tiles), sel)

    def read(self, field: int, stream=None) -> np.ndarray:
        c = self.cfg
        nh = (c.batch, c.n_q_heads)
        shape, dt = {FIELD_A_OUT: (nh + (c.block_size, c.head_dim), np.float32),
                     FIELD_L_OUT: (nh + (c.block_size,), np.float32),
                     FIELD_SIM: (nh, np.float32), FIELD_REUSE: (nh, np.uint8),
                     FIELD_VALID: (nh, np.uint8), FIELD_WAIT_ERR: ((1,), np.uint32)}[field]
        buf = np.empty(shape, dtype=dt)
        _check(self.lib.fb_cache_read(self.h, field, buf.ctypes.data, buf.nbytes, _stream(stream)))
        return buf

    def info(self):
        nb, ns = ctypes.c_size_t(), ctypes.c_int32()
        _check(self.lib.fb_cache_info(self.h, ctypes.byref(nb), ctypes.byref(ns)))
        return {"device_bytes": nb.value, "kv_splits": ns.value}

    def profile_enable(self, on: bool = True) -> None:
        _check(self.lib.fb_profile_enable(self.h, 1 if on else 0))

    def profile_read(self):
        st = FBProfileStats()
        _check(self.lib.fb_profile_read(self.h, ctypes.byref(st)))
        return {KIND_NAMES[k]: (st.launches[k], st.ms[k]) for k in range(len(KIND_NAMES))}

    def close(self) -> None:
        if getattr(self, "h", None):
            self.lib.fb_cache_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


NOALLOC_SCRATCH_BYTES = 64 << 20


def step_noalloc(q, k_blk, v_blk, k_prefix, v_prefix, prefix_len: int, a_out, l_out, out,
                 softmax_scale: float = 0.0, stream=None) -> None:
    """fb_step_noalloc: one always-recompute step with no cache and no
    allocation.  Shapes: q, out [B, Hq, Bs, D]; k_blk, v_blk [B, Hkv, Bs, D];
    k_prefix, v_prefix [B, Hkv, max_prefix, D] (working dtype); a_out float32
    [B, Hq, Bs, D]; l_out float32 [B, Hq, Bs]; all contiguous device tensors."""
    lib = load()
    b, hq, bs, d = q.shape
    hkv, max_prefix = k_prefix.shape[1], k_prefix.shape[2]
    dt = FB_F32 if q.dtype == torch.float32 else FB_BF16 if q.dtype == torch.bfloat16 else -1
    cfg = FBConfig(b, hq, hkv, d, bs, max_prefix, dt, softmax_scale)
    for t, shape, name in ((q, (b, hq, bs, d), "q"), (out, (b, hq, bs, d), "out"), (k_blk, (b, hkv, bs, d), "k_blk"),
                           (v_blk, (b, hkv, bs, d), "v_blk"), (v_prefix, tuple(k_prefix.shape), "v_prefix"),
                           (a_out, (b, hq, bs, d), "a_out"), (l_out, (b, hq, bs), "l_out")):
        if tuple(t.shape) != shape or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor of shape {shape}")
    if a_out.dtype != torch.float32 or l_out.dtype != torch.float32:
        raise TypeError("a_out and l_out are float32")
    for t, name in ((k_blk, "k_blk"), (v_blk, "v_blk"), (k_prefix, "k_prefix"), (v_prefix, "v_prefix"), (out, "out")):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, q has {q.dtype}")
    _check(lib.fb_step_noalloc(ctypes.byref(cfg), q.data_ptr(), k_blk.data_ptr(), v_blk.data_ptr(),
                               k_prefix.data_ptr(), v_prefix.data_ptr(), int(prefix_len), a_out.data_ptr(),
                               l_out.data_ptr(), out.data_ptr(), _stream(stream)))


class PreparedStep:
    """fb_step on buffers checked once by Cache.prepare (they are kept alive
    here).  n_updated is copied into a preallocated int32 array per call."""

    def __init__(self, cache: Cache, q, kb, vb, kp, vp, out, keep, sel=None):
        self.cache, self.keep = cache, keep
        self.sel = sel
        self.ptrs = (q, kb, vb, kp, vp)
        self.out = out
        self.m = (ctypes.c_int32 * cache.cfg.batch)()
        self.m_ptr = ctypes.cast(self.m, ctypes.POINTER(ctypes.c_int32))
        self.args = FBPolicyArgs(0, 0, 0.0, self.m_ptr)
        self.args_ref = ctypes.byref(self.args)
        self.opts = step_opts(None)
        self.opts_ref = ctypes.byref(self.opts)
        self.fn = cache.lib.fb_step

    def __call__(self, policy: int, prefix_len: int, n_updated=None, tau: int = 0, gamma: float = 0.0,
                 stream=None, n_updated_dev: Optional[int] = None) -> None:
        """n_updated_dev: device address of B int32 counts (decisions on the
        device); n_updated is then ignored."""
        a = self.args
        a.policy, a.tau, a.gamma = policy, tau, gamma
        opts = None
        if n_updated_dev is not None:
            a.n_updated = None
            self.opts.n_updated_dev = n_updated_dev
            opts = self.opts_ref
        else:
            a.n_updated = self.m_ptr
            if n_updated is not None:
                for i, v in enumerate(n_updated):
                    self.m[i] = int(v)
        q, kb, vb, kp, vp = self.ptrs
        st = _stream(stream) if stream is None or not isinstance(stream, int) else stream
        if self.sel is not None:
            code = self.cache.lib.fb_step_sparse(self.cache.h, self.args_ref, opts, q, kb, vb, kp, vp, prefix_len,
                                                 self.sel[0], self.sel[1], self.out, st)
        elif opts is not None:
            code = self.cache.lib.fb_step_ex(self.cache.h, self.args_ref, opts, q, kb, vb, kp, vp, prefix_len,
                                             self.out, st)
        else:
            code = self.fn(self.cache.h, self.args_ref, q, kb, vb, kp, vp, prefix_len, self.out, st)
        if code != FB_OK:
            _check(code)
