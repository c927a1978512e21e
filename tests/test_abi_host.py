"""The C ABI on the CPU: every symbol include/fb.h declares is exported by
libfb.so, and argument/config checks return their FB_E_* codes before any
device work (no GPU is needed for any call here)."""
import ctypes
import os
import re

import pytest

from cached_attention_fb_amd import fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fb.h")).read()
    return sorted(set(re.findall(r"\b(fb_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["fb_cache_alloc", "fb_cache_free", "fb_cache_reset", "fb_external_attn",
              "fb_internal_attn_merge", "fb_step", "fb_cache_read", "fb_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = fb.load()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert sorted(fb.EXPORTED) == declared_functions()


def cfg(**kw):
    base = dict(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=128, block_size=32, max_prefix=1024,
                dtype=fb.FB_BF16, softmax_scale=0.0, kv_splits=0)
    base.update(kw)
    return fb.FBConfig(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), fb.FB_E_DTYPE),
    (dict(batch=0), fb.FB_E_SHAPE),
    (dict(batch=1025), fb.FB_E_SHAPE),
    (dict(n_q_heads=6, n_kv_heads=4), fb.FB_E_SHAPE),
    (dict(n_kv_heads=0), fb.FB_E_SHAPE),
    (dict(block_size=0), fb.FB_E_SHAPE),
    (dict(max_prefix=-1), fb.FB_E_SHAPE),
    (dict(head_dim=96), fb.FB_E_UNSUPPORTED),
    (dict(head_dim=256), fb.FB_E_UNSUPPORTED),
    (dict(kv_splits=-1), fb.FB_E_ARG),
    (dict(kv_splits=65), fb.FB_E_ARG),
    (dict(softmax_scale=float("nan")), fb.FB_E_ARG),
])
def test_config_checks(kw, code):
    lib = fb.load()
    h = ctypes.c_void_p()
    c = cfg(**kw)
    assert lib.fb_cache_alloc(ctypes.byref(c), ctypes.byref(h)) == code
    assert h.value is None
    assert lib.fb_last_error() != b""


def test_valid_config_without_device_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    lib = fb.load()
    h = ctypes.c_void_p()
    c = cfg()
    assert lib.fb_cache_alloc(ctypes.byref(c), ctypes.byref(h)) == fb.FB_E_HIP
    assert h.value is None


def test_null_arguments():
    lib = fb.load()
    assert lib.fb_cache_alloc(None, None) == fb.FB_E_ARG
    h = ctypes.c_void_p()
    assert lib.fb_cache_alloc(None, ctypes.byref(h)) == fb.FB_E_ARG
    assert lib.fb_cache_free(None) == fb.FB_OK
    assert lib.fb_last_error() == b""
    assert lib.fb_cache_reset(None, None) == fb.FB_E_ARG
    assert lib.fb_external_attn(None, None, None, None, 0, None, None) == fb.FB_E_ARG
    assert lib.fb_internal_attn_merge(None, None, None, None, None, None) == fb.FB_E_ARG
    pa = fb.FBPolicyArgs(fb.POLICY_ALWAYS, 0, 0.0, None)
    assert lib.fb_step(None, ctypes.byref(pa), None, None, None, None, None, 0, None, None) == fb.FB_E_ARG
    assert lib.fb_cache_read(None, 0, None, 0, None) == fb.FB_E_ARG
    assert lib.fb_cache_info(None, None, None) == fb.FB_E_ARG
    assert lib.fb_profile_enable(None, 1) == fb.FB_E_ARG
    assert lib.fb_profile_read(None, None) == fb.FB_E_ARG
    assert b"null" in lib.fb_last_error()


def test_binding_refuses_missing_library(tmp_path, monkeypatch):
    monkeypatch.setattr(fb, "_lib", None)
    monkeypatch.setattr(fb, "LIB_PATH", str(tmp_path / "libfb.so"))
    with pytest.raises(ImportError):
        fb.load()
