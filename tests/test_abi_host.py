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
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # declarations only, not the comments
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
                dtype=fb.FB_BF16, softmax_scale=0.0)
    base.update(kw)
    return fb.FBConfig(**base)


# The boundary's two structs exactly as the hot-path contract lays them out:
# eight 4-byte fields, and three 4-byte fields then a host pointer.  Declared
# here independently of the binding, so that a layout drift on either side
# shows up.
class ContractConfig(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32), ("max_prefix", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


class ContractPolicyArgs(ctypes.Structure):
    _fields_ = [("policy", ctypes.c_int32), ("tau", ctypes.c_int32), ("gamma", ctypes.c_float),
                ("n_updated", ctypes.POINTER(ctypes.c_int32))]


def test_contract_struct_layouts():
    """fb_config and fb_policy_args keep the contract's layout (no field added):
    the binding's structs match field by field, and the header declares
    exactly these fields."""
    assert ctypes.sizeof(ContractConfig) == 32
    assert ctypes.sizeof(ContractPolicyArgs) == 24
    for mine, theirs in ((fb.FBConfig, ContractConfig), (fb.FBPolicyArgs, ContractPolicyArgs)):
        assert ctypes.sizeof(mine) == ctypes.sizeof(theirs)
        assert [(n, t, getattr(mine, n).offset) for n, t in mine._fields_] == \
               [(n, t, getattr(theirs, n).offset) for n, t in theirs._fields_]
    text = open(os.path.join(ROOT, "include", "fb.h")).read()
    for name, fields in (("fb_config", [f for f, _ in ContractConfig._fields_]),
                         ("fb_policy_args", [f for f, _ in ContractPolicyArgs._fields_])):
        body = re.search(r"typedef struct \{([^}]*)\} " + name + ";", text).group(1)
        body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
        declared = re.findall(r"(\w+)\s*;", body)
        assert declared == fields, (name, declared)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=9), fb.FB_E_DTYPE), (dict(head_dim=80), fb.FB_E_UNSUPPORTED), (dict(batch=-3), fb.FB_E_SHAPE),
    (dict(n_q_heads=5, n_kv_heads=2), fb.FB_E_SHAPE), (dict(softmax_scale=float("inf")), fb.FB_E_ARG),
])
def test_contract_config_is_read_field_by_field(kw, code):
    """A contract-layout fb_config passed through the C ABI: each field's bad
    value is reported with its own code, so every field is read where the
    contract puts it."""
    lib = fb.load()
    base = dict(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=128, block_size=32, max_prefix=64,
                dtype=fb.FB_BF16, softmax_scale=0.0)
    base.update(kw)
    c = ContractConfig(**base)
    h = ctypes.c_void_p()
    assert lib.fb_cache_alloc(ctypes.cast(ctypes.byref(c), ctypes.POINTER(fb.FBConfig)), ctypes.byref(h)) == code
    assert h.value is None


@pytest.mark.parametrize("opts,code", [
    (dict(struct_size=0, kv_splits=0), fb.FB_E_ARG),
    (dict(struct_size=8, kv_splits=-1), fb.FB_E_ARG),
    (dict(struct_size=8, kv_splits=65), fb.FB_E_ARG),
])
def test_cache_opts_checks(opts, code):
    lib = fb.load()
    h = ctypes.c_void_p()
    c = cfg()
    o = fb.FBCacheOpts(**opts)
    assert lib.fb_cache_alloc_ex(ctypes.byref(c), ctypes.byref(o), ctypes.byref(h)) == code
    assert h.value is None
    assert lib.fb_last_error() != b""


def test_cache_opts_shorter_struct_takes_defaults():
    """struct_size 4 (a caller whose struct ends before kv_splits): the out-of-range
    kv_splits behind it is not read, so only the missing device is reported."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    lib = fb.load()
    h = ctypes.c_void_p()
    c = cfg()
    o = fb.FBCacheOpts(struct_size=4, kv_splits=999)
    assert lib.fb_cache_alloc_ex(ctypes.byref(c), ctypes.byref(o), ctypes.byref(h)) == fb.FB_E_HIP


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
    assert lib.fb_step_ex(None, ctypes.byref(pa), None, None, None, None, None, None, 0, None, None) == fb.FB_E_ARG
    assert lib.fb_step_sparse(None, ctypes.byref(pa), None, None, None, None, None, None, 0, None, 0, None,
                              None) == fb.FB_E_ARG
    assert lib.fb_cache_alloc_ex(None, None, None) == fb.FB_E_ARG
    assert lib.fb_step_noalloc(None, None, None, None, None, None, 0, None, None, None, None) == fb.FB_E_ARG
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
