"""The host runtime under AddressSanitizer and UndefinedBehaviorSanitizer.

fb_runtime.cpp is compiled for the host with both sanitizers (g++, no device
code: the kernel launchers are replaced by stand-ins that are never reached)
and linked with tests/native/abi_sanitize.cpp, which drives every entry point
through its argument, config and option checks on a machine without a GPU.
The program must report no failed check and no sanitizer finding (leak
detection on)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "native")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists("/opt/rocm/include/hip"),
                                reason="needs g++ and the HIP headers")


def test_runtime_checks_under_sanitizers(tmp_path):
    import torch
    if torch.cuda.is_available():
        pytest.skip("the program expects no device")
    exe = str(tmp_path / "abi_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "cached_attention_fb_amd", "csrc"),
           os.path.join(HERE, "abi_sanitize.cpp"), os.path.join(HERE, "launch_stubs.cpp"),
           os.path.join(ROOT, "cached_attention_fb_amd", "csrc", "fb_runtime.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "0 failures" in r.stdout
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out and "LeakSanitizer" not in out, out[-3000:]
