"""Build libfb.so (gfx950) in-tree with hipcc.

    python -m cached_attention_fb_amd.build
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfb.so")
SOURCES = ["fb_attn_bf16.hip", "fb_attn_f32.hip", "fb_aux.hip", "fb_runtime.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


COMPILE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17",
    # keep fp32 arithmetic off the packed-fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the softmax works on them without AGPR copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc_command(out=LIB, extra=()):
    return [HIPCC, *COMPILE_FLAGS, "-fPIC", "-shared",
            *[os.path.join(CSRC, s) for s in SOURCES], *extra, "-o", out]


def device_asm_command(source, out):
    """The gfx950 assembly of one source file, built with the library's flags."""
    return [HIPCC, *COMPILE_FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, source), "-o", out]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
