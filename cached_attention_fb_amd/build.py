"""Build libfb.so (gfx950) in-tree with hipcc.

Each source is compiled on its own (in parallel), then the objects are linked
into the shared library.

    python -m cached_attention_fb_amd.build
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfb.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMPILE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17",
    # keep fp32 arithmetic off the packed-fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
# MFMA results in VGPRs: the softmax works on them without AGPR copies (the
# kernels whose accumulators fit the 256 architectural VGPRs)
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]

# source -> its extra flags
SOURCES = {
    "fb_attn_bf16.hip": VGPR_FORM,
    "fb_attn_r64.hip": VGPR_FORM,
    "fb_attn_f32.hip": VGPR_FORM,
    "fb_aux.hip": VGPR_FORM,
    "fb_noalloc.hip": [],
    "fb_runtime.cpp": [],
}


def flags_for(source):
    return [*COMPILE_FLAGS, *SOURCES[source]]


def compile_command(source, out):
    return [HIPCC, *flags_for(source), "-fPIC", "-c", os.path.join(CSRC, source), "-o", out]


def link_command(objs, out):
    return [HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", out]


def device_asm_command(source, out):
    """The gfx950 assembly of one source file, built with the library's flags."""
    return [HIPCC, *flags_for(source), "--cuda-device-only", "-S", os.path.join(CSRC, source), "-o", out]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, errs


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for src in SOURCES:
        jobs.append((compile_command(src, os.path.join(OBJ, src + ".o")), src))
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda j: (j[1], j[0], _run(j[0])), jobs))
    for src, cmd, (rc, errs) in results:
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{errs}")
        if verbose and errs.strip():
            print(errs, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = link_command([os.path.join(OBJ, s + ".o") for s in SOURCES], tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    rc, errs = _run(cmd)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{errs}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
