"""Properties of the kernels' gfx950 assembly (built here from the sources,
with the library's own flags), checked without a GPU.

- Every K/V/Q DMA load (global_load_lds_dwordx4, issued from inline asm, where
  the compiler's hazard checks do not reach) is directly preceded by the wait
  states it needs: one after the scalar write of M0 that sets its LDS
  address, five where its SGPR base may have been written by a vector
  instruction just before.  A missing wait reads a stale register: the load
  goes to a wrong address.
- The LDS address of every DMA load (M0) is written in the same basic block,
  by a scalar instruction, or by a vector one far enough back.
- No packed-fp32 vector instruction (v_pk_add/mul/fma_f32) appears: the
  build turns the feature off and no code writes them by hand.
- The attention kernels use no scratch memory (nothing spills).
"""
import os
import re
import shutil
import subprocess

import pytest

from cached_attention_fb_amd import build as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc is not installed")


def _asm(source, tmp_path):
    out = str(tmp_path / (source + ".s"))
    r = subprocess.run(B.device_asm_command(source, out), capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return [l.strip() for l in open(out).read().splitlines()]


ATTN_SOURCES = ["fb_attn_bf16.hip", "fb_attn_r64.hip"]


@pytest.fixture(scope="module", params=ATTN_SOURCES)
def attn_asm(request, tmp_path_factory):
    """The assembly of each bf16 attention kernel file."""
    return _asm(request.param, tmp_path_factory.mktemp("asm"))


def _instructions(lines):
    return [l for l in lines if l and not l.startswith((";", ".", "#")) and not l.endswith(":")]


def test_dma_loads_carry_their_wait_states(attn_asm):
    ins = _instructions(attn_asm)
    loads = [i for i, l in enumerate(ins) if l.startswith("global_load_lds_dwordx4")]
    assert len(loads) > 50   # the attention kernels issue their tiles this way
    for i in loads:
        uniform_base = re.search(r",\s*s\[\d+:\d+\]", ins[i]) is not None
        need = "s_nop 4" if uniform_base else "s_nop 0"
        assert ins[i - 1] == need, f"{ins[i]!r} preceded by {ins[i - 1]!r}, needs {need}"


def _wait_states_between(lines, j, i):
    """Wait states the instructions strictly between lines j and i provide:
    s_nop N gives N + 1, any other instruction one."""
    n = 0
    for t in lines[j + 1:i]:
        if not t or t.startswith((";", ".", "#")):
            continue
        m = re.match(r"s_nop\s+(\d+)", t)
        n += int(m.group(1)) + 1 if m else 1
    return n


def test_dma_lds_address_is_set_by_a_scalar_write(attn_asm):
    """M0 holds a DMA load's LDS address.  Its last writer before every load
    sits in the same basic block, and is a scalar instruction (which needs one
    wait state, supplied by the asm) or else a vector one at least five wait
    states back (v_readfirstlane into M0: the compiler does not see the asm's
    use of M0, so nothing else would space them)."""
    lines = attn_asm
    checked = 0
    for i, l in enumerate(lines):
        if not l.startswith("global_load_lds_dwordx4"):
            continue
        j = i - 1
        while j >= 0:
            t = lines[j]
            assert not (t.endswith(":") and not t.startswith(";")), \
                f"line {i}: M0 is set in another basic block than the DMA load"
            if re.match(r"^[a-z_0-9]+\s+m0\b", t):
                break
            j -= 1
        assert j >= 0, f"line {i}: no write of M0 before the DMA load"
        writer = lines[j].split()[0]
        need = 1 if writer.startswith("s_") else 5
        got = _wait_states_between(lines, j, i)
        assert got >= need, f"line {i}: {lines[j]!r} then {got} wait states before {l!r}, needs {need}"
        checked += 1
    assert checked > 50


def test_no_packed_fp32_instructions(attn_asm, tmp_path):
    for name, lines in (("attention", attn_asm), ("fb_aux.hip", _asm("fb_aux.hip", tmp_path)),
                        ("fb_attn_f32.hip", _asm("fb_attn_f32.hip", tmp_path))):
        bad = [l for l in _instructions(lines) if re.match(r"v_pk_(add|mul|fma)_f32\b", l)]
        assert not bad, f"{name}: {bad[:3]}"


def test_attention_kernels_do_not_spill(attn_asm):
    kernels = [l.split()[1] for l in attn_asm if l.startswith(".amdhsa_kernel ")]
    assert kernels
    text = "\n".join(attn_asm)
    sizes = re.findall(r"\.amdhsa_private_segment_fixed_size (\d+)", text)
    assert len(sizes) == len(kernels)
    assert all(int(s) == 0 for s in sizes), list(zip(kernels, sizes))
    assert not any(l.startswith("scratch_") for l in _instructions(attn_asm))


DIV_CHECK = r"""
#include <cstdio>
#include "fb_internal.h"
// n / d through div_magic's multiplier, as the work-item decode does it
static long long via(long long n, uint64_t m) { return (long long)(((uint64_t)(uint32_t)n * m) >> 32); }
int main() {
  long bad = 0;
  for (int d = 1; d <= 5000; ++d) {
    const long long n_max = ((1LL << 32) - 1) / d;   // every n below keeps n * d < 2^32
    const uint64_t m = fbk::div_magic(d, n_max);
    if (m == 0) { ++bad; continue; }
    for (long long n = 0; n < n_max && n < (1 << 16); ++n) bad += via(n, m) != n / d;
    for (long long n = n_max - 1; n >= 0 && n > n_max - 4096; --n) bad += via(n, m) != n / d;
  }
  bad += fbk::div_magic(3, 1LL << 31) != 0;   // a bound it cannot meet: ordinary division
  bad += fbk::div_magic(0, 10) != 0;
  std::printf("%ld\n", bad);
  return bad != 0;
}
"""


def test_decode_multiplier_is_exact(tmp_path):
    """The attention work-item decode replaces n / d by a multiply with
    div_magic(d) = ceil(2^32 / d): exact for every index n with n d < 2^32."""
    src, exe = tmp_path / "div_check.cpp", tmp_path / "div_check"
    src.write_text(DIV_CHECK)
    r = subprocess.run([B.HIPCC, "-O2", "-std=c++17", "-I", os.path.join(B.ROOT, "include"), "-I", B.CSRC,
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "0", r.stdout + r.stderr
