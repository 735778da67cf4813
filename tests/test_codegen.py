"""Checks of the generated gfx950 code that the kernels' correctness relies on (host only: hipcc
cross-compiles the device code to assembly without a GPU).

The prefill tile copies K/V stages into LDS with global_load_lds_dwordx4, issued from inline
assembly that sets M0 (the LDS base of the copy) right before each copy.  M0 is a register the
compiler reserves: declaring it clobbered would not make the compiler preserve it, so the kernels
are only correct while the compiler itself uses M0 for nothing else.  This test compiles every
source that uses the copy and checks that each M0 access is one of the copies' own
`s_mov_b32 m0, sN; s_nop 0; global_load_lds_dwordx4` sequences.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_256_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")


def _device_asm(src: str, out: str) -> str:
    cmd = [HIPCC, "-S", "--offload-device-only", "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return open(out).read()


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
@pytest.mark.parametrize("src", ["pa_prefill.hip", "pa_mixed.hip"])
def test_m0_is_used_only_by_the_lds_copies(src, tmp_path):
    asm = _device_asm(src, str(tmp_path / (src + ".s")))
    lines = [l.strip() for l in asm.splitlines()]
    code = [l for l in lines if l and not l.startswith((";", ".")) and not l.endswith(":")]
    copies = 0
    for i, l in enumerate(code):
        if not re.search(r"\bm0\b", l):
            continue
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", l), f"{src}: M0 used outside a copy: {l!r}"
        assert code[i + 1] == "s_nop 0" and code[i + 2].startswith("global_load_lds_dwordx4"), \
            f"{src}: M0 set without the copy right after it: {code[i:i + 3]!r}"
        copies += 1
    assert copies > 0, f"{src}: no LDS copies found (the check would be vacuous)"
