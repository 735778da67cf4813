"""Checks of the generated gfx950 code that the kernels' correctness relies on (host only: hipcc
cross-compiles the device code to assembly without a GPU).

The prefill tile copies K/V stages into LDS with global_load_lds_dwordx4, issued from inline
assembly that sets M0 (the LDS base of the copy) right before each copy.  M0 is a register the
compiler reserves: declaring it clobbered would not make the compiler preserve it, so the kernels
are only correct while the compiler itself uses M0 for nothing else.  The builder runs that check
on every build and refuses to link libpa.so when it fails; these tests run the builder's check on
freshly compiled assembly and show that it rejects the misuses it exists to catch.
"""

import importlib.util
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")


def _builder():
    spec = importlib.util.spec_from_file_location(
        "_pa_build_for_codegen", os.path.join(ROOT, "paged_kv_cache_256_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
@pytest.mark.parametrize("src", ["pa_prefill.hip", "pa_mixed.hip"])
def test_m0_is_used_only_by_the_lds_copies(src, tmp_path):
    b = _builder()
    out = str(tmp_path / (src + ".s"))
    r = subprocess.run(b.device_asm_cmd(HIPCC, src, out), capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert b.check_m0_use(open(out).read(), src) > 0


def test_m0_check_rejects_stray_uses():
    b = _builder()
    good = "s_mov_b32 m0, s12\ns_nop 0\nglobal_load_lds_dwordx4 v[2:3], off offset:16\n"
    assert b.check_m0_use(good + good, "ok") == 2
    for bad in ("s_mov_b32 m0, -1\nds_read_b32 v1, v2\n",                 # compiler's own M0 write
                "s_mov_b32 m0, s4\nv_add_u32 v1, v2, v3\nglobal_load_lds_dwordx4 v[2:3], off\n",
                good + "v_readfirstlane_b32 s3, v1\ns_mov_b32 s5, m0\n",  # M0 read elsewhere
                "v_add_u32 v1, v2, v3\n"):                               # no copy at all
        with pytest.raises(RuntimeError):
            b.check_m0_use(bad, "bad")
