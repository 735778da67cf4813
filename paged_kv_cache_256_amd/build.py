"""Build libpa.so (the paged-attention HIP library for gfx950) in place.

Usage: python paged_kv_cache_256_amd/build.py [-v]
(run as a script: the package itself does not import until libpa.so exists)

Every HIP source is compiled with hipcc for gfx950 only; the objects go to _build/ at the
repository root and the shared library to paged_kv_cache_256_amd/libpa.so, next to the
Python binding that loads it.  Packed fp32 instructions are disabled for device code.

The prefill tile copies K/V stages into LDS with global_load_lds_dwordx4, issued from inline
assembly that sets M0 (the copy's LDS base) right before each copy.  The compiler reserves M0,
and declaring it clobbered would not make the compiler preserve it, so those kernels are correct
only while the compiler itself uses M0 for nothing else.  Every build therefore also compiles the
sources that issue the copies to gfx950 assembly and refuses to produce the library when an M0
access is not one of the copies' own `s_mov_b32 m0, sN; s_nop 0; global_load_lds_dwordx4`
sequences.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpa.so")
ARCH = "gfx950"

SOURCES = ["pa_api.cpp", "pa_block_manager.cpp", "pa_cache.hip", "pa_decode.hip", "pa_mixed.hip",
           "pa_prefill.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
M0_SOURCES = ("pa_prefill.hip", "pa_mixed.hip")  # the sources that issue LDS-DMA copies


def check_m0_use(asm: str, name: str) -> int:
    """Check gfx950 assembly: every M0 access must be `s_mov_b32 m0, sN` followed by `s_nop 0`
    and a `global_load_lds_dwordx4`.  Returns the number of copies; raises RuntimeError on any
    other M0 access, or when there is no copy at all (the check would then be vacuous)."""
    lines = [l.strip() for l in asm.splitlines()]
    code = [l for l in lines if l and not l.startswith((";", ".")) and not l.endswith(":")]
    copies = 0
    for i, l in enumerate(code):
        if not re.search(r"\bm0\b", l):
            continue
        if not re.fullmatch(r"s_mov_b32 m0, s\d+", l):
            raise RuntimeError(f"{name}: M0 used outside an LDS copy: {l!r}")
        nxt = code[i + 1:i + 3]
        if len(nxt) < 2 or nxt[0] != "s_nop 0" or not nxt[1].startswith("global_load_lds_dwordx4"):
            raise RuntimeError(f"{name}: M0 set without the LDS copy right after it: {code[i:i + 3]!r}")
        copies += 1
    if copies == 0:
        raise RuntimeError(f"{name}: no LDS copies found in the assembly")
    return copies


def device_asm_cmd(cc: str, src: str, out: str, dflags=()) -> list:
    return [cc, "-S", "--offload-device-only", *COMMON[:2], "-I", os.path.join(ROOT, "include"),
            "-I", CSRC, *dflags, *DEVICE, os.path.join(CSRC, src), "-o", out]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, jobs: int | None = None, defines=(), lib_path: str | None = None,
          obj_dir: str | None = None) -> str:
    """Compile and link libpa.so.  `defines` (NAME=VALUE strings) and `lib_path` / `obj_dir`
    build a variant of the library elsewhere (tuning experiments); the default build writes
    paged_kv_cache_256_amd/libpa.so."""
    cc = hipcc()
    out_dir = obj_dir or OUT_DIR
    lib = lib_path or LIB
    os.makedirs(out_dir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.rsplit(".", 1)[0] + ".o")
        objs.append(obj)
        path = os.path.join(CSRC, src)
        if src.endswith(".hip"):
            cmds.append([cc, *COMMON, *dflags, *DEVICE, "-c", path, "-o", obj])
        else:
            cmds.append([cc, *COMMON, *dflags, "-c", path, "-o", obj])
    asms = []
    for src in M0_SOURCES:
        asm = os.path.join(out_dir, src.rsplit(".", 1)[0] + ".gfx950.s")
        asms.append((src, asm))
        cmds.append(device_asm_cmd(cc, src, asm, dflags))
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    for src, asm in asms:
        with open(asm) as f:
            n = check_m0_use(f.read(), src)
        if verbose:
            print(f"{src}: M0 used by its {n} LDS copies only", flush=True)
    tmp = lib + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
          "-Wl,-rpath,/opt/rocm/lib"], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser()
    ap.add_argument("-v", action="store_true")
    ap.add_argument("-D", action="append", default=[], help="preprocessor define NAME=VALUE")
    ap.add_argument("--lib", default=None, help="output library path (default: in the package)")
    ap.add_argument("--objdir", default=None)
    a = ap.parse_args()
    print(build(verbose=a.v, defines=a.D, lib_path=a.lib, obj_dir=a.objdir))
