"""Compile the HIP sources into dynamic_rope_context_amd/libbifocal.so (gfx950).

Usage: python -m dynamic_rope_context_amd.build  (or build() from Python)
Every HIP source is compiled with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libbifocal.so")
SOURCES = ["api.cpp", "tables.hip", "rope.hip", "decode.hip", "decode_mfma.hip",
           "prefill_f32.hip", "prefill_mfma.hip", "prefill_ie.hip", "noalloc.hip"]
ARCH = os.environ.get("BIFOCAL_ARCH", "gfx950")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wno-unused-result"]
# Per-source additions.  The prefill kernel's softmax maxima are fmaxf chains over
# MFMA results; without NaN semantics the compiler drops the canonicalizing moves it
# puts before each of them (about 5 VALU instructions per 32-key tile and wave).  The
# compiler may then assume that no value is a NaN: the prefill's result for inputs that
# hold NaN or infinity is unspecified (finite inputs, the documented domain, are
# unaffected).
EXTRA_FLAGS = {"prefill_mfma.hip": ["-fno-honor-nans"]}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False, jobs: int = 6) -> str:
    hipcc = _hipcc()
    objdir = os.path.join(ROOT, "_build", ARCH)
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"]
        cmd = [hipcc, *FLAGS, *EXTRA_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
