"""The C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

api.cpp and noalloc.hip are compiled with the sanitizers on their host side, and linked
with tests/sanitizer_stubs.cpp in place of the kernel launchers: each stand-in touches
every byte its kernel would reach through the arguments it receives.  The driver
(tests/sanitizer_driver.py) calls every entry point with buffers of exactly the sizes
the calls need, in a Python process that preloads the sanitizer runtime.  A workspace
layout or bookkeeping error that points past a buffer, or undefined behaviour in the
host code, fails the run."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dynamic_rope_context_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


def _asan_runtime():
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)) or _asan_runtime() is None:
        pytest.skip("hipcc / clang sanitizer runtime not available")
    out = tmp_path_factory.mktemp("asan")
    objs = []
    for src in (os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "noalloc.hip"),
                os.path.join(ROOT, "tests", "sanitizer_stubs.cpp")):
        obj = str(out / (os.path.basename(src) + ".o"))
        # each sanitizer flag applies to the host side only; noalloc.hip keeps its device
        # part (a device array the host code registers), the others compile host-only
        only = [] if src.endswith("noalloc.hip") else ["--cuda-host-only"]
        cmd = [HIPCC, "-x", "hip", *only, "--offload-arch=gfx950", "-O1", "-g", "-fPIC",
               "-std=c++17",
               "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=undefined", "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    lib = str(out / "libbifocal_host_sanitized.so")
    cmd = [CLANG, "-shared", "-fsanitize=address,undefined", "-shared-libasan", *objs,
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return lib


def test_abi_under_address_and_undefined_behaviour_sanitizers(sanitized_lib):
    env = dict(os.environ)
    env["LD_PRELOAD"] = _asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitizer_driver.py"),
                        sanitized_lib], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout[-2000:],
                                                                  r.stderr[-6000:])
