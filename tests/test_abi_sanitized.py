"""The C-ABI checks of test_abi.py, run against a build of the library whose host code carries
AddressSanitizer and UndefinedBehaviorSanitizer instrumentation (device code unchanged). No
GPU is needed: every call in those checks returns from host-side validation before any launch.
The sanitizers watch the argument validation, the error-message formatting and the workspace
arithmetic of the entry points."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "structured_sparse_nvfp4_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "host_sanitized")
LIB = os.path.join(OUT, "libssnvfp4_hostsan.so")
HIPCC = "/opt/rocm/bin/hipcc"
# each sanitizer applies to the host compilation only
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer".split()


def _runtime():
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


def _build():
    os.makedirs(OUT, exist_ok=True)
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]
    procs, objs = [], []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(OUT, os.path.basename(src).replace(".hip", ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *common, *HOST_SAN, "-c", src, "-o", obj], stdout=subprocess.PIPE,
                                      stderr=subprocess.PIPE, text=True))
    for p in procs:
        _, err = p.communicate()
        assert p.returncode == 0, err[-4000:]
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan", *HOST_SAN, *objs,
                        "-o", LIB], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]


@pytest.mark.skipif(not os.path.exists(HIPCC) or _runtime() is None, reason="hipcc or the ASan runtime is missing")
def test_abi_checks_under_host_sanitizers():
    _build()
    nm = subprocess.run(["nm", "-D", "--undefined-only", LIB], capture_output=True, text=True).stdout
    assert "__asan_init" in nm and "__ubsan_handle" in nm, "the build is not instrumented"
    env = dict(os.environ, LD_PRELOAD=_runtime(), ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import sys, pytest\n"
            "import structured_sparse_nvfp4_amd as s\n"
            f"s.LIB_PATH = {LIB!r}\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', 'tests/test_abi.py']))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert " passed" in r.stdout and "skipped" not in r.stdout
