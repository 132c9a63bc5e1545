"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds a copy of ``libkvx`` whose host side is instrumented (``-Xarch_host``
sanitizer flags; device code as usual) and the C program
``tests/sanitize/host_checks.c``, then runs it.  The program only makes calls
that are pure host logic or that the argument checks refuse before any HIP
runtime call, with host arrays of exactly the documented lengths, so an
out-of-bounds host read, a use after free or a signed overflow in the size
arithmetic ends the run with a sanitizer report.  CPU only: no kernel runs.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "cross_model_kv_kvx_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
CHECKS = os.path.join(ROOT, "tests", "sanitize", "host_checks.c")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"

# Each sanitizer flag applies to the host compilation only.
HOST_SAN = []
for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer"):
    HOST_SAN += ["-Xarch_host", flag]


def runtime_dir():
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return os.path.dirname(hits[0]) if hits else None


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.timeout(600)
def test_host_checks_under_asan_and_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG) and runtime_dir()):
        pytest.skip("ROCm clang with the sanitizer runtimes is needed")
    if not os.path.exists(CHECKS):
        pytest.skip("the host checks are not part of this tree")
    out = str(tmp_path)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src):
        obj = os.path.join(out, os.path.basename(src) + ".o")
        run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", *HOST_SAN, "-c", src, "-o", obj])
        return obj

    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "8"))))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = os.path.join(out, "libkvx_san.so")
    run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN, "-Xarch_host", "-shared-libsan", *objs,
         "-o", lib])
    exe = os.path.join(out, "host_checks")
    run([CLANG, "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-shared-libsan", f"-I{INCLUDE}", CHECKS, f"-L{out}", "-lkvx_san", f"-Wl,-rpath,{out}", "-o", exe])
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = runtime_dir() + (":" + env["LD_LIBRARY_PATH"] if env.get("LD_LIBRARY_PATH") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    # no device is opened: every call returns before the HIP runtime is used
    env["HIP_VISIBLE_DEVICES"] = ""
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"sanitized host checks failed (status {r.returncode}):\n{r.stdout}\n{r.stderr}"
    assert "host checks passed" in r.stdout
    shutil.rmtree(out, ignore_errors=True)
