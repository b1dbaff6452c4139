"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of the library is compiled with both sanitizers on its host
pass (the device code is built as usual and never launched), and linked with
the C driver in tests/host_sanitize/abi_host_checks.c into one executable.  The driver calls
every entry point with arguments its checks must reject, the workspace-size
queries over a sweep of shapes (the tiling plan's integer arithmetic), the
flag rules of deferred chains, the overlap rules of the sketch-space update
and the kernel-choice setter; the sanitizers abort on the first finding.
"""
import concurrent.futures
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rank_gradient_sketching_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "abi_host_checks.c")
ROCM = "/opt/rocm"
SOURCES = ["abi.cpp", "regen.hip", "sketch.hip", "merge.hip", "kl.hip", "kl_sweep.hip",
           "optim.hip", "noalloc.hip", "calib.hip"]
# each sanitizer flag applies to the host pass only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _tools():
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    asan = glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                  "libclang_rt.asan-x86_64.a"))
    if not (os.path.exists(hipcc) and os.path.exists(clang) and asan):
        pytest.skip("hipcc, clang++ or the sanitizer runtimes are not installed")
    return hipcc, clang


def _run(cmd, cwd):
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout[-4000:]}\n{res.stderr[-4000:]}"
    return res


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    hipcc, clang = _tools()
    out = str(tmp_path)

    def compile_one(src):
        obj = os.path.join(out, os.path.splitext(src)[0] + ".o")
        _run([hipcc, "--offload-arch=gfx950", "-O2", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Xarch_host", "-g", f"-I{INCLUDE}", f"-I{CSRC}", *SAN, "-c", os.path.join(CSRC, src),
              "-o", obj], out)
        return obj

    with concurrent.futures.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    exe = os.path.join(out, "abi_host_checks")
    _run([clang, "-x", "c", "-std=c11", "-O1", "-g", "-D__HIP_PLATFORM_AMD__",
          f"-I{INCLUDE}", f"-I{ROCM}/include", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-c", DRIVER, "-o", exe + ".o"], out)
    _run([hipcc, "--offload-arch=gfx950", *SAN, exe + ".o", *objs,
          f"-L{ROCM}/lib", f"-Wl,-rpath,{ROCM}/lib", "-lamdhip64", "-o", exe], out)
    # the library's own objects carry the instrumentation, not only the driver
    # (UBSan checks appear where there is arithmetic to check: the argument
    # checks and the tiling plan)
    for obj in objs:
        syms = _run(["nm", obj], out).stdout
        assert "__asan_" in syms, obj
        if os.path.basename(obj) in ("abi.o", "sketch.o"):
            assert "__ubsan_handle" in syms, obj
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([exe], cwd=out, capture_output=True, text=True, env=env, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-8000:]
    assert "0 failed" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr
    shutil.rmtree(out, ignore_errors=True)
