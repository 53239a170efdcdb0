"""Host-side validation under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU).

Every libmoe source is compiled as the product build compiles it, with ASan
and UBSan added to the host pass only (the device code is unchanged and never
runs here: the consumer makes only calls that validation answers before any
launch), and linked into a private copy of the library. The plain C11 consumer tests/c_abi_check.c, built with
the same sanitizers, then drives every entry point's argument checks,
including extreme sizes whose products would overflow a 32-bit int. Any
out-of-bounds access, use of freed memory, signed overflow, misaligned access
or invalid shift in the host code ends the run with a report.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

from mixture_experts_layer_count_amd.build import FLAGS as PRODUCT_FLAGS, _file_flags

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_count_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("hipcc / clang not available")
    out = tmp_path_factory.mktemp("san")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def compile_one(src):
        obj = str(out / (os.path.basename(src) + ".o"))
        _run([HIPCC, *PRODUCT_FLAGS, *_file_flags(src), "-Xarch_host", "-g", *SAN, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(out / "libmoe.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, "-o", lib, *objs])
    exe = str(out / "c_abi_check")
    _run([CLANG, "-std=c11", "-g", "-Wall", "-Wextra", "-Werror", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", "-I/opt/rocm/include",
          os.path.join(ROOT, "tests", "c_abi_check.c"), "-o", exe, f"-L{out}", "-lmoe", f"-Wl,-rpath,{out}"])
    return exe


def test_c_abi_validation_under_asan_ubsan(sanitized):
    env = dict(os.environ)
    # the HIP runtime is not instrumented and keeps allocations for the
    # process lifetime: leak reports would be about it, not this code
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    run = subprocess.run([sanitized], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all checks passed" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
