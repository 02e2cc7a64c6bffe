"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The HIP sources are compiled with the sanitizers on their host side only (the
GPU code is built as usual), linked with ``tests/host/abi_host_check.cpp``,
and run on the CPU: every call there returns before any HIP call (layout and
workspace queries, the host-side W12 format check, plan creation on a
27B-like model description, argument validation of the launching entry
points).  A sanitizer finding aborts the program."""

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tree_verification_pass_amd", "csrc")
ROCM = "/opt/rocm"
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="ROCm toolchain not found")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_abi_host_paths_clean_under_sanitizers(tmp_path):
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_hip(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *inc,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_hip, sorted(glob.glob(os.path.join(CSRC, "*.hip")))))
    drv = str(tmp_path / "drv.o")
    _run([CLANG, "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", *inc,
          "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-c",
          os.path.join(ROOT, "tests", "host", "abi_host_check.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_host_check")
    _run([CLANG, "-fsanitize=address,undefined", drv, *objs, f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = _run([exe], env=env, timeout=300)
    assert "abi host checks passed" in r.stdout
