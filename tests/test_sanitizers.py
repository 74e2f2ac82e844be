"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs are built with the sanitizers and must run clean:
  * the C oracle (oracle/kdaref.c) driven by tests/c_abi/oracle_check.c
    (every dtype, several threads, the epilogue, argument errors, and a
    one-token closed form);
  * libkda's host ABI code (kda_api.hip, instrumented on the host side only;
    the device code is built as usual) driven by tests/c_abi/abi_check.c, the
    plain C caller of the documented host-side behaviour.  The other kernel
    objects are the in-tree build's.
Any sanitizer report aborts the program with a nonzero status.
"""
import os
import shutil
import subprocess

import pytest

from gated_delta_rule_14_amd import build as kbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CABI = os.path.join(ROOT, "tests", "c_abi")
ROCM = "/opt/rocm"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    run([gcc, "-std=c11", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-pthread", os.path.join(CABI, "oracle_check.c"),
         os.path.join(ROOT, "oracle", "kdaref.c"), "-o", exe, "-lm"])
    r = run([exe], env=dict(SAN_ENV, ASAN_OPTIONS="abort_on_error=1:detect_leaks=1"))
    assert r.stdout.strip() == "ok"


def test_host_abi_under_sanitizers(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not all(os.path.exists(p) for p in (hipcc, clang, clangxx)):
        pytest.skip("ROCm toolchain not available")
    objs = [os.path.join(kbuild.OBJ, os.path.basename(s) + ".o") for s in kbuild.sources()
            if os.path.basename(s) != "kda_api.hip"]
    if not all(os.path.exists(o) for o in objs):
        pytest.fail("kernel objects missing; run __graft_entry__.build() first")
    api = str(tmp_path / "kda_api_san.o")
    # host-side instrumentation only: -Xarch_host before each sanitizer flag
    run([hipcc, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"),
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=all",
         "-c", os.path.join(kbuild.CSRC, "kda_api.hip"), "-o", api])
    caller = str(tmp_path / "abi_check.o")
    run([clang, "-std=c11", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-I" + os.path.join(ROOT, "include"), "-c", os.path.join(CABI, "abi_check.c"), "-o", caller])
    exe = str(tmp_path / "abi_san")
    run([clangxx, "-fsanitize=address,undefined", caller, api] + objs +
        ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    # the HIP runtime's own allocations at exit are not this code's: leaks off
    r = run([exe], env=dict(SAN_ENV, ASAN_OPTIONS="abort_on_error=1:detect_leaks=0"))
    assert r.stdout.strip() == "ok"
