"""CPU hygiene: the oracle and the C ABI's host validation layer built with
AddressSanitizer and UndefinedBehaviorSanitizer, their tests run against
those builds in a child process (uninstrumented Python with the sanitizer
runtime preloaded).  Any report fails the run: the builds abort on the
first error."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_TESTS = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
CHILD_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
             "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run_child(code, extra_env, timeout=600):
    env = dict(os.environ, **CHILD_ENV, **extra_env)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_under_asan_ubsan():
    gcc_asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(gcc_asan) or not os.path.exists(gcc_asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    from oracle import build as ob
    lib = ob.build(sanitize=True)
    code = ("import sys, pytest, oracle\n"
            f"assert oracle._LIB_PATH == {lib!r}\n"
            f"sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', *{ORACLE_TESTS!r}]))\n")
    out = _run_child(code, {"LD_PRELOAD": gcc_asan, "MXQ_ORACLE_LIB": lib})
    assert " passed" in out


def test_abi_validation_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not os.path.exists(hipcc) or not rt:
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "libmxq_san.so")
    csrc = os.path.join(ROOT, "mxfp4_precision_numerics_amd", "csrc")
    # host code only is instrumented (each -fsanitize after -Xarch_host)
    cmd = [hipcc, "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared", "-O1", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), os.path.join(csrc, "mxq_api.hip"),
           os.path.join(ROOT, "tests", "sanitize", "abi_stubs.hip"), "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    code = ("import sys, pytest\n"
            "import mxfp4_precision_numerics_amd as m\n"
            f"m.LIB_PATH = {lib!r}\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', 'tests/test_abi.py', "
            "'tests/test_binding_checks.py']))\n")
    out = _run_child(code, {"LD_PRELOAD": rt[-1]})
    assert " passed" in out
