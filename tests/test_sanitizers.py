"""CPU sanitizer runs: the C oracle and the host side of the HIP library (the
C-ABI entry points' argument validation, workspace layout and error paths)
are built with AddressSanitizer and UndefinedBehaviorSanitizer, and the
oracle's pin tests and the C-ABI validation tests run against those builds in
a child process with the sanitizer runtime preloaded.  Any report (an
out-of-bounds or freed-memory access, a signed overflow, a misaligned access,
an out-of-range shift or conversion) aborts the child and fails the test.  No GPU is used: the device
code of the HIP library is compiled as usual and never launched here."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_runtime(name):
    try:
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                           check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _run_child(tests, env_extra):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *tests]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    from oracle import build as oracle_build
    lib = oracle_build.build(lib=str(tmp_path / "libmoe_oracle_san.so"), sanitize=True)
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    out = _run_child(tests, {"MOE_ORACLE_LIBRARY": lib, "LD_PRELOAD": f"{asan} {ubsan}"})
    print(out.strip().splitlines()[-1])


def test_host_validation_under_asan_ubsan(tmp_path):
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rts or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc or clang's ASan runtime not installed")
    from sparse_moe_layer_04_amd import build as hip_build
    lib = hip_build.build(lib=str(tmp_path / "libmoe_hip_san.so"),
                          build_dir=str(tmp_path / "obj"), sanitize=True)
    out = _run_child([os.path.join(ROOT, "tests", "test_abi.py")],
                     {"MOE_HIP_LIBRARY": lib, "LD_PRELOAD": sorted(rts)[-1]})
    print(out.strip().splitlines()[-1])
