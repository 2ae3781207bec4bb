"""Host sanitizers over the CPU oracle (no GPU): oracle/sanitize_check.cpp, which calls every
exported oracle function in both precisions on inputs that reach each branch, built together with
the oracle source under AddressSanitizer + UndefinedBehaviorSanitizer (g++), and under
ThreadSanitizer with the OpenMP runtime's Archer tool (clang++), which supplies the happens-before
edges of OpenMP's barriers and task scheduling that an uninstrumented runtime hides."""
import os
import shutil
import subprocess

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(REPO, "oracle")
DRIVER = os.path.join(ORACLE, "sanitize_check.cpp")
ROCM_LLVM = "/opt/rocm/llvm"


def _build_and_run(tmp_path, compiler, flags, env_extra):
    exe = str(tmp_path / "sanitize_check")
    subprocess.run([compiler, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *flags, "-fopenmp", "-I", ORACLE,
                    DRIVER, "-o", exe], check=True, capture_output=True, timeout=300)
    env = dict(os.environ, OMP_NUM_THREADS="4", **env_extra)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    return r


def test_address_and_undefined_behaviour_sanitizers(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    r = _build_and_run(tmp_path, "g++", ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"],
                       {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0", "UBSAN_OPTIONS": "print_stacktrace=1"})
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "ERROR: LeakSanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and "0 unexpected values" in out, out[-4000:]


def test_thread_sanitizer_with_openmp_archer(tmp_path):
    clang = os.path.join(ROCM_LLVM, "bin", "clang++")
    archer = os.path.join(ROCM_LLVM, "lib", "libarcher.so")
    if not (os.path.exists(clang) and os.path.exists(archer)):
        pytest.skip("clang++ with the Archer OpenMP tool not found")
    r = _build_and_run(tmp_path, clang, ["-fsanitize=thread", f"-Wl,-rpath,{ROCM_LLVM}/lib"],
                       {"OMP_TOOL_LIBRARIES": archer, "TSAN_OPTIONS": "ignore_noninstrumented_modules=1"})
    out = r.stdout + r.stderr
    assert "WARNING: ThreadSanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and "0 unexpected values" in out, out[-4000:]
