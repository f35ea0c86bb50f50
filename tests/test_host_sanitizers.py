"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two checked builds, each run in a child process with its sanitizer runtime preloaded:
  * the C oracle, built by gcc with -fsanitize=address,undefined, under the oracle's pin tests;
  * the library's host code (argument validation, plan choice, launch set-up), built by hipcc
    with the sanitizers on the host pass only, under the ABI tests, which include a sweep of
    every planner over shapes, paths and splits. No GPU is visible to that process, so every
    accepted configuration stops at its first HIP call.
Any sanitizer report ends the child process with a non-zero status and fails the test. Leak
checking is off: the Python interpreter keeps its own allocations until exit.
"""
import ctypes
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ENV_OPTS = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
            "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _device_visible() -> bool:
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return False
    n = ctypes.c_int(0)
    return hip.hipGetDeviceCount(ctypes.byref(n)) == 0 and n.value > 0


def _instrumented(lib: str) -> bool:
    res = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    syms = res.stdout
    return "__asan_report_load" in syms and "__ubsan_handle_" in syms


def _run_child(code: str, lib: str, runtime: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, **ENV_OPTS)
    env["LD_PRELOAD"] = runtime
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    return subprocess.run([sys.executable, "-c", code, lib], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=600)


def _check(res: subprocess.CompletedProcess, what: str):
    out = res.stdout + res.stderr
    assert res.returncode == 0, f"{what} under ASan/UBSan: status {res.returncode}\n{out[-6000:]}"
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]


ORACLE_CHILD = r"""
import glob, os, sys, pytest
import oracle
from oracle import build
build.LIB = sys.argv[1]
rc = pytest.main(["-q", "-x", "-s", "-p", "no:cacheprovider", "-m", "not gpu"]
                 + sorted(glob.glob("tests/test_oracle_*.py")))
assert os.path.samefile(oracle.lib()._name, sys.argv[1]), "the checked oracle was not the one loaded"
sys.exit(int(rc))
"""

LIBRARY_CHILD = r"""
import os, sys, pytest
from skinny_gemm_nvfp4_amd import binding, build
build.LIB = sys.argv[1]
rc = pytest.main(["-q", "-x", "-s", "-p", "no:cacheprovider", "tests/test_abi.py"])
assert os.path.samefile(binding.load_library()._name, sys.argv[1]), "the checked library was not the one loaded"
sys.exit(int(rc))
"""


def test_oracle_under_asan_ubsan(tmp_path):
    from oracle import sanitize
    runtime = sanitize.asan_runtime()
    if not runtime:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    lib = sanitize.build_checked(str(tmp_path / "libnvfp4_oracle_checked.so"))
    assert _instrumented(lib)
    _check(_run_child(ORACLE_CHILD, lib, runtime), "oracle pin tests")


def test_library_host_code_under_asan_ubsan(tmp_path):
    from skinny_gemm_nvfp4_amd import hostcheck
    if _device_visible():
        pytest.skip("a GPU is visible: the checked library is for processes that have none")
    runtime = hostcheck.asan_runtime()
    if not runtime:
        pytest.skip("the clang AddressSanitizer runtime is not installed")
    lib = hostcheck.build_checked(str(tmp_path / "libnvfp4_checked.so"))
    assert _instrumented(lib)
    res = _run_child(LIBRARY_CHILD, lib, runtime)
    _check(res, "ABI tests")
    # the planner sweeps ran (they skip only where a GPU is visible, which the CPU suite never has)
    assert "skipped" not in res.stdout, res.stdout[-3000:]
