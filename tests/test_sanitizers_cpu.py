"""CPU sanitizer leg: the float64 oracle and the attention library's host code
(argument validation, dispatch, the C ABI) built with AddressSanitizer and
UndefinedBehaviorSanitizer, each exercised by the existing CPU tests in a child
process that preloads the matching ASan runtime (gcc's for the oracle, clang's
for the library's host code). Any sanitizer report fails the child process and
so this test. Leak checking is off: the child is a Python interpreter whose own
allocations are not the code under test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_child(preload, fa_lib, oracle_lib, tests):
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join(x for x in (preload, os.environ.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "2"
    env.pop("PYTEST_XDIST_WORKER", None)
    cmd = [sys.executable, os.path.join(ROOT, "tests", "sanitize_driver.py"), fa_lib, oracle_lib,
           "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(ROOT, "tests", t) for t in tests]]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    """The oracle pins (every oracle entry point on small and edge inputs)."""
    from oracle import build_oracle
    lib = build_oracle.build(sanitize_dir=str(tmp_path))
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    if not os.path.exists(asan):
        pytest.skip("gcc's libasan is not installed")
    out = _run_child(asan, "-", lib, ["test_oracle_pins.py", "test_oracle_mask_pins.py",
                                      "test_oracle_bwd_pins.py", "test_oracle_decode_pins.py"])
    assert " passed" in out


def test_host_code_under_asan_ubsan(tmp_path):
    """Every argument-validation path of every C entry point (the CPU ABI
    tests call them with invalid or empty arguments, which return before any
    HIP call), plus the binding's own checks."""
    from tests.conftest import gpu_available
    if gpu_available():
        pytest.skip("the ABI validation tests run only where no GPU is visible")
    from exact_attention_91_amd import build
    lib = build.build_host_sanitized(str(tmp_path))
    out = _run_child(build.host_sanitizer_runtime(), lib, "-", ["test_abi_cpu.py"])
    assert " passed" in out
