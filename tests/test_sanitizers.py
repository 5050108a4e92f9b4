"""The CPU-side code under AddressSanitizer and UndefinedBehaviorSanitizer:
the oracle (every pin of tests/test_oracle_pins.py) and the argument
validation of the C ABI (every check of tests/test_abi.py), each built with
the sanitizers and run in a child process with the sanitizer runtime
preloaded.  Any sanitizer report fails the test.  CPU only."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_child(env_extra, tests):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           *tests]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_under_sanitizers():
    from oracle import build
    lib = build.build_sanitized()
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isfile(asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    out = run_child({"ORACLE_LIB": lib, "LD_PRELOAD": asan},
                    ["tests/test_oracle_pins.py"])
    assert " passed" in out


def test_abi_validation_under_sanitizers():
    from quantized_gguf_block_amd import build
    try:
        lib = build.build_host_sanitized()
    except FileNotFoundError as e:
        pytest.skip(f"library objects not built: {e}")
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    out = run_child({"CQ_TEST_LIB": lib, "LD_PRELOAD": rt[-1]}, ["tests/test_abi.py"])
    assert " passed" in out
