"""Sanitizer runs on the host, no GPU needed: the C oracle and the host side
of the C-ABI library (argument validation, launch planning, error strings),
each built with AddressSanitizer and UndefinedBehaviorSanitizer, run the oracle
pins and the host ABI tests in a child process that preloads the sanitizer
runtime. A positive control plants an out-of-bounds read in a copy of the
oracle source and checks that the same setup reports it.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
ORACLE_SRC = os.path.join(ROOT, "oracle", "qmv_oracle.c")
SAN_CFLAGS = ["-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
              "-fno-fast-math", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=undefined"]


def asan_runtime():
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return rts[-1] if rts else None


def build_oracle(src, out):
    subprocess.run([CLANG] + SAN_CFLAGS + ["-o", out, src, "-lm"], check=True)
    return out


def child_env(oracle_lib, host_lib=None):
    env = dict(os.environ, LD_PRELOAD=asan_runtime(), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               QMV_SANITIZED_ORACLE=oracle_lib)
    if host_lib:
        env["QMV_SANITIZED_LIB"] = host_lib
    return env


@pytest.fixture(scope="module")
def san_builds(tmp_path_factory):
    if asan_runtime() is None or not os.path.exists(CLANG):
        pytest.skip("no clang sanitizer runtime in this image")
    from block_quantized_matvec_gguf_amd import build
    if not os.path.exists(build.SAN_LIB):
        build.build()
    d = tmp_path_factory.mktemp("san")
    return build_oracle(ORACLE_SRC, str(d / "liboracle_san.so")), build.SAN_LIB, d


def test_pins_and_host_abi_under_sanitizers(san_builds):
    oracle_lib, host_lib, _ = san_builds
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
         "tests/test_host_abi.py", "tests/test_oracle_pins.py",
         "tests/test_sanitizers.py::test_child_loads_the_sanitizer_builds",
         # (these two import torch, which is not run under the preloaded runtime)
         "-k", "not bf16_every_pattern and not create_without_a_device"],
        cwd=ROOT, env=child_env(oracle_lib, host_lib), capture_output=True, text=True,
        timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in r.stdout and " skipped" not in r.stdout.splitlines()[-1], out[-2000:]


def test_child_loads_the_sanitizer_builds():
    """Inside the child run: the preloaded runtime is active and both
    libraries in use are the sanitizer builds."""
    if "QMV_SANITIZED_LIB" not in os.environ:
        pytest.skip("checked inside the sanitizer child run")
    import ctypes

    import oracle
    from block_quantized_matvec_gguf_amd import binding
    assert hasattr(ctypes.CDLL(None), "__asan_report_load1")
    assert oracle._lib._name == os.environ["QMV_SANITIZED_ORACLE"]
    assert binding._lib._name == os.environ["QMV_SANITIZED_LIB"]


def test_planted_out_of_bounds_read_is_reported(san_builds):
    """Positive control: a copy of the oracle whose Q8_0 decode reads the code
    byte one block too far is run on one 34-byte block; the sanitizer must
    stop it with a heap-buffer-overflow report."""
    _, _, d = san_builds
    src = open(ORACLE_SRC).read()
    good = "case ORACLE_Q8_0: return oracle_q8_0_elem(row + (i / 32) * 34, (int)(i % 32));"
    assert good in src
    bad = src.replace(good, "case ORACLE_Q8_0: return oracle_q8_0_elem(row + (i / 32 + 1) * 34,"
                            " (int)(i % 32));")
    (d / "bad.c").write_text(bad)
    lib = build_oracle(str(d / "bad.c"), str(d / "libbad.so"))
    script = ("import sys, numpy as np; sys.path.insert(0, %r); import oracle; "
              "lib = oracle.load_library(%r); blk = np.zeros(34, np.uint8); "
              "print(lib.oracle_elem(6, blk.ctypes.data, 5))" % (ROOT, lib))
    r = subprocess.run([sys.executable, "-c", script], env=child_env(lib), capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr, r.stderr[-3000:]
