"""AddressSanitizer and UndefinedBehaviorSanitizer over the host code (CPU).

Two child processes, each with its compiler's sanitizer runtime preloaded:
  * the HIP library's host side (argument validation: view overlap and span
    arithmetic, launch configuration, dispatch; the kernels' launch helpers)
    built with -fsanitize=address,undefined behind -Xarch_host, under the CPU
    boundary tests;
  * the C oracles built with gcc's sanitizers, under the oracle-pin tests.
A sanitizer report stops the child with a nonzero status, which fails here.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
sys.path.insert(0, os.path.join(TESTS, "sanitize"))

import sanitized_build as sb  # noqa: E402

pytestmark = pytest.mark.slow


def _gpu_visible():
    import torch

    return torch.cuda.device_count() > 0


def run_sanitized(preload, setup, test_files, deselect=""):
    env = dict(os.environ)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:exitcode=99"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=98"
    code = ("import sys\nsys.path.insert(0, %r)\nsys.path.insert(0, %r)\n%s\nimport pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-m', 'not gpu and not slow', '-p', "
            "'no:cacheprovider'] + %r + %r))\n"
            % (ROOT, TESTS, setup, ["-k", deselect] if deselect else [], test_files))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=1500)
    report = r.stdout[-4000:] + "\n" + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in r.stderr, report
    assert "runtime error:" not in r.stderr, report
    return r.stdout


@pytest.mark.skipif(_gpu_visible(), reason="the boundary tests use fake addresses: CPU only")
def test_library_host_code_under_asan_and_ubsan():
    lib = sb.library()
    setup = "import bf16_rounding_numerics_amd as arn\narn.LIBRARY = %r" % lib
    out = run_sanitized(sb.clang_asan_runtime(), setup,
                        [os.path.join(TESTS, "test_boundary.py")])
    assert " passed" in out


def test_oracles_under_asan_and_ubsan():
    lib, log1p = sb.oracles()
    setup = ("import oracle\noracle._default = oracle.Oracle(%r)\n"
             "oracle._default_log1p = oracle.Log1pOracle(%r)" % (lib, log1p))
    files = [os.path.join(TESTS, f) for f in (
        "test_oracle_converters.py", "test_oracle_fused.py", "test_oracle_plain.py",
        "test_oracle_quant.py", "test_oracle_fp8.py", "test_oracle_qk.py",
        "test_oracle_log1p.py")]
    # The planted-mistake tests run mutated copies of the oracle, not this
    # build; the second 72-call chain repeats the first one's code path.
    out = run_sanitized(sb.gcc_runtime("libasan.so"), setup, files,
                        deselect="not planted_mistake and not chain_gate")
    assert " passed" in out


@pytest.mark.parametrize("fn,kind", [("heap_overflow", "AddressSanitizer"),
                                     ("signed_overflow", "runtime error")])
def test_the_harness_reports_planted_errors(tmp_path, fn, kind):
    """The same preload and options catch a planted heap overflow and a signed
    overflow in a small library of their own (run in a child process)."""
    src = tmp_path / "planted.c"
    src.write_text(
        "#include <limits.h>\n#include <stdlib.h>\n"
        "int heap_overflow(int n) { int* p = malloc(n * sizeof(int)); int v = p[n];"
        " free(p); return v; }\n"
        "int signed_overflow(int a) { return a + 1; }\n")
    lib = tmp_path / "libplanted.so"
    subprocess.run(["gcc", "-O0", "-shared", "-fPIC", *sb.GCC_SANITIZERS, "-o", str(lib),
                    str(src)], check=True)
    arg = 4 if fn == "heap_overflow" else 2147483647
    env = dict(os.environ)
    env["LD_PRELOAD"] = sb.gcc_runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:exitcode=99"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=98"
    code = "import ctypes; print(ctypes.CDLL(%r).%s(%d))" % (str(lib), fn, arg)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0 and kind in r.stderr, r.stderr[-2000:]
