"""The public headers as plain C: a C99 program (tests/c_abi/abi_check.c)
compiled with -Wall -Wextra -Werror -pedantic against include/ only, linked
with the built library and run.  It checks the ABI version, the build
identity, the status texts, zero-size calls and host-side argument errors;
it never launches a kernel (CPU only)."""
import os
import subprocess

import pytest

import bf16_rounding_numerics_amd as arn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_visible():
    import torch

    return torch.cuda.device_count() > 0


@pytest.mark.skipif(_gpu_visible(), reason="fake device addresses: CPU only")
def test_c99_caller_of_the_abi(tmp_path):
    exe = str(tmp_path / "abi_check")
    lib_dir = os.path.dirname(arn.LIBRARY)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I" + os.path.join(ROOT, "include"), "-o", exe,
                    os.path.join(ROOT, "tests", "c_abi", "abi_check.c"), arn.LIBRARY,
                    "-Wl,-rpath," + lib_dir], check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_headers_compile_as_cxx_too(tmp_path):
    src = tmp_path / "inc.cpp"
    src.write_text('#include "add_rmsnorm.h"\n#include "log1p_f32.h"\nint main() { return 0; }\n')
    subprocess.run(["g++", "-std=c++11", "-Wall", "-Werror", "-fsyntax-only",
                    "-I" + os.path.join(ROOT, "include"), str(src)], check=True)
