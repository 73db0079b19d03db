"""Builds the C callers of the library's ABI (test helpers, plain C with gcc):
gpu_caller, a C99 program that runs the library on the GPU with HIP's C
runtime API and no Python.  The executable finds the library next to the
package through its run path, so it runs from any working directory."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(ROOT, "bf16_rounding_numerics_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
GPU_CALLER = os.path.join(HERE, "gpu_caller")


def build(force: bool = True) -> str:
    src = GPU_CALLER + ".c"
    if force or not os.path.exists(GPU_CALLER) or (
            os.path.getmtime(GPU_CALLER) < os.path.getmtime(src)):
        tmp = GPU_CALLER + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-D__HIP_PLATFORM_AMD__", "-I" + INCLUDE,
                        "-isystem", os.path.join(ROCM, "include"), "-o", tmp, src,
                        "-L" + LIB_DIR, "-laddrmsnorm", "-L" + os.path.join(ROCM, "lib"),
                        "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../bf16_rounding_numerics_amd",
                        "-Wl,-rpath," + os.path.join(ROCM, "lib")], check=True)
        os.replace(tmp, GPU_CALLER)
    return GPU_CALLER
