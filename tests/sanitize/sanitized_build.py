"""Builds of the library's host code and of the oracle with AddressSanitizer
and UndefinedBehaviorSanitizer, for CPU tests.

The HIP library is compiled from the same sources and flags as the shipped
one, with the sanitizers on the host side only (each -fsanitize= behind
-Xarch_host: device code is never instrumented), against the shared
sanitizer runtime of the compiler (clang's, preloaded at run time).  The C
oracles are compiled with gcc's sanitizers.  Results are cached under
tests/sanitize/_build by source digest.
"""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
BUILD = os.path.join(HERE, "_build")

HOST_SANITIZERS = ["-g", "-fno-omit-frame-pointer",
                   "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=all", "-shared-libsan"]
GCC_SANITIZERS = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]


def clang_asan_runtime() -> str:
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise FileNotFoundError("clang's shared AddressSanitizer runtime is not installed")
    return found[-1]


def gcc_runtime(name: str) -> str:
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True,
                          check=True).stdout.strip()
    if not os.path.isabs(path):
        raise FileNotFoundError("gcc's %s is not installed" % name)
    return path


def _digest(paths, extra):
    h = hashlib.sha256(extra.encode())
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def library() -> str:
    """The HIP library with host-side ASan and UBSan (built if missing)."""
    from bf16_rounding_numerics_amd import build as hip_build

    digest = hip_build.source_digest()
    out = os.path.join(BUILD, "libaddrmsnorm_san_%s.so" % digest[:16])
    if os.path.exists(out):
        return out
    os.makedirs(BUILD, exist_ok=True)
    info = "arch=%s flags=%s sources_sha256=%s" % (hip_build.ARCH, " ".join(hip_build.FLAGS),
                                                   digest)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "--offload-arch=" + hip_build.ARCH, *hip_build.FLAGS, *HOST_SANITIZERS,
           "-I" + hip_build.INCLUDE, "-I" + hip_build.CSRC,
           '-DADD_RMSNORM_BUILD_INFO="%s"' % info, "-o", tmp, *hip_build.SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized hipcc build failed:\n" + r.stderr[-4000:])
    os.replace(tmp, out)
    return out


def oracles() -> tuple:
    """The C oracles (fused op and log1p) with gcc's ASan and UBSan."""
    import oracle

    d = _digest([oracle.SOURCE, oracle.LOG1P_SOURCE], " ".join(oracle.CFLAGS + GCC_SANITIZERS))
    lib = os.path.join(BUILD, "liboracle_san_%s.so" % d)
    log1p = os.path.join(BUILD, "liblog1p_oracle_san_%s.so" % d)
    if not (os.path.exists(lib) and os.path.exists(log1p)):
        os.makedirs(BUILD, exist_ok=True)
        flags = oracle.CFLAGS + GCC_SANITIZERS
        subprocess.run(["gcc", *flags, "-o", lib, oracle.SOURCE, "-lm"], check=True)
        flags11 = [f if f != "-std=c11" else "-std=gnu11" for f in flags]
        subprocess.run(["gcc", *flags11, "-o", log1p, oracle.LOG1P_SOURCE, "-lquadmath", "-lm"],
                       check=True)
    return lib, log1p
