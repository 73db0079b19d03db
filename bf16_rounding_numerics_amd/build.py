"""Build the HIP library libaddrmsnorm.so for gfx950, in place.

The build records its own target, flags and source digest in the library
(add_rmsnorm_build_info), so a stale or differently built binary is visible
to whoever loads it.
"""
from __future__ import annotations

import hashlib
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libaddrmsnorm.so")
SOURCES = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "log1p.hip"),
           os.path.join(CSRC, "api.cpp")]
HEADERS = [os.path.join(CSRC, "launch.h"), os.path.join(CSRC, "log1p_table.h"),
           os.path.join(INCLUDE, "add_rmsnorm.h"), os.path.join(INCLUDE, "log1p_f32.h")]

ARCH = "gfx950"
# Numerics flags: no contraction (every fma is written out), IEEE denormals,
# correctly rounded fp32 division and square root, no fast-math.  Packed fp32
# instructions are disabled for the device (the host pass warns it does not
# know that feature; harmless).
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def source_digest() -> str:
    h = hashlib.sha256()
    for p in SOURCES + HEADERS:
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()


def build() -> str:
    """Compile the library; returns its path."""
    digest = source_digest()
    info = "arch=%s flags=%s sources_sha256=%s" % (ARCH, " ".join(FLAGS), digest)
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "--offload-arch=" + ARCH, *FLAGS, "-I" + INCLUDE, "-I" + CSRC,
           '-DADD_RMSNORM_BUILD_INFO="%s"' % info, "-o", tmp, *SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s\n%s" % (r.returncode, r.stdout, r.stderr))
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build())
