"""The gfx950 assembly of this library's own kernels, built here with the
library's own flags (CPU only: hipcc cross-compiles).

Checks, per kernel:
  * fp32 denormals are kept (.amdhsa_float_denorm_mode_32 3, no flush to
    zero): the IEEE gradual underflow the oracle assumes;
  * no private (scratch) segment: no register spills, no stack;
  * and, over the whole file: the stores round through the hardware packed
    fp32 -> bf16 conversion (v_cvt_pk_bf16_f32, round to nearest even), and
    no packed fp32 arithmetic instruction is emitted (the build disables them).
"""
import os
import re
import subprocess

import pytest

from bf16_rounding_numerics_amd import build as hip_build

pytestmark = pytest.mark.slow


def _device_asm(tmp_path, source):
    out = tmp_path / (os.path.basename(source) + ".s")
    flags = [f for f in hip_build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = ["hipcc", "--offload-arch=" + hip_build.ARCH, "--cuda-device-only", "-S", *flags,
           "-I" + hip_build.INCLUDE, "-I" + hip_build.CSRC, "-o", str(out), source]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernel_descriptors(asm):
    """{kernel symbol: {directive: value}} from the .amdhsa_kernel blocks."""
    kernels = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", asm, re.S):
        fields = dict(re.findall(r"\.(amdhsa_\w+) (\S+)", m.group(2)))
        kernels[m.group(1)] = fields
    return kernels


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")
    return {os.path.basename(s): _device_asm(d, s)
            for s in hip_build.SOURCES if s.endswith(".hip")}


def test_every_kernel_keeps_denormals_and_has_no_scratch(asm):
    total = 0
    for name, text in asm.items():
        kernels = _kernel_descriptors(text)
        assert kernels, name
        for k, f in kernels.items():
            assert f.get("amdhsa_float_denorm_mode_32") == "3", (name, k, f.get(
                "amdhsa_float_denorm_mode_32"))
            assert f.get("amdhsa_private_segment_fixed_size") == "0", (name, k)
        total += len(kernels)
    # every template instance the dispatch can reach is compiled
    assert total > 600, total


def test_rounding_uses_the_hardware_rne_convert(asm):
    text = asm["kernels.hip"]
    assert len(re.findall(r"\bv_cvt_pk_bf16_f32\b", text)) > 1000


def test_no_packed_fp32_arithmetic(asm):
    for name, text in asm.items():
        found = re.findall(r"\bv_pk_(?:add|mul|fma)_f32\b", text)
        assert not found, (name, found[:3])
