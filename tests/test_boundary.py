"""The C-ABI boundary, on the CPU: the library loads, exports every entry point
include/*.h declares, and rejects bad arguments on the host before any HIP
call.  (No computation runs here; that needs the GPU.)"""
import ctypes
import glob
import math
import os
import re
import subprocess

import pytest

import bf16_rounding_numerics_amd as arn
from bf16_rounding_numerics_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M):
            if not m.group(0).lstrip().startswith("#"):
                names.add(m.group(1))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert set(arn.EXPORTS) == set(names), names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", arn.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(arn.lib(), name)


def test_abi_version_matches_header():
    hdr = open(os.path.join(ROOT, "include", "add_rmsnorm.h")).read()
    v = int(re.search(r"#define ADD_RMSNORM_ABI_VERSION (\d+)", hdr).group(1))
    assert arn.add_rmsnorm_abi_version() == v == arn.ABI_VERSION
    m = int(re.search(r"#define ADD_RMSNORM_MAX_HIDDEN (\d+)", hdr).group(1))
    assert m == arn.MAX_HIDDEN


def test_build_info_names_target_flags_and_current_sources():
    info = arn.add_rmsnorm_build_info()
    assert "arch=gfx950" in info
    for flag in ("-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
                 "-fhip-fp32-correctly-rounded-divide-sqrt", "-packed-fp32-ops"):
        assert flag in info
    # A library built from other sources than the tree's is stale.
    assert "sources_sha256=" + hip_build.source_digest() in info


def test_strerror_texts():
    texts = {s: arn.add_rmsnorm_strerror(s) for s in (0, -1, -2, -3, -4, -5)}
    assert len(set(texts.values())) == 6
    assert arn.add_rmsnorm_strerror(-99) == "unknown status"


# ---------------------------------------------------------------- validation

A = 1 << 20  # fake, 16-byte aligned "device" addresses far apart
MB = 1 << 24


def _gpu_visible():
    import torch

    return torch.cuda.device_count() > 0


# Every call below must be rejected before a launch; where a GPU is visible
# they are skipped anyway, so that fake addresses can never reach a kernel.
fake_addresses = pytest.mark.skipif(_gpu_visible(), reason="fake device addresses: CPU only")


def call(out=A, res=A + MB, x=A + 2 * MB, r=A + 3 * MB, w=A + 4 * MB, n=4, h=64, eps=1e-6,
         cfg=None):
    L = arn.lib()
    if cfg is None:
        return L.add_rmsnorm_fwd(out, res, x, r, w, n, h, eps, None)
    c = arn.LaunchCfg(*cfg)
    return L.add_rmsnorm_fwd_cfg(out, res, x, r, w, n, h, eps, ctypes.byref(c), None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), arn.EINVAL),
    (dict(h=0), arn.EINVAL),
    (dict(h=-8), arn.EINVAL),
    (dict(eps=-1.0), arn.EINVAL),
    (dict(eps=math.nan), arn.EINVAL),
    (dict(eps=math.inf), arn.EINVAL),
    (dict(h=12, cfg=(arn.PATH_WG_ROW, 0, 0, 0)), arn.EALIGN),   # a fast path forced on
    (dict(h=4, cfg=(arn.PATH_WAVE_ROW, 0, 0, 0)), arn.EALIGN),  # what only the general takes
    (dict(h=32776), arn.ERANGE),
    (dict(out=0), arn.EINVAL),
    (dict(res=0), arn.EINVAL),
    (dict(x=0), arn.EINVAL),
    (dict(r=0), arn.EINVAL),
    (dict(w=0), arn.EINVAL),
    (dict(x=A + 2 * MB + 1), arn.EALIGN),               # odd address
    (dict(w=A + 4 * MB + 1), arn.EALIGN),
    (dict(x=A + 2 * MB + 8, cfg=(arn.PATH_LDS_TWO_PASS, 0, 0, 0)), arn.EALIGN),
    (dict(out=A + 2 * MB + 16), arn.EALIAS),            # out partly overlaps x
    (dict(res=A + 3 * MB - 16), arn.EALIAS),            # residual_out partly overlaps residual
    (dict(res=A + 4 * 64 * 2 - 16), arn.EALIAS),        # residual_out overlaps out's tail
    (dict(res=A + 4 * MB + 64), arn.EALIAS),            # residual_out overlaps weight
    (dict(out=A + 4 * MB), arn.EALIAS),                 # out is the weight
    (dict(out=A + 2 * MB, res=A + 2 * MB), arn.EALIAS), # both outputs in place on x
    (dict(n=1 << 62, h=8), arn.ERANGE),                 # byte count overflows
])
@fake_addresses
def test_argument_errors(kw, status):
    assert call(**kw) == status


@fake_addresses
def test_zero_rows_is_a_no_op_without_pointer_checks():
    assert call(out=0, res=0, x=0, r=0, w=0, n=0) == arn.OK
    assert call(n=0) == arn.OK


@fake_addresses
def test_adjacent_buffers_are_not_overlap():
    # residual_out right after out: touching, not overlapping.  A forced path
    # that cannot take hidden = 8192 is rejected after the overlap checks, so
    # ERANGE (not EALIAS) shows the adjacent buffers passed, and nothing is
    # launched with these fake addresses.
    assert call(res=A + 4 * 8192 * 2, h=8192, x=A + 8 * MB, r=A + 9 * MB, w=A + 10 * MB,
                cfg=(arn.PATH_WAVE_ROW, 0, 0, 0)) == arn.ERANGE
    assert call(res=A + 4 * 8192 * 2 - 16, h=8192, x=A + 8 * MB, r=A + 9 * MB, w=A + 10 * MB,
                cfg=(arn.PATH_WAVE_ROW, 0, 0, 0)) == arn.EALIAS


@pytest.mark.parametrize("kw", [
    dict(out=A + 2 * MB),                       # out == x
    dict(res=A + 3 * MB),                       # residual_out == residual
    dict(out=A + 2 * MB, res=A + 3 * MB),       # both in place
    dict(out=A + 3 * MB, res=A + 2 * MB),       # crosswise
])
@fake_addresses
def test_exact_in_place_aliases_pass_validation(kw):
    # Exact aliases are accepted.  A forced path that cannot take hidden 8192
    # is rejected after the alias checks, so ERANGE (not EALIAS) shows that
    # they passed, and nothing is launched with the fake addresses.
    assert call(h=8192, cfg=(arn.PATH_WAVE_ROW, 0, 0, 0), **kw) == arn.ERANGE


@pytest.mark.parametrize("cfg,status", [
    ((0, 0, 0, 1), arn.EINVAL),                 # flags must be 0
    ((9, 0, 0, 0), arn.EINVAL),                 # unknown path
    ((6, 0, 0, 0), arn.EINVAL),
    ((arn.PATH_PACKED, 0, 0, 3), arn.EINVAL),   # rows per lane 1, 2 or 4
    ((arn.PATH_PACKED, 0, 0, 8), arn.EINVAL),
    ((arn.PATH_WAVE_ROW, 0, 0, 2), arn.EINVAL),  # flags only on the packed and register paths
    ((arn.PATH_WAVE_ROW, 0, 0, 1), arn.EINVAL),
    ((arn.PATH_WG_ROW, 0, 0, 2), arn.EINVAL),   # the register path's only flag is 1
    ((arn.PATH_LDS_TWO_PASS, 0, 0, 1), arn.EINVAL),
    ((arn.PATH_GENERAL, 0, 0, 1), arn.EINVAL),
    ((-1, 0, 0, 0), arn.EINVAL),
    ((0, 100, 0, 0), arn.EINVAL),               # not a supported workgroup size
    ((0, 2048, 0, 0), arn.EINVAL),
    ((0, 0, -2, 0), arn.EINVAL),                # grid_blocks below -1
])
@fake_addresses
def test_bad_launch_configuration(cfg, status):
    assert call(cfg=cfg) == status


@pytest.mark.parametrize("path,block,h", [
    (arn.PATH_WAVE_ROW, 0, 8192),       # more than 8 segments per lane
    (arn.PATH_WAVE_ROW, 1024, 4096),    # 8 per lane at 1024 threads is not built
    (arn.PATH_WG_ROW, 64, 8192),
    (arn.PATH_WG_ROW, 1024, 32768),     # 4 per thread at 1024 threads is not built
    (arn.PATH_WG_ROW, 0, 32768),
    (arn.PATH_PACKED, 0, 520),          # more than 64 segments
    (arn.PATH_PACKED, 0, 8192),
])
@fake_addresses
def test_forced_path_outside_its_range(path, block, h):
    assert call(h=h, cfg=(path, block, 0, 0)) == arn.ERANGE
    if path == arn.PATH_WG_ROW:
        assert call(h=h, cfg=(path, block, 0, arn.FLAG_LATE_WEIGHT)) == arn.ERANGE


@fake_addresses
def test_cvt_range_errors():
    L = arn.lib()
    assert L.add_rmsnorm_test_cvt_range(A, 0, -8, None) == arn.EINVAL
    assert L.add_rmsnorm_test_cvt_range(A, 0, 12, None) == arn.EALIGN
    assert L.add_rmsnorm_test_cvt_range(A + 4, 0, 16, None) == arn.EALIGN
    assert L.add_rmsnorm_test_cvt_range(0, 0, 16, None) == arn.EINVAL
    assert L.add_rmsnorm_test_cvt_range(0, 0, 0, None) == arn.OK
    assert L.add_rmsnorm_test_cvt_e4m3_range(A, 0, -8, None) == arn.EINVAL
    assert L.add_rmsnorm_test_cvt_e4m3_range(A, 0, 12, None) == arn.EALIGN
    assert L.add_rmsnorm_test_cvt_e4m3_range(A + 8, 0, 16, None) == arn.EALIGN
    assert L.add_rmsnorm_test_cvt_e4m3_range(0, 0, 16, None) == arn.EINVAL
    assert L.add_rmsnorm_test_cvt_e4m3_range(0, 0, 0, None) == arn.OK


def qcall(q=A + 5 * MB, sc=A + 6 * MB, res=A + MB, x=A + 2 * MB, r=A + 3 * MB, w=A + 4 * MB,
          n=4, h=64, eps=1e-6, cfg=None, fp8=False):
    L = arn.lib()
    name = "add_rmsnorm_quant_fp8_fwd" if fp8 else "add_rmsnorm_quant_fwd"
    if cfg is None:
        return getattr(L, name)(q, sc, res, x, r, w, n, h, eps, None)
    c = arn.LaunchCfg(*cfg)
    return getattr(L, name + "_cfg")(q, sc, res, x, r, w, n, h, eps, ctypes.byref(c), None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), arn.EINVAL),
    (dict(h=12), arn.EALIGN),
    (dict(h=32776), arn.ERANGE),
    (dict(eps=math.nan), arn.EINVAL),
    (dict(q=0), arn.EINVAL),
    (dict(sc=0), arn.EINVAL),
    (dict(q=A + 5 * MB + 8), arn.EALIGN),
    (dict(sc=A + 6 * MB + 2), arn.EALIGN),
    (dict(q=A + 2 * MB), arn.EALIAS),                   # codes on x
    (dict(sc=A + 3 * MB + 64), arn.EALIAS),             # scales inside residual
    (dict(sc=A + 5 * MB + 16), arn.EALIAS),             # scales inside the codes
    (dict(q=A + MB + 128), arn.EALIAS),                 # codes inside residual_out
    (dict(res=A + 3 * MB - 16), arn.EALIAS),            # residual_out partly on residual
    (dict(res=A + 4 * MB), arn.EALIAS),                 # residual_out on the weight
])
@pytest.mark.parametrize("fp8", [False, True], ids=["int8", "fp8"])
@fake_addresses
def test_quant_argument_errors(kw, status, fp8):
    assert qcall(fp8=fp8, **kw) == status


@pytest.mark.parametrize("fp8", [False, True], ids=["int8", "fp8"])
@fake_addresses
def test_quant_packed_path_configuration(fp8):
    # the packed path takes quantised rows up to hidden 512; rows per lane 1, 2, 4
    assert qcall(fp8=fp8, h=520, cfg=(arn.PATH_PACKED, 0, 0, 0)) == arn.ERANGE
    assert qcall(fp8=fp8, h=1024, cfg=(arn.PATH_PACKED, 256, -1, 4)) == arn.ERANGE
    assert qcall(fp8=fp8, cfg=(arn.PATH_PACKED, 0, 0, 3)) == arn.EINVAL
    assert qcall(fp8=fp8, cfg=(arn.PATH_GENERAL, 0, 0, 0)) == arn.EINVAL
    assert qcall(fp8=fp8, cfg=(arn.PATH_WG_ROW, 0, 0, 2)) == arn.EINVAL
    # the late weight read is built for bf16 out only
    assert qcall(fp8=fp8, cfg=(arn.PATH_WG_ROW, 0, 0, arn.FLAG_LATE_WEIGHT)) == arn.EINVAL


@pytest.mark.parametrize("fp8", [False, True], ids=["int8", "fp8"])
@fake_addresses
def test_quant_zero_rows_and_in_place_validation(fp8):
    assert qcall(q=0, sc=0, res=0, x=0, r=0, w=0, n=0, fp8=fp8) == arn.OK
    # The fused entry points need both residual pointers.
    assert qcall(res=0, r=0, fp8=fp8) == arn.EINVAL
    assert qcall(res=0, fp8=fp8) == arn.EINVAL
    # residual_out == residual passes the alias checks (ERANGE from the forced
    # path comes after them; nothing is launched).
    assert qcall(res=A + 3 * MB, h=8192, cfg=(arn.PATH_WAVE_ROW, 0, 0, 0), fp8=fp8) == arn.ERANGE


def pcall(out=A, x=A + 2 * MB, w=A + 4 * MB, n=4, h=64, eps=1e-6, cfg=None):
    L = arn.lib()
    if cfg is None:
        return L.rmsnorm_fwd(out, x, w, n, h, eps, None)
    c = arn.LaunchCfg(*cfg)
    return L.rmsnorm_fwd_cfg(out, x, w, n, h, eps, ctypes.byref(c), None)


def pqcall(q=A + 5 * MB, sc=A + 6 * MB, x=A + 2 * MB, w=A + 4 * MB, n=4, h=64, eps=1e-6,
           cfg=None, fp8=False):
    L = arn.lib()
    name = "rmsnorm_quant_fp8_fwd" if fp8 else "rmsnorm_quant_fwd"
    if cfg is None:
        return getattr(L, name)(q, sc, x, w, n, h, eps, None)
    c = arn.LaunchCfg(*cfg)
    return getattr(L, name + "_cfg")(q, sc, x, w, n, h, eps, ctypes.byref(c), None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), arn.EINVAL),
    (dict(h=0), arn.EINVAL),
    (dict(eps=-1.0), arn.EINVAL),
    (dict(h=12, cfg=(arn.PATH_WG_ROW, 0, 0, 0)), arn.EALIGN),
    (dict(h=32776), arn.ERANGE),
    (dict(out=0), arn.EINVAL),
    (dict(x=0), arn.EINVAL),
    (dict(w=0), arn.EINVAL),
    (dict(out=A + 1), arn.EALIGN),
    (dict(out=A + 8, cfg=(arn.PATH_WG_ROW, 0, 0, 0)), arn.EALIGN),
    (dict(out=A + 2 * MB + 16), arn.EALIAS),            # out partly overlaps x
    (dict(out=A + 4 * MB - 16), arn.EALIAS),            # out's tail on the weight
    (dict(n=1 << 62, h=8), arn.ERANGE),
    (dict(cfg=(0, 0, 0, 1)), arn.EINVAL),
    (dict(cfg=(arn.PATH_WAVE_ROW, 0, 0, 0), h=8192), arn.ERANGE),
])
@fake_addresses
def test_plain_argument_errors(kw, status):
    assert pcall(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), arn.EINVAL),
    (dict(h=12), arn.EALIGN),
    (dict(q=0), arn.EINVAL),
    (dict(sc=0), arn.EINVAL),
    (dict(x=0), arn.EINVAL),
    (dict(q=A + 5 * MB + 8), arn.EALIGN),
    (dict(sc=A + 6 * MB + 2), arn.EALIGN),
    (dict(q=A + 2 * MB), arn.EALIAS),                   # codes on x
    (dict(sc=A + 2 * MB + 64), arn.EALIAS),             # scales inside x
    (dict(sc=A + 5 * MB + 16), arn.EALIAS),             # scales inside the codes
    (dict(q=A + 4 * MB - 64), arn.EALIAS),              # codes reach the weight
    (dict(cfg=(arn.PATH_WG_ROW, 64, 0, 0), h=8192), arn.ERANGE),
])
@pytest.mark.parametrize("fp8", [False, True], ids=["int8", "fp8"])
@fake_addresses
def test_plain_quant_argument_errors(kw, status, fp8):
    assert pqcall(fp8=fp8, **kw) == status


@fake_addresses
def test_plain_zero_rows_and_in_place_validation():
    assert pcall(out=0, x=0, w=0, n=0) == arn.OK
    assert pqcall(q=0, sc=0, x=0, w=0, n=0) == arn.OK
    assert pqcall(q=0, sc=0, x=0, w=0, n=0, fp8=True) == arn.OK
    # out == x passes the alias checks; the forced path's ERANGE comes after
    # them, so nothing is launched.
    assert pcall(out=A + 2 * MB, h=8192, cfg=(arn.PATH_WAVE_ROW, 0, 0, 0)) == arn.ERANGE


@fake_addresses
def test_copy2_errors():
    L = arn.lib()
    assert L.add_rmsnorm_test_copy2(A, A + MB, A + 2 * MB, A + 3 * MB, -8, None) == arn.EINVAL
    assert L.add_rmsnorm_test_copy2(A, A + MB, A + 2 * MB, A + 3 * MB, 12, None) == arn.EALIGN
    assert L.add_rmsnorm_test_copy2(A + 2, A + MB, A + 2 * MB, A + 3 * MB, 16, None) == arn.EALIGN
    assert L.add_rmsnorm_test_copy2(0, A + MB, A + 2 * MB, A + 3 * MB, 16, None) == arn.EINVAL
    assert L.add_rmsnorm_test_copy2(A, A + 16, A + 2 * MB, A + 3 * MB, 16, None) == arn.EALIAS
    assert L.add_rmsnorm_test_copy2(A, A + MB, A, A + 3 * MB, 16, None) == arn.EALIAS
    assert L.add_rmsnorm_test_copy2(0, 0, 0, 0, 0, None) == arn.OK


@fake_addresses
def test_copy_rows_errors():
    L = arn.lib()
    c = L.add_rmsnorm_test_copy_rows
    args = (A, A + MB, A + 2 * MB, A + 3 * MB)
    assert c(*args, -1, 1024, 1, None) == arn.EINVAL        # negative rows
    assert c(*args, 4, 0, 1, None) == arn.EINVAL            # hidden <= 0
    assert c(*args, 4, 1024, 3, None) == arn.EINVAL         # rows per burst 1, 2 or 4
    assert c(*args, 4, 1020, 1, None) == arn.EALIGN         # hidden % 8 != 0
    assert c(*args, 4, 16392, 1, None) == arn.ERANGE        # hidden above 16384
    assert c(*args, (1 << 30) + 1, 8, 1, None) == arn.ERANGE
    assert c(A + 2, A + MB, A + 2 * MB, A + 3 * MB, 4, 1024, 1, None) == arn.EALIGN
    assert c(0, A + MB, A + 2 * MB, A + 3 * MB, 4, 1024, 1, None) == arn.EINVAL
    assert c(A, A + 4096, A + 2 * MB, A + 3 * MB, 4, 1024, 1, None) == arn.EALIAS
    assert c(A, A + MB, A + 2 * MB, A + 16, 4, 1024, 2, None) == arn.EALIAS
    assert c(0, 0, 0, 0, 0, 1024, 4, None) == arn.OK        # no rows: nothing checked further


@fake_addresses
def test_stream_hook_errors():
    L = arn.lib()
    assert L.add_rmsnorm_test_stream(A, A + MB, -8, 0, None) == arn.EINVAL
    assert L.add_rmsnorm_test_stream(A, A + MB, 16, 2, None) == arn.EINVAL   # unknown mode
    assert L.add_rmsnorm_test_stream(A, A + MB, 12, 0, None) == arn.EALIGN
    assert L.add_rmsnorm_test_stream(A + 2, A + MB, 16, 0, None) == arn.EALIGN
    assert L.add_rmsnorm_test_stream(A, 0, 16, 0, None) == arn.EINVAL        # read needs src
    assert L.add_rmsnorm_test_stream(A, A + 16, 16, 0, None) == arn.EALIAS
    assert L.add_rmsnorm_test_stream(0, 0, 0, 1, None) == arn.OK


# ---------------------------------------------------------------- binding

def test_binding_refuses_cpu_tensors():
    import torch

    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    w = torch.ones(64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        arn.add_rmsnorm_fwd(torch.empty_like(x), torch.empty_like(x), x, x.clone(), w)


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(arn, "_lib", None)
    monkeypatch.setattr(arn, "LIBRARY", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        arn.lib()


def test_status_codes_match_header():
    hdr = open(os.path.join(ROOT, "include", "add_rmsnorm.h")).read()
    for name in ("OK", "EINVAL", "EALIGN", "EALIAS", "ERANGE", "EHIP"):
        m = re.search(r"#define ADD_RMSNORM_%s \(?(-?\d+)\)?" % name, hdr)
        assert int(m.group(1)) == getattr(arn, name), name
    for name in ("AUTO", "WAVE_ROW", "WG_ROW", "LDS_TWO_PASS"):
        m = re.search(r"#define ADD_RMSNORM_PATH_%s (\d+)" % name, hdr)
        assert int(m.group(1)) == getattr(arn, "PATH_" + name), name


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), arn.EINVAL),
    (dict(out=0), arn.EINVAL),
    (dict(x=0), arn.EINVAL),
    (dict(out=A + 4), arn.EALIGN),
    (dict(x=A + 2 * MB + 8), arn.EALIGN),
    (dict(out=A + 2 * MB + 16), arn.EALIAS),            # out partly overlaps x
    (dict(cfg=(100, 0, 0, 0)), arn.EINVAL),             # workgroup size
    (dict(cfg=(0, 3, 0, 0)), arn.EINVAL),               # elements per thread
    (dict(cfg=(0, 0, -2, 0)), arn.EINVAL),              # grid
    (dict(cfg=(0, 0, 0, 2)), arn.EINVAL),               # unknown flag
    (dict(n=1 << 62), arn.ERANGE),
])
@fake_addresses
def test_log1p_argument_errors(kw, status):
    L = arn.lib()
    out, x, n = kw.get("out", A), kw.get("x", A + 2 * MB), kw.get("n", 64)
    if "cfg" in kw:
        c = arn.Log1pCfg(*kw["cfg"])
        assert L.log1p_f32_cfg(out, x, n, ctypes.byref(c), None) == status
    else:
        assert L.log1p_f32(out, x, n, None) == status


@fake_addresses
def test_log1p_zero_length_is_a_no_op():
    L = arn.lib()
    assert L.log1p_f32(0, 0, 0, None) == arn.OK
    assert L.log1p_f32_cfg(0, 0, 0, None, None) == arn.OK


def test_log1p_binding_refuses_cpu_tensors():
    import torch

    x = torch.zeros(16, dtype=torch.float32)
    with pytest.raises(ValueError):
        arn.log1p_f32(torch.empty_like(x), x)


# ---------------------------------------------------------------- strided views

def scall(out=A, so=None, res=A + MB, sro=None, x=A + 2 * MB, sx=None, r=A + 3 * MB, sr=None,
          w=A + 4 * MB, n=4, h=4104, eps=1e-6, cfg=(1, 0, 0, 0)):
    """add_rmsnorm_fwd_strided with fake addresses.  The default forced path
    (one wavefront per row) cannot take hidden 4104: a call that passes every
    argument and alias check returns ERANGE, or EALIGN when only the general
    kernel could take the layout; nothing is launched."""
    L = arn.lib()
    st = [v if v is not None else h for v in (so, sro, sx, sr)]
    c = arn.LaunchCfg(*cfg)
    return L.add_rmsnorm_fwd_strided(out, st[0], res, st[1], x, st[2], r, st[3], w, n, h, eps,
                                     ctypes.byref(c), None)


PASSED = (arn.ERANGE, arn.EALIGN)


@fake_addresses
def test_strided_argument_errors():
    assert scall(so=4103) == arn.EINVAL                 # stride below hidden
    assert scall(sx=100) == arn.EINVAL
    assert scall(out=A + 1) == arn.EALIGN
    assert scall(n=1 << 40, sx=1 << 30) == arn.ERANGE   # span overflows
    assert scall(out=0) == arn.EINVAL
    assert scall(n=0, out=0, res=0, x=0, r=0, w=0, cfg=(0, 0, 0, 0)) == arn.OK
    L = arn.lib()
    c = arn.LaunchCfg(1, 0, 0, 0)
    assert L.rmsnorm_fwd_strided(A, 4100, A + MB, 4104, A + 4 * MB, 4, 4104, 1e-6,
                                 ctypes.byref(c), None) == arn.EINVAL


@fake_addresses
def test_strided_column_blocks_of_one_matrix():
    h, ld = 4104, 3 * 4104
    # x, residual, out as three interleaved column blocks of one [4, 3h] matrix
    base = A
    assert scall(x=base, sx=ld, r=base + 2 * h, sr=ld, out=base + 4 * h, so=ld) in PASSED
    # out shifted half a row width into x's columns: shares elements
    assert scall(x=base, sx=ld, r=base + 4 * h, sr=ld, out=base + h, so=ld) == arn.EALIAS
    # in place on a strided view
    assert scall(x=base, sx=ld, out=base, so=ld, r=base + 2 * h, sr=ld) in PASSED
    # same base, other stride: not the same view
    assert scall(x=base, sx=ld, out=base, so=ld + 8, r=base + 2 * h, sr=ld) == arn.EALIAS
    # the weight inside the gap between out's rows, then on one of them
    assert scall(out=base, so=ld, w=base + 2 * h + 64) in PASSED
    assert scall(out=base, so=ld, w=base + 2 * ld + 64) == arn.EALIAS


def _bytes_of(base, stride, n, h):
    return {base + 2 * (i * stride) + k for i in range(n) for k in range(2 * h)}


@fake_addresses
def test_strided_alias_check_against_brute_force():
    import random

    rnd = random.Random(5)
    h = 4104
    for _ in range(200):
        n = rnd.choice([1, 2, 3, 5])
        s_out = h + rnd.choice([0, 8, 1000, 4104, 5000])
        s_x = s_out if rnd.random() < 0.7 else h + rnd.choice([0, 16, 3000])
        out = A + 2 * rnd.randrange(0, 4 * h)
        x = A + 2 * rnd.randrange(0, 4 * h)
        got = scall(out=out, so=s_out, x=x, sx=s_x, res=A + 6 * MB, r=A + 8 * MB, n=n)
        shared = bool(_bytes_of(out, s_out, n, h) & _bytes_of(x, s_x, n, h))
        if out == x and s_out == s_x:
            expect_alias = False                              # in place
        elif s_out == s_x:
            expect_alias = shared                             # exact, element by element
        else:
            lo_o, hi_o = out, out + 2 * ((n - 1) * s_out + h)
            lo_x, hi_x = x, x + 2 * ((n - 1) * s_x + h)
            expect_alias = lo_o < hi_x and lo_x < hi_o        # spans
        assert (got == arn.EALIAS) == expect_alias, (n, s_out, s_x, out - A, x - A, got)
        if not expect_alias:
            assert got in PASSED


# ------------------------------------------------------------------ per-head q/k norm

def qkcall(qo=A, ko=A + MB, q=A + 2 * MB, k=A + 3 * MB, qw=A + 4 * MB, kw=A + 5 * MB, t=4,
          hq=4, hk=2, d=520, sq=None, sk=None, sqo=None, sko=None, eps=1e-6, cfg=None):
    """qk_rmsnorm_fwd(_cfg) with fake addresses.  The default head_dim 520 is
    beyond the kernel's 512 and is rejected after every other check, so a
    call that passes them returns ERANGE and launches nothing."""
    L = arn.lib()
    sq = hq * d if sq is None else sq
    sk = hk * d if sk is None else sk
    sqo = hq * d if sqo is None else sqo
    sko = hk * d if sko is None else sko
    args = (qo, ko, q, k, qw, kw, t, hq, hk, d, sq, sk, sqo, sko, eps)
    if cfg is None:
        return L.qk_rmsnorm_fwd(*args, None)
    c = arn.LaunchCfg(*cfg)
    return L.qk_rmsnorm_fwd_cfg(*args, ctypes.byref(c), None)


@pytest.mark.parametrize("kw,status", [
    (dict(), arn.ERANGE),                       # every check passed, head_dim too large
    (dict(t=-1), arn.EINVAL),
    (dict(hq=-1), arn.EINVAL),
    (dict(d=0), arn.EINVAL),
    (dict(eps=math.nan), arn.EINVAL),
    (dict(eps=-1e-6), arn.EINVAL),
    (dict(d=12), arn.EALIGN),
    (dict(d=40000), arn.ERANGE),
    (dict(q=0), arn.EINVAL),
    (dict(ko=0), arn.EINVAL),
    (dict(kw=0), arn.EINVAL),
    (dict(q=A + 2 * MB + 8), arn.EALIGN),
    (dict(kw=A + 5 * MB + 2), arn.EALIGN),
    (dict(sq=4 * 520 - 8), arn.EINVAL),         # token stride below the heads' width
    (dict(sko=2 * 520 + 4), arn.EALIGN),        # stride not on 8 elements
    (dict(cfg=(arn.PATH_WAVE_ROW, 0, 0, 0)), arn.EINVAL),
    (dict(cfg=(arn.PATH_PACKED, 0, 0, 3)), arn.EINVAL),
    (dict(cfg=(arn.PATH_PACKED, 96, 0, 0)), arn.EINVAL),
    (dict(cfg=(arn.PATH_PACKED, 0, -2, 0)), arn.EINVAL),
    (dict(cfg=(arn.PATH_PACKED, 256, -1, 4)), arn.ERANGE),
    (dict(qo=A + 2 * MB + 16), arn.EALIAS),     # q_out partly over q
    (dict(qo=A + 3 * MB), arn.EALIAS),          # q_out on k
    (dict(ko=A + 2 * MB + 1040), arn.EALIAS),   # k_out inside q
    (dict(ko=A + 64), arn.EALIAS),              # k_out over q_out
    (dict(qo=A + 5 * MB - 1040), arn.EALIAS),   # q_out runs over k's weight
    (dict(qo=A + 2 * MB, ko=A + 3 * MB), arn.ERANGE),  # both in place: accepted
    (dict(t=1 << 28, hq=8, hk=0, qo=A, q=A + (1 << 44), qw=A + (1 << 46)),
     arn.ERANGE),                               # 2^31 head rows
])
@fake_addresses
def test_qk_argument_errors(kw, status):
    assert qkcall(**kw) == status


@fake_addresses
def test_qk_no_tokens_or_no_heads_are_no_ops():
    assert qkcall(qo=0, ko=0, q=0, k=0, qw=0, kw=0, t=0, d=128) == arn.OK
    assert qkcall(qo=0, ko=0, q=0, k=0, qw=0, kw=0, hq=0, hk=0, d=128) == arn.OK
    # k absent: its pointers may be NULL, q is still checked
    assert qkcall(ko=0, k=0, kw=0, hk=0) == arn.ERANGE
    assert qkcall(ko=0, k=0, kw=0, hk=0, q=0) == arn.EINVAL


@fake_addresses
def test_qk_fused_qkv_layout_in_place():
    # q, k, v as column blocks of one [t, (hq + 2 hk) d] tensor, normalised in place
    d, hq, hk = 520, 4, 2
    ld = (hq + 2 * hk) * d
    base = A
    kq = base + 2 * hq * d
    assert qkcall(qo=base, q=base, ko=kq, k=kq, sq=ld, sk=ld, sqo=ld, sko=ld) == arn.ERANGE
    # k_out shifted one head left: it covers q's last head
    assert qkcall(qo=base, q=base, ko=kq - 2 * d, k=kq, sq=ld, sk=ld, sqo=ld,
                 sko=ld) == arn.EALIAS
    # q_out a separate contiguous tensor, k in place: accepted
    assert qkcall(qo=A + 8 * MB, q=base, ko=kq, k=kq, sq=ld, sk=ld, sqo=hq * d,
                  sko=ld) == arn.ERANGE
    # q_out on v's columns: as wide as q, so it runs into the next token's q
    assert qkcall(qo=kq + 2 * hk * d, q=base, ko=kq, k=kq, sq=ld, sk=ld, sqo=ld,
                  sko=ld) == arn.EALIAS


@fake_addresses
def test_qk_alias_check_against_brute_force():
    import random

    rnd = random.Random(9)
    d = 520
    for _ in range(300):
        t = rnd.choice([1, 2, 3, 5])
        hq, hk = rnd.choice([1, 2, 3]), rnd.choice([1, 2])
        ld = rnd.choice([(hq + 2 * hk) * d, (hq + hk) * d + 8, 4 * (hq + hk) * d])
        sq = ld
        sk = ld if rnd.random() < 0.8 else ld + 8
        q = A + 16 * rnd.randrange(0, 2 * d)
        k = A + 16 * rnd.randrange(0, 2 * d)
        qo = A + 4 * MB
        ko = A + 6 * MB
        got = qkcall(qo=qo, ko=ko, q=q, k=k, qw=A + 10 * MB, kw=A + 11 * MB, t=t, hq=hq, hk=hk,
                    d=d, sq=sq, sk=sk, sqo=ld, sko=ld)
        # outputs far away; only the inputs may overlap each other, which is allowed
        assert got == arn.ERANGE, (t, hq, hk, ld, sq, sk, q - A, k - A, got)
        # now put k_out on top of q's region
        ko2 = q + 16 * rnd.randrange(-d // 4, d // 2)
        got = qkcall(qo=qo, ko=ko2, q=q, k=k, qw=A + 10 * MB, kw=A + 11 * MB, t=t, hq=hq,
                    hk=hk, d=d, sq=sq, sk=sk, sqo=ld, sko=sk)
        shared = bool(_bytes_of(ko2, sk, t, hk * d) & _bytes_of(q, sq, t, hq * d))
        if not shared and sk == sq:
            shared_k = ko2 == k or bool(_bytes_of(ko2, sk, t, hk * d) & _bytes_of(k, sk, t, hk * d))
            if ko2 == k:
                shared_k = False                        # exactly k's view: in place
            expect = shared_k
        elif sk == sq:
            expect = True
        else:
            lo_a, hi_a = ko2, ko2 + 2 * ((t - 1) * sk + hk * d)
            lo_b, hi_b = q, q + 2 * ((t - 1) * sq + hq * d)
            span = lo_a < hi_b and lo_b < hi_a
            shared_k = ko2 != k and bool(_bytes_of(ko2, sk, t, hk * d) &
                                         _bytes_of(k, sk, t, hk * d))
            expect = span or shared_k
        assert (got == arn.EALIAS) == expect, (t, hq, hk, ld, sq, sk, q - A, k - A, ko2 - A, got)


# ------------------------------------------------------------------ strided quantised views

def sqcall(q=A + 10 * MB, sc=A + 12 * MB, res=A, sro=None, x=A + 2 * MB, sx=None, r=A + 4 * MB,
           sr=None, w=A + 6 * MB, n=4, h=8192, cfg=(1, 0, 0, 0), fp8=False, plain=False):
    """The strided quantised entry points with fake addresses.  The default
    forced path (one wavefront per row) cannot take hidden 8192, so a call
    that passes every check returns ERANGE and launches nothing."""
    L = arn.lib()
    c = arn.LaunchCfg(*cfg)
    sx = h if sx is None else sx
    if plain:
        fn = L.rmsnorm_quant_fp8_fwd_strided if fp8 else L.rmsnorm_quant_fwd_strided
        return fn(q, sc, x, sx, w, n, h, 1e-6, ctypes.byref(c), None)
    sro = h if sro is None else sro
    sr = h if sr is None else sr
    fn = L.add_rmsnorm_quant_fp8_fwd_strided if fp8 else L.add_rmsnorm_quant_fwd_strided
    return fn(q, sc, res, sro, x, sx, r, sr, w, n, h, 1e-6, ctypes.byref(c), None)


@pytest.mark.parametrize("fp8", [False, True], ids=["int8", "fp8"])
@fake_addresses
def test_strided_quant_validation(fp8):
    h = 8192
    assert sqcall(fp8=fp8) == arn.ERANGE                       # every check passed
    assert sqcall(fp8=fp8, sx=h - 8) == arn.EINVAL             # stride below hidden
    assert sqcall(fp8=fp8, sro=h + 4) == arn.EALIGN            # stride off 8 elements
    assert sqcall(fp8=fp8, x=A + 2 * MB + 8) == arn.EALIGN
    assert sqcall(fp8=fp8, n=1 << 40, sx=1 << 30) == arn.ERANGE  # span overflows
    # codes: inside x's first row, then in the gap between x's strided rows
    assert sqcall(fp8=fp8, q=A + 2 * MB + 64) == arn.EALIAS
    assert sqcall(fp8=fp8, sx=3 * h, q=A + 2 * MB + 2 * h) == arn.ERANGE
    assert sqcall(fp8=fp8, sx=3 * h, q=A + 2 * MB + 2 * h + 16) == arn.EALIAS
    # scales on residual_out's last row
    assert sqcall(fp8=fp8, sc=A + 3 * 2 * h + 32) == arn.EALIAS
    # residual_out in place on residual (same view), then the same pointer with another stride
    assert sqcall(fp8=fp8, res=A + 4 * MB) == arn.ERANGE
    assert sqcall(fp8=fp8, res=A + 4 * MB, sro=2 * h) == arn.EALIAS
    # residual_out interleaved with x as column blocks of one matrix: accepted
    assert sqcall(fp8=fp8, x=A + 2 * MB, sx=2 * h, res=A + 2 * MB + 2 * h, sro=2 * h) == arn.ERANGE
    # the plain forms
    assert sqcall(fp8=fp8, plain=True) == arn.ERANGE
    assert sqcall(fp8=fp8, plain=True, sx=h - 8) == arn.EINVAL
    assert sqcall(fp8=fp8, plain=True, q=A + 2 * MB + 3 * 2 * h) == arn.EALIAS
    # zero rows: a no-op whatever the pointers
    assert sqcall(fp8=fp8, n=0, q=0, sc=0, res=0, x=0, r=0, w=0) == arn.OK
