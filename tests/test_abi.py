"""The C ABI library, without a GPU: it loads, exports every symbol that
include/dg.h declares, and rejects invalid arguments on the host before any
HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

import moe_grouped_gemm_nt_amd as dgpkg
from moe_grouped_gemm_nt_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from moe_grouped_gemm_nt_amd import build
        build.build()
    return _lib.load()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_entry_points():
    syms = declared_symbols()
    for s in ["dg_fp8_gemm_nt", "dg_m_grouped_fp8_gemm_nt_contiguous", "dg_m_grouped_fp8_gemm_nt_masked"]:
        assert s in syms


def test_library_exports_every_declared_symbol(lib):
    for s in declared_symbols():
        assert hasattr(lib, s), s
    assert sorted(_lib.EXPORTED) == declared_symbols()
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (dg_[a-z0-9_]+)", out))
    assert set(declared_symbols()) <= exported


def test_version(lib):
    assert lib.dg_version() >= 100


FAKE = ctypes.c_void_p(0x100000)          # aligned, never dereferenced: validation fails first


def _dense(lib, a=FAKE, sfa=FAKE, b=FAKE, sfb=FAKE, c=None, d=FAKE, M=64, N=64, K=128):
    return lib.dg_fp8_gemm_nt(a, sfa, b, sfb, c, d, M, N, K, None)


@pytest.mark.parametrize("kw,needle", [
    (dict(a=None), "NULL"),
    (dict(d=None), "NULL"),
    (dict(K=100), "multiple of 128"),
    (dict(M=-1), "negative"),
    (dict(a=ctypes.c_void_p(0x100001)), "16-byte"),
    (dict(sfb=ctypes.c_void_p(0x100002)), "4-byte"),
    (dict(d=ctypes.c_void_p(0x100001)), "2-byte"),
])
def test_dense_rejects_invalid_arguments(lib, kw, needle):
    assert _dense(lib, **kw) == _lib.DG_ERR_INVALID_ARG
    assert needle in lib.dg_last_error().decode()


def test_dense_empty_is_noop(lib):
    assert _dense(lib, M=0) == _lib.DG_OK
    assert _dense(lib, N=0) == _lib.DG_OK


def test_grouped_reject_invalid_arguments(lib):
    f = lib.dg_m_grouped_fp8_gemm_nt_contiguous
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, 128, 64, 128, 0, FAKE, None) == _lib.DG_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, 128, 64, 128, 2, None, None) == _lib.DG_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, 64, 128, 2, FAKE, None) == _lib.DG_OK
    g = lib.dg_m_grouped_fp8_gemm_nt_masked
    assert g(FAKE, FAKE, FAKE, FAKE, None, FAKE, 256, 64, 128, 4, None, 128, None) == _lib.DG_ERR_INVALID_ARG
    assert g(FAKE, FAKE, FAKE, FAKE, None, FAKE, 256, 64, 128, 4, FAKE, -1, None) == _lib.DG_ERR_INVALID_ARG
    assert g(FAKE, FAKE, FAKE, FAKE, None, FAKE, 256, 64, 128, 4096, FAKE, 1, None) == _lib.DG_ERR_UNSUPPORTED
    assert g(FAKE, FAKE, FAKE, FAKE, None, FAKE, 256, 64, 129, 4, FAKE, 1, None) == _lib.DG_ERR_INVALID_ARG
    assert g(FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, 64, 128, 4, FAKE, 1, None) == _lib.DG_OK


def test_python_binding_rejects_host_tensors(lib):
    import torch
    a = torch.zeros(4, 128, dtype=torch.uint8)
    with pytest.raises(ValueError):
        dgpkg.dg_fp8_gemm_nt(a, torch.ones(1, 4), a, torch.ones(1, 1), None, torch.zeros(4, 4, dtype=torch.bfloat16))


def test_no_oracle_in_product_package():
    pkg = os.path.join(ROOT, "moe_grouped_gemm_nt_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
                assert "inputgen" not in src, f
