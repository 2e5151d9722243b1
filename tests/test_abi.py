"""The C ABI library, without a GPU: it loads, exports every symbol that
include/dg.h declares, and rejects invalid arguments on the host before any
HIP call."""
import ctypes
import os
import re
import subprocess

import numpy as np
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


def _dense(lib, a=FAKE, sfa=FAKE, b=FAKE, sfb=FAKE, c=None, d=FAKE, M=64, N=64, K=128, fn="dg_fp8_gemm_nt"):
    return getattr(lib, fn)(a, sfa, b, sfb, c, d, M, N, K, None)


@pytest.mark.parametrize("kw,needle", [
    (dict(a=None), "NULL"),
    (dict(d=None), "NULL"),
    (dict(K=100), "multiple of 128"),
    (dict(M=-1), "negative"),
    (dict(a=ctypes.c_void_p(0x100001)), "16-byte"),
    (dict(sfb=ctypes.c_void_p(0x100002)), "4-byte"),
    (dict(d=ctypes.c_void_p(0x100001)), "2-byte"),
])
@pytest.mark.parametrize("fn", ["dg_fp8_gemm_nt", "dg_fp8_gemm_nt_noalloc"])
def test_dense_rejects_invalid_arguments(lib, kw, needle, fn):
    assert _dense(lib, fn=fn, **kw) == _lib.DG_ERR_INVALID_ARG
    assert needle in lib.dg_last_error().decode()


@pytest.mark.parametrize("fn", ["dg_fp8_gemm_nt", "dg_fp8_gemm_nt_noalloc"])
def test_dense_empty_is_noop(lib, fn):
    assert _dense(lib, M=0, fn=fn) == _lib.DG_OK
    assert _dense(lib, N=0, fn=fn) == _lib.DG_OK


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


def test_python_binding_checks_shapes():
    # the library sees pointers and sizes only, so the binding checks every
    # tensor's shape against the sizes it passes (before the device check:
    # host tensors reach the shape check)
    import torch
    u8 = torch.uint8
    a, b = torch.zeros(64, 256, dtype=u8), torch.zeros(300, 256, dtype=u8)
    d = torch.zeros(64, 300, dtype=torch.bfloat16)
    sfa, sfb = torch.ones(2, 64), torch.ones(3, 2)
    bad = {
        "sfa": (a, torch.ones(64, 2), b, sfb, None, d),          # [M][K/128] instead of [K/128][M]
        "sfb": (a, sfa, b, torch.ones(2, 3), None, d),
        "d": (a, sfa, b, sfb, None, torch.zeros(300, 64, dtype=torch.bfloat16)),
        "c": (a, sfa, b, sfb, torch.zeros(64, 299, dtype=torch.bfloat16), d),
    }
    for name, args in bad.items():
        with pytest.raises(ValueError, match=f"^{name} has shape"):
            dgpkg.dg_fp8_gemm_nt(*args)
    with pytest.raises(ValueError, match="device tensor"):
        dgpkg.dg_fp8_gemm_nt(a, sfa, b, sfb, None, d)           # shapes right, host memory
    with pytest.raises(ValueError, match="^b has shape"):      # nn: B stored [K][N]
        dgpkg.dg_fp8_gemm_nn(a, sfa, torch.zeros(255, 300, dtype=u8), sfb, None, d)
    ga = torch.zeros(4, 32, 256, dtype=u8)
    gb = torch.zeros(4, 300, 256, dtype=u8)
    with pytest.raises(ValueError, match="^sfa has shape"):   # masked A scales [G][K/128][max_m]
        dgpkg.dg_m_grouped_fp8_gemm_nt_masked(ga, torch.ones(2, 4, 32), gb, torch.ones(4, 3, 2), None,
                                              torch.zeros(4, 32, 300, dtype=torch.bfloat16),
                                              torch.zeros(4, dtype=torch.int32), 16)
    with pytest.raises(ValueError, match="^grouped_layout has shape"):
        dgpkg.dg_m_grouped_fp8_gemm_nt_contiguous(a, sfa, gb, torch.ones(4, 3, 2), None, d,
                                                  torch.zeros(63, dtype=torch.int32))
    with pytest.raises(ValueError, match="^b has shape"):      # FP4: two codes per byte
        dgpkg.dg_fp8_fp4_gemm_nt(a, sfa, b, torch.zeros(2, 300, dtype=torch.int32), None, d)
    ka, kbm = torch.zeros(384, 64, dtype=u8), torch.zeros(384, 48, dtype=u8)
    with pytest.raises(ValueError, match="sum to 256"):
        dgpkg.dg_k_grouped_fp8_gemm_tn_contiguous(ka, torch.ones(3, 64), kbm, torch.ones(3, 48), None,
                                                  torch.zeros(2, 64, 48), [128, 128])


def test_ceilings_library_exports_every_declared_symbol():
    # the microbenchmarks of include/dg_ceilings.h live in their own library
    from moe_grouped_gemm_nt_amd import build, ceilings
    if not os.path.exists(ceilings.CEILINGS_PATH):
        build.build_ceilings()
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "dg_ceilings.h")).read(), flags=re.S)
    syms = sorted(set(re.findall(r"\b(dgc_[a-z0-9_]+)\s*\(", text)))
    assert syms == ["dgc_chase", "dgc_empty", "dgc_fill", "dgc_mfma", "dgc_stream"]
    out = subprocess.run(["nm", "-D", "--defined-only", ceilings.CEILINGS_PATH], capture_output=True, text=True).stdout
    assert set(syms) <= set(re.findall(r" T (dgc_[a-z0-9_]+)", out))
    lib = ceilings.load()
    # invalid arguments are refused on the host, before any HIP call
    assert lib.dgc_stream(None, 4096, 1, 0, None, None) == -1
    assert lib.dgc_stream(ctypes.c_void_p(0x1000), 1000, 1, 0, ctypes.c_void_p(0x1000), None) == -1
    assert lib.dgc_empty(0, None) == -1
    assert lib.dgc_mfma(0, 1, 0, ctypes.c_void_p(0x1000), None) == -1
    assert lib.dgc_chase(ctypes.c_void_p(0x1000), 10, 3, ctypes.c_void_p(0x1000), None) == -1
    assert lib.dgc_chase(None, 10, 0, ctypes.c_void_p(0x1000), None) == -1
    assert lib.dgc_fill(ctypes.c_void_p(0x1000), 65536, 2, 8, ctypes.c_void_p(0x1000), None) == -1   # steps overflow
    assert lib.dgc_fill(ctypes.c_void_p(0x1000), 65536, 1, 3, ctypes.c_void_p(0x1000), None) == -1   # share must divide 32


def test_layout_check_on_host(lib):
    ok = np.array([0] * 128 + [1] * 100 + [-1] * 28 + [7] * 20, dtype=np.int32)
    dgpkg.dg_check_grouped_layout(ok, 2)                  # ids >= G count as padding
    bad = np.array([0] * 100 + [1] * 28 + [1] * 10, dtype=np.int32)
    with pytest.raises(dgpkg.DGError) as e:
        dgpkg.dg_check_grouped_layout(bad, 2)
    assert e.value.status == _lib.DG_ERR_INVALID_ARG and "rows 0..127" in str(e.value)
    tail = np.array([3] * 128 + [3] * 5 + [0] * 2, dtype=np.int32)   # the ragged last block
    with pytest.raises(dgpkg.DGError) as e:
        dgpkg.dg_check_grouped_layout(tail, 4)
    assert "rows 128..134" in str(e.value)


def test_stream_workspace_binding_rejects_bad_buffers(lib):
    lib.dg_bind_stream_workspace.restype = ctypes.c_int
    assert lib.dg_bind_stream_workspace(None, ctypes.c_void_p(0x100010), ctypes.c_size_t(1 << 20)) == _lib.DG_ERR_INVALID_ARG
    assert "256-byte" in lib.dg_last_error().decode()
    assert lib.dg_bind_stream_workspace(None, ctypes.c_void_p(0x100000), ctypes.c_size_t(128)) == _lib.DG_ERR_INVALID_ARG
    assert "smaller" in lib.dg_last_error().decode()
