"""The host side of the library (argument validation, the configuration
chooser, the layout check) built with AddressSanitizer and
UndefinedBehaviorSanitizer on the host code only, and driven through the C ABI
on every entry point's host-side paths in a subprocess that preloads the ASan
runtime.  No GPU: every call here returns before any HIP call."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "moe_grouped_gemm_nt_amd")


def _hipcc():
    import shutil
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    from moe_grouped_gemm_nt_amd import build
    objdir = os.path.join(PKG, "_build")
    kernels = [os.path.join(objdir, f) for f in ("fp8_gemm.o", "fp8_gemm_e8m0.o")]
    if not all(os.path.exists(k) for k in kernels):
        build.build()
    out = tmp_path_factory.mktemp("asan")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    obj = str(out / "dg_api_san.o")
    lib = str(out / "libdg_san.so")
    flags = [f for f in build.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"]
    r = subprocess.run([_hipcc()] + flags + san + ["-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(PKG, "csrc", "dg_api.hip"), "-o", obj], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + san + [obj] + kernels + ["-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    rt = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    assert os.path.exists(rt), rt
    return lib, rt


DRIVER = textwrap.dedent(r"""
    import ctypes, sys
    lib = ctypes.CDLL(sys.argv[1])
    lib.dg_last_error.restype = ctypes.c_char_p
    vp, ci = ctypes.c_void_p, ctypes.c_int
    F = vp(0x100000)                     # aligned, never dereferenced: validation fails first
    bad = {"a16": vp(0x100001), "a4": vp(0x100002), "a2": vp(0x100001)}
    calls = 0

    def expect(rc, want, what):
        global calls
        calls += 1
        assert rc == want, (what, rc, lib.dg_last_error())

    dense = ["dg_fp8_gemm_nt", "dg_fp8_gemm_nt_noalloc", "dg_fp8_gemm_nn", "dg_fp8_gemm_tn", "dg_fp8_gemm_tt",
             "dg_fp8_fp4_gemm_nt"]
    for name in dense:
        f = getattr(lib, name)
        f.restype = ci
        for args, want in [((None, F, F, F, None, F, 64, 64, 128), -1), ((F, F, F, F, None, None, 64, 64, 128), -1),
                           ((F, F, F, F, None, F, 64, 64, 100), -1), ((F, F, F, F, None, F, -1, 64, 128), -1),
                           ((F, F, F, F, None, F, 64, -5, 128), -1), ((bad["a16"], F, F, F, None, F, 64, 64, 128), -1),
                           ((F, bad["a4"], F, F, None, F, 64, 64, 128), -1), ((F, F, F, F, bad["a2"], F, 64, 64, 128), -1),
                           ((F, F, F, F, None, F, 0, 64, 128), 0), ((F, F, F, F, None, F, 64, 0, 128), 0)]:
            expect(f(*args, None), want, (name, args))
    for name in ("dg_m_grouped_fp8_gemm_nt_contiguous", "dg_m_grouped_fp8_fp4_gemm_nt_contiguous"):
        f = getattr(lib, name)
        f.restype = ci
        expect(f(F, F, F, F, None, F, 128, 64, 128, 0, F, None), -1, name)
        expect(f(F, F, F, F, None, F, 128, 64, 128, 2, None, None), -1, name)
        expect(f(F, F, F, F, None, F, 128, 64, 128, 2, bad["a2"], None), -1, name)
        expect(f(F, F, F, F, None, F, 0, 64, 128, 2, F, None), 0, name)
    for name in ("dg_m_grouped_fp8_gemm_nt_masked", "dg_m_grouped_fp8_fp4_gemm_nt_masked"):
        f = getattr(lib, name)
        f.restype = ci
        expect(f(F, F, F, F, None, F, 128, 64, 128, 0, F, 64, None), -1, name)
        expect(f(F, F, F, F, None, F, 128, 64, 128, 4096, F, 64, None), -2, name)
        expect(f(F, F, F, F, None, F, 128, 64, 128, 2, None, 64, None), -1, name)
        expect(f(F, F, F, F, None, F, 128, 64, 128, 2, F, -1, None), -1, name)
        expect(f(F, F, F, F, None, F, 0, 64, 128, 2, F, 64, None), 0, name)
    kg = lib.dg_k_grouped_fp8_gemm_tn_contiguous
    kg.restype = ci
    ks = (ctypes.c_int32 * 3)(128, 0, 256)
    badks = (ctypes.c_int32 * 3)(128, 100, 256)
    negks = (ctypes.c_int32 * 3)(128, -128, 256)
    expect(kg(F, F, F, F, None, F, 64, 64, 3, badks, None), -1, "ks not a multiple of 128")
    expect(kg(F, F, F, F, None, F, 64, 64, 3, negks, None), -1, "negative ks")
    expect(kg(F, F, F, F, None, F, 64, 64, 0, ks, None), -1, "no groups")
    expect(kg(F, F, F, F, None, F, 64, 64, 300, ks, None), -2, "too many groups")
    expect(kg(F, F, F, F, None, F, 60, 64, 3, ks, None), -2, "M not a multiple of 16")
    expect(kg(F, F, F, F, None, F, 0, 64, 3, ks, None), 0, "empty")
    # the chooser over a grid of shapes, including extreme sizes
    ch = lib.dg_choose_config
    ch.restype = ci
    cfg, spl = ci(), ci()
    for form in (0, 1, 2):
        for rows in (1, 16, 64, 100, 128, 1000, 4096, 65536, 2**30):
            for N in (1, 64, 2112, 7168, 2**30):
                for K in (0, 128, 7168, 16384, 2**30):
                    for lay in range(5):
                        for has_c in (0, 1):
                            expect(ch(form, rows, N, K, 8, 256, lay, has_c, ctypes.byref(cfg), ctypes.byref(spl)), 0,
                                   (form, rows, N, K))
                            assert 0 <= cfg.value < 13 and spl.value >= 1
    expect(ch(3, 8, 8, 128, 1, 256, 0, 0, ctypes.byref(cfg), ctypes.byref(spl)), -1, "bad form")
    expect(ch(0, 8, 8, 128, 1, 256, 0, 0, None, ctypes.byref(spl)), -1, "null out")
    # the layout check
    chk = lib.dg_check_grouped_layout
    chk.restype = ci
    good = (ctypes.c_int32 * 300)(*([0] * 128 + [1] * 100 + [-1] * 28 + [5] * 44))
    expect(chk(good, 300, 2), 0, "valid layout (ids >= G are padding)")
    mixed = (ctypes.c_int32 * 256)(*([0] * 100 + [1] * 156))
    expect(chk(mixed, 256, 2), -1, "two experts in one block")
    assert b"rows 0..127" in lib.dg_last_error()
    expect(chk(None, 10, 2), -1, "null layout")
    expect(chk(None, 0, 2), 0, "empty layout")
    bind = lib.dg_bind_stream_workspace
    bind.restype = ci
    bind.argtypes = [vp, vp, ctypes.c_size_t]
    expect(bind(None, vp(0x100010), 1 << 20), -1, "misaligned workspace")
    expect(bind(None, F, 100), -1, "workspace too small")
    print(f"SANITIZED_OK {calls}")
""")


def test_host_code_under_address_and_undefined_behaviour_sanitizers(sanitized_lib, tmp_path):
    lib, rt = sanitized_lib
    # the host code is instrumented by both sanitizers
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms
    script = tmp_path / "drive.py"
    script.write_text(DRIVER)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, str(script), lib], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "SANITIZED_OK" in r.stdout, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
