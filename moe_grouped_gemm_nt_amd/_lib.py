"""ctypes binding of libdg.so (the C ABI in include/dg.h).

Argument marshalling only: torch tensors in, device pointers and the current
HIP stream out.  Every step of the computation runs in the library's kernels;
there is no fallback path.  A missing library raises at first use."""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libdg.so")

DG_OK = 0
DG_ERR_INVALID_ARG = -1
DG_ERR_UNSUPPORTED = -2
DG_ERR_HIP = -3

EXPORTED = [
    "dg_fp8_gemm_nt",
    "dg_fp8_gemm_nt_noalloc",
    "dg_fp8_gemm_nn",
    "dg_fp8_gemm_tn",
    "dg_fp8_gemm_tt",
    "dg_fp8_fp4_gemm_nt",
    "dg_m_grouped_fp8_gemm_nt_contiguous",
    "dg_m_grouped_fp8_gemm_nt_masked",
    "dg_m_grouped_fp8_fp4_gemm_nt_contiguous",
    "dg_m_grouped_fp8_fp4_gemm_nt_masked",
    "dg_k_grouped_fp8_gemm_tn_contiguous",
    "dg_choose_config",
    "dg_check_grouped_layout",
    "dg_bind_stream_workspace",
    "dg_init",
    "dg_last_error",
    "dg_version",
]

_lock = threading.Lock()
_lib = None


class DGError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libdg.so once; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m moe_grouped_gemm_nt_amd.build`")
        lib = ctypes.CDLL(path)
        vp, fp, i32p, ci = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
        for name in ("dg_fp8_gemm_nt", "dg_fp8_gemm_nt_noalloc", "dg_fp8_gemm_nn", "dg_fp8_gemm_tn", "dg_fp8_gemm_tt"):
            getattr(lib, name).argtypes = [vp, fp, vp, fp, vp, vp, ci, ci, ci, vp]
            getattr(lib, name).restype = ci
        lib.dg_fp8_fp4_gemm_nt.argtypes = [vp, fp, vp, vp, vp, vp, ci, ci, ci, vp]
        lib.dg_fp8_fp4_gemm_nt.restype = ci
        lib.dg_m_grouped_fp8_gemm_nt_contiguous.argtypes = [vp, fp, vp, fp, vp, vp, ci, ci, ci, ci, i32p, vp]
        lib.dg_m_grouped_fp8_gemm_nt_contiguous.restype = ci
        lib.dg_m_grouped_fp8_gemm_nt_masked.argtypes = [vp, fp, vp, fp, vp, vp, ci, ci, ci, ci, i32p, ci, vp]
        lib.dg_m_grouped_fp8_gemm_nt_masked.restype = ci
        lib.dg_m_grouped_fp8_fp4_gemm_nt_contiguous.argtypes = [vp, fp, vp, vp, vp, vp, ci, ci, ci, ci, i32p, vp]
        lib.dg_m_grouped_fp8_fp4_gemm_nt_contiguous.restype = ci
        lib.dg_m_grouped_fp8_fp4_gemm_nt_masked.argtypes = [vp, fp, vp, vp, vp, vp, ci, ci, ci, ci, i32p, ci, vp]
        lib.dg_m_grouped_fp8_fp4_gemm_nt_masked.restype = ci
        lib.dg_k_grouped_fp8_gemm_tn_contiguous.argtypes = [vp, fp, vp, fp, vp, vp, ci, ci, ci, vp, vp]
        lib.dg_k_grouped_fp8_gemm_tn_contiguous.restype = ci
        lib.dg_choose_config.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci, ctypes.POINTER(ci), ctypes.POINTER(ci)]
        lib.dg_choose_config.restype = ci
        lib.dg_bind_stream_workspace.argtypes = [vp, vp, ctypes.c_size_t]
        lib.dg_bind_stream_workspace.restype = ci
        lib.dg_check_grouped_layout.argtypes = [vp, ci, ci]
        lib.dg_check_grouped_layout.restype = ci
        lib.dg_init.argtypes = []
        lib.dg_init.restype = ci
        lib.dg_last_error.argtypes = []
        lib.dg_last_error.restype = ctypes.c_char_p
        lib.dg_version.argtypes = []
        lib.dg_version.restype = ci
        _lib = lib
        return lib


def _check(fn: str, status: int):
    if status != DG_OK:
        raise DGError(fn, status, (load().dg_last_error() or b"").decode())


_CODE_DTYPES = (torch.uint8, torch.float8_e4m3fn)
_BF16_DTYPES = (torch.bfloat16, torch.int16, torch.uint16)
_F32 = (torch.float32,)
_I32 = (torch.int32,)
_U8 = (torch.uint8,)


def _ptr(t, name, dtypes, shape, allow_none=False):
    """The address of t after checking its dtype, shape and layout: the
    library sees pointers and sizes only, so a tensor of another
    shape would be read or written out of bounds by the kernels.  shape None
    skips the shape check (scales when K is not a multiple of 128, which the
    library rejects itself)."""
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} must not be None")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}; expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _on_device(**tensors):
    """Every tensor must live on the current device: the library runs the
    call there (checked after all shapes, so shape errors name the tensor
    even for host tensors)."""
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor")
        if t.device.index is not None and t.device.index != torch.cuda.current_device():
            raise ValueError(f"{name} is on {t.device}; the call runs on the current device "
                             f"cuda:{torch.cuda.current_device()}")


def _kb(K):
    """K blocks of 128, or None when K is not a multiple of 128 (rejected by the library)."""
    return K // 128 if K % 128 == 0 else None


def _sh(*dims):
    """A shape, or None when one of its sizes is unknown."""
    return None if any(x is None for x in dims) else dims


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def dg_init() -> None:
    _check("dg_init", load().dg_init())


FORMS = {"dense": 0, "contiguous": 1, "masked": 2}
AB_LAYOUTS = {"nt": 0, "tt": 1, "nn": 2, "tn": 3, "fp4": 4}


def dg_choose_config(form, rows, N, K, num_groups=1, num_cus=256, ab_layout="nt", has_c=False):
    """(configuration id, decode K splits) the calls would choose; host-only,
    touches no device.  rows is M, or expected_m for the masked form."""
    cfg, splits = ctypes.c_int(-1), ctypes.c_int(0)
    _check("dg_choose_config", load().dg_choose_config(
        FORMS[form], int(rows), int(N), int(K), int(num_groups), int(num_cus), AB_LAYOUTS[ab_layout],
        1 if has_c else 0, ctypes.byref(cfg), ctypes.byref(splits)))
    return cfg.value, splits.value


def dg_bind_stream_workspace(stream, workspace) -> None:
    """Binds a device tensor (256-byte aligned, at least 256 bytes) as the
    workspace of every later call on `stream`; workspace None removes the binding."""
    if workspace is None:
        ptr, nbytes = None, 0
    else:
        _on_device(workspace=workspace)
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        ptr, nbytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check("dg_bind_stream_workspace", load().dg_bind_stream_workspace(_stream(stream), ptr, nbytes))


def dg_check_grouped_layout(grouped_layout, num_groups) -> None:
    """Host-side check of a contiguous layout (a host int32 array or tensor) against
    the one-expert-per-128-row-block contract; raises DGError naming the first
    offending block."""
    import numpy as np
    h = np.ascontiguousarray(np.asarray(grouped_layout.cpu() if isinstance(grouped_layout, torch.Tensor)
                                        else grouped_layout, dtype=np.int32))
    _check("dg_check_grouped_layout", load().dg_check_grouped_layout(
        h.ctypes.data_as(ctypes.c_void_p), int(h.size), int(num_groups)))


def dg_version() -> int:
    return load().dg_version()


def _dense(fn, a, sfa, b, sfb, c, d, M, N, K, a_shape, b_shape, stream):
    """The dense calls (every operand storage): scales sfa [K/128][M] and
    sfb [ceil(N/128)][K/128], c and d [M][N]."""
    kb, nb = _kb(K), (N + 127) // 128
    args = (_ptr(a, "a", _CODE_DTYPES, a_shape), _ptr(sfa, "sfa", _F32, _sh(kb, M)),
            _ptr(b, "b", _CODE_DTYPES, b_shape), _ptr(sfb, "sfb", _F32, _sh(nb, kb)),
            _ptr(c, "c", _BF16_DTYPES, (M, N), True), _ptr(d, "d", _BF16_DTYPES, (M, N)),
            M, N, K)
    _on_device(a=a, sfa=sfa, b=b, sfb=sfb, c=c, d=d)
    _check(fn, getattr(load(), fn)(*args, _stream(stream)))


def dg_fp8_gemm_nt(a, sfa, b, sfb, c, d, stream=None) -> None:
    """d[M][N] = bf16(c + a[M][K] . b[N][K]^T) with sfa [K/128][M], sfb [ceil(N/128)][K/128]."""
    M, K = a.shape
    N = b.shape[0]
    _dense("dg_fp8_gemm_nt", a, sfa, b, sfb, c, d, M, N, K, (M, K), (N, K), stream)


def dg_fp8_gemm_nt_noalloc(a, sfa, b, sfb, c, d, stream=None) -> None:
    """As dg_fp8_gemm_nt, with the kernels' scratch in the library's fixed
    per-device array: the call allocates no device memory."""
    M, K = a.shape
    N = b.shape[0]
    _dense("dg_fp8_gemm_nt_noalloc", a, sfa, b, sfb, c, d, M, N, K, (M, K), (N, K), stream)


def dg_fp8_gemm_nn(a, sfa, b, sfb, c, d, stream=None) -> None:
    """d[M][N] = bf16(c + a[M][K] . b[K][N]) (B stored K-major), scales as in the NT call."""
    M, K = a.shape
    N = b.shape[1]
    _dense("dg_fp8_gemm_nn", a, sfa, b, sfb, c, d, M, N, K, (M, K), (K, N), stream)


def dg_fp8_gemm_tn(a, sfa, b, sfb, c, d, stream=None) -> None:
    """d[M][N] = bf16(c + a[K][M]^T . b[K][N]) (both operands stored K-major)."""
    K, M = a.shape
    N = b.shape[1]
    _dense("dg_fp8_gemm_tn", a, sfa, b, sfb, c, d, M, N, K, (K, M), (K, N), stream)


def dg_fp8_gemm_tt(a, sfa, b, sfb, c, d, stream=None) -> None:
    """d[M][N] = bf16(c + a[K][M]^T . b[N][K]^T) (A stored K-major)."""
    K, M = a.shape
    N = b.shape[0]
    _dense("dg_fp8_gemm_tt", a, sfa, b, sfb, c, d, M, N, K, (K, M), (N, K), stream)


def dg_fp8_fp4_gemm_nt(a, sfa, b, sfb, c, d, stream=None) -> None:
    """d[M][N] = bf16(c + a[M][K] . dequant(b)^T): b packed E2M1 [N][K/2], sfb int32 [K/128][N]
    (four E8M0 exponents per int, one per 32 K values)."""
    M, K = a.shape
    N = b.shape[0]
    kb = _kb(K)
    args = (_ptr(a, "a", _CODE_DTYPES, (M, K)), _ptr(sfa, "sfa", _F32, _sh(kb, M)),
            _ptr(b, "b", _U8, (N, K // 2)), _ptr(sfb, "sfb", _I32, _sh(kb, N)),
            _ptr(c, "c", _BF16_DTYPES, (M, N), True), _ptr(d, "d", _BF16_DTYPES, (M, N)),
            M, N, K)
    _on_device(a=a, sfa=sfa, b=b, sfb=sfb, c=c, d=d)
    _check("dg_fp8_fp4_gemm_nt", load().dg_fp8_fp4_gemm_nt(*args, _stream(stream)))


def dg_m_grouped_fp8_gemm_nt_contiguous(a, sfa, b, sfb, c, d, grouped_layout, stream=None) -> None:
    """Contiguous M-grouped form: a [M][K], b [G][N][K], sfa [K/128][M],
    sfb [G][ceil(N/128)][K/128], grouped_layout int32 [M]."""
    M, K = a.shape
    G, N, _ = b.shape
    kb = _kb(K)
    args = (_ptr(a, "a", _CODE_DTYPES, (M, K)), _ptr(sfa, "sfa", _F32, _sh(kb, M)),
            _ptr(b, "b", _CODE_DTYPES, (G, N, K)), _ptr(sfb, "sfb", _F32, _sh(G, (N + 127) // 128, kb)),
            _ptr(c, "c", _BF16_DTYPES, (M, N), True), _ptr(d, "d", _BF16_DTYPES, (M, N)), M, N, K, G,
            _ptr(grouped_layout, "grouped_layout", _I32, (M,)))
    _on_device(a=a, sfa=sfa, b=b, sfb=sfb, c=c, d=d, grouped_layout=grouped_layout)
    _check("dg_m_grouped_fp8_gemm_nt_contiguous", load().dg_m_grouped_fp8_gemm_nt_contiguous(*args, _stream(stream)))


def dg_m_grouped_fp8_gemm_nt_masked(a, sfa, b, sfb, c, d, masked_m, expected_m, stream=None) -> None:
    """Masked M-grouped form: a [G][max_m][K], b [G][N][K], sfa [G][K/128][max_m],
    sfb [G][ceil(N/128)][K/128], masked_m int32 [G] on the device."""
    G, max_m, K = a.shape
    N = b.shape[1]
    kb = _kb(K)
    args = (_ptr(a, "a", _CODE_DTYPES, (G, max_m, K)), _ptr(sfa, "sfa", _F32, _sh(G, kb, max_m)),
            _ptr(b, "b", _CODE_DTYPES, (G, N, K)), _ptr(sfb, "sfb", _F32, _sh(G, (N + 127) // 128, kb)),
            _ptr(c, "c", _BF16_DTYPES, (G, max_m, N), True), _ptr(d, "d", _BF16_DTYPES, (G, max_m, N)),
            max_m, N, K, G, _ptr(masked_m, "masked_m", _I32, (G,)), int(expected_m))
    _on_device(a=a, sfa=sfa, b=b, sfb=sfb, c=c, d=d, masked_m=masked_m)
    _check("dg_m_grouped_fp8_gemm_nt_masked", load().dg_m_grouped_fp8_gemm_nt_masked(*args, _stream(stream)))


def dg_k_grouped_fp8_gemm_tn_contiguous(a, sfa, b, sfb, c, d, ks, stream=None) -> None:
    """K-grouped TN form: a [K][M], b [K][N], sfa [K/128][M], sfb [K/128][N], c and d fp32
    [G][M][N]; ks is a host sequence of per-group K sizes (multiples of 128) summing to K."""
    K, M = a.shape
    N = b.shape[1]
    ks = [int(k) for k in ks]
    # sizes that are negative or not multiples of 128 are the library's to reject
    if all(k >= 0 and k % 128 == 0 for k in ks) and sum(ks) != K:
        raise ValueError(f"the group sizes sum to {sum(ks)}; a has K = {K} rows")
    G = len(ks)
    kb = _kb(K)
    ks_host = (ctypes.c_int32 * G)(*ks)
    args = (_ptr(a, "a", _CODE_DTYPES, (K, M)), _ptr(sfa, "sfa", _F32, _sh(kb, M)),
            _ptr(b, "b", _CODE_DTYPES, (K, N)), _ptr(sfb, "sfb", _F32, _sh(kb, N)),
            _ptr(c, "c", _F32, (G, M, N), True), _ptr(d, "d", _F32, (G, M, N)), M, N, G,
            ctypes.cast(ks_host, ctypes.c_void_p))
    _on_device(a=a, sfa=sfa, b=b, sfb=sfb, c=c, d=d)
    _check("dg_k_grouped_fp8_gemm_tn_contiguous", load().dg_k_grouped_fp8_gemm_tn_contiguous(*args, _stream(stream)))


def dg_m_grouped_fp8_fp4_gemm_nt_contiguous(a, sfa, b, sfb, c, d, grouped_layout, stream=None) -> None:
    """Contiguous M-grouped FP8 x FP4 form: a [M][K], b packed [G][N][K/2], sfb int32 [G][K/128][N]."""
    M, K = a.shape
    G, N, _ = b.shape
    kb = _kb(K)
    args = (_ptr(a, "a", _CODE_DTYPES, (M, K)), _ptr(sfa, "sfa", _F32, _sh(kb, M)),
            _ptr(b, "b", _U8, (G, N, K // 2)), _ptr(sfb, "sfb", _I32, _sh(G, kb, N)),
            _ptr(c, "c", _BF16_DTYPES, (M, N), True), _ptr(d, "d", _BF16_DTYPES, (M, N)), M, N, K, G,
            _ptr(grouped_layout, "grouped_layout", _I32, (M,)))
    _on_device(a=a, sfa=sfa, b=b, sfb=sfb, c=c, d=d, grouped_layout=grouped_layout)
    _check("dg_m_grouped_fp8_fp4_gemm_nt_contiguous", load().dg_m_grouped_fp8_fp4_gemm_nt_contiguous(*args, _stream(stream)))


def dg_m_grouped_fp8_fp4_gemm_nt_masked(a, sfa, b, sfb, c, d, masked_m, expected_m, stream=None) -> None:
    """Masked M-grouped FP8 x FP4 form: a [G][max_m][K], b packed [G][N][K/2], sfb int32 [G][K/128][N]."""
    G, max_m, K = a.shape
    N = b.shape[1]
    kb = _kb(K)
    args = (_ptr(a, "a", _CODE_DTYPES, (G, max_m, K)), _ptr(sfa, "sfa", _F32, _sh(G, kb, max_m)),
            _ptr(b, "b", _U8, (G, N, K // 2)), _ptr(sfb, "sfb", _I32, _sh(G, kb, N)),
            _ptr(c, "c", _BF16_DTYPES, (G, max_m, N), True), _ptr(d, "d", _BF16_DTYPES, (G, max_m, N)),
            max_m, N, K, G, _ptr(masked_m, "masked_m", _I32, (G,)), int(expected_m))
    _on_device(a=a, sfa=sfa, b=b, sfb=sfb, c=c, d=d, masked_m=masked_m)
    _check("dg_m_grouped_fp8_fp4_gemm_nt_masked", load().dg_m_grouped_fp8_fp4_gemm_nt_masked(*args, _stream(stream)))
