"""Plain fp64 CPU oracle for the FP8 x FP4 dense GEMM (NT).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: [likun] likun.im/craft/deepgemm.html, section 一 (the GEMM family
"fp8_fp4_gemm_{nt,nn,tn,tt}", D = C + A @ B in the NT layout) and section 五
(scale factors for the newer architecture are packed UE8M0, four to an int);
[lqnn] lqnn.cn/news/208760 (the 2026-04 release adds an FP8 x FP4 GEMM);
[zwt] zwt0204.github.io DeepGEMM deep dive (FP4 among the GEMM precisions).

What is computed (every step in fp64):

    D[m,n] = RNE_bf16( C[m,n] + sum_kb sa[kb,m]
                       * sum_{k in kb} dec8(A[m,k]) * dec4(B[n,k]) * 2**(e[n, k//32] - 127) )

Readings where the pages are silent:
  * FP4 is OCP E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; no
    infinities or NaN; magnitudes 0, 1/2, 1, 3/2, 2, 3, 4, 6.
  * B holds two codes per byte, element 2i in the low nibble, K contiguous:
    b [N][K/2].
  * B's scales are E8M0 (2**(byte - 127)), one per row per 32 K values, packed
    four to an int32 in K order: sfb [K/128][N], byte j of sfb[kb][n] scaling
    K values 128*kb + 32*j .. +31 of row n.
  * A is e4m3 with 1x128 fp32 scales sfa [K/128][M], exactly as in the FP8 GEMM.
"""
from __future__ import annotations

import numpy as np

from .fp8_gemm import BLOCK, bf16_bits_to_f64, decode_e4m3, round_f64_to_bf16_bits


def _build_e2m1_table() -> np.ndarray:
    """The 16 E2M1 codes decoded from the format's bit fields."""
    t = np.zeros(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 8 else 1.0
        e = (code >> 1) & 3
        m = code & 1
        mag = (m / 2.0) if e == 0 else (2.0 ** (e - 1)) * (1.0 + m / 2.0)
        t[code] = sign * mag
    return t


E2M1_VALUES = _build_e2m1_table()


def decode_e2m1_packed(b: np.ndarray) -> np.ndarray:
    """Packed codes [N][K/2] -> fp64 values [N][K] (low nibble = even element)."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty((b.shape[0], b.shape[1] * 2), dtype=np.float64)
    out[:, 0::2] = E2M1_VALUES[b & 0xF]
    out[:, 1::2] = E2M1_VALUES[b >> 4]
    return out


def e8m0_scales(sfb: np.ndarray, N: int, K: int) -> np.ndarray:
    """Packed E8M0 int32 [K/128][N] -> fp64 scales [N][K/32]."""
    q = np.asarray(sfb).view(np.uint32)
    assert q.shape == (K // BLOCK, N), q.shape
    e = np.empty((N, K // 32), dtype=np.int64)
    for j in range(4):
        e[:, j::4] = ((q >> (8 * j)) & 0xFF).T.astype(np.int64)
    return np.ldexp(1.0, e - 127)


def gemm_fp8_fp4_nt_acc(a, sfa, b, sfb, c=None, rows=None, cols=None) -> np.ndarray:
    """Unrounded fp64 result for the selected rows and columns."""
    M, K = a.shape
    N = b.shape[0]
    assert b.shape == (N, K // 2) and K % BLOCK == 0 and sfa.shape == (K // BLOCK, M)
    rows = np.arange(M) if rows is None else np.asarray(rows)
    cols = np.arange(N) if cols is None else np.asarray(cols)
    A = decode_e4m3(a[rows])                                      # [R][K]
    scale_b = e8m0_scales(sfb, N, K)[cols]                        # [Cn][K/32]
    B = decode_e2m1_packed(b[cols]) * np.repeat(scale_b, 32, axis=1)   # scaled B [Cn][K]
    sa = sfa[:, rows].astype(np.float64)                          # [KB][R]
    acc = np.zeros((len(rows), len(cols)), dtype=np.float64)
    for kb in range(K // BLOCK):
        ks = slice(kb * BLOCK, (kb + 1) * BLOCK)
        acc += sa[kb][:, None] * (A[:, ks] @ B[:, ks].T)
    if c is not None:
        acc += bf16_bits_to_f64(np.asarray(c)[np.ix_(rows, cols)])
    return acc


def gemm_fp8_fp4_nt(a, sfa, b, sfb, c=None, rows=None, cols=None) -> np.ndarray:
    """bf16 bits of D (see the module docstring)."""
    return round_f64_to_bf16_bits(gemm_fp8_fp4_nt_acc(a, sfa, b, sfb, c, rows, cols))


def m_grouped_fp8_fp4_contiguous(a, sfa, b, sfb, grouped_layout, c=None, rows=None, cols=None):
    """M-grouped contiguous FP8 x FP4 form ([likun] section 二 lists
    "m_grouped_fp8_fp4_gemm_nt_contiguous" with grouped_layout): row m is the
    dense FP8 x FP4 product of A[m] with expert grouped_layout[m]'s B (packed
    [G][N][K/2]) and scales (sfb [G][K/128][N]); rows whose id lies outside
    [0, G) are not part of the result.  Returns (bits [R][Cn], written [R])."""
    M, K = a.shape
    G, N, _ = b.shape
    layout = np.asarray(grouped_layout)
    rows = np.arange(M) if rows is None else np.asarray(rows)
    cols = np.arange(N) if cols is None else np.asarray(cols)
    out = np.zeros((len(rows), len(cols)), dtype=np.uint16)
    ids = layout[rows]
    written = (ids >= 0) & (ids < G)
    for g in np.unique(ids[written]):
        sel = np.nonzero(ids == g)[0]
        rsel = rows[sel]
        cg = None if c is None else np.asarray(c)[rsel]
        out[sel] = gemm_fp8_fp4_nt(a[rsel], sfa[:, rsel], b[g], sfb[g], cg, None, cols)
    return out, written


def m_grouped_fp8_fp4_masked(a, sfa, b, sfb, masked_m, c=None, groups=None, cols=None):
    """M-grouped masked FP8 x FP4 form ([likun] section 二,
    "m_grouped_fp8_fp4_gemm_nt_masked"): group g's first min(masked_m[g], max_m)
    rows are the dense FP8 x FP4 product with B[g]; later rows are not part of
    the result.  Returns (bits [G'][max_m][Cn], written [G'][max_m])."""
    G, max_m, K = a.shape
    N = b.shape[1]
    groups = np.arange(G) if groups is None else np.asarray(groups)
    cols = np.arange(N) if cols is None else np.asarray(cols)
    out = np.zeros((len(groups), max_m, len(cols)), dtype=np.uint16)
    written = np.zeros((len(groups), max_m), dtype=bool)
    for i, g in enumerate(groups):
        m = int(min(max(int(masked_m[g]), 0), max_m))
        if m == 0:
            continue
        cg = None if c is None else np.asarray(c)[g][:m]
        out[i, :m] = gemm_fp8_fp4_nt(a[g][:m], sfa[g][:, :m], b[g], sfb[g], cg, None, cols)
        written[i, :m] = True
    return out, written
