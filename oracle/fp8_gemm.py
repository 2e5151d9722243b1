"""Plain fp64 CPU oracle for D = C + A.B^T with fine-grained FP8 block scaling.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (web pages on DeepGEMM):
  [likun]  likun.im/craft/deepgemm.html, section 一 (the GEMM family and its
           naming convention: D = C + A @ B in the NT layout) and section 二
           (the register_apis listing: the dense call, the M-grouped contiguous
           call taking grouped_layout, the M-grouped masked call taking
           masked_m and expected_m).
  [aitang] aitangshan.cn/news/1491278, "基本使用示例" (the usage example:
           D = C + A @ B.T, A and B passed with their scale factors) and
           "4. FP8 精度优化的核心" (block-wise scaling: the matrices are cut into
           blocks, each with one scale, and each block's GEMM result is
           multiplied by its scales).
  [zwt]    zwt0204.github.io DeepGEMM deep dive, "它的公开接口..." list
           (contiguous and masked grouped GEMM; masked layout for decoding).

What is computed (the plain definition, every step in fp64):

    D[m,n] = RNE_bf16( C[m,n] + sum_kb  sa[kb,m] * sb[n//128,kb]
                                        * sum_{k in kb} dec(A[m,k]) * dec(B[n,k]) )

with kb running over the 128-wide K blocks in ascending order.  The inner
block sum of decoded e4m3 products is exact in fp64 (products carry at most 8
significant bits and are multiples of 2**-18; 128 of them stay far below
2**53 units).  The scale product and the accumulation round only at fp64
precision.  The final rounding goes straight from fp64 to bf16 (never through
fp32) with round-to-nearest, ties to even.

Readings where the pages are silent:
  * e4m3 is the OCP E4M3FN format: bias 7, no infinities, 0x7F/0xFF are NaN,
    largest finite value 448.
  * A scales are 1x128 (one per row per K block), stored K-block-major
    ("MN-major") as sfa[K/128][M]; B scales are 128x128, sfb[ceil(N/128)][K/128].
  * C is bf16 in D's layout, or absent (zero).
  * contiguous form: row m uses expert g = grouped_layout[m]; rows whose id
    lies outside [0, G) are not part of the result (not written).
  * masked form: in group g only the first min(masked_m[g], max_m) rows are
    part of the result; the rest are not written.
"""
from __future__ import annotations

import numpy as np

BLOCK = 128


def _build_e4m3_table() -> np.ndarray:
    """All 256 OCP E4M3FN codes decoded from the format definition.

    code = s eeee mmm; bias 7.  e >= 1: (-1)^s 2^(e-7) (1 + m/8);
    e == 0: (-1)^s 2^-6 (m/8) (subnormal, and +-0); e == 15, m == 7: NaN."""
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = s * (2.0 ** -6) * (m / 8.0)
        else:
            t[code] = s * (2.0 ** (e - 7)) * (1.0 + m / 8.0)
    return t


E4M3_VALUES = _build_e4m3_table()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def round_f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 values straight to bf16 (8 significant bits, exponent range of
    fp32), nearest-even.  Returns the uint16 bit patterns.

    For a finite nonzero x = f * 2**e (0.5 <= |f| < 1) the bf16 grid spacing at
    x is 2**(e-8), but never finer than the smallest subnormal 2**-133.
    x / spacing is exact in fp64; np.rint rounds it to the nearest integer,
    ties to even.  Results beyond the largest finite bf16 become +-inf."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    _, e = np.frexp(np.where(finite, x, 0.0))
    spacing_exp = np.maximum(e - 8, -133)
    q = np.ldexp(np.where(finite, x, 0.0), -spacing_exp)
    r = np.ldexp(np.rint(q), spacing_exp)
    max_bf16 = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > max_bf16, np.copysign(np.inf, r), r)
    out[...] = np.where(finite, r, x)
    # every value in `out` is representable in bf16, hence in fp32 exactly
    bits32 = out.astype(np.float32).view(np.uint32)
    nan = np.isnan(out)
    bits16 = (bits32 >> 16).astype(np.uint16)
    bits16[nan] = np.uint16(0x7FC0)
    return bits16


def _check_dims(a, sfa, b, sfb, M, N, K):
    assert a.shape == (M, K), a.shape
    assert b.shape == (N, K), b.shape
    assert K % BLOCK == 0
    assert sfa.shape == (K // BLOCK, M), sfa.shape
    assert sfb.shape == ((N + BLOCK - 1) // BLOCK, K // BLOCK), sfb.shape


def gemm_nt_acc(a, sfa, b, sfb, c=None, rows=None, cols=None) -> np.ndarray:
    """Unrounded fp64 result C + sum_kb scale * blockGEMM, for the selected rows
    and columns (all by default).  [aitang] section 4: per-block GEMM, then the
    block's result is multiplied by its scale factors; [likun] section 一: D = C + A@B
    in the NT layout (B stored N x K)."""
    M, K = a.shape
    N = b.shape[0]
    _check_dims(a, sfa, b, sfb, M, N, K)
    rows = np.arange(M) if rows is None else np.asarray(rows)
    cols = np.arange(N) if cols is None else np.asarray(cols)
    A = decode_e4m3(a[rows])                       # [R][K] fp64
    B = decode_e4m3(b[cols])                       # [Cn][K] fp64
    sa = sfa[:, rows].astype(np.float64)           # [KB][R]
    sb = sfb[cols // BLOCK, :].astype(np.float64)  # [Cn][KB]
    acc = np.zeros((len(rows), len(cols)), dtype=np.float64)
    for kb in range(K // BLOCK):
        ks = slice(kb * BLOCK, (kb + 1) * BLOCK)
        partial = A[:, ks] @ B[:, ks].T            # exact block sum
        acc += (sa[kb][:, None] * sb[:, kb][None, :]) * partial
    if c is not None:
        acc += bf16_bits_to_f64(np.asarray(c)[np.ix_(rows, cols)])
    return acc


def gemm_nt(a, sfa, b, sfb, c=None, rows=None, cols=None) -> np.ndarray:
    """bf16 bits of D = C + A.B^T (dense fp8_gemm_nt; [likun] sections 一 and 二)."""
    return round_f64_to_bf16_bits(gemm_nt_acc(a, sfa, b, sfb, c, rows, cols))


def gemm_layout(layout, a, sfa, b, sfb, c=None, rows=None, cols=None) -> np.ndarray:
    """bf16 bits of D = C + A.B for the four storage layouts of the dense GEMM
    family ([likun] section 一: fp8_gemm_{nt,nn,tn,tt}).

    layout is two letters: the first gives A's storage ("n": [M][K], "t":
    [K][M]), the second B's ("t": [N][K], "n": [K][N]).  Scales are indexed by
    the logical row, column and K block exactly as in gemm_nt, whatever the
    storage.  Transposing a stored operand only relabels its values, so the
    operands are brought to the NT storage and gemm_nt computes."""
    assert len(layout) == 2 and layout[0] in "nt" and layout[1] in "nt", layout
    a_nt = np.asarray(a) if layout[0] == "n" else np.ascontiguousarray(np.asarray(a).T)
    b_nt = np.asarray(b) if layout[1] == "t" else np.ascontiguousarray(np.asarray(b).T)
    return gemm_nt(a_nt, sfa, b_nt, sfb, c, rows, cols)


def m_grouped_contiguous(a, sfa, b, sfb, grouped_layout, c=None, rows=None, cols=None):
    """M-grouped contiguous form ([likun] section 二, grouped_layout; [zwt] list).

    a [M][K], sfa [KB][M], b [G][N][K], sfb [G][NB][KB], grouped_layout int [M].
    Row m is the dense product of A[m] with expert grouped_layout[m]'s B.
    Returns (bits [R][Cn], written [R]) where written marks rows whose expert
    id is valid; other rows hold 0 and are not part of the result."""
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
        csel = None if c is None else np.asarray(c)[rsel][:, :]
        sub = gemm_nt(a[rsel], sfa[:, rsel], b[g], sfb[g],
                      None if csel is None else csel, None, cols)
        out[sel] = sub
    return out, written


def m_grouped_masked(a, sfa, b, sfb, masked_m, c=None, groups=None, cols=None):
    """M-grouped masked form ([likun] section 二, masked_m / expected_m; [zwt]
    list: masked layout for inference decoding).

    a [G][max_m][K], sfa [G][KB][max_m], b [G][N][K], sfb [G][NB][KB],
    masked_m int [G].  Group g's first min(masked_m[g], max_m) rows are the
    dense product with B[g]; later rows are not part of the result.
    Returns (bits [G'][max_m][Cn], written [G'][max_m]) over the chosen groups."""
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
        out[i, :m] = gemm_nt(a[g][:m], sfa[g][:, :m], b[g], sfb[g], cg, None, cols)
        written[i, :m] = True
    return out, written


def k_grouped_tn_acc(a, sfa, b, sfb, ks, c=None, groups=None):
    """Unrounded fp64 results of the K-grouped TN form and their magnitudes.

    [likun] section 一 lists a GEMM grouped along K ("k_grouped_fp8_gemm_tn",
    for the MoE backward pass) and section 二 its call with per-group K sizes
    (ks) and the (1, 1, 128) scale recipe.  Group g owns the K rows
    k_start[g] .. k_start[g] + ks[g] - 1 of both operands; A is stored [K][M]
    and B [K][N] (the "tn" storage); sfa[kb][m] and sfb[kb][n] scale one
    column of one 128-row K block (1x128 along K for both operands).  Per group:

        D[g][m][n] = C[g][m][n] + sum_kb sfa[kb][m] * sfb[kb][n]
                                  * sum_{k in kb} dec(A[k][m]) * dec(B[k][n])

    over the group's K blocks in ascending order, every step in fp64 (the
    block sums are exact).  Returns (acc [G'][M][N], mag [G'][M][N]) where mag
    is |C| plus the sum of the absolute values of every scaled product, the
    scale against which an fp32 accumulation's rounding error is bounded."""
    K, M = a.shape
    N = b.shape[1]
    ks = np.asarray(ks, dtype=np.int64)
    assert b.shape[0] == K and sfa.shape == (K // BLOCK, M) and sfb.shape == (K // BLOCK, N)
    assert np.all(ks % BLOCK == 0) and int(ks.sum()) == K
    starts = np.concatenate([[0], np.cumsum(ks)])
    groups = np.arange(len(ks)) if groups is None else np.asarray(groups)
    acc = np.zeros((len(groups), M, N), dtype=np.float64)
    mag = np.zeros((len(groups), M, N), dtype=np.float64)
    for i, g in enumerate(groups):
        for kb in range(int(starts[g]) // BLOCK, int(starts[g + 1]) // BLOCK):
            rows = slice(kb * BLOCK, (kb + 1) * BLOCK)
            A = decode_e4m3(a[rows])                         # [128][M]
            B = decode_e4m3(b[rows])                         # [128][N]
            s = sfa[kb].astype(np.float64)[:, None] * sfb[kb].astype(np.float64)[None, :]
            acc[i] += s * (A.T @ B)                          # exact block sum, then scaled
            mag[i] += np.abs(s) * (np.abs(A).T @ np.abs(B))
        if c is not None:
            cg = np.asarray(c)[g].astype(np.float64)
            acc[i] += cg
            mag[i] += np.abs(cg)
    return acc, mag


def k_grouped_tn(a, sfa, b, sfb, ks, c=None, groups=None):
    """fp32 result of the K-grouped TN form (see k_grouped_tn_acc): each fp64
    value rounded once to fp32, to nearest with ties to even."""
    acc, _ = k_grouped_tn_acc(a, sfa, b, sfb, ks, c, groups)
    return acc.astype(np.float32)

