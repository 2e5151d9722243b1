"""Pins of the CPU oracle against facts fixed outside it: the e4m3 and bf16
formats (library special cases), exact rational arithmetic on tiny inputs,
closed forms in the exact regime, and invariants of block scaling.

The pages print no worked numeric example for this GEMM, so every pin here is
mathematical or a library special case."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import inputgen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# exact-rational helpers written independently of the oracle
# ----------------------------------------------------------------------------
def frac_e4m3(code: int) -> Fraction:
    """e4m3 value as an exact rational, computed from the bit fields."""
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 64)
    return s * (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))


def frac_rne_bf16_bits(x: Fraction) -> int:
    """Exact round-to-nearest-even of a rational to bf16, as bit pattern."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    ax = -x if x < 0 else x
    e = ax.numerator.bit_length() - ax.denominator.bit_length()
    # adjust so that 2**e <= ax < 2**(e+1)
    while Fraction(2) ** e > ax:
        e -= 1
    while Fraction(2) ** (e + 1) <= ax:
        e += 1
    spacing_exp = max(e - 7, -133)
    q = ax / (Fraction(2) ** spacing_exp)
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = Fraction(fl) * (Fraction(2) ** spacing_exp)
    f32 = np.array([float(val)], dtype=np.float32)
    assert Fraction(float(f32[0])) == val
    return sign | int(f32.view(np.uint32)[0] >> 16)


def frac_rne_f32(x: Fraction) -> np.float32:
    """Exact round-to-nearest-even of a rational to fp32 (normal range)."""
    if x == 0:
        return np.float32(0.0)
    ax = -x if x < 0 else x
    e = ax.numerator.bit_length() - ax.denominator.bit_length()
    while Fraction(2) ** e > ax:
        e -= 1
    while Fraction(2) ** (e + 1) <= ax:
        e += 1
    spacing_exp = max(e - 23, -149)
    q = ax / (Fraction(2) ** spacing_exp)
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = Fraction(fl) * (Fraction(2) ** spacing_exp)
    out = np.float32(float(val))            # val has <= 24 significant bits: exact
    assert Fraction(float(out)) == val
    return -out if x < 0 else out


def frac_f32(v) -> Fraction:
    return Fraction(float(np.float32(v)))


def frac_bf16(bits: int) -> Fraction:
    return Fraction(float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]))


def brute_force_bits(a, sfa, b, sfb, c, rows, cols):
    """D[m,n] from the definition with exact rationals: scale each decoded
    element by its own block scale, sum over all of K, add C, round once."""
    K = a.shape[1]
    out = np.zeros((len(rows), len(cols)), dtype=np.uint16)
    for i, m in enumerate(rows):
        for j, n in enumerate(cols):
            tot = Fraction(0)
            for k in range(K):
                av = frac_e4m3(int(a[m, k])) * frac_f32(sfa[k // 128, m])
                bv = frac_e4m3(int(b[n, k])) * frac_f32(sfb[n // 128, k // 128])
                tot += av * bv
            if c is not None:
                tot += frac_bf16(int(c[m, n]))
            out[i, j] = frac_rne_bf16_bits(tot)
    return out


# ----------------------------------------------------------------------------
# format pins
# ----------------------------------------------------------------------------
def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = oracle.decode_e4m3(np.arange(256))
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan_ref)
    assert set(np.nonzero(nan_ref)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(mine[~nan_ref], ref[~nan_ref])
    assert mine[0x01] == 2.0 ** -9 and mine[0x7E] == 448.0 and mine[0x38] == 1.0
    # independent exact decode agrees too
    for code in range(256):
        if code & 0x7F == 0x7F:
            continue
        assert Fraction(mine[code]) == frac_e4m3(code)


def test_bf16_rounding_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # add exact ties and neighbours
    extra = np.array([257.0, 259.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2.0 ** -130,
                      3 * 2.0 ** -134, 0.0, -0.0, 3.3895313892515355e38], dtype=np.float32)
    x = np.concatenate([x, extra])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = oracle.round_f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(mine, ref)


def test_bf16_rounding_is_direct_not_through_fp32():
    # 1 + 2**-8 + 2**-40 lies above the tie between 1 and 1 + 2**-7; through fp32
    # it would collapse onto the tie and round to even (1.0)
    x = np.array([1 + 2.0 ** -8 + 2.0 ** -40, -(1 + 2.0 ** -8 + 2.0 ** -40), 1 + 2.0 ** -8])
    got = oracle.round_f64_to_bf16_bits(x)
    assert got.tolist() == [0x3F81, 0xBF81, 0x3F80]


def test_bf16_rounding_against_exact_rationals():
    rng = np.random.default_rng(2)
    vals = rng.standard_normal(2000) * np.exp2(rng.integers(-140, 120, size=2000))
    got = oracle.round_f64_to_bf16_bits(vals)
    for v, g in zip(vals, got):
        assert frac_rne_bf16_bits(Fraction(float(v))) == int(g)


# ----------------------------------------------------------------------------
# brute force on tiny inputs (exact rationals)
# ----------------------------------------------------------------------------
def _random_codes(rng, shape):
    codes = rng.integers(0, 256, size=shape).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00        # no NaN codes
    return codes


@pytest.mark.parametrize("M,N,K,seed", [(3, 5, 128, 0), (8, 8, 256, 1), (5, 7, 384, 2), (1, 1, 128, 3)])
def test_brute_force_tiny(M, N, K, seed):
    rng = np.random.default_rng(seed)
    a = _random_codes(rng, (M, K))
    b = _random_codes(rng, (N, K))
    sfa = rng.uniform(0.01, 3.0, size=(K // 128, M)).astype(np.float32)
    sfb = rng.uniform(0.01, 3.0, size=((N + 127) // 128, K // 128)).astype(np.float32)
    c = inputgen.bf16_bits_from_f32(rng.standard_normal((M, N)).astype(np.float32) * 50)
    ref = brute_force_bits(a, sfa, b, sfb, c, range(M), range(N))
    got = oracle.gemm_nt(a, sfa, b, sfb, c)
    assert np.array_equal(got, ref)
    got0 = oracle.gemm_nt(a, sfa, b, sfb, None)
    ref0 = brute_force_bits(a, sfa, b, sfb, None, range(M), range(N))
    assert np.array_equal(got0, ref0)


def test_brute_force_across_n_blocks_and_row_subsets():
    # N spans three 128-row B blocks; checks the sfb block index and the
    # row/column subset path used for sampled parity at full size
    rng = np.random.default_rng(7)
    M, N, K = 6, 300, 256
    a = _random_codes(rng, (M, K))
    b = _random_codes(rng, (N, K))
    sfa = rng.uniform(0.01, 3.0, size=(K // 128, M)).astype(np.float32)
    sfb = rng.uniform(0.01, 3.0, size=((N + 127) // 128, K // 128)).astype(np.float32)
    rows = np.array([0, 3, 5])
    cols = np.array([0, 127, 128, 255, 256, 299])
    ref = brute_force_bits(a, sfa, b, sfb, None, rows, cols)
    got = oracle.gemm_nt(a, sfa, b, sfb, None, rows=rows, cols=cols)
    assert np.array_equal(got, ref)
    full = oracle.gemm_nt(a, sfa, b, sfb, None)
    assert np.array_equal(full[np.ix_(rows, cols)], ref)


# ----------------------------------------------------------------------------
# exact regime: closed form with Python integers
# ----------------------------------------------------------------------------
def closed_form_exact_bits(p, e_min):
    """Integer-only evaluation: codes are integers, scales are 2**e, so the
    result in units of 2**(2*e_min) is an integer sum."""
    A = oracle_free_int_values(p.a)
    B = oracle_free_int_values(p.b)
    ea = np.log2(p.sfa).astype(np.int64) - e_min       # [KB][M]
    eb = np.log2(p.sfb).astype(np.int64) - e_min       # [NB][KB]
    M, N, K = p.M, p.N, p.K
    tot = np.zeros((M, N), dtype=np.int64)
    for kb in range(K // 128):
        part = A[:, kb * 128:(kb + 1) * 128] @ B[:, kb * 128:(kb + 1) * 128].T
        shift = ea[kb][:, None] + eb[np.arange(N) // 128, kb][None, :]
        tot += part << shift
    if p.c is not None:
        cint = np.rint(oracle_free_bf16_values(p.c)).astype(np.int64)
        tot += cint << (-2 * e_min)
    assert np.abs(tot).max() < 2 ** 24
    val = tot.astype(np.float64) * 2.0 ** (2 * e_min)
    return torch.from_numpy(val.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def oracle_free_int_values(codes):
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(v, np.rint(v))
    return v.astype(np.int64)


def oracle_free_bf16_values(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("M,N,K,e_min,span", [(64, 256, 1024, -2, 3), (33, 200, 7168, -2, 3), (16, 130, 16384, -1, 2)])
def test_exact_regime_closed_form(M, N, K, e_min, span):
    p = inputgen.exact_dense(M, N, K, seed=5, e_min=e_min, e_span=span)
    ref = closed_form_exact_bits(p, e_min)
    got = oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)
    assert np.array_equal(got, ref)


def test_subnormal_exact_case_matches_brute_force():
    p = inputgen.exact_subnormal_dense(4, 6, 256, seed=3)
    assert (p.a < 8).any() or (p.a & 0x78 == 0).any()       # subnormal codes present
    ref = brute_force_bits(p.a, p.sfa, p.b, p.sfb, None, range(4), range(6))
    assert np.array_equal(oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb), ref)


# ----------------------------------------------------------------------------
# invariants of block scaling
# ----------------------------------------------------------------------------
def _dec_bits(bits):
    return oracle_free_bf16_values(bits)


def test_linearity_under_power_of_two_scale_changes():
    rng = np.random.default_rng(11)
    p = inputgen.make_dense(40, 300, 512, seed=4, b_std=0.02)
    base = _dec_bits(oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb))
    # A row scale: row m of D scales by 2**j
    for m, j in [(0, 3), (17, -4), (39, 1)]:
        sfa2 = p.sfa.copy()
        sfa2[:, m] *= np.float32(2.0 ** j)
        d2 = _dec_bits(oracle.gemm_nt(p.a, sfa2, p.b, p.sfb))
        assert np.array_equal(d2[m], base[m] * 2.0 ** j)
        others = np.arange(40) != m
        assert np.array_equal(d2[others], base[others])
    # one B block's scale (all K blocks): exactly its 128 columns scale
    sfb2 = p.sfb.copy()
    sfb2[1, :] *= np.float32(4.0)
    d3 = _dec_bits(oracle.gemm_nt(p.a, p.sfa, p.b, sfb2))
    assert np.array_equal(d3[:, 128:256], base[:, 128:256] * 4.0)
    assert np.array_equal(d3[:, :128], base[:, :128])
    assert np.array_equal(d3[:, 256:], base[:, 256:])
    # a single (row, K block) scale: only that row changes
    sfa3 = p.sfa.copy()
    sfa3[2, 5] *= np.float32(2.0)
    d4 = _dec_bits(oracle.gemm_nt(p.a, sfa3, p.b, p.sfb))
    assert not np.array_equal(d4[5], base[5])
    assert np.array_equal(np.delete(d4, 5, axis=0), np.delete(base, 5, axis=0))
    del rng


def test_moving_a_factor_two_from_codes_into_scale():
    rng = np.random.default_rng(12)
    M, N, K = 8, 16, 384
    even = inputgen.encode_e4m3(rng.choice([-4.0, -2.0, 0.0, 2.0, 4.0], size=(M, K)).astype(np.float32))
    half = inputgen.encode_e4m3(oracle_free_int_values(even).astype(np.float32) / 2)
    b = inputgen.encode_e4m3(rng.integers(-4, 5, size=(N, K)).astype(np.float32))
    sfa = np.ldexp(1.0, rng.integers(-3, 2, size=(K // 128, M))).astype(np.float32)
    sfb = np.ldexp(1.0, rng.integers(-3, 2, size=(1, K // 128))).astype(np.float32)
    d1 = oracle.gemm_nt(even, sfa, b, sfb)
    # halve codes of K block 1 of every row, double its scale
    a2 = even.copy()
    a2[:, 128:256] = half[:, 128:256]
    sfa2 = sfa.copy()
    sfa2[1] *= 2
    assert np.array_equal(oracle.gemm_nt(a2, sfa2, b, sfb), d1)
    # a change that is not compensated must show
    assert not np.array_equal(oracle.gemm_nt(a2, sfa, b, sfb), d1)


def test_k_additivity_exact_regime():
    p = inputgen.exact_dense(24, 160, 1024, seed=9, with_c=False)
    full = oracle.gemm_nt_acc(p.a, p.sfa, p.b, p.sfb)
    k1 = 384
    left = oracle.gemm_nt_acc(p.a[:, :k1], p.sfa[:k1 // 128], p.b[:, :k1], p.sfb[:, :k1 // 128])
    right = oracle.gemm_nt_acc(p.a[:, k1:], p.sfa[k1 // 128:], p.b[:, k1:], p.sfb[:, k1 // 128:])
    assert np.array_equal(full, left + right)


def test_plain_definition_cross_check():
    """C + dequant(A) dequant(B)^T with one numpy matmul over all of K."""
    p = inputgen.make_dense(96, 260, 1024, seed=6, b_std=0.02, c_std=0.1, pow2=False)
    A = torch.from_numpy(p.a).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    B = torch.from_numpy(p.b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    Aq = A * np.repeat(p.sfa.T.astype(np.float64), 128, axis=1)
    Bq = B * np.repeat(np.repeat(p.sfb.astype(np.float64), 128, axis=1), 128, axis=0)[:p.N]
    ref = Aq @ Bq.T + oracle_free_bf16_values(p.c)
    acc = oracle.gemm_nt_acc(p.a, p.sfa, p.b, p.sfb, p.c)
    assert np.max(np.abs(acc - ref)) <= 1e-12 * np.max(np.abs(ref))
    got = oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)
    ref_bits = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # rounding through fp32 may differ only at near-ties
    assert np.mean(got != ref_bits) <= 1e-3


# ----------------------------------------------------------------------------
# storage layouts of the dense form (nt, nn, tn, tt)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("layout", ["nt", "nn", "tn", "tt"])
def test_layouts_brute_force_on_stored_arrays(layout):
    # the brute force reads the stored arrays with the layout's own indexing
    # (A[k][m] for "t", B[k][n] for a second "n"), independent of the
    # transposition gemm_layout performs
    rng = np.random.default_rng(40 + "nt nn tn tt".split().index(layout))
    M, N, K = 6, 5, 256
    a = _random_codes(rng, (M, K) if layout[0] == "n" else (K, M))
    b = _random_codes(rng, (N, K) if layout[1] == "t" else (K, N))
    sfa = rng.uniform(0.05, 3.0, size=(K // 128, M)).astype(np.float32)
    sfb = rng.uniform(0.05, 3.0, size=(1, K // 128)).astype(np.float32)
    c = inputgen.bf16_bits_from_f32(rng.standard_normal((M, N)).astype(np.float32) * 20)
    got = oracle.gemm_layout(layout, a, sfa, b, sfb, c)
    for m in range(M):
        for n in range(N):
            tot = frac_bf16(int(c[m, n]))
            for k in range(K):
                av = frac_e4m3(int(a[m, k] if layout[0] == "n" else a[k, m])) * frac_f32(sfa[k // 128, m])
                bv = frac_e4m3(int(b[n, k] if layout[1] == "t" else b[k, n])) * frac_f32(sfb[n // 128, k // 128])
                tot += av * bv
            assert int(got[m, n]) == frac_rne_bf16_bits(tot), (layout, m, n)


def test_layouts_agree_on_transposed_storage():
    # the same logical product stored four ways gives one result
    rng = np.random.default_rng(44)
    M, N, K = 9, 130, 384
    a = _random_codes(rng, (M, K))
    b = _random_codes(rng, (N, K))
    sfa = rng.uniform(0.1, 2.0, size=(K // 128, M)).astype(np.float32)
    sfb = rng.uniform(0.1, 2.0, size=(2, K // 128)).astype(np.float32)
    ref = oracle.gemm_nt(a, sfa, b, sfb)
    stored = {"nt": (a, b), "nn": (a, b.T.copy()), "tn": (a.T.copy(), b.T.copy()), "tt": (a.T.copy(), b)}
    for layout, (aa, bb) in stored.items():
        assert np.array_equal(oracle.gemm_layout(layout, aa, sfa, bb, sfb), ref), layout


# ----------------------------------------------------------------------------
# K-grouped TN form
# ----------------------------------------------------------------------------
def test_k_grouped_brute_force_tiny():
    # exact rationals over the stored arrays (A[k][m], B[k][n], sfa[k//128][m],
    # sfb[k//128][n]), group g summing only its own K rows, one rounding to fp32
    rng = np.random.default_rng(51)
    G, M, N = 3, 5, 4
    ks = np.array([128, 0, 256], dtype=np.int32)
    K = int(ks.sum())
    a = _random_codes(rng, (K, M))
    b = _random_codes(rng, (K, N))
    sfa = rng.uniform(0.05, 3.0, size=(K // 128, M)).astype(np.float32)
    sfb = rng.uniform(0.05, 3.0, size=(K // 128, N)).astype(np.float32)
    c = (rng.standard_normal((G, M, N)) * 30).astype(np.float32)
    got = oracle.k_grouped_tn(a, sfa, b, sfb, ks, c)
    assert got.dtype == np.float32 and got.shape == (G, M, N)
    start = 0
    for g in range(G):
        for m in range(M):
            for n in range(N):
                tot = frac_f32(c[g, m, n])
                for k in range(start, start + int(ks[g])):
                    tot += (frac_e4m3(int(a[k, m])) * frac_f32(sfa[k // 128, m])
                            * frac_e4m3(int(b[k, n])) * frac_f32(sfb[k // 128, n]))
                assert got[g, m, n].view(np.uint32) == frac_rne_f32(tot).view(np.uint32), (g, m, n)
        start += int(ks[g])
    # an empty group gives C exactly; without C it gives zeros
    assert np.array_equal(got[1], c[1])
    assert not np.any(oracle.k_grouped_tn(a, sfa, b, sfb, ks)[1])


def test_k_grouped_magnitude_brute_force():
    # The second output of k_grouped_tn_acc (likun.im section 二, the
    # k_grouped_fp8_gemm_tn_contiguous call with per-group K sizes) is the
    # error scale of an fp32 accumulation: |C| plus the sum of the absolute
    # values of every scaled product a*sa*b*sb of the group's K rows.  Exact
    # rationals over the stored arrays, with mixed-sign codes (subnormals
    # included), scales that are not powers of two (some negative, so that a
    # dropped absolute value shows), an empty group and C; every value here
    # has few significant bits, so the fp64 sums are exact and the two must
    # agree exactly, for acc as well as for mag.
    rng = np.random.default_rng(52)
    G, M, N = 4, 3, 5
    ks = np.array([256, 0, 128, 384], dtype=np.int32)
    K = int(ks.sum())
    a = _random_codes(rng, (K, M))
    b = _random_codes(rng, (K, N))
    a[0, 0], a[1, 0], b[0, 0] = 0x01, 0x85, 0x03        # subnormal codes of both signs
    sfa = (rng.integers(1, 16, size=(K // 128, M)) * rng.choice([-1, 1], size=(K // 128, M)) / 8.0).astype(np.float32)
    sfb = (rng.integers(1, 16, size=(K // 128, N)) / 4.0).astype(np.float32)
    sfb[0, 1] = -0.75
    c = rng.integers(-40, 41, size=(G, M, N)).astype(np.float32)
    acc, mag = oracle.k_grouped_tn_acc(a, sfa, b, sfb, ks, c)
    assert mag.shape == (G, M, N) and acc.shape == (G, M, N)
    start = 0
    for g in range(G):
        for m in range(M):
            for n in range(N):
                tot = frac_f32(c[g, m, n])
                mg = abs(frac_f32(c[g, m, n]))
                for k in range(start, start + int(ks[g])):
                    term = (frac_e4m3(int(a[k, m])) * frac_f32(sfa[k // 128, m])
                            * frac_e4m3(int(b[k, n])) * frac_f32(sfb[k // 128, n]))
                    tot += term
                    mg += abs(term)
                assert Fraction(float(acc[g, m, n])) == tot, (g, m, n)
                assert Fraction(float(mag[g, m, n])) == mg, (g, m, n)
        start += int(ks[g])
    # the empty group: |C| only; without C, zero
    assert np.array_equal(mag[1], np.abs(c[1]).astype(np.float64))
    assert not np.any(oracle.k_grouped_tn_acc(a, sfa, b, sfb, ks)[1][1])
    # a term-wise bound: mag dominates |acc| everywhere
    assert np.all(mag >= np.abs(acc))


def test_k_grouped_exact_regime_closed_form():
    # integer codes and power-of-two scales: Python integers (scaled by the
    # smallest scale product) give the exact value, which fp32 holds exactly
    p = inputgen.exact_kgrouped(3, 16, 32, [256, 128, 0], seed=5, e_min=-2, e_span=3)
    got = oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, p.c)
    ia = oracle_free_int_values(p.a).astype(np.int64)            # [K][M]
    ib = oracle_free_int_values(p.b).astype(np.int64)            # [K][N]
    ea = np.log2(p.sfa).astype(np.int64)                         # [KB][M]
    eb = np.log2(p.sfb).astype(np.int64)
    unit = 2 * -2                                                # exponent of the smallest scale product
    start = 0
    for g in range(p.G):
        tot = (p.c[g].astype(np.int64) << (-unit))               # C in units of 2**unit
        for k in range(start, start + int(p.ks[g])):
            kb = k // 128
            sh = ea[kb][:, None] + eb[kb][None, :] - unit        # >= 0
            tot = tot + ((ia[k][:, None] * ib[k][None, :]) << sh)
        start += int(p.ks[g])
        exact = tot.astype(np.float64) * 2.0 ** unit
        assert np.array_equal(got[g], exact.astype(np.float32)), g
        assert np.all(np.abs(tot) < 2 ** 53)


# ----------------------------------------------------------------------------
# grouped forms
# ----------------------------------------------------------------------------
def test_contiguous_brute_force_tiny():
    rng = np.random.default_rng(21)
    G, N, K = 3, 5, 256
    layout = np.array([0, 0, 2, 2, 2, -1, 1, 3, 1, 7], dtype=np.int32)   # 3 (== G), 7 and -1 are not valid
    M = len(layout)
    a = _random_codes(rng, (M, K))
    b = _random_codes(rng, (G, N, K))
    sfa = rng.uniform(0.1, 2, size=(K // 128, M)).astype(np.float32)
    sfb = rng.uniform(0.1, 2, size=(G, 1, K // 128)).astype(np.float32)
    c = inputgen.bf16_bits_from_f32(rng.standard_normal((M, N)).astype(np.float32))
    got, written = oracle.m_grouped_contiguous(a, sfa, b, sfb, layout, c)
    assert written.tolist() == [True, True, True, True, True, False, True, False, True, False]
    for m in range(M):
        g = layout[m]
        if not (0 <= g < G):
            continue
        ref = brute_force_bits(a, sfa, b[g], sfb[g], c, [m], range(N))
        assert np.array_equal(got[m], ref[0]), m


def test_masked_brute_force_tiny():
    rng = np.random.default_rng(22)
    G, max_m, N, K = 4, 5, 3, 128
    masked_m = np.array([0, 5, 2, 9], dtype=np.int32)   # 9 clamps to max_m
    a = _random_codes(rng, (G, max_m, K))
    b = _random_codes(rng, (G, N, K))
    sfa = rng.uniform(0.1, 2, size=(G, 1, max_m)).astype(np.float32)
    sfb = rng.uniform(0.1, 2, size=(G, 1, 1)).astype(np.float32)
    got, written = oracle.m_grouped_masked(a, sfa, b, sfb, masked_m)
    assert written.sum(axis=1).tolist() == [0, 5, 2, 5]
    for g in range(G):
        for m in range(int(written[g].sum())):
            ref = brute_force_bits(a[g], sfa[g], b[g], sfb[g], None, [m], range(N))
            assert np.array_equal(got[g, m], ref[0])
        assert (got[g][~written[g]] == 0).all()


# ----------------------------------------------------------------------------
# hand-derived closed-form fixtures
# ----------------------------------------------------------------------------
def _expand(spec, shape):
    arr = np.full(shape, spec["fill"], dtype=np.float64)
    for r, v in spec.get("rows", []):
        arr[r, :] = v
    for idx, v in spec.get("set", []):
        arr[tuple(idx)] = v
    return arr


def test_golden_closed_form_fixtures():
    with open(os.path.join(GOLDEN, "closed_form.json")) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 3
    for case in cases:
        M, N, K = case["M"], case["N"], case["K"]
        a = inputgen.encode_e4m3(_expand(case["a"], (M, K)).astype(np.float32))
        b = inputgen.encode_e4m3(_expand(case["b"], (N, K)).astype(np.float32))
        sfa = _expand(case["sfa"], (K // 128, M)).astype(np.float32)
        sfb = _expand(case["sfb"], ((N + 127) // 128, K // 128)).astype(np.float32)
        c = None
        if "c" in case:
            c = inputgen.bf16_bits_from_f32(_expand(case["c"], (M, N)).astype(np.float32))
        got = _dec_bits(oracle.gemm_nt(a, sfa, b, sfb, c))
        for (m, n), v in case["expect"]:
            assert got[m, n] == v, (case["name"], m, n, got[m, n], v)


# ----------------------------------------------------------------------------
# FP8 x FP4 form
# ----------------------------------------------------------------------------
def test_e2m1_table_against_the_format_value_list():
    # OCP Microscaling Formats v1.0, FP4 (E2M1) element data type: the eight
    # magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6; the top bit is the sign
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(oracle.E2M1_VALUES[:8]) == mags
    assert list(oracle.E2M1_VALUES[8:]) == [-m for m in mags]


def _nibble(b, n, k):
    byte = int(b[n, k // 2])
    return (byte >> 4) if k % 2 else (byte & 0xF)


def frac_e2m1(code: int) -> Fraction:
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
    return -mags[code & 7] if code & 8 else mags[code & 7]


@pytest.mark.parametrize("M,N,K,seed", [(3, 5, 128, 60), (4, 3, 256, 61)])
def test_fp8_fp4_brute_force_tiny(M, N, K, seed):
    # exact rationals from the stored arrays: nibbles of b, the E8M0 byte of
    # each 32 K values taken from the packed int, one rounding to bf16
    rng = np.random.default_rng(seed)
    a = _random_codes(rng, (M, K))
    b = rng.integers(0, 256, size=(N, K // 2)).astype(np.uint8)
    sfa = rng.uniform(0.05, 3.0, size=(K // 128, M)).astype(np.float32)
    ebytes = rng.integers(120, 135, size=(K // 128, N, 4)).astype(np.uint32)
    sfb = (ebytes[..., 0] | (ebytes[..., 1] << 8) | (ebytes[..., 2] << 16) | (ebytes[..., 3] << 24)).view(np.int32)
    c = inputgen.bf16_bits_from_f32(rng.standard_normal((M, N)).astype(np.float32) * 10)
    got = oracle.gemm_fp8_fp4_nt(a, sfa, b, sfb, c)
    for m in range(M):
        for n in range(N):
            tot = frac_bf16(int(c[m, n]))
            for k in range(K):
                e = int(ebytes[k // 128, n, (k % 128) // 32]) - 127
                tot += (frac_e4m3(int(a[m, k])) * frac_f32(sfa[k // 128, m])
                        * frac_e2m1(_nibble(b, n, k)) * Fraction(2) ** e)
            assert int(got[m, n]) == frac_rne_bf16_bits(tot), (m, n)


def test_fp8_fp4_quantiser_round_trip():
    # every code decodes to a value the quantiser maps back to that code, and
    # scales are powers of two with the block maximum within 6 * scale
    x = np.random.default_rng(62).standard_normal((8, 256)).astype(np.float32)
    packed, e = inputgen.quantize_fp4_rows(x)
    vals = oracle.decode_e2m1_packed(packed) * np.repeat(np.ldexp(1.0, e.astype(np.int64) - 127), 32, axis=1)
    amax = np.abs(x).reshape(8, 8, 32).max(axis=2)
    s = np.ldexp(1.0, e.astype(np.int64) - 127)
    assert np.all(amax <= 6 * s) and np.all(amax > 3 * s)
    err = np.abs(vals - x)
    assert np.all(err <= np.repeat(s, 32, axis=1) * 1.0 + 1e-12)     # half the widest E2M1 step (4 -> 6) times the scale
    codes = np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(8, 256)
    assert np.array_equal(inputgen.encode_e2m1(oracle.E2M1_VALUES[codes]), np.where(codes == 8, 0, codes))


def test_fp8_fp4_grouped_forms_reduce_to_brute_force_rows():
    # contiguous: every valid row equals the exact-rational result with its
    # expert's B; masked: the first masked_m rows of each group likewise
    rng = np.random.default_rng(63)
    G, N, K = 3, 4, 128
    layout = np.array([0, 2, 2, -1, 1, 5], dtype=np.int32)
    M = len(layout)
    a = _random_codes(rng, (M, K))
    b = rng.integers(0, 256, size=(G, N, K // 2)).astype(np.uint8)
    sfa = rng.uniform(0.1, 2.0, size=(K // 128, M)).astype(np.float32)
    eb = rng.integers(124, 131, size=(G, K // 128, N, 4)).astype(np.uint32)
    sfb = (eb[..., 0] | (eb[..., 1] << 8) | (eb[..., 2] << 16) | (eb[..., 3] << 24)).view(np.int32)
    got, written = oracle.m_grouped_fp8_fp4_contiguous(a, sfa, b, sfb, layout)
    assert written.tolist() == [True, True, True, False, True, False]
    for m in range(M):
        g = int(layout[m])
        if not 0 <= g < G:
            continue
        for n in range(N):
            tot = Fraction(0)
            for k in range(K):
                tot += (frac_e4m3(int(a[m, k])) * frac_f32(sfa[k // 128, m]) * frac_e2m1(_nibble(b[g], n, k))
                        * Fraction(2) ** (int(eb[g, k // 128, n, (k % 128) // 32]) - 127))
            assert int(got[m, n]) == frac_rne_bf16_bits(tot), (m, n)
    masked_m = np.array([2, 0, 7], dtype=np.int32)
    am = a[:6].reshape(3, 2, K).repeat(2, axis=1)[:, :3]            # [G][max_m=3][K]
    sfam = np.ascontiguousarray(np.repeat(sfa[:, None, :3], G, axis=1).transpose(1, 0, 2))   # [G][KB][3]
    gm, wm = oracle.m_grouped_fp8_fp4_masked(am, sfam, b, sfb, masked_m)
    assert wm.tolist() == [[True, True, False], [False, False, False], [True, True, True]]
    for g in range(G):
        m = min(int(masked_m[g]), 3)
        if m:
            ref = oracle.gemm_fp8_fp4_nt(am[g][:m], sfam[g][:, :m], b[g], sfb[g])
            assert np.array_equal(gm[g, :m], ref)

