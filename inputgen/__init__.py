"""Seeded synthetic inputs for the FP8 block-scaled GEMM (NT), its M-grouped
forms and the K-grouped TN form.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds no GEMM arithmetic: it draws random numbers, quantises
them to OCP e4m3 codes with per-block scales (the input recipe), and lays the
results out in the memory formats the library takes.  Neither the oracle nor
the GPU path is imported here.

Layouts (all row-major, numpy):
  a    uint8   [M][K]          e4m3 codes, K contiguous (masked form: [G][max_m][K])
  sfa  float32 [K/128][M]      one scale per row per 128-wide K slice, M contiguous
                               (masked form: [G][K/128][max_m])
  b    uint8   [N][K]          e4m3 codes (grouped forms: [G][N][K])
  sfb  float32 [ceil(N/128)][K/128]  one scale per 128x128 block (grouped: [G][..][..])
  c    uint16  [M][N]          bf16 bit patterns, or None for C = 0

Quantisation recipe (fine-grained block scaling, DeepGEMM pages "FP8 precision
core" section of the aitangshan.cn article; block shapes 1x128 for A and
128x128 for B): amax over the block in fp32, scale = amax/448 (fp32), rounded
up to a power of two when ``pow2`` is set, scale 1 for an all-zero block;
code = RNE_e4m3(clamp(x / scale, -448, 448)).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

BLOCK = 128
E4M3_MAX = 448.0


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


# ----------------------------------------------------------------------------
# scale and code helpers (input preparation only)
# ----------------------------------------------------------------------------
def _pow2_ceil(v: np.ndarray) -> np.ndarray:
    """Smallest power of two >= v for positive fp32 v (exact via frexp)."""
    v = np.asarray(v, dtype=np.float32)
    m, e = np.frexp(v.astype(np.float64))
    # v = m * 2**e with 0.5 <= m < 1; an exact power of two has m == 0.5
    e = np.where(m == 0.5, e - 1, e)
    return np.ldexp(np.ones_like(v, dtype=np.float64), e).astype(np.float32)


def _scales_from_amax(amax: np.ndarray, pow2: bool) -> np.ndarray:
    amax = np.asarray(amax, dtype=np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    if pow2:
        s = np.where(amax > 0, _pow2_ceil(np.where(s > 0, s, 1.0)), np.float32(1.0))
    else:
        s = np.where(s > 0, s, np.float32(1.0))
    return s.astype(np.float32)


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3 codes, round to nearest even, saturating at +-448."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.clamp(-E4M3_MAX, E4M3_MAX)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


E2M1_MAX = 6.0
_E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def encode_e2m1(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP E2M1 (FP4) codes 0..15, round to nearest with ties to the
    even code (even mantissa bit), saturating at +-6."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), E2M1_MAX)
    # distances to the 8 magnitudes; ties go to the even code
    d = np.abs(mag[..., None] - _E2M1_VALUES)
    best = np.argmin(d + 1e-9 * (np.arange(8) % 2), axis=-1)   # prefer even codes on ties
    code = best.astype(np.uint8)
    code[(x < 0) & (code != 0)] |= 8
    return code


def quantize_fp4_rows(x: np.ndarray):
    """1x32 FP4 quantisation of x [N][K] with E8M0 scales: per row per 32 K
    values, scale = 2**ceil(log2(amax/6)) (1 for an all-zero group), code =
    RNE_e2m1(x / scale).  Returns (packed codes [N][K/2] u8, element 2i in the
    low nibble, scale exponents [N][K/32] as biased E8M0 bytes)."""
    N, K = x.shape
    assert K % 32 == 0
    xb = x.reshape(N, K // 32, 32).astype(np.float32)
    amax = np.abs(xb).max(axis=2)
    e = np.zeros_like(amax, dtype=np.int64)
    nz = amax > 0
    # smallest e with 6 * 2**e >= amax, exactly via frexp of amax / 6 in fp64
    m, ex = np.frexp(amax[nz].astype(np.float64) / E2M1_MAX)
    e[nz] = np.where(m == 0.5, ex - 1, ex)
    codes = encode_e2m1(xb / np.ldexp(1.0, e)[:, :, None]).reshape(N, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def quantize_rows(x: np.ndarray, pow2: bool):
    """1x128 quantisation of x [R][K] -> (codes [R][K] u8, scales [K/128][R] f32)."""
    R, K = x.shape
    assert K % BLOCK == 0
    xb = x.reshape(R, K // BLOCK, BLOCK)
    amax = np.abs(xb).max(axis=2)                     # [R][KB]
    s = _scales_from_amax(amax, pow2)                 # [R][KB]
    q = (xb / s[:, :, None]).astype(np.float32)
    codes = encode_e4m3(q.reshape(R, K))
    return codes, np.ascontiguousarray(s.T)


def quantize_blocks(x: np.ndarray, pow2: bool):
    """128x128 quantisation of x [N][K] -> (codes [N][K] u8, scales [ceil(N/128)][K/128] f32).

    The last N block may hold fewer than 128 rows; its amax is taken over the
    rows present."""
    N, K = x.shape
    assert K % BLOCK == 0
    KB = K // BLOCK
    NB = (N + BLOCK - 1) // BLOCK
    s = np.empty((NB, KB), dtype=np.float32)
    codes = np.empty((N, K), dtype=np.uint8)
    for nb in range(NB):
        rows = x[nb * BLOCK:(nb + 1) * BLOCK]
        r = rows.shape[0]
        xb = rows.reshape(r, KB, BLOCK)
        amax = np.abs(xb).max(axis=(0, 2))            # [KB]
        sb = _scales_from_amax(amax, pow2)
        s[nb] = sb
        q = (xb / sb[None, :, None]).astype(np.float32)
        codes[nb * BLOCK:(nb + 1) * BLOCK] = encode_e4m3(q.reshape(r, K))
    return codes, s


# ----------------------------------------------------------------------------
# problem containers
# ----------------------------------------------------------------------------
@dataclass
class Dense:
    a: np.ndarray
    sfa: np.ndarray
    b: np.ndarray
    sfb: np.ndarray
    c: Optional[np.ndarray]
    M: int
    N: int
    K: int
    name: str = "dense"

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


@dataclass
class Contiguous:
    a: np.ndarray            # [M][K]
    sfa: np.ndarray          # [KB][M]
    b: np.ndarray            # [G][N][K]
    sfb: np.ndarray          # [G][NB][KB]
    c: Optional[np.ndarray]
    grouped_layout: np.ndarray  # int32 [M]
    counts: np.ndarray       # real rows per expert
    M: int
    N: int
    K: int
    G: int
    name: str = "contiguous"

    @property
    def real_rows(self) -> int:
        return int(self.counts.sum())

    @property
    def flops(self) -> float:
        return 2.0 * self.real_rows * self.N * self.K


@dataclass
class Masked:
    a: np.ndarray            # [G][max_m][K]
    sfa: np.ndarray          # [G][KB][max_m]
    b: np.ndarray            # [G][N][K]
    sfb: np.ndarray          # [G][NB][KB]
    c: Optional[np.ndarray]  # [G][max_m][N] or None
    masked_m: np.ndarray     # int32 [G]
    expected_m: int
    max_m: int
    N: int
    K: int
    G: int
    name: str = "masked"

    @property
    def flops(self) -> float:
        return 2.0 * float(np.minimum(self.masked_m, self.max_m).sum()) * self.N * self.K


@dataclass
class DenseFP4:
    """FP8 x FP4 dense problem: A e4m3 with 1x128 fp32 scales as in Dense; B
    holds OCP E2M1 codes two to a byte (element 2i in the low nibble) with one
    E8M0 scale per row per 32 K values, packed four to an int32 in K order."""
    a: np.ndarray            # [M][K] e4m3 codes
    sfa: np.ndarray          # [K/128][M] fp32
    b: np.ndarray            # [N][K/2] packed E2M1
    sfb: np.ndarray          # [K/128][N] int32: byte j = E8M0 of K values 32j..32j+31 of the block
    c: Optional[np.ndarray]  # [M][N] bf16 bits or None
    M: int
    N: int
    K: int
    name: str = "dense_fp4"

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


def pack_e8m0_blocks(e: np.ndarray) -> np.ndarray:
    """E8M0 bytes [N][K/32] -> int32 [K/128][N], byte j of an int holding the
    scale of K values 32j..32j+31 of that 128-wide block."""
    N, KS = e.shape
    assert KS % 4 == 0
    q = e.reshape(N, KS // 4, 4).astype(np.uint32)
    packed = q[:, :, 0] | (q[:, :, 1] << 8) | (q[:, :, 2] << 16) | (q[:, :, 3] << 24)
    return np.ascontiguousarray(packed.T).view(np.int32)


@dataclass
class KGrouped:
    """K-grouped TN problem (MoE weight gradient): group g owns K rows
    k_start[g] .. k_start[g+1]-1 of both operands (its tokens), ks[g] of them,
    each a multiple of 128."""
    a: np.ndarray            # [K][M] e4m3 codes, M contiguous (stored K-major)
    sfa: np.ndarray          # [K/128][M] fp32, one per column m per 128 K rows
    b: np.ndarray            # [K][N] e4m3 codes, N contiguous
    sfb: np.ndarray          # [K/128][N] fp32, one per column n per 128 K rows
    c: Optional[np.ndarray]  # [G][M][N] fp32 or None
    ks: np.ndarray           # int32 [G], multiples of 128
    counts: np.ndarray       # real tokens per group (<= ks)
    M: int
    N: int
    K: int
    G: int
    name: str = "kgrouped"

    @property
    def k_start(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.ks)]).astype(np.int64)

    @property
    def flops(self) -> float:
        return 2.0 * float(self.counts.sum()) * self.M * self.N


# ----------------------------------------------------------------------------
# random problems
# ----------------------------------------------------------------------------
def _normal(rng, shape, std):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def make_dense(M, N, K, seed=0, a_std=1.0, b_std=1.0, c_std=None, pow2=True, name="dense"):
    """Draw order: A, B, C."""
    rng = rng_for(seed)
    a, sfa = quantize_rows(_normal(rng, (M, K), a_std), pow2)
    b, sfb = quantize_blocks(_normal(rng, (N, K), b_std), pow2)
    c = None
    if c_std is not None:
        c = bf16_bits_from_f32(_normal(rng, (M, N), c_std))
    return Dense(a, sfa, b, sfb, c, M, N, K, name)


def make_contiguous(G, N, K, total_rows, seed=0, a_std=1.0, b_std=0.02, pow2=True,
                    with_c=False, c_std=0.1, pad_id=None, name="contiguous"):
    """Draw order: counts (multinomial, equal probabilities), A (real rows), B expert by expert, C.

    Each expert's segment is its count padded up to a multiple of 128.  Padding
    rows hold zero codes and unit scales.  ``pad_id`` None gives padding rows
    their segment's expert id; an integer (e.g. -1) marks them with that id."""
    rng = rng_for(seed)
    counts = rng.multinomial(total_rows, [1.0 / G] * G).astype(np.int64)
    seg = ((counts + BLOCK - 1) // BLOCK) * BLOCK
    M = int(seg.sum())
    layout = np.empty(M, dtype=np.int32)
    real_mask = np.zeros(M, dtype=bool)
    off = 0
    for g in range(G):
        layout[off:off + seg[g]] = g
        if pad_id is not None:
            layout[off + counts[g]:off + seg[g]] = pad_id
        real_mask[off:off + counts[g]] = True
        off += seg[g]
    x = np.zeros((M, K), dtype=np.float32)
    x[real_mask] = _normal(rng, (int(counts.sum()), K), a_std)
    a, sfa = quantize_rows(x, pow2)
    b = np.empty((G, N, K), dtype=np.uint8)
    sfb = np.empty((G, (N + BLOCK - 1) // BLOCK, K // BLOCK), dtype=np.float32)
    for g in range(G):
        b[g], sfb[g] = quantize_blocks(_normal(rng, (N, K), b_std), pow2)
    c = bf16_bits_from_f32(_normal(rng, (M, N), c_std)) if with_c else None
    return Contiguous(a, sfa, b, sfb, c, layout, counts, M, N, K, G, name)


def make_masked(G, max_m, N, K, seed=0, expected_m=128, a_std=1.0, b_std=0.02, pow2=True,
                with_c=False, c_std=0.1, masked_m=None, name="masked"):
    """Draw order: masked_m (integers 0..max_m inclusive), A, B expert by expert, C."""
    rng = rng_for(seed)
    if masked_m is None:
        masked_m = rng.integers(0, max_m + 1, size=G).astype(np.int32)
    else:
        masked_m = np.asarray(masked_m, dtype=np.int32)
    a = np.empty((G, max_m, K), dtype=np.uint8)
    sfa = np.empty((G, K // BLOCK, max_m), dtype=np.float32)
    for g in range(G):
        a[g], sfa[g] = quantize_rows(_normal(rng, (max_m, K), a_std), pow2)
    b = np.empty((G, N, K), dtype=np.uint8)
    sfb = np.empty((G, (N + BLOCK - 1) // BLOCK, K // BLOCK), dtype=np.float32)
    for g in range(G):
        b[g], sfb[g] = quantize_blocks(_normal(rng, (N, K), b_std), pow2)
    c = bf16_bits_from_f32(_normal(rng, (G, max_m, N), c_std)) if with_c else None
    return Masked(a, sfa, b, sfb, c, masked_m, expected_m, max_m, N, K, G, name)


# ----------------------------------------------------------------------------
# the five workloads (sizes and distributions of the DeepSeek-V3/R1 shapes)
# ----------------------------------------------------------------------------
CONFIG_NAMES = [
    "dense_128x256x512",
    "dense_decode_64x2112x7168",
    "dense_prefill_4096x7168x16384",
    "contiguous_8x4096x7168_rows8192",
    "masked_32x256x4096x7168",
]


def make_kgrouped(G, M, N, total_tokens, seed=0, a_std=1.0, b_std=1.0, pow2=True, with_c=False,
                  c_std=1.0, counts=None, name="kgrouped"):
    """Draw order: counts (multinomial, equal probabilities, unless given), A, B, C.

    Group g's tokens are padded to ks[g] = ceil(count/128)*128 K rows whose
    padding holds zero codes and unit scales.  A is drawn as [tokens][M] and
    quantised per column per 128 K rows (1x128 along K, the (1, 1, 128)
    recipe); B likewise as [tokens][N]."""
    rng = rng_for(seed)
    if counts is None:
        counts = rng.multinomial(total_tokens, [1.0 / G] * G)
    counts = np.asarray(counts, dtype=np.int64)
    ks = ((counts + BLOCK - 1) // BLOCK) * BLOCK
    K = int(ks.sum())
    real = np.zeros(K, dtype=bool)
    off = 0
    for g in range(G):
        real[off:off + counts[g]] = True
        off += ks[g]
    xa = np.zeros((K, M), dtype=np.float32)
    xa[real] = _normal(rng, (int(counts.sum()), M), a_std)
    xb = np.zeros((K, N), dtype=np.float32)
    xb[real] = _normal(rng, (int(counts.sum()), N), b_std)
    # quantise along K: the transposed arrays are [M][K] rows with 1x128 blocks
    ca, sfa = quantize_rows(np.ascontiguousarray(xa.T), pow2)
    cb, sfb = quantize_rows(np.ascontiguousarray(xb.T), pow2)
    c = _normal(rng, (G, M, N), c_std) if with_c else None
    return KGrouped(np.ascontiguousarray(ca.T), sfa, np.ascontiguousarray(cb.T), sfb, c,
                    ks.astype(np.int32), counts, M, N, K, G, name)


def make_dense_fp4(M, N, K, seed=0, a_std=1.0, b_std=1.0, c_std=None, pow2=True, name="dense_fp4"):
    """Draw order: A, B, C.  A as in make_dense; B quantised to FP4 per row per 32."""
    rng = rng_for(seed)
    a, sfa = quantize_rows(_normal(rng, (M, K), a_std), pow2)
    b, e = quantize_fp4_rows(_normal(rng, (N, K), b_std))
    c = bf16_bits_from_f32(_normal(rng, (M, N), c_std)) if c_std is not None else None
    return DenseFP4(a, sfa, b, pack_e8m0_blocks(e), c, M, N, K, name)


def exact_dense_fp4(M, N, K, seed=0, e_min=-2, e_span=2, with_c=True, name="exact_dense_fp4"):
    """FP8 x FP4 problem in the exact regime: A integer codes in [-4, 4] with
    scales 2**e (e in [e_min, e_min+e_span]); B codes from every E2M1 value
    (multiples of 1/2, |b| <= 6) with E8M0 scales 2**e, e in the same range;
    C an integer in [-64, 64].  Every scaled product is a multiple of
    2**(2*e_min - 1) of at most 48 * 4**e_span such units, so with
    K*48*4**e_span + 64*2**(1 - 2*e_min) < 2**24 every fp32 partial sum,
    promotion and accumulation is exact in any order."""
    assert K * 48 * 4 ** e_span + 64 * 2 ** (1 - 2 * e_min) < 2 ** 24
    rng = rng_for(seed)
    a = _int_codes(rng, (M, K))
    codes = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    b = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    KB = K // BLOCK
    sfa = np.ldexp(1.0, rng.integers(e_min, e_min + e_span + 1, size=(KB, M))).astype(np.float32)
    e = (rng.integers(e_min, e_min + e_span + 1, size=(N, K // 32)) + 127).astype(np.uint8)
    c = None
    if with_c:
        c = bf16_bits_from_f32(rng.integers(-64, 65, size=(M, N)).astype(np.float32))
    return DenseFP4(a, sfa, b, pack_e8m0_blocks(e), c, M, N, K, name)


def make_config(i: int, seed: int = 0):
    if i == 0:
        return make_dense(128, 256, 512, seed, 1.0, 1.0, None, True, CONFIG_NAMES[0])
    if i == 1:
        return make_dense(64, 2112, 7168, seed, 1.0, 0.02, 0.1, True, CONFIG_NAMES[1])
    if i == 2:
        return make_dense(4096, 7168, 16384, seed, 1.0, 0.02, None, False, CONFIG_NAMES[2])
    if i == 3:
        return make_contiguous(8, 4096, 7168, 8192, seed, name=CONFIG_NAMES[3])
    if i == 4:
        return make_masked(32, 256, 4096, 7168, seed, expected_m=128, name=CONFIG_NAMES[4])
    raise ValueError(i)


# ----------------------------------------------------------------------------
# the exact regime: small-integer codes with power-of-two scales
# ----------------------------------------------------------------------------
def _int_codes(rng, shape, lo=-4, hi=4):
    v = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return encode_e4m3(v)


def exact_dense(M, N, K, seed=0, e_min=-2, e_span=3, with_c=True, name="exact_dense"):
    """Integer codes in [-4, 4], scales 2**e with e in [e_min, e_min+e_span], C an
    integer in [-64, 64].  With K*16*4**e_span + 64*4**(-e_min) < 2**24 every fp32
    partial sum, scale product, accumulation and the final C addition are exact,
    so the result is unique and both sides must agree bit for bit."""
    assert K * 16 * (4 ** e_span) + 64 * 4 ** (-e_min) < 2 ** 24
    rng = rng_for(seed)
    a = _int_codes(rng, (M, K))
    b = _int_codes(rng, (N, K))
    KB = K // BLOCK
    NB = (N + BLOCK - 1) // BLOCK
    sfa = np.ldexp(1.0, rng.integers(e_min, e_min + e_span + 1, size=(KB, M))).astype(np.float32)
    sfb = np.ldexp(1.0, rng.integers(e_min, e_min + e_span + 1, size=(NB, KB))).astype(np.float32)
    c = None
    if with_c:
        c = bf16_bits_from_f32(rng.integers(-64, 65, size=(M, N)).astype(np.float32))
    return Dense(a, sfa, b, sfb, c, M, N, K, name)


def exact_kgrouped(G, M, N, ks, seed=0, e_min=-2, e_span=3, with_c=True, name="exact_kgrouped"):
    """K-grouped problem in the exact regime: integer codes in [-4, 4], scales
    2**e with e in [e_min, e_min+e_span] per column per 128 K rows, C an integer
    in [-64, 64] (fp32).  With every group's K below the exact_dense bound, every
    fp32 partial sum, scale product and accumulation is exact."""
    ks = np.asarray(ks, dtype=np.int32)
    assert np.all(ks % BLOCK == 0) and np.all(ks >= 0)
    assert int(ks.max(initial=0)) * 16 * (4 ** e_span) + 64 * 4 ** (-e_min) < 2 ** 24
    rng = rng_for(seed)
    K = int(ks.sum())
    a = _int_codes(rng, (K, M))
    b = _int_codes(rng, (K, N))
    KB = K // BLOCK
    sfa = np.ldexp(1.0, rng.integers(e_min, e_min + e_span + 1, size=(KB, M))).astype(np.float32)
    sfb = np.ldexp(1.0, rng.integers(e_min, e_min + e_span + 1, size=(KB, N))).astype(np.float32)
    c = rng.integers(-64, 65, size=(G, M, N)).astype(np.float32) if with_c else None
    return KGrouped(a, sfa, b, sfb, c, ks, ks.astype(np.int64), M, N, K, G, name)


def exact_subnormal_dense(M, N, K, seed=0, name="exact_subnormal"):
    """Codes drawn from every finite e4m3 value of magnitude below 1/4
    (biased exponent <= 4: subnormals and +-0 included), unit scales, K <= 512.
    Every product is a multiple of 2**-18 and below 1/16, so every partial sum
    of up to 512 terms stays below 32 = 2**23 * 2**-18: exact in fp32 in any
    order, and the result is unique."""
    assert K <= 512
    rng = rng_for(seed)
    allowed = np.array([c for c in range(256) if ((c >> 3) & 0xF) <= 4], dtype=np.uint8)
    a = allowed[rng.integers(0, len(allowed), size=(M, K))]
    b = allowed[rng.integers(0, len(allowed), size=(N, K))]
    sfa = np.ones((K // BLOCK, M), dtype=np.float32)
    sfb = np.ones(((N + BLOCK - 1) // BLOCK, K // BLOCK), dtype=np.float32)
    return Dense(a, sfa, b, sfb, None, M, N, K, name)
