"""Parity of the FP8 x FP4 call (B packed E2M1 with per-32 E8M0 scales) with
the oracle, through the C ABI.  Exact-regime inputs must match bit for bit;
random inputs meet the NT call's bf16 tolerance."""
import numpy as np
import pytest
import torch

import inputgen
import oracle
from tests.gpu_util import bf16_bits_dev, bits_host, check_tolerance, dev, sentinel_like

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_grouped_gemm_nt_amd as m
    m.dg_init()
    return m


def log(msg):
    print(msg, flush=True)


def run_fp4(dg, p):
    d = sentinel_like((p.M, p.N))
    c = bf16_bits_dev(p.c) if p.c is not None else None
    dg.dg_fp8_fp4_gemm_nt(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), c, d)
    torch.cuda.synchronize()
    return bits_host(d)


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (300, 400, 512), (17, 48, 256), (64, 2112, 7168), (528, 272, 1024)])
def test_fp4_exact(dg, M, N, K):
    log(f"case: fp8 x fp4 exact {M}x{N}x{K}")
    p = inputgen.exact_dense_fp4(M, N, K, seed=M + N)
    assert np.array_equal(run_fp4(dg, p), oracle.gemm_fp8_fp4_nt(p.a, p.sfa, p.b, p.sfb, p.c))


@pytest.mark.parametrize("cfg", ["0", "1", "6", "11"])
def test_fp4_every_tile_config_exact(dg, monkeypatch, cfg):
    log(f"case: fp8 x fp4 exact, forced config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    p = inputgen.exact_dense_fp4(400, 592, 640, seed=3)
    assert np.array_equal(run_fp4(dg, p), oracle.gemm_fp8_fp4_nt(p.a, p.sfa, p.b, p.sfb, p.c))


@pytest.mark.parametrize("cfg,sk", [("0", None), ("0", "16"), ("6", "3")])
def test_fp4_split_tail_exact(dg, monkeypatch, cfg, sk):
    # the tile kernels' last partial round split over K, with an FP4 B
    log(f"case: fp8 x fp4 split tail, config {cfg}, splits {sk}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    if sk is not None:
        monkeypatch.setenv("DG_SK_SPLITS", sk)
    p = inputgen.exact_dense_fp4(1000, 2112, 1024, seed=15)
    assert np.array_equal(run_fp4(dg, p), oracle.gemm_fp8_fp4_nt(p.a, p.sfa, p.b, p.sfb, p.c))


@pytest.mark.parametrize("cfg", ["1", "12"])
@pytest.mark.parametrize("splits", ["1", "3", "16"])
@pytest.mark.parametrize("M,N,K", [(64, 2112, 7168), (100, 200, 2048), (1, 64, 128)])
def test_fp4_decode_splits_exact(dg, monkeypatch, cfg, splits, M, N, K):
    # the decode kernel (64x64 tiles, K split over workgroups) with a forced
    # split count: one split writes the result itself, more go through the
    # fp32 partials and the split-K reduction (1) or the in-launch hand-off (12)
    log(f"case: fp8 x fp4 decode exact {M}x{N}x{K}, config {cfg}, forced splits {splits}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    monkeypatch.setenv("DG_FORCE_SPLITS", splits)
    p = inputgen.exact_dense_fp4(M, N, K, seed=M + 7)
    assert np.array_equal(run_fp4(dg, p), oracle.gemm_fp8_fp4_nt(p.a, p.sfa, p.b, p.sfb, p.c))


def test_fp4_decode_random_tolerance(dg):
    log("case: fp8 x fp4 random, decode shape 64x2112x7168")
    p = inputgen.make_dense_fp4(64, 2112, 7168, 11, 1.0, 0.02, 0.1, False)
    check_tolerance(run_fp4(dg, p), oracle.gemm_fp8_fp4_nt(p.a, p.sfa, p.b, p.sfb, p.c), "fp4 decode")


@pytest.mark.parametrize("pow2", [True, False])
def test_fp4_random_tolerance(dg, pow2):
    log(f"case: fp8 x fp4 random, A pow2 scales {pow2}")
    p = inputgen.make_dense_fp4(256, 384, 2048, 9, 1.0, 0.02, 0.1, pow2)
    check_tolerance(run_fp4(dg, p), oracle.gemm_fp8_fp4_nt(p.a, p.sfa, p.b, p.sfb, p.c), "fp4")


def test_fp4_wide_scale_range(dg):
    # E8M0 exponents spread over 2^-20 .. 2^20 on the first 32-K slice of every
    # block: checks that each slice takes its own scale byte (sums of very
    # different magnitudes round in fp32, so the bound is the bf16 tolerance)
    log("case: fp8 x fp4 with scale exponents spread over 2^-20 .. 2^20")
    p = inputgen.exact_dense_fp4(64, 128, 256, seed=4, with_c=False)
    q = p.sfb.view(np.uint32).copy()
    rng = np.random.default_rng(5)
    shift = rng.integers(-20, 21, size=q.shape).astype(np.int64)
    b0 = ((q & 0xFF).astype(np.int64) + shift).clip(1, 254).astype(np.uint32)
    q = (q & ~np.uint32(0xFF)) | b0
    p.sfb = q.view(np.int32)
    check_tolerance(run_fp4(dg, p), oracle.gemm_fp8_fp4_nt(p.a, p.sfa, p.b, p.sfb, p.c), "fp4 scales")


def _fp4_experts(G, N, K, seed):
    ps = [inputgen.exact_dense_fp4(1, N, K, seed=seed + g, with_c=False) for g in range(G)]
    return np.stack([q.b for q in ps]), np.stack([q.sfb for q in ps])


@pytest.mark.parametrize("cfg,sk", [(None, None), ("0", None), ("6", None), ("11", None), ("0", "5"), ("6", "3")])
def test_fp4_contiguous_exact(dg, monkeypatch, cfg, sk):
    log(f"case: fp8 x fp4 contiguous exact, config {cfg}, split tail {sk}")
    if cfg is not None:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    if sk is not None:
        monkeypatch.setenv("DG_SK_SPLITS", sk)
    G, N, K = 3, 272, 512
    counts = [200, 5, 300]
    segs = [((c + 127) // 128) * 128 for c in counts]
    layout = np.full(sum(segs), -1, dtype=np.int32)
    off = 0
    for g, (cnt, sg) in enumerate(zip(counts, segs)):
        layout[off:off + cnt] = g
        off += sg
    base = inputgen.exact_dense_fp4(len(layout), N, K, seed=21)
    b, sfb = _fp4_experts(G, N, K, 30)
    d = sentinel_like((len(layout), N))
    dg.dg_m_grouped_fp8_fp4_gemm_nt_contiguous(dev(base.a), dev(base.sfa), dev(b), dev(sfb),
                                               bf16_bits_dev(base.c), d, dev(layout))
    torch.cuda.synchronize()
    got = bits_host(d)
    ref, written = oracle.m_grouped_fp8_fp4_contiguous(base.a, base.sfa, b, sfb, layout, base.c)
    assert np.array_equal(got[written], ref[written])
    assert np.all(got[~written] == 0xDEAD)


@pytest.mark.parametrize("cfg", [None, "0", "6", "11"])
def test_fp4_masked_exact(dg, monkeypatch, cfg):
    log(f"case: fp8 x fp4 masked exact, config {cfg}")
    if cfg is not None:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    G, max_m, N, K = 4, 288, 256, 384
    base = inputgen.exact_dense_fp4(G * max_m, N, K, seed=22, with_c=False)
    a = base.a.reshape(G, max_m, K)
    sfa = np.ascontiguousarray(base.sfa.reshape(K // 128, G, max_m).transpose(1, 0, 2))
    b, sfb = _fp4_experts(G, N, K, 40)
    masked_m = np.array([288, 0, 1, 140], dtype=np.int32)
    d = sentinel_like((G, max_m, N))
    dg.dg_m_grouped_fp8_fp4_gemm_nt_masked(dev(a), dev(sfa), dev(b), dev(sfb), None, d, dev(masked_m), 128)
    torch.cuda.synchronize()
    got = bits_host(d)
    ref, written = oracle.m_grouped_fp8_fp4_masked(a, sfa, b, sfb, masked_m)
    assert np.array_equal(got[written], ref[written])
    assert np.all(got[~written] == 0xDEAD)


@pytest.mark.parametrize("cfg", ["1", "0", "6"])
def test_fp4_in_place_c_equals_d(dg, monkeypatch, cfg):
    log(f"case: fp8 x fp4 in place (c == d), forced config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    p = inputgen.exact_dense_fp4(200, 464, 1024, seed=23)
    cd = bf16_bits_dev(p.c)
    dg.dg_fp8_fp4_gemm_nt(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), cd, cd)
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(cd), oracle.gemm_fp8_fp4_nt(p.a, p.sfa, p.b, p.sfb, p.c))


def test_fp4_masked_with_c(dg):
    # masked FP8 x FP4 with a bf16 C [G][max_m][N]
    log("case: fp8 x fp4 masked with C")
    G, max_m, N, K = 3, 160, 272, 512
    base = inputgen.exact_dense_fp4(G * max_m, N, K, seed=24)
    a = base.a.reshape(G, max_m, K)
    sfa = np.ascontiguousarray(base.sfa.reshape(K // 128, G, max_m).transpose(1, 0, 2))
    c = base.c.reshape(G, max_m, N)
    b, sfb = _fp4_experts(G, N, K, 50)
    masked_m = np.array([160, 3, 77], dtype=np.int32)
    d = sentinel_like((G, max_m, N))
    dg.dg_m_grouped_fp8_fp4_gemm_nt_masked(dev(a), dev(sfa), dev(b), dev(sfb), bf16_bits_dev(c), d,
                                           dev(masked_m), 64)
    torch.cuda.synchronize()
    got = bits_host(d)
    ref, written = oracle.m_grouped_fp8_fp4_masked(a, sfa, b, sfb, masked_m, c)
    assert np.array_equal(got[written], ref[written])
    assert np.all(got[~written] == 0xDEAD)
