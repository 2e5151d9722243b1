"""Parity of the dense nn / tn / tt calls (K-major operands) with the oracle,
through the C ABI.  Exact-regime inputs must match bit for bit; random inputs
meet the same tolerance as the NT call."""
import numpy as np
import pytest
import torch

import inputgen
import oracle
from tests.gpu_util import bf16_bits_dev, bits_host, check_tolerance, dev, sentinel_like

pytestmark = pytest.mark.gpu

CALLS = {"nn": "dg_fp8_gemm_nn", "tn": "dg_fp8_gemm_tn", "tt": "dg_fp8_gemm_tt", "nt": "dg_fp8_gemm_nt"}


@pytest.fixture(scope="module")
def dg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_grouped_gemm_nt_amd as m
    m.dg_init()
    return m


def log(msg):
    print(msg, flush=True)


def stored(layout, p):
    """The problem's operands in the layout's storage: A [K][M] for "t", B [K][N] for a second "n"."""
    a = p.a if layout[0] == "n" else np.ascontiguousarray(p.a.T)
    b = p.b if layout[1] == "t" else np.ascontiguousarray(p.b.T)
    return a, b


def run_layout(dg, layout, p, c=True):
    a, b = stored(layout, p)
    d = sentinel_like((p.M, p.N))
    cc = bf16_bits_dev(p.c) if (c and p.c is not None) else None
    getattr(dg, CALLS[layout])(dev(a), dev(p.sfa), dev(b), dev(p.sfb), cc, d)
    torch.cuda.synchronize()
    return bits_host(d), a, b


# several tiles of every configuration, ragged M and N tails (multiples of 16
# where the operand is K-major), a single K block and a long K
SHAPES = [(128, 128, 128), (304, 400, 512), (16, 48, 256), (528, 272, 1024), (64, 2112, 7168)]


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_layout_exact(dg, layout, M, N, K):
    log(f"case: {layout} exact {M}x{N}x{K}")
    p = inputgen.exact_dense(M, N, K, seed=M + N + K)
    got, a, b = run_layout(dg, layout, p)
    ref = oracle.gemm_layout(layout, a, p.sfa, b, p.sfb, p.c)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("cfg", ["0", "1", "6", "11"])
def test_layout_every_tile_config_exact(dg, monkeypatch, layout, cfg):
    log(f"case: {layout} exact, forced config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    M, N, K = 400, 592, 640
    p = inputgen.exact_dense(M, N, K, seed=7)
    got, a, b = run_layout(dg, layout, p)
    assert np.array_equal(got, oracle.gemm_layout(layout, a, p.sfa, b, p.sfb, p.c))


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_layout_random_tolerance(dg, layout):
    log(f"case: {layout} random")
    p = inputgen.make_dense(256, 384, 2048, 3, 1.0, 0.02, 0.1, False, "random")
    got, a, b = run_layout(dg, layout, p)
    check_tolerance(got, oracle.gemm_layout(layout, a, p.sfa, b, p.sfb, p.c), layout)


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("cfg", ["0", "11"])
def test_layout_matches_nt_call(dg, monkeypatch, layout, cfg):
    # one logical product, stored two ways, on the same tile configuration:
    # identical bits from both calls
    log(f"case: {layout} against the nt call, config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    p = inputgen.make_dense(512, 512, 1024, 5, 1.0, 0.02, None, True, "random")
    got, _, _ = run_layout(dg, layout, p)
    ref, _, _ = run_layout(dg, "nt", p)
    assert np.array_equal(got, ref)


def test_layout_sizes_rejected(dg):
    log("case: K-major operands with sizes that are not multiples of 16")
    p = inputgen.exact_dense(40, 48, 128, seed=1)            # M = 40
    for layout in ("tn", "tt"):
        with pytest.raises(dg.DGError) as e:
            run_layout(dg, layout, p)
        assert e.value.status == -2
    q = inputgen.exact_dense(32, 40, 128, seed=2)            # N = 40
    for layout in ("nn", "tn"):
        with pytest.raises(dg.DGError) as e:
            run_layout(dg, layout, q)
        assert e.value.status == -2
    got, a, b = run_layout(dg, "nn", p)                       # nn with M = 40 is fine
    assert np.array_equal(got, oracle.gemm_layout("nn", a, p.sfa, b, p.sfb, p.c))


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("cfg,sk", [("0", None), ("0", "16"), ("6", None), ("6", "3")])
def test_layout_split_tail_exact(dg, monkeypatch, layout, cfg, sk):
    # the items of a last partial round split over K (fp32 partials, then the
    # split reduction), with K-major operands
    log(f"case: {layout} split tail, config {cfg}, splits {sk}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    if sk is not None:
        monkeypatch.setenv("DG_SK_SPLITS", sk)
    p = inputgen.exact_dense(992, 2112, 1024, seed=14)
    got, a, b = run_layout(dg, layout, p)
    assert np.array_equal(got, oracle.gemm_layout(layout, a, p.sfa, b, p.sfb, p.c))


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_layout_decode_shape_random_tolerance(dg, layout):
    log(f"case: {layout} random, decode shape 64x2112x7168")
    p = inputgen.make_dense(64, 2112, 7168, 5, 1.0, 0.02, 0.1, True, "random")
    got, a, b = run_layout(dg, layout, p)
    check_tolerance(got, oracle.gemm_layout(layout, a, p.sfa, b, p.sfb, p.c), layout)


@pytest.mark.parametrize("cfg", ["1", "12"])
@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("splits", ["1", "3", "16"])
@pytest.mark.parametrize("M,N,K", [(64, 2112, 7168), (96, 160, 2048), (16, 16, 128)])
def test_layout_decode_kernel_exact(dg, monkeypatch, cfg, layout, splits, M, N, K):
    # the decode kernel (64x64 tiles, K split over workgroups) with K-major
    # operands staged in octets and read with transposing LDS reads; one split
    # writes D itself, more go through the fp32 partials and the reduction (1)
    # or the in-launch hand-off (12)
    log(f"case: {layout} decode kernel exact {M}x{N}x{K}, config {cfg}, forced splits {splits}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    monkeypatch.setenv("DG_FORCE_SPLITS", splits)
    p = inputgen.exact_dense(M, N, K, seed=M + K)
    got, a, b = run_layout(dg, layout, p)
    assert np.array_equal(got, oracle.gemm_layout(layout, a, p.sfa, b, p.sfb, p.c))


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("cfg", ["1", "12", "0", "11"])
def test_layout_in_place_c_equals_d(dg, monkeypatch, layout, cfg):
    log(f"case: {layout} in place (c == d), forced config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    p = inputgen.exact_dense(192, 336, 1024, seed=19)
    a, b = stored(layout, p)
    cd = bf16_bits_dev(p.c)
    getattr(dg, CALLS[layout])(dev(a), dev(p.sfa), dev(b), dev(p.sfb), cd, cd)
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(cd), oracle.gemm_layout(layout, a, p.sfa, b, p.sfb, p.c))
