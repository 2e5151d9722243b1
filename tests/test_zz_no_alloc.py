"""The allocation-free dense call (dg_fp8_gemm_nt_noalloc) against the
allocating one (dg_fp8_gemm_nt), through the C ABI: two calls in a row, the
second smaller, on exact-regime inputs (bit for bit, and against the oracle)
and on random inputs (the bf16 tolerance); and the refusal of a configuration
forced beyond its scratch."""
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
    return m


def both(dg, p):
    a, b, sfa, sfb = dev(p.a), dev(p.b), dev(p.sfa), dev(p.sfb)
    c = bf16_bits_dev(p.c) if p.c is not None else None
    d0, d1 = sentinel_like((p.M, p.N)), sentinel_like((p.M, p.N))
    dg.dg_fp8_gemm_nt_noalloc(a, sfa, b, sfb, c, d1)
    torch.cuda.synchronize()
    got = bits_host(d1)
    dg.dg_fp8_gemm_nt(a, sfa, b, sfb, c, d0)
    torch.cuda.synchronize()
    return got, bits_host(d0)


# (M, N, K): the decode shape (split-K partials in the scratch), a mid-size
# shape (the split tail of the tile kernels), then smaller ones
SEQUENCES = [
    [(64, 2112, 7168), (16, 512, 1024)],
    [(512, 4096, 7168), (128, 256, 512)],
]


@pytest.mark.parametrize("shapes", SEQUENCES)
def test_exact_two_calls_bit_for_bit(dg, shapes):
    for i, (M, N, K) in enumerate(shapes):
        print(f"case: noalloc exact {M}x{N}x{K} (call {i + 1} of {len(shapes)})", flush=True)
        p = inputgen.exact_dense(M, N, K, seed=70 + i)
        got, ref_entry = both(dg, p)
        assert np.array_equal(got, ref_entry)
        if M * N * K <= 64 * 2112 * 7168:
            assert np.array_equal(got, oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c))


@pytest.mark.parametrize("shapes", SEQUENCES)
def test_random_two_calls_within_tolerance(dg, shapes):
    for i, (M, N, K) in enumerate(shapes):
        print(f"case: noalloc random {M}x{N}x{K} (call {i + 1} of {len(shapes)})", flush=True)
        p = inputgen.make_dense(M, N, K, seed=80 + i, a_std=1.0, b_std=0.02, c_std=0.1, pow2=False, name="noalloc")
        got, ref_entry = both(dg, p)
        check_tolerance(got, ref_entry, f"noalloc vs allocating entry {M}x{N}x{K}")
        if M * N * K <= 64 * 2112 * 7168:
            check_tolerance(got, oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c), f"noalloc vs oracle {M}x{N}x{K}")


def test_forced_beyond_scratch_is_refused(dg, monkeypatch):
    print("case: noalloc forced 56 splits at 64x2112x7168 (29.6 MB of partials)", flush=True)
    p = inputgen.exact_dense(64, 2112, 7168, seed=90)
    monkeypatch.setenv("DG_FORCE_CONFIG", "1")
    monkeypatch.setenv("DG_FORCE_SPLITS", "56")
    d = sentinel_like((p.M, p.N))
    with pytest.raises(dg.DGError) as e:
        dg.dg_fp8_gemm_nt_noalloc(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), bf16_bits_dev(p.c), d)
    assert e.value.status == -2 and "workspace" in str(e.value)
    torch.cuda.synchronize()
    # the allocating call has room for it and still runs
    dg.dg_fp8_gemm_nt(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), bf16_bits_dev(p.c), d)
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(d), oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c))


def test_one_launch_decode_counters_left_at_zero(dg, monkeypatch):
    # the one-launch decode keeps one counter per tile in the scratch array:
    # they start at zero with the array and every call leaves them there, so
    # calls in a row (the second on fewer tiles, the third on more) agree with
    # the allocating call and the oracle bit for bit
    monkeypatch.setenv("DG_FORCE_CONFIG", "12")
    for i, (M, N, K) in enumerate([(64, 2112, 7168), (100, 640, 4096), (64, 2112, 7168)]):
        print(f"case: noalloc one-launch decode {M}x{N}x{K} (call {i + 1} of 3)", flush=True)
        p = inputgen.exact_dense(M, N, K, seed=95 + i)
        got, ref_entry = both(dg, p)
        assert np.array_equal(got, ref_entry)
        assert np.array_equal(got, oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c))
