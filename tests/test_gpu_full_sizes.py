"""Parity at the full sizes of the benchmark's layout, K-grouped and FP8 x FP4
workloads, through the C ABI and on the configuration each call chooses, on
sampled rows that the oracle computes one by one:

* the prefill problem 4096x7168x16384 stored nn, tn and tt (A stored [K][M]
  for a first "t", B stored [K][N] for a second "n"),
* the K-grouped TN call of 8 experts, M=4096 x N=7168 each, 8192 tokens,
* FP8 x FP4 at 4096x7168x16384 and at the decode shape 64x2112x7168 (with C).

Random data: the bf16 results meet |d - ref| <= 8e-3 |ref| + 1e-3 rms(ref)
and a relative Frobenius error <= 2e-3; the fp32 K-grouped results stay within
the fp32 accumulation bound of the K-grouped tests."""
import numpy as np
import pytest
import torch

import inputgen
import oracle
from tests.gpu_util import bf16_bits_dev, bits_host, check_tolerance, dev, sentinel_like

pytestmark = pytest.mark.gpu

CALLS = {"nn": "dg_fp8_gemm_nn", "tn": "dg_fp8_gemm_tn", "tt": "dg_fp8_gemm_tt"}
_PREFILL = {}


@pytest.fixture(scope="module")
def dg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_grouped_gemm_nt_amd as m
    m.dg_init()
    return m


def log(msg):
    print(msg, flush=True)


def sample_rows(M, seed, extra=(0, 1, 127, 128, 255)):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[r for r in extra if r < M], [M - 1], rng.integers(0, M, size=12)]))


def prefill():
    """The prefill problem, as generated for the benchmark (seed 0)."""
    if "p" not in _PREFILL:
        _PREFILL["p"] = inputgen.make_config(2, seed=0)
    return _PREFILL["p"]


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_prefill_layout_full_size_sampled(dg, layout):
    log(f"case: prefill 4096x7168x16384 stored {layout}, sampled rows")
    p = prefill()
    a = p.a if layout[0] == "n" else np.ascontiguousarray(p.a.T)
    b = p.b if layout[1] == "t" else np.ascontiguousarray(p.b.T)
    d = sentinel_like((p.M, p.N))
    getattr(dg, CALLS[layout])(dev(a), dev(p.sfa), dev(b), dev(p.sfb), None, d)
    torch.cuda.synchronize()
    got = bits_host(d)
    rows = sample_rows(p.M, 1)
    check_tolerance(got[rows], oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, None, rows=rows), f"prefill {layout}")


def test_kgrouped_full_size_sampled(dg):
    log("case: k-grouped 8 x 4096 x 7168, 8192 tokens, sampled rows of three groups")
    p = inputgen.make_kgrouped(8, 4096, 7168, 8192, seed=0)
    d = torch.full((p.G, p.M, p.N), -12345.5, dtype=torch.float32, device="cuda")
    dg.dg_k_grouped_fp8_gemm_tn_contiguous(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), None, d, p.ks)
    torch.cuda.synchronize()
    starts = np.concatenate([[0], np.cumsum(p.ks)])
    for g in (0, 3, 7):
        rows = sample_rows(p.M, 10 + g)
        k0, k1 = int(starts[g]), int(starts[g + 1])
        # the group's K rows and the sampled M columns form a one-group problem
        acc, mag = oracle.k_grouped_tn_acc(np.ascontiguousarray(p.a[k0:k1, rows]),
                                           np.ascontiguousarray(p.sfa[k0 // 128:k1 // 128, rows]),
                                           p.b[k0:k1], p.sfb[k0 // 128:k1 // 128], [k1 - k0])
        got = d[g][torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
        bound = 2.0 ** -24 * (2 * 128 + (k1 - k0) // 128 + 4) * mag[0] + 1e-30
        err = np.abs(got - acc[0])
        assert np.all(np.isfinite(got)), g
        assert np.all(err <= bound), f"group {g}: {int(np.sum(err > bound))} elements out of bound"


def test_fp8_fp4_prefill_full_size_sampled(dg):
    log("case: fp8 x fp4 4096x7168x16384, sampled rows")
    p = inputgen.make_dense_fp4(4096, 7168, 16384, 0, 1.0, 0.02, None, False)
    d = sentinel_like((p.M, p.N))
    dg.dg_fp8_fp4_gemm_nt(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), None, d)
    torch.cuda.synchronize()
    got = bits_host(d)
    rows = sample_rows(p.M, 2)
    check_tolerance(got[rows], oracle.gemm_fp8_fp4_nt(p.a, p.sfa, p.b, p.sfb, None, rows=rows), "fp4 prefill")


def test_fp8_fp4_decode_full_size(dg):
    log("case: fp8 x fp4 64x2112x7168 with C, every row")
    p = inputgen.make_dense_fp4(64, 2112, 7168, 0, 1.0, 0.02, 0.1, False)
    d = sentinel_like((p.M, p.N))
    dg.dg_fp8_fp4_gemm_nt(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), bf16_bits_dev(p.c), d)
    torch.cuda.synchronize()
    check_tolerance(bits_host(d), oracle.gemm_fp8_fp4_nt(p.a, p.sfa, p.b, p.sfb, p.c), "fp4 decode")
