"""DG_VALIDATE=1: the M-grouped calls check their device-resident control data
on the host before launching (a debugging aid that synchronises)."""
import numpy as np
import pytest
import torch

import inputgen
import oracle
from tests.gpu_util import bits_host, dev, sentinel_like

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_grouped_gemm_nt_amd as m
    m.dg_init()
    return m


def test_contiguous_mixed_block_is_refused(dg, monkeypatch):
    print("case: DG_VALIDATE contiguous, a block holding two experts", flush=True)
    G, N, K, M = 2, 128, 256, 256
    base = inputgen.exact_dense(M, N, K, seed=3)
    b = np.stack([inputgen.exact_dense(1, N, K, seed=5 + g).b for g in range(G)])
    sfb = np.stack([inputgen.exact_dense(1, N, K, seed=7 + g).sfb for g in range(G)])
    layout = np.array([0] * 100 + [1] * 156, dtype=np.int32)
    d = sentinel_like((M, N))
    monkeypatch.setenv("DG_VALIDATE", "1")
    with pytest.raises(dg.DGError) as e:
        dg.dg_m_grouped_fp8_gemm_nt_contiguous(dev(base.a), dev(base.sfa), dev(b), dev(sfb), None, d, dev(layout))
    assert e.value.status == -1 and "rows 0..127" in str(e.value)
    # a valid layout runs, and gives the oracle's result
    layout = np.array([0] * 100 + [-1] * 28 + [1] * 128, dtype=np.int32)
    dg.dg_m_grouped_fp8_gemm_nt_contiguous(dev(base.a), dev(base.sfa), dev(b), dev(sfb), None, d, dev(layout))
    torch.cuda.synchronize()
    ref, written = oracle.m_grouped_contiguous(base.a, base.sfa, b, sfb, layout)
    assert np.array_equal(bits_host(d)[written], ref[written])


def test_masked_out_of_range_is_refused(dg, monkeypatch):
    print("case: DG_VALIDATE masked, masked_m beyond max_m", flush=True)
    G, max_m, N, K = 3, 64, 128, 256
    base = inputgen.exact_dense(G * max_m, N, K, seed=11)
    a = base.a.reshape(G, max_m, K)
    sfa = np.ascontiguousarray(base.sfa.reshape(K // 128, G, max_m).transpose(1, 0, 2))
    b = np.stack([inputgen.exact_dense(1, N, K, seed=12 + g).b for g in range(G)])
    sfb = np.stack([inputgen.exact_dense(1, N, K, seed=15 + g).sfb for g in range(G)])
    d = sentinel_like((G, max_m, N))
    monkeypatch.setenv("DG_VALIDATE", "1")
    for bad in ([64, 65, 0], [-1, 3, 4]):
        with pytest.raises(dg.DGError) as e:
            dg.dg_m_grouped_fp8_gemm_nt_masked(dev(a), dev(sfa), dev(b), dev(sfb), None, d,
                                               dev(np.array(bad, dtype=np.int32)), 32)
        assert e.value.status == -1 and "masked_m" in str(e.value)
    mm = np.array([64, 1, 0], dtype=np.int32)
    dg.dg_m_grouped_fp8_gemm_nt_masked(dev(a), dev(sfa), dev(b), dev(sfb), None, d, dev(mm), 32)
    torch.cuda.synchronize()
    ref, written = oracle.m_grouped_masked(a, sfa, b, sfb, mm)
    assert np.array_equal(bits_host(d)[written], ref[written])
