"""Parity of the K-grouped TN call (MoE weight gradient) with the oracle,
through the C ABI.  Exact-regime inputs must match bit for bit (fp32).
Random inputs must stay within an fp32 accumulation bound,
|d - ref| <= 2**-24 * (2*128 + KB + 4) * mag, where mag is |C| plus the sum of
the absolute scaled products (from the oracle) and KB the group's K blocks:
each 128-term MFMA block sum is allowed an error of one fp32 unit per addition
(2**-23 relative, which covers truncating as well as rounding adders), and the
scale product, the promotion FMA of each block and the C addition one
rounding each (2**-24 relative to mag)."""
import numpy as np
import pytest
import torch

import inputgen
import oracle
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

SENTINEL_F32 = np.float32(-12345.5)


@pytest.fixture(scope="module")
def dg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_grouped_gemm_nt_amd as m
    m.dg_init()
    return m


def log(msg):
    print(msg, flush=True)


def run_kg(dg, p, c=True, d_init=None):
    d = torch.full((p.G, p.M, p.N), float(SENTINEL_F32), dtype=torch.float32, device="cuda") \
        if d_init is None else d_init
    cc = dev(p.c) if (c and p.c is not None) else None
    dg.dg_k_grouped_fp8_gemm_tn_contiguous(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), cc, d, p.ks)
    torch.cuda.synchronize()
    return d.cpu().numpy()


def check_bound(got, p, c=True):
    acc, mag = oracle.k_grouped_tn_acc(p.a, p.sfa, p.b, p.sfb, p.ks, p.c if c else None)
    kb = (np.asarray(p.ks) // 128).astype(np.float64)[:, None, None]
    bound = 2.0 ** -24 * (2 * 128 + kb + 4) * mag + 1e-30
    err = np.abs(got.astype(np.float64) - acc)
    assert np.all(np.isfinite(got))
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{len(bad)} elements out of bound, e.g. {bad[:3]} err {err[tuple(bad[0])]} bound {bound[tuple(bad[0])]}"
    return float(np.max(err / np.maximum(mag, 1e-30)))


@pytest.mark.parametrize("ks", [[256, 0, 384], [128], [0, 128, 0, 1024, 256]])
def test_kgrouped_exact(dg, ks):
    log(f"case: k-grouped exact ks={ks}")
    p = inputgen.exact_kgrouped(len(ks), 288, 400, ks, seed=len(ks))
    got = run_kg(dg, p)
    ref = oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, p.c)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("cfg", ["0", "6", "11"])
def test_kgrouped_every_tile_config_exact(dg, monkeypatch, cfg):
    log(f"case: k-grouped exact, forced config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    p = inputgen.exact_kgrouped(4, 528, 272, [384, 128, 0, 640], seed=11)
    got = run_kg(dg, p)
    assert np.array_equal(got.view(np.uint32), oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, p.c).view(np.uint32))


@pytest.mark.parametrize("window", ["1", "4", "16"])
def test_kgrouped_k_window_orders(dg, monkeypatch, window):
    # the K order inside each group's range: groups of 1 to 9 K blocks
    log(f"case: k-grouped exact, K window {window}")
    monkeypatch.setenv("DG_K_WINDOW", window)
    p = inputgen.exact_kgrouped(5, 528, 400, [128, 512, 1152, 640, 0], seed=5)
    got = run_kg(dg, p)
    assert np.array_equal(got.view(np.uint32), oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, p.c).view(np.uint32))


def test_kgrouped_without_c_and_in_place(dg):
    log("case: k-grouped without C, then accumulating into C in place")
    p = inputgen.exact_kgrouped(3, 64, 128, [128, 256, 0], seed=3)
    got = run_kg(dg, p, c=False)
    ref0 = oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, None)
    assert np.array_equal(got.view(np.uint32), ref0.view(np.uint32))
    assert not np.any(got[2])                          # empty group without C: zeros
    d = dev(p.c.copy())                                # d == c: gradient accumulation
    dg.dg_k_grouped_fp8_gemm_tn_contiguous(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), d, d, p.ks)
    torch.cuda.synchronize()
    ref = oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, p.c)
    assert np.array_equal(d.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("pow2,cfg", [(True, None), (False, None), (False, "0"), (False, "6"), (False, "11")])
def test_kgrouped_random_bound(dg, monkeypatch, pow2, cfg):
    # with an fp32 C: the tiles up to 128x256 start their accumulators at C,
    # the 256x256 tile adds it after the K loop
    log(f"case: k-grouped random, pow2={pow2}, config {cfg}")
    if cfg is not None:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    p = inputgen.make_kgrouped(4, 512, 768, 3000, seed=7, pow2=pow2, with_c=True)
    got = run_kg(dg, p)
    rel = check_bound(got, p)
    log(f"  max error / magnitude: {rel:.3e}")


def test_kgrouped_rejects(dg):
    log("case: k-grouped argument errors")
    p = inputgen.exact_kgrouped(2, 32, 48, [128, 128], seed=1)
    d = torch.zeros((2, 32, 48), dtype=torch.float32, device="cuda")
    args = (dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), None, d)
    with pytest.raises(dg.DGError) as e:
        dg.dg_k_grouped_fp8_gemm_tn_contiguous(*args, [128, 100])          # not a multiple of 128
    assert e.value.status == -1
    q = inputgen.exact_kgrouped(1, 40, 48, [128], seed=2)                 # M = 40
    with pytest.raises(dg.DGError) as e:
        dg.dg_k_grouped_fp8_gemm_tn_contiguous(dev(q.a), dev(q.sfa), dev(q.b), dev(q.sfb), None,
                                               torch.zeros((1, 40, 48), dtype=torch.float32, device="cuda"), [128])
    assert e.value.status == -2


def test_kgrouped_rejects_too_many_groups(dg):
    log("case: k-grouped with 257 groups (the limit is 256)")
    p = inputgen.exact_kgrouped(1, 32, 48, [128], seed=5)
    d = torch.zeros((257, 32, 48), dtype=torch.float32, device="cuda")
    with pytest.raises(dg.DGError) as e:
        dg.dg_k_grouped_fp8_gemm_tn_contiguous(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), None, d,
                                               [128] + [0] * 256)
    assert e.value.status == -2
