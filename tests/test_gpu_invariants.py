"""Invariants of the HIP path that hold at any size, checked at the full
workload sizes the benchmark times, plus grouped calls against per-expert
dense calls.

* Linearity under power-of-two scale changes: multiplying the row scales of
  one row (one expert's B block scale) by 2^j multiplies that row (those
  columns of that expert's rows) of D by exactly 2^j when C = 0, because a
  power-of-two factor commutes with every fp32 and bf16 rounding on the way
  (no result here comes near overflow or the subnormal range); every other
  element stays bit-identical (the kernels sum in a fixed order).
* A grouped call equals, row for row and bit for bit, dense calls on each
  expert's rows with that expert's B when both run the same tile kernel
  (forced configuration, no split tail, K blocks in order): the grouping only
  selects operands.

The scale layouts follow the DeepGEMM pages (fine-grained scaling: one scale
per row per 128 K values for A, per 128x128 block for B)."""
import numpy as np
import pytest
import torch

import inputgen
from tests.gpu_util import bits_host, bits_to_f64, dev, sentinel_like

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


def call(dg, p, sfa=None, sfb=None):
    """One call with C = 0 (the linearity holds for D - C only)."""
    sfa = p.sfa if sfa is None else sfa
    sfb = p.sfb if sfb is None else sfb
    if isinstance(p, inputgen.Dense):
        d = sentinel_like((p.M, p.N))
        dg.dg_fp8_gemm_nt(dev(p.a), dev(sfa), dev(p.b), dev(sfb), None, d)
    elif isinstance(p, inputgen.Contiguous):
        d = sentinel_like((p.M, p.N))
        dg.dg_m_grouped_fp8_gemm_nt_contiguous(dev(p.a), dev(sfa), dev(p.b), dev(sfb), None, d,
                                               dev(p.grouped_layout))
    else:
        d = sentinel_like((p.G, p.max_m, p.N))
        dg.dg_m_grouped_fp8_gemm_nt_masked(dev(p.a), dev(sfa), dev(p.b), dev(sfb), None, d,
                                           dev(p.masked_m), p.expected_m)
    torch.cuda.synchronize()
    return bits_host(d)


def computed_rows(p):
    """(index tuple prefix, expert) of rows that hold results."""
    if isinstance(p, inputgen.Dense):
        return [((m,), None) for m in range(p.M)]
    if isinstance(p, inputgen.Contiguous):
        return [((m,), int(g)) for m, g in enumerate(p.grouped_layout) if 0 <= g < p.G]
    return [((g, m), g) for g in range(p.G) for m in range(min(int(p.masked_m[g]), p.max_m))]


def check_scaled(d0, d1, mask, factor, what):
    """d1 == d0 * factor exactly where mask holds, d1 == d0 bit for bit elsewhere."""
    v0, v1 = bits_to_f64(d0), bits_to_f64(d1)
    assert np.all(np.isfinite(v0[mask])), what
    assert np.array_equal(v1[mask], v0[mask] * factor[mask]), what
    assert np.array_equal(d1[~mask], d0[~mask]), what


def row_scale_change(p, rng):
    """Row scales of 8 computed rows times 2^j; returns (sfa, factor, mask)."""
    rows = computed_rows(p)
    pick = rng.choice(len(rows), size=min(8, len(rows)), replace=False)
    exps = rng.choice([-3, -1, 1, 2, 4], size=len(pick))
    sfa = p.sfa.copy()
    factor = np.ones(out_shape(p))
    mask = np.zeros(out_shape(p), dtype=bool)
    for k, e in zip(pick, exps):
        idx, _ = rows[k]
        if isinstance(p, inputgen.Masked):
            sfa[idx[0], :, idx[1]] *= 2.0 ** e
        else:
            sfa[:, idx[0]] *= 2.0 ** e
        factor[idx] = 2.0 ** e
        mask[idx] = True
    return sfa, factor, mask


def block_scale_change(p, rng):
    """Up to three B block scales (one expert's, for grouped calls) times 2^j;
    returns (sfb, factor, mask)."""
    nb_count = (p.N + 127) // 128
    sfb = p.sfb.copy()
    factor = np.ones(out_shape(p))
    mask = np.zeros(out_shape(p), dtype=bool)
    picks = []
    for _ in range(3):
        nb = int(rng.integers(0, nb_count))
        e = int(rng.choice([-2, 1, 3]))
        g = None if isinstance(p, inputgen.Dense) else int(rng.integers(0, p.G))
        if any(q[0] == nb and q[1] == g for q in picks):
            continue
        picks.append((nb, g, e))
    rows = computed_rows(p)
    for nb, g, e in picks:
        cols = slice(nb * 128, min(p.N, nb * 128 + 128))
        if g is None:
            sfb[nb, :] *= 2.0 ** e
            factor[:, cols] *= 2.0 ** e
            mask[:, cols] = True
        else:
            sfb[g, nb, :] *= 2.0 ** e
            for idx, gg in rows:
                if gg == g:
                    factor[idx + (cols,)] *= 2.0 ** e
                    mask[idx + (cols,)] = True
    return sfb, factor, mask


def out_shape(p):
    return (p.G, p.max_m, p.N) if isinstance(p, inputgen.Masked) else (p.M, p.N)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_linearity_in_scales(dg, cfg):
    log(f"case: linearity in A's row scales and B's block scales, workload {cfg}")
    p = inputgen.make_config(cfg, seed=0)
    rng = np.random.default_rng(100 + cfg)
    d0 = call(dg, p)
    sfa, factor, mask = row_scale_change(p, rng)
    check_scaled(d0, call(dg, p, sfa=sfa), mask, factor, f"workload {cfg} row scales")
    sfb, factor, mask = block_scale_change(p, rng)
    check_scaled(d0, call(dg, p, sfb=sfb), mask, factor, f"workload {cfg} block scales")


def dense_bits(dg, a, sfa, b, sfb):
    d = sentinel_like((a.shape[0], b.shape[0]))
    dg.dg_fp8_gemm_nt(dev(a), dev(np.ascontiguousarray(sfa)), dev(b), dev(sfb), None, d)
    torch.cuda.synchronize()
    return bits_host(d)


@pytest.mark.parametrize("cfg", ["0", "6"])
def test_contiguous_equals_per_expert_dense(dg, monkeypatch, cfg):
    log(f"case: contiguous vs per-expert dense calls, config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    monkeypatch.setenv("DG_SK_SPLITS", "0")
    monkeypatch.setenv("DG_K_WINDOW", "1")      # the dense calls in the M-grouped forms' K order
    p = inputgen.make_contiguous(5, 384, 1024, 900, seed=8)
    got = call(dg, p)
    for g in range(p.G):
        rows = np.nonzero(p.grouped_layout == g)[0]
        if rows.size == 0:
            continue
        ref = dense_bits(dg, p.a[rows], p.sfa[:, rows], p.b[g], p.sfb[g])
        assert np.array_equal(got[rows], ref), f"expert {g}"


@pytest.mark.parametrize("cfg", ["0", "11"])
def test_masked_equals_per_expert_dense(dg, monkeypatch, cfg):
    log(f"case: masked vs per-expert dense calls, config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    monkeypatch.setenv("DG_SK_SPLITS", "0")
    monkeypatch.setenv("DG_K_WINDOW", "1")      # the dense calls in the M-grouped forms' K order
    p = inputgen.make_masked(5, 320, 512, 768, seed=9, masked_m=[0, 320, 1, 129, 255])
    got = call(dg, p)
    for g in range(p.G):
        m = int(p.masked_m[g])
        if m == 0:
            continue
        ref = dense_bits(dg, p.a[g][:m], p.sfa[g][:, :m], p.b[g], p.sfb[g])
        assert np.array_equal(got[g][:m], ref), f"expert {g}"
