"""Calls captured in a HIP graph and replayed several times, with eager calls
and synchronisations between the replays; every replay is checked against the
oracle.  Covers the launch shapes beyond the decode path: the split tail (tile
kernel plus its reduction), the masked form reading masked_m on the device
(changed between replays: a replay must use the current values), the K-grouped
form, FP8 x FP4 decode, and the power-of-two scale gate (scales changed between
replays: the on-device check must pick the kernel for the current scales).
Exact-regime inputs, so every comparison is bit for bit."""
import numpy as np
import pytest
import torch

import inputgen
import oracle
from tests.gpu_util import SENTINEL, bf16_bits_dev, bits_host, dev, sentinel_like

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


def capture(fn):
    """Runs fn once eagerly (library set-up), then captures it in a graph."""
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        fn()
    torch.cuda.synchronize()
    return graph


def reset(t):
    t.view(torch.int16).fill_(SENTINEL - 0x10000)


@pytest.mark.parametrize("cfg,sk", [("0", "3"), ("6", "4")])
def test_split_tail_graph(dg, monkeypatch, cfg, sk):
    log(f"case: split tail under graph replay, config {cfg}, splits {sk}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    monkeypatch.setenv("DG_SK_SPLITS", sk)
    p = inputgen.exact_dense(1000, 2112, 1024, seed=60)
    ref = oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)
    a, sfa, b, sfb, c = dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), bf16_bits_dev(p.c)
    out, eager = sentinel_like((p.M, p.N)), sentinel_like((p.M, p.N))
    graph = capture(lambda: dg.dg_fp8_gemm_nt(a, sfa, b, sfb, c, out))
    for rep in range(3):
        reset(out)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(out), ref), rep
        dg.dg_fp8_gemm_nt(a, sfa, b, sfb, c, eager)
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(eager), ref), rep


def test_masked_graph_reads_current_masked_m(dg):
    log("case: masked under graph replay, masked_m changed between replays")
    G, max_m, N, K = 4, 256, 384, 512
    p = inputgen.exact_dense(G * max_m, N, K, seed=61, with_c=False)
    a = p.a.reshape(G, max_m, K)
    sfa = np.ascontiguousarray(p.sfa.reshape(K // 128, G, max_m).transpose(1, 0, 2))
    bs = [inputgen.exact_dense(1, N, K, seed=70 + g, with_c=False) for g in range(G)]
    b = np.stack([q.b for q in bs])
    sfb = np.stack([q.sfb for q in bs])
    mms = [np.array(v, dtype=np.int32) for v in ([256, 0, 17, 130], [1, 255, 0, 64], [128, 128, 300, 3])]
    a_d, sfa_d, b_d, sfb_d = dev(a), dev(sfa), dev(b), dev(sfb)
    mm_d = dev(mms[0])
    out = sentinel_like((G, max_m, N))
    graph = capture(lambda: dg.dg_m_grouped_fp8_gemm_nt_masked(a_d, sfa_d, b_d, sfb_d, None, out, mm_d, 128))
    for rep, mm in enumerate(mms):
        mm_d.copy_(torch.from_numpy(mm))
        reset(out)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = bits_host(out)
        ref, written = oracle.m_grouped_masked(a, sfa, b, sfb, mm)
        assert np.array_equal(got[written], ref[written]), rep
        assert np.all(got[~written] == SENTINEL), rep


def test_kgrouped_graph(dg):
    log("case: k-grouped under graph replay")
    p = inputgen.exact_kgrouped(3, 256, 272, [384, 0, 256], seed=62)
    ref = oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, p.c)
    a, sfa, b, sfb, c = dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), dev(p.c)
    out = torch.empty((p.G, p.M, p.N), dtype=torch.float32, device="cuda")
    ks = list(p.ks)
    graph = capture(lambda: dg.dg_k_grouped_fp8_gemm_tn_contiguous(a, sfa, b, sfb, c, out, ks))
    for rep in range(3):
        out.fill_(-1.0)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), rep
        dg.dg_k_grouped_fp8_gemm_tn_contiguous(a, sfa, b, sfb, c, torch.empty_like(out), ks)
        torch.cuda.synchronize()


def test_fp4_decode_graph(dg):
    log("case: fp8 x fp4 decode (split K, two launches) under graph replay")
    p = inputgen.exact_dense_fp4(64, 2112, 7168, seed=63)
    ref = oracle.gemm_fp8_fp4_nt(p.a, p.sfa, p.b, p.sfb, p.c)
    a, sfa, b, sfb, c = dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), bf16_bits_dev(p.c)
    out = sentinel_like((p.M, p.N))
    graph = capture(lambda: dg.dg_fp8_fp4_gemm_nt(a, sfa, b, sfb, c, out))
    for rep in range(3):
        reset(out)
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(out), ref), rep
        dg.dg_fp8_fp4_gemm_nt(a, sfa, b, sfb, c, sentinel_like((p.M, p.N)))
        torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", ["7", "10"])
def test_scale_gate_graph_follows_current_scales(dg, monkeypatch, cfg):
    # a gated pair (the scale check, the MFMA-scaled kernel and the general
    # kernel) in one graph: with power-of-two scales the MFMA-scaled kernel
    # works; after one A scale is changed on the device to a value that is not
    # a power of two, a replay of the same graph must run the general kernel
    log(f"case: scale gate under graph replay, config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    p = inputgen.exact_dense(512, 768, 512, seed=64)
    a, b, sfb, c = dev(p.a), dev(p.b), dev(p.sfb), bf16_bits_dev(p.c)
    sfa = dev(p.sfa)
    out = sentinel_like((p.M, p.N))
    graph = capture(lambda: dg.dg_fp8_gemm_nt(a, sfa, b, sfb, c, out))
    sfa_odd = p.sfa.copy()
    sfa_odd[1, 7] *= 1.5                       # not a power of two: the general kernel's case
    for rep, s in enumerate([p.sfa, sfa_odd, p.sfa]):
        sfa.copy_(torch.from_numpy(s))
        reset(out)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = oracle.gemm_nt(p.a, s, p.b, p.sfb, p.c)
        if rep == 1:
            # 1.5 x a power of two keeps the exact regime only up to rounding of
            # row 7: compare the other rows bit for bit and row 7 within 1 ulp
            got = bits_host(out)
            mask = np.ones(p.M, dtype=bool)
            mask[7] = False
            assert np.array_equal(got[mask], ref[mask]), rep
            assert np.max(np.abs(got[7].astype(np.int32) - ref[7].astype(np.int32))) <= 1, rep
        else:
            assert np.array_equal(bits_host(out), ref), rep
