"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Exact-regime inputs (small-integer codes, power-of-two scales) must match bit
for bit; random inputs must meet |d - ref| <= 8e-3 |ref| + 1e-3 rms(ref) and a
relative Frobenius error <= 2e-3.  The five workloads at their full sizes are
checked on every element they write (the prefill, contiguous and masked ones
take tens of seconds of fp64 BLAS in the oracle), rows they must not write on
the sentinel left in them."""
import os

import numpy as np
import pytest
import torch

import inputgen
import oracle
from tests.gpu_util import (SENTINEL, bf16_bits_dev, bits_host, check_tolerance, dev,
                            sentinel_like)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_grouped_gemm_nt_amd as m
    m.dg_init()
    return m


def run_dense(dg, p, c_dev=None, out=None):
    a, b = dev(p.a), dev(p.b)
    sfa, sfb = dev(p.sfa), dev(p.sfb)
    c = c_dev if c_dev is not None else (bf16_bits_dev(p.c) if p.c is not None else None)
    d = out if out is not None else sentinel_like((p.M, p.N))
    dg.dg_fp8_gemm_nt(a, sfa, b, sfb, c, d)
    torch.cuda.synchronize()
    return bits_host(d)


def log(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------------------
# dense
# ---------------------------------------------------------------------------
def test_dense_config0_full(dg):
    log("case: dense config 0 (128x256x512) full oracle")
    p = inputgen.make_config(0)
    got = run_dense(dg, p)
    ref = oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)
    check_tolerance(got, ref, "config0")


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_dense_config0_seeds_exact_regime(dg, seed):
    log(f"case: exact regime 128x256x512 seed {seed}")
    p = inputgen.exact_dense(128, 256, 512, seed=seed)
    got = run_dense(dg, p)
    ref = oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)
    assert np.array_equal(got, ref)


def test_dense_config1_decode_full(dg):
    log("case: dense config 1 (64x2112x7168, C) full oracle")
    p = inputgen.make_config(1)
    got = run_dense(dg, p)
    ref = oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)
    check_tolerance(got, ref, "config1")


def test_dense_decode_exact_regime(dg):
    log("case: exact regime 64x2112x7168")
    p = inputgen.exact_dense(64, 2112, 7168, seed=4)
    got = run_dense(dg, p)
    ref = oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("M,N,K", [
    (1, 8, 128), (7, 64, 256), (64, 2112, 128), (100, 200, 256), (129, 136, 384),
    (257, 300, 640), (33, 130, 1024), (500, 520, 256), (16, 4096, 1024),
])
def test_dense_edge_shapes_exact(dg, M, N, K):
    log(f"case: exact edge shape {M}x{N}x{K}")
    p = inputgen.exact_dense(M, N, K, seed=M + N)
    got = run_dense(dg, p)
    ref = oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)
    assert np.array_equal(got, ref), f"{np.sum(got != ref)} mismatches"


def test_dense_subnormal_codes_exact(dg):
    log("case: subnormal codes 70x90x512")
    p = inputgen.exact_subnormal_dense(70, 90, 512, seed=8)
    got = run_dense(dg, p)
    assert np.array_equal(got, oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb))


@pytest.mark.parametrize("M,N,K,pow2", [(200, 384, 1536, False), (64, 520, 2048, True), (300, 1000, 512, False)])
def test_dense_random_tolerance(dg, M, N, K, pow2):
    log(f"case: random {M}x{N}x{K} pow2={pow2}")
    p = inputgen.make_dense(M, N, K, seed=3, b_std=0.02, c_std=0.1, pow2=pow2)
    got = run_dense(dg, p)
    check_tolerance(got, oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c), f"{M}x{N}x{K}")


def test_dense_in_place_c_equals_d(dg):
    log("case: in-place c == d")
    p = inputgen.exact_dense(96, 200, 512, seed=12)
    cd = bf16_bits_dev(p.c)
    got = run_dense(dg, p, c_dev=cd, out=cd)
    assert np.array_equal(got, oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c))


def test_dense_k_zero_gives_c(dg):
    log("case: K = 0")
    rng = np.random.default_rng(0)
    c = inputgen.bf16_bits_from_f32(rng.standard_normal((5, 9)).astype(np.float32))
    a = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
    b = torch.zeros((9, 0), dtype=torch.uint8, device="cuda")
    sfa = torch.zeros((0, 5), dtype=torch.float32, device="cuda")
    sfb = torch.zeros((1, 0), dtype=torch.float32, device="cuda")
    # empty tensors may carry null data pointers: give the library valid ones
    a = torch.zeros((5, 16), dtype=torch.uint8, device="cuda")[:, :0]
    d = sentinel_like((5, 9))
    import moe_grouped_gemm_nt_amd._lib as L
    lib = L.load()
    scratch = torch.zeros(64, dtype=torch.float32, device="cuda")
    rc = lib.dg_fp8_gemm_nt(scratch.data_ptr(), scratch.data_ptr(), scratch.data_ptr(), scratch.data_ptr(),
                            bf16_bits_dev(c).data_ptr(), d.data_ptr(), 5, 9, 0, None)
    assert rc == 0
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(d), c)
    del a, b, sfa, sfb


@pytest.mark.parametrize("window", ["1", "2", "4", "8", "16", "3", "32"])
def test_dense_k_window_orders(dg, monkeypatch, window):
    # every K order of the tile kernels sums the same blocks, so the exact
    # regime stays bit for bit: K block counts below, at and past whole
    # windows, several tiles (each starts at its own offset in a window), and
    # the split tail (each split orders its own range); a window that is not
    # a power of two up to 16 falls back to the default order
    log(f"case: dense K window {window}")
    monkeypatch.setenv("DG_K_WINDOW", window)
    for cfg, (M, N, K) in [("11", (512, 512, 13 * 128)), ("6", (384, 768, 16 * 128)),
                           ("0", (256, 384, 3 * 128)), ("5", (512, 256, 21 * 128))]:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
        p = inputgen.exact_dense(M, N, K, seed=int(window) + M)
        assert np.array_equal(run_dense(dg, p), oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)), (cfg, M, N, K)
    monkeypatch.setenv("DG_FORCE_CONFIG", "6")
    monkeypatch.setenv("DG_SK_SPLITS", "3")
    p = inputgen.exact_dense(1152, 2048, 40 * 128, seed=int(window))
    assert np.array_equal(run_dense(dg, p), oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)), "split tail"


# decode configurations: 1 = partials, then the reduction kernel; 12 = one
# launch, the tile's last split summing the others' device-coherent partials
DECODE_CFGS = ["1", "12"]


@pytest.mark.parametrize("cfg", DECODE_CFGS)
def test_dense_split_k_forced_matches(dg, monkeypatch, cfg):
    log(f"case: forced split-K, config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    p = inputgen.exact_dense(64, 640, 4096, seed=13)
    ref = oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)
    for splits in ["1", "2", "3", "8"]:
        monkeypatch.setenv("DG_FORCE_SPLITS", splits)
        got = run_dense(dg, p)
        assert np.array_equal(got, ref), splits
    monkeypatch.delenv("DG_FORCE_SPLITS")


@pytest.mark.parametrize("cfg", DECODE_CFGS)
def test_decode_split_k_exact(dg, monkeypatch, cfg):
    log(f"case: decode split-K, several split counts, config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    for M, N, K in [(64, 2112, 7168), (17, 200, 2048), (100, 640, 4096)]:
        p = inputgen.exact_dense(M, N, K, seed=M + K)
        ref = oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)
        for splits in ["0", "5", "8"]:
            monkeypatch.setenv("DG_FORCE_SPLITS", splits)
            got = run_dense(dg, p)
            assert np.array_equal(got, ref), (M, N, K, splits)
    monkeypatch.delenv("DG_FORCE_SPLITS")


@pytest.mark.parametrize("cfg", DECODE_CFGS)
def test_decode_split_k_no_stale_partials(dg, monkeypatch, cfg):
    log(f"case: decode split-K, alternating inputs on one workspace, config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    probs = [inputgen.exact_dense(64, 2112, 7168, seed=s) for s in (40, 41, 42)]
    refs = [oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c) for p in probs]
    devs = [(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), bf16_bits_dev(p.c)) for p in probs]
    outs = [sentinel_like((64, 2112)) for _ in probs]
    for rep in range(4):
        for i in range(3):
            dg.dg_fp8_gemm_nt(*devs[i], outs[i])
        torch.cuda.synchronize()
        for i in range(3):
            assert np.array_equal(bits_host(outs[i]), refs[i]), (rep, i)


@pytest.mark.parametrize("cfg", DECODE_CFGS)
def test_decode_split_k_graph_replays(dg, monkeypatch, cfg):
    # the call's launches (partials, then their reduction; or the one-launch
    # form with its counters) captured in a graph and replayed several times,
    # with eager calls between the replays
    log(f"case: decode split-K under graph replay, config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    probs = [inputgen.exact_dense(64, 2112, 7168, seed=s) for s in (50, 51)]
    refs = [oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c) for p in probs]
    devs = [(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), bf16_bits_dev(p.c)) for p in probs]
    outs = [sentinel_like((64, 2112)) for _ in probs]
    eager = sentinel_like((64, 2112))
    for i in range(2):                      # warm-up outside the capture (library set-up)
        dg.dg_fp8_gemm_nt(*devs[i], outs[i])
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(2):
            dg.dg_fp8_gemm_nt(*devs[i], outs[i])
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.view(torch.int16).fill_(SENTINEL - 0x10000)
        graph.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert np.array_equal(bits_host(outs[i]), refs[i]), (rep, i)
        dg.dg_fp8_gemm_nt(*devs[rep % 2], eager)
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(eager), refs[rep % 2]), rep


def test_decode_one_launch_many_tiles(dg, monkeypatch):
    # the one-launch decode past one round of the chip: 128 tiles in 7 splits
    # (896 items, 3.5 rounds), 99 tiles in 3 splits, 64 tiles in 2 splits,
    # then the default shape
    log("case: one-launch decode, several rounds of items per XCD")
    monkeypatch.setenv("DG_FORCE_CONFIG", "12")
    for M, N, K in [(128, 4096, 7168), (130, 2112, 3072), (200, 1000, 1280), (64, 2112, 7168)]:
        p = inputgen.exact_dense(M, N, K, seed=M + N)
        assert np.array_equal(run_dense(dg, p), oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)), (M, N, K)


# "7", "8" and "10" are the power-of-two-scale kernels, run behind the scale check beside
# configuration 4: exact inputs take it, the non-power-of-two case must not.
@pytest.mark.parametrize("cfg", ["0", "1", "2", "3", "4", "5", "6", "7", "8", "9", "10", "11", "12"])
def test_dense_every_tile_config(dg, monkeypatch, cfg):
    log(f"case: forced config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    p = inputgen.exact_dense(300, 520, 768, seed=14)
    got = run_dense(dg, p)
    assert np.array_equal(got, oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c))
    q = inputgen.make_dense(200, 300, 1024, seed=15, b_std=0.02, c_std=0.1, pow2=False)
    check_tolerance(run_dense(dg, q), oracle.gemm_nt(q.a, q.sfa, q.b, q.sfb, q.c), f"cfg{cfg}")


@pytest.mark.parametrize("M,N,K", [(64, 2112, 7168), (1, 8, 128), (17, 200, 640), (100, 520, 1024),
                                   (64, 2112, 128), (33, 4096, 512), (16, 48, 384), (64, 130, 896)])
def test_dense_narrow_kernel_exact(dg, monkeypatch, M, N, K):
    # the whole-K kernel for few rows: exact regime, ragged M, N and block counts
    log(f"case: narrow kernel exact {M}x{N}x{K}")
    monkeypatch.setenv("DG_FORCE_CONFIG", "9")
    p = inputgen.exact_dense(M, N, K, seed=M * 7 + K)
    got = run_dense(dg, p)
    ref = oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)
    assert np.array_equal(got, ref), f"{np.sum(got != ref)} mismatches"


def test_dense_narrow_kernel_decode_random(dg, monkeypatch):
    log("case: narrow kernel, dense config 1 (64x2112x7168, C) full oracle")
    monkeypatch.setenv("DG_FORCE_CONFIG", "9")
    p = inputgen.make_config(1)
    check_tolerance(run_dense(dg, p), oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c), "narrow config1")


@pytest.mark.parametrize("cfg", ["8", "10"])
@pytest.mark.parametrize("pow2", [True, False])
def test_dense_scale_gate_random(dg, monkeypatch, pow2, cfg):
    # the scale check picks the power-of-two kernel or the general one
    log(f"case: gated pair cfg {cfg}, 1024x1040x2048 pow2={pow2}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    p = inputgen.make_dense(1024, 1040, 2048, seed=21, b_std=0.02, c_std=0.1, pow2=pow2)
    got = run_dense(dg, p)
    check_tolerance(got, oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c), f"gate pow2={pow2}")


def test_dense_scale_gate_one_bad_scale(dg, monkeypatch):
    # power-of-two scales except one A scale and, separately, one B scale that
    # are not: the general kernel must do the work both times
    log("case: gated pair, a single non-power-of-two scale")
    monkeypatch.setenv("DG_FORCE_CONFIG", "7")
    p = inputgen.exact_dense(300, 520, 768, seed=22)
    for which in ("sfa", "sfb"):
        s = getattr(p, which).copy()
        flat = s.reshape(-1)
        flat[flat.size // 2] *= np.float32(1.5)       # exact: small-integer codes times 3/2
        args = dict(a=p.a, sfa=p.sfa, b=p.b, sfb=p.sfb)
        args[which] = s
        d = sentinel_like((p.M, p.N))
        dg.dg_fp8_gemm_nt(dev(args["a"]), dev(args["sfa"]), dev(args["b"]), dev(args["sfb"]),
                          bf16_bits_dev(p.c), d)
        torch.cuda.synchronize()
        ref = oracle.gemm_nt(args["a"], args["sfa"], args["b"], args["sfb"], p.c)
        assert np.array_equal(bits_host(d), ref), which


def test_dense_scale_gate_after_other_verdicts(dg, monkeypatch):
    # alternate pow2 and non-pow2 calls on one stream: each call's verdicts
    # must be its own
    log("case: gated pair, alternating scale kinds")
    monkeypatch.setenv("DG_FORCE_CONFIG", "7")
    good = inputgen.exact_dense(256, 384, 512, seed=23)
    bad = inputgen.make_dense(256, 384, 512, seed=24, b_std=0.02, c_std=0.1, pow2=False)
    outs = []
    for rep in range(3):
        for p in (good, bad):
            d = sentinel_like((p.M, p.N))
            dg.dg_fp8_gemm_nt(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), bf16_bits_dev(p.c), d)
            outs.append((p, d))
    torch.cuda.synchronize()
    ref_good = oracle.gemm_nt(good.a, good.sfa, good.b, good.sfb, good.c)
    ref_bad = oracle.gemm_nt(bad.a, bad.sfa, bad.b, bad.sfb, bad.c)
    for p, d in outs:
        if p is good:
            assert np.array_equal(bits_host(d), ref_good)
        else:
            check_tolerance(bits_host(d), ref_bad, "alternating non-pow2")


@pytest.mark.slow
def test_dense_config2_prefill_full(dg):
    # every element of the 4096 x 7168 result against the oracle's (about a
    # TFLOP of fp64 BLAS on the host: tens of seconds)
    log("case: dense config 2 (4096x7168x16384) full oracle")
    p = inputgen.make_config(2)
    got = run_dense(dg, p)
    ref = oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, None)
    check_tolerance(got, ref, "config2 full")


@pytest.mark.slow
def test_dense_prefill_exact_regime_sampled(dg):
    log("case: exact regime 1024x7168x16384 sampled")
    p = inputgen.exact_dense(1024, 7168, 16384, seed=16, e_min=-1, e_span=2)
    got = run_dense(dg, p)
    rows = np.array([0, 5, 130, 511, 700, 1023])
    assert np.array_equal(got[rows], oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c, rows=rows))


# ---------------------------------------------------------------------------
# contiguous
# ---------------------------------------------------------------------------
def run_contig(dg, p, c=None):
    d = sentinel_like((p.M, p.N))
    dg.dg_m_grouped_fp8_gemm_nt_contiguous(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb),
                                           c, d, dev(p.grouped_layout))
    torch.cuda.synchronize()
    return bits_host(d)


def test_contiguous_small_random(dg):
    log("case: contiguous 4 experts, N=384, K=1024")
    p = inputgen.make_contiguous(4, 384, 1024, 700, seed=1)
    got = run_contig(dg, p)
    ref, written = oracle.m_grouped_contiguous(p.a, p.sfa, p.b, p.sfb, p.grouped_layout)
    assert written.all()
    check_tolerance(got, ref, "contiguous small")


@pytest.mark.parametrize("cfg", ["0", "2", "3", "4", "5", "6", "7", "8", "10", "11"])
def test_contiguous_every_tile_config_exact(dg, monkeypatch, cfg):
    log(f"case: contiguous exact, forced config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    G, N, K = 3, 384, 768
    counts = np.array([200, 5, 300])
    segs = [((c + 127) // 128) * 128 for c in counts]
    M = sum(segs)
    layout = np.full(M, -1, dtype=np.int32)
    off = 0
    for g, (cnt, sg) in enumerate(zip(counts, segs)):
        layout[off:off + cnt] = g
        off += sg
    base = inputgen.exact_dense(M, N, K, seed=9)
    b = np.stack([inputgen.exact_dense(1, N, K, seed=60 + g).b for g in range(G)])
    sfb = np.stack([inputgen.exact_dense(1, N, K, seed=70 + g).sfb for g in range(G)])
    d = sentinel_like((M, N))
    dg.dg_m_grouped_fp8_gemm_nt_contiguous(dev(base.a), dev(base.sfa), dev(b), dev(sfb),
                                           bf16_bits_dev(base.c), d, dev(layout))
    torch.cuda.synchronize()
    got = bits_host(d)
    ref, written = oracle.m_grouped_contiguous(base.a, base.sfa, b, sfb, layout, base.c)
    assert np.array_equal(got[written], ref[written])
    assert np.all(got[~written] == SENTINEL)


@pytest.mark.parametrize("cfg", ["0", "3", "4", "5", "6", "7", "8", "10", "11"])
def test_masked_every_tile_config_exact(dg, monkeypatch, cfg):
    log(f"case: masked exact, forced config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    G, max_m, N, K = 5, 320, 256, 512
    base = inputgen.exact_dense(G * max_m, N, K, seed=33)
    a = base.a.reshape(G, max_m, K)
    sfa = np.ascontiguousarray(base.sfa.reshape(K // 128, G, max_m).transpose(1, 0, 2))
    b = np.stack([inputgen.exact_dense(1, N, K, seed=80 + g).b for g in range(G)])
    sfb = np.stack([inputgen.exact_dense(1, N, K, seed=90 + g).sfb for g in range(G)])
    masked_m = np.array([320, 0, 1, 129, 257], dtype=np.int32)
    d = sentinel_like((G, max_m, N))
    dg.dg_m_grouped_fp8_gemm_nt_masked(dev(a), dev(sfa), dev(b), dev(sfb), None, d, dev(masked_m), 128)
    torch.cuda.synchronize()
    got = bits_host(d)
    ref, written = oracle.m_grouped_masked(a, sfa, b, sfb, masked_m)
    assert np.array_equal(got[written], ref[written])
    assert np.all(got[~written] == SENTINEL)


@pytest.mark.parametrize("cfg", [None, "5", "11"])
def test_contiguous_exact_with_padding_ids_and_empty_expert(dg, monkeypatch, cfg):
    # with 256-row tiles two of the three tiles hold two experts each
    log(f"case: contiguous exact, -1 padding rows, an empty expert, C, config {cfg}")
    if cfg is not None:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    G, N, K = 5, 200, 512
    rng = np.random.default_rng(3)
    counts = np.array([130, 0, 7, 256, 1])
    segs = [((c + 127) // 128) * 128 for c in counts]
    M = sum(segs)
    layout = np.full(M, -1, dtype=np.int32)
    off = 0
    for g, (cnt, sg) in enumerate(zip(counts, segs)):
        layout[off:off + cnt] = g
        off += sg
    base = inputgen.exact_dense(M, N, K, seed=4)
    b = np.stack([inputgen.exact_dense(1, N, K, seed=10 + g).b for g in range(G)])
    sfb = np.stack([inputgen.exact_dense(1, N, K, seed=20 + g).sfb for g in range(G)])
    c = base.c
    d = sentinel_like((M, N))
    dg.dg_m_grouped_fp8_gemm_nt_contiguous(dev(base.a), dev(base.sfa), dev(b), dev(sfb),
                                           bf16_bits_dev(c), d, dev(layout))
    torch.cuda.synchronize()
    got = bits_host(d)
    ref, written = oracle.m_grouped_contiguous(base.a, base.sfa, b, sfb, layout, c)
    assert np.array_equal(got[written], ref[written])
    assert np.all(got[~written] == SENTINEL)
    del rng


@pytest.mark.parametrize("cfg,sk", [(None, "0"), (None, "4"), ("0", "0"), ("0", "4"), ("6", "4"), ("11", None),
                                    ("7", None), ("8", None), ("10", None)])
def test_contiguous_exact_out_of_range_padding_ids(dg, monkeypatch, cfg, sk):
    # padding rows carry ids outside [0, G) other than -1 (G, G + 3, a large
    # id): a block's valid rows must still be computed, and the padding rows
    # left untouched, with the split tail on and off
    log(f"case: contiguous exact, padding ids >= G, config {cfg}, split tail {sk}")
    if cfg is not None:
        monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    if sk is not None:
        monkeypatch.setenv("DG_SK_SPLITS", sk)
    G, N, K = 4, 200, 768
    counts = np.array([130, 7, 256, 1])
    segs = [((c + 127) // 128) * 128 for c in counts]
    M = sum(segs)
    pad_ids = np.array([G, G + 3, 1 << 20, -1], dtype=np.int32)
    layout = np.empty(M, dtype=np.int32)
    off = 0
    for g, (cnt, sg) in enumerate(zip(counts, segs)):
        layout[off:off + cnt] = g
        layout[off + cnt:off + sg] = pad_ids[np.arange(sg - cnt) % len(pad_ids)]
        off += sg
    base = inputgen.exact_dense(M, N, K, seed=41)
    b = np.stack([inputgen.exact_dense(1, N, K, seed=110 + g).b for g in range(G)])
    sfb = np.stack([inputgen.exact_dense(1, N, K, seed=120 + g).sfb for g in range(G)])
    d = sentinel_like((M, N))
    dg.dg_m_grouped_fp8_gemm_nt_contiguous(dev(base.a), dev(base.sfa), dev(b), dev(sfb),
                                           bf16_bits_dev(base.c), d, dev(layout))
    torch.cuda.synchronize()
    got = bits_host(d)
    ref, written = oracle.m_grouped_contiguous(base.a, base.sfa, b, sfb, layout, base.c)
    assert written.sum() == counts.sum()
    assert np.array_equal(got[written], ref[written])
    assert np.all(got[~written] == SENTINEL)


@pytest.mark.slow
def test_contiguous_config3_full(dg):
    # every row of every expert against the oracle; padding rows untouched
    log("case: contiguous config 3 (8 experts, 8192 rows, N=4096, K=7168) full oracle")
    p = inputgen.make_config(3)
    got = run_contig(dg, p)
    ref, written = oracle.m_grouped_contiguous(p.a, p.sfa, p.b, p.sfb, p.grouped_layout)
    assert written.sum() == p.real_rows or written.sum() == p.M    # padding carries -1 or its expert's id
    check_tolerance(got[written], ref[written], "config3 full")
    assert np.all(got[~written] == SENTINEL)


# ---------------------------------------------------------------------------
# masked
# ---------------------------------------------------------------------------
def run_masked(dg, p, expected_m=None, c=None):
    d = sentinel_like((p.G, p.max_m, p.N))
    dg.dg_m_grouped_fp8_gemm_nt_masked(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), c, d,
                                       dev(p.masked_m), p.expected_m if expected_m is None else expected_m)
    torch.cuda.synchronize()
    return bits_host(d)


def test_masked_small_random(dg):
    log("case: masked 6 groups, max_m 192, N=256, K=768")
    p = inputgen.make_masked(6, 192, 256, 768, seed=2, masked_m=[0, 1, 127, 128, 192, 300])
    got = run_masked(dg, p)
    ref, written = oracle.m_grouped_masked(p.a, p.sfa, p.b, p.sfb, p.masked_m)
    check_tolerance(got[written], ref[written], "masked small")
    assert np.all(got[~written] == SENTINEL)


@pytest.mark.parametrize("expected_m", [1, 64, 128, 256])
def test_masked_exact_independent_of_expected_m(dg, expected_m):
    log(f"case: masked exact, expected_m {expected_m}")
    G, max_m, N, K = 4, 256, 320, 1024
    base = inputgen.exact_dense(G * max_m, N, K, seed=31)
    a = base.a.reshape(G, max_m, K)
    sfa = np.ascontiguousarray(base.sfa.reshape(K // 128, G, max_m).transpose(1, 0, 2))
    b = np.stack([inputgen.exact_dense(1, N, K, seed=40 + g).b for g in range(G)])
    sfb = np.stack([inputgen.exact_dense(1, N, K, seed=50 + g).sfb for g in range(G)])
    masked_m = np.array([0, 255, 256, 17], dtype=np.int32)
    c = base.c.reshape(G, max_m, N)
    d = sentinel_like((G, max_m, N))
    dg.dg_m_grouped_fp8_gemm_nt_masked(dev(a), dev(sfa), dev(b), dev(sfb), bf16_bits_dev(c), d,
                                       dev(masked_m), expected_m)
    torch.cuda.synchronize()
    got = bits_host(d)
    ref, written = oracle.m_grouped_masked(a, sfa, b, sfb, masked_m, c)
    assert np.array_equal(got[written], ref[written])
    assert np.all(got[~written] == SENTINEL)


@pytest.mark.slow
def test_masked_config4_full(dg):
    # every group's first masked_m rows against the oracle; the rest untouched
    log("case: masked config 4 (32 experts, max_m 256, N=4096, K=7168) full oracle")
    p = inputgen.make_config(4)
    got = run_masked(dg, p)
    ref, written = oracle.m_grouped_masked(p.a, p.sfa, p.b, p.sfb, p.masked_m)
    check_tolerance(got[written], ref[written], "config4 full")
    assert np.all(got[~written] == SENTINEL)
    for g in range(p.G):
        m = int(min(max(p.masked_m[g], 0), p.max_m))
        if m:
            assert not np.any(got[g, :m] == SENTINEL)


# ---------------------------------------------------------------------------
# split tail: the last, partly filled round of tile-kernel items split over K
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,sk", [("6", None), ("6", "2"), ("6", "7"), ("6", "0"), ("0", "2"), ("3", "4")])
def test_dense_split_tail_exact(dg, monkeypatch, cfg, sk):
    log(f"case: dense split tail, config {cfg}, splits {sk}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    if sk is not None:
        monkeypatch.setenv("DG_SK_SPLITS", sk)
    p = inputgen.exact_dense(1000, 2112, 1024, seed=12)
    got = run_dense(dg, p)
    assert np.array_equal(got, oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c))


@pytest.mark.parametrize("sk", [None, "3", "8"])
def test_contiguous_split_tail_exact(dg, monkeypatch, sk):
    log(f"case: contiguous split tail, splits {sk}")
    monkeypatch.setenv("DG_FORCE_CONFIG", "6")
    if sk is not None:
        monkeypatch.setenv("DG_SK_SPLITS", sk)
    G, N, K = 3, 2048, 1024
    counts = [300, 500, 200]
    segs = [((c + 127) // 128) * 128 for c in counts]
    M = sum(segs)
    layout = np.full(M, -1, dtype=np.int32)
    off = 0
    for g, (cnt, sg) in enumerate(zip(counts, segs)):
        layout[off:off + cnt] = g
        off += sg
    base = inputgen.exact_dense(M, N, K, seed=13)
    b = np.stack([inputgen.exact_dense(1, N, K, seed=90 + g).b for g in range(G)])
    sfb = np.stack([inputgen.exact_dense(1, N, K, seed=95 + g).sfb for g in range(G)])
    d = sentinel_like((M, N))
    dg.dg_m_grouped_fp8_gemm_nt_contiguous(dev(base.a), dev(base.sfa), dev(b), dev(sfb),
                                           bf16_bits_dev(base.c), d, dev(layout))
    torch.cuda.synchronize()
    got = bits_host(d)
    ref, written = oracle.m_grouped_contiguous(base.a, base.sfa, b, sfb, layout, base.c)
    assert np.array_equal(got[written], ref[written])
    assert np.all(got[~written] == SENTINEL)


def test_dense_split_tail_random_tolerance(dg, monkeypatch):
    log("case: dense split tail, random inputs")
    monkeypatch.setenv("DG_FORCE_CONFIG", "6")
    p = inputgen.make_dense(1000, 2112, 3072, 7, 1.0, 0.02, 0.1, False, "random")
    check_tolerance(run_dense(dg, p), oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c), "split tail")


def test_dense_long_k_wide_n_decode_shape(dg):
    # 64 rows, N = 16000, K = 16384: few enough 128x128 tiles for the decode
    # kernel's range, but its K splits would need more than two rounds of the
    # chip and more fp32 partials than the workspace holds, so the call takes
    # a tile kernel
    log("case: dense 64x16000x16384 (decode-shaped, long K, wide N), sampled rows")
    p = inputgen.make_dense(64, 16000, 16384, 17, 1.0, 0.02, 0.1, True, "wide")
    got = run_dense(dg, p)
    rows = np.array([0, 1, 31, 32, 63])
    check_tolerance(got[rows], oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c, rows=rows), "64x16000x16384")


def test_dense_rejects_too_wide_n(dg):
    # N = 2**22: the tile kernels' column offsets would leave 32 bits; real
    # buffers of that shape, so nothing is out of bounds even if it launched
    log("case: dense 1 x 4194304 x 128 is rejected")
    N = 1 << 22
    a = torch.zeros((1, 128), dtype=torch.uint8, device="cuda")
    b = torch.zeros((N, 128), dtype=torch.uint8, device="cuda")
    sfa = torch.ones((1, 1), dtype=torch.float32, device="cuda")
    sfb = torch.ones((N // 128, 1), dtype=torch.float32, device="cuda")
    d = torch.zeros((1, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dg.DGError) as e:
        dg.dg_fp8_gemm_nt(a, sfa, b, sfb, None, d)
    assert e.value.status == -2


@pytest.mark.parametrize("cfg", ["1", "0", "6", "11"])
def test_dense_in_place_every_path(dg, monkeypatch, cfg):
    # c == d through the decode kernel (one split writes D itself; several go
    # through the reduction), the tile kernels that read C a strip ahead of
    # their stores (0, 6) and the one that reads it per element (11), and the
    # split tail
    log(f"case: in-place c == d, forced config {cfg}")
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    for M, N, K in [(96, 200, 512), (300, 2112, 1024)]:
        p = inputgen.exact_dense(M, N, K, seed=M + 1)
        cd = bf16_bits_dev(p.c)
        got = run_dense(dg, p, c_dev=cd, out=cd)
        assert np.array_equal(got, oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)), (M, N, K)
