"""Seeded random cases across the calls, operand storages, forced
configurations and split settings, each compared bit for bit with the oracle
on exact-regime inputs (integer codes, power-of-two scales, integer C: every
fp32 sum the kernels form is exact in any order).

The cases are drawn once from a fixed seed, so a failure names a case that
reruns identically.  Shapes are ragged (M and N not multiples of the tiles,
1 row, 1 column where the storage allows it) and K runs from one K block to
24 (K-grouped: groups of 0 to 9 K blocks, fp32 C and D).  Forced configurations that do not apply to a call are ignored by the
library (it then chooses by itself), so every drawn combination is valid.

A second set of cases draws random data (A ~ N(0,1), B ~ N(0,0.02), C ~
N(0,0.1), scales amax/448 not rounded to powers of two, so the general
promotion path runs) and checks the bf16 bound |d - ref| <= 8e-3 |ref| +
1e-3 rms(ref) with a relative Frobenius error <= 2e-3 (K-grouped: the fp32
accumulation bound of the K-grouped tests)."""
import numpy as np
import pytest
import torch

import inputgen
import oracle
from tests.gpu_util import SENTINEL, bf16_bits_dev, bits_host, check_tolerance, dev, sentinel_like

pytestmark = pytest.mark.gpu

FORMS = ["nt"] * 12 + ["nn", "tn", "tt"] * 3 + ["fp4"] * 7 + ["contiguous"] * 7 + ["masked"] * 7 + \
        ["fp4_contiguous"] * 3 + ["fp4_masked"] * 3 + ["kgrouped"] * 5
CALLS = {"nt": "dg_fp8_gemm_nt", "nn": "dg_fp8_gemm_nn", "tn": "dg_fp8_gemm_tn", "tt": "dg_fp8_gemm_tt"}


def draw_cases(n=160, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        form = str(rng.choice(FORMS))
        K = 128 * int(rng.integers(1, 25))
        a_kmajor = form in ("tn", "tt", "kgrouped")
        b_kmajor = form in ("nn", "tn", "kgrouped")
        M = int(rng.choice([1, 16, 64, 100, 128, 250, 333, 512, 700]))
        M = max(16, M // 16 * 16) if a_kmajor else M
        N = int(rng.choice([1, 48, 130, 256, 400, 777, 1100, 2112]))
        N = max(16, N // 16 * 16) if b_kmajor else N
        cfg = rng.choice([None, None, "0", "1", "2", "3", "4", "5", "6", "7", "8", "9", "10", "11", "12"])
        env = {}
        if cfg is not None:
            env["DG_FORCE_CONFIG"] = str(cfg)
        r = rng.random()
        if r < 0.25:
            env["DG_SK_SPLITS"] = "0"
        elif r < 0.5:
            env["DG_SK_SPLITS"] = str(int(rng.integers(2, 17)))
        if cfg in ("1", "12") and rng.random() < 0.5:
            env["DG_FORCE_SPLITS"] = str(int(rng.integers(1, 9)))
        case = dict(i=i, form=form, M=M, N=N, K=K, env=env, with_c=bool(rng.random() < 0.5),
                    seed=int(rng.integers(0, 1 << 30)))
        if form in ("contiguous", "fp4_contiguous", "masked", "fp4_masked"):
            G = int(rng.integers(1, 6))
            case["G"] = G
            if "contiguous" in form:
                # counts include empty experts; each segment is padded to 128 rows
                case["counts"] = [int(x) for x in rng.choice([0, 1, 5, 100, 128, 129, 300], size=G)]
            else:
                max_m = int(rng.choice([1, 64, 129, 256, 320]))
                case["max_m"] = max_m
                case["masked_m"] = [int(x) for x in rng.integers(0, max_m + 1, size=G)]
                case["expected_m"] = int(rng.choice([1, 64, 128, 256]))
        if form == "kgrouped":
            case["ks"] = [128 * int(x) for x in rng.choice([0, 1, 2, 5, 9], size=int(rng.integers(1, 6)))]
        cases.append(case)
    return cases


CASES = draw_cases()


def case_id(c):
    if "counts" in c:
        shape = f"counts{'_'.join(map(str, c['counts']))}x{c['N']}x{c['K']}"
    elif "masked_m" in c:
        shape = f"G{c['G']}x{c['max_m']}x{c['N']}x{c['K']}-m{'_'.join(map(str, c['masked_m']))}"
    elif "ks" in c:
        shape = f"{c['M']}x{c['N']}-ks{'_'.join(map(str, c['ks']))}"
    else:
        shape = f"{c['M']}x{c['N']}x{c['K']}"
    return f"{c['i']}-{c['form']}-{shape}" + ("-c" if c["with_c"] else "") + \
        "".join(f"-{k[3:].lower()}{v}" for k, v in sorted(c["env"].items()))


@pytest.fixture(scope="module")
def dg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_grouped_gemm_nt_amd as m
    m.dg_init()
    return m


def expert_weights(G, N, K, seed, fp4):
    """Per-expert B and its scales, stacked on a leading group axis."""
    make = inputgen.exact_dense_fp4 if fp4 else inputgen.exact_dense
    ps = [make(1, N, K, seed=seed + g, with_c=False) for g in range(G)]
    return np.stack([q.b for q in ps]), np.stack([q.sfb for q in ps])


def run_dense_case(dg, c):
    M, N, K = c["M"], c["N"], c["K"]
    if c["form"] == "fp4":
        p = inputgen.exact_dense_fp4(M, N, K, seed=c["seed"], with_c=c["with_c"])
        ref = oracle.gemm_fp8_fp4_nt(p.a, p.sfa, p.b, p.sfb, p.c)
        a, b, fn = p.a, p.b, "dg_fp8_fp4_gemm_nt"
    else:
        p = inputgen.exact_dense(M, N, K, seed=c["seed"], with_c=c["with_c"])
        layout = c["form"]
        a = p.a if layout[0] == "n" else np.ascontiguousarray(p.a.T)
        b = p.b if layout[1] == "t" else np.ascontiguousarray(p.b.T)
        ref = oracle.gemm_layout(layout, a, p.sfa, b, p.sfb, p.c)
        fn = CALLS[layout]
    d = sentinel_like((M, N))
    cc = bf16_bits_dev(p.c) if p.c is not None else None
    getattr(dg, fn)(dev(a), dev(p.sfa), dev(b), dev(p.sfb), cc, d)
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(d), ref)


def run_contiguous_case(dg, c):
    N, K, G = c["N"], c["K"], c["G"]
    fp4 = c["form"].startswith("fp4")
    segs = [(n + 127) // 128 * 128 for n in c["counts"]]
    M = max(sum(segs), 128)                    # all-empty: one padding block
    layout = np.full(M, -1, dtype=np.int32)
    off = 0
    for g, (cnt, sg) in enumerate(zip(c["counts"], segs)):
        layout[off:off + cnt] = g
        off += sg
    base = inputgen.exact_dense(M, N, K, seed=c["seed"], with_c=c["with_c"])
    b, sfb = expert_weights(G, N, K, c["seed"] + 1, fp4)
    d = sentinel_like((M, N))
    cc = bf16_bits_dev(base.c) if base.c is not None else None
    fn = dg.dg_m_grouped_fp8_fp4_gemm_nt_contiguous if fp4 else dg.dg_m_grouped_fp8_gemm_nt_contiguous
    fn(dev(base.a), dev(base.sfa), dev(b), dev(sfb), cc, d, dev(layout))
    torch.cuda.synchronize()
    got = bits_host(d)
    ref_fn = oracle.m_grouped_fp8_fp4_contiguous if fp4 else oracle.m_grouped_contiguous
    ref, written = ref_fn(base.a, base.sfa, b, sfb, layout, base.c)
    assert np.array_equal(got[written], ref[written])
    assert np.all(got[~written] == SENTINEL)


def run_masked_case(dg, c):
    N, K, G, max_m = c["N"], c["K"], c["G"], c["max_m"]
    fp4 = c["form"].startswith("fp4")
    base = inputgen.exact_dense(G * max_m, N, K, seed=c["seed"], with_c=c["with_c"])
    a = base.a.reshape(G, max_m, K)
    sfa = np.ascontiguousarray(base.sfa.reshape(K // 128, G, max_m).transpose(1, 0, 2))
    cm = base.c.reshape(G, max_m, N) if base.c is not None else None
    b, sfb = expert_weights(G, N, K, c["seed"] + 1, fp4)
    masked_m = np.array(c["masked_m"], dtype=np.int32)
    d = sentinel_like((G, max_m, N))
    cc = bf16_bits_dev(cm) if cm is not None else None
    fn = dg.dg_m_grouped_fp8_fp4_gemm_nt_masked if fp4 else dg.dg_m_grouped_fp8_gemm_nt_masked
    fn(dev(a), dev(sfa), dev(b), dev(sfb), cc, d, dev(masked_m), c["expected_m"])
    torch.cuda.synchronize()
    got = bits_host(d)
    ref_fn = oracle.m_grouped_fp8_fp4_masked if fp4 else oracle.m_grouped_masked
    ref, written = ref_fn(a, sfa, b, sfb, masked_m, cm)
    assert np.array_equal(got[written], ref[written])
    assert np.all(got[~written] == SENTINEL)


def run_kgrouped_case(dg, c):
    p = inputgen.exact_kgrouped(len(c["ks"]), c["M"], c["N"], c["ks"], seed=c["seed"], with_c=c["with_c"])
    ref = oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, p.c)
    d = torch.full((p.G, p.M, p.N), -12345.5, dtype=torch.float32, device="cuda")
    cc = dev(p.c) if p.c is not None else None
    dg.dg_k_grouped_fp8_gemm_tn_contiguous(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), cc, d, p.ks)
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("case", CASES, ids=case_id)
def test_random_case_exact(dg, monkeypatch, case):
    print(f"case: {case_id(case)}", flush=True)
    for k, v in case["env"].items():
        monkeypatch.setenv(k, v)
    if case["form"] == "kgrouped":
        run_kgrouped_case(dg, case)
    elif "contiguous" in case["form"]:
        run_contiguous_case(dg, case)
    elif "masked" in case["form"]:
        run_masked_case(dg, case)
    else:
        run_dense_case(dg, case)


RANDOM_FORMS = ("nt", "nn", "tn", "tt", "fp4", "contiguous", "masked", "kgrouped")
RANDOM_CASES = [c for c in draw_cases(n=96, seed=2027) if c["form"] in RANDOM_FORMS][:56]


def run_random_case(dg, c):
    M, N, K, form, seed = c["M"], c["N"], c["K"], c["form"], c["seed"]
    c_std = 0.1 if c["with_c"] else None
    if form == "fp4":
        p = inputgen.make_dense_fp4(M, N, K, seed, 1.0, 0.02, c_std, False)
        d = sentinel_like((M, N))
        dg.dg_fp8_fp4_gemm_nt(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb),
                              bf16_bits_dev(p.c) if p.c is not None else None, d)
        torch.cuda.synchronize()
        check_tolerance(bits_host(d), oracle.gemm_fp8_fp4_nt(p.a, p.sfa, p.b, p.sfb, p.c), form)
    elif form in CALLS:
        p = inputgen.make_dense(M, N, K, seed, 1.0, 0.02, c_std, False)
        a = p.a if form[0] == "n" else np.ascontiguousarray(p.a.T)
        b = p.b if form[1] == "t" else np.ascontiguousarray(p.b.T)
        d = sentinel_like((M, N))
        getattr(dg, CALLS[form])(dev(a), dev(p.sfa), dev(b), dev(p.sfb),
                                 bf16_bits_dev(p.c) if p.c is not None else None, d)
        torch.cuda.synchronize()
        check_tolerance(bits_host(d), oracle.gemm_layout(form, a, p.sfa, b, p.sfb, p.c), form)
    elif form == "contiguous":
        p = inputgen.make_contiguous(c["G"], N, K, max(1, sum(c["counts"])), seed, pow2=False,
                                     with_c=c["with_c"], pad_id=-1)
        d = sentinel_like((p.M, N))
        dg.dg_m_grouped_fp8_gemm_nt_contiguous(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb),
                                               bf16_bits_dev(p.c) if p.c is not None else None, d,
                                               dev(p.grouped_layout))
        torch.cuda.synchronize()
        got = bits_host(d)
        ref, written = oracle.m_grouped_contiguous(p.a, p.sfa, p.b, p.sfb, p.grouped_layout, p.c)
        check_tolerance(got[written], ref[written], form)
        assert np.all(got[~written] == SENTINEL)
    elif form == "masked":
        p = inputgen.make_masked(c["G"], c["max_m"], N, K, seed, c["expected_m"], pow2=False,
                                 with_c=c["with_c"], masked_m=c["masked_m"])
        d = sentinel_like((p.G, p.max_m, N))
        dg.dg_m_grouped_fp8_gemm_nt_masked(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb),
                                           bf16_bits_dev(p.c) if p.c is not None else None, d,
                                           dev(p.masked_m), p.expected_m)
        torch.cuda.synchronize()
        got = bits_host(d)
        ref, written = oracle.m_grouped_masked(p.a, p.sfa, p.b, p.sfb, p.masked_m, p.c)
        if written.any():
            check_tolerance(got[written], ref[written], form)
        assert np.all(got[~written] == SENTINEL)
    else:
        p = inputgen.make_kgrouped(len(c["ks"]), M, N, max(1, sum(c["ks"])), seed, pow2=False,
                                   with_c=c["with_c"])
        d = torch.full((p.G, p.M, p.N), -12345.5, dtype=torch.float32, device="cuda")
        dg.dg_k_grouped_fp8_gemm_tn_contiguous(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb),
                                               dev(p.c) if p.c is not None else None, d, p.ks)
        torch.cuda.synchronize()
        got = d.cpu().numpy().astype(np.float64)
        acc, mag = oracle.k_grouped_tn_acc(p.a, p.sfa, p.b, p.sfb, p.ks, p.c)
        kb = (np.asarray(p.ks) // 128).astype(np.float64)[:, None, None]
        bound = 2.0 ** -24 * (2 * 128 + kb + 4) * mag + 1e-30
        assert np.all(np.isfinite(got)) and np.all(np.abs(got - acc) <= bound)


@pytest.mark.parametrize("case", RANDOM_CASES, ids=case_id)
def test_random_case_tolerance(dg, monkeypatch, case):
    print(f"case: random data {case_id(case)}", flush=True)
    for k, v in case["env"].items():
        monkeypatch.setenv(k, v)
    run_random_case(dg, case)
