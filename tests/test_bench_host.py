"""Host-side checks of the benchmark (no GPU): the algorithmic work it divides
by, and its refusal of more than one GPU."""
import os
import subprocess
import sys

import inputgen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_headline_algorithmic_bytes_and_flops():
    # dense decode 64x2112x7168 with C: A 64*7168, B 2112*7168, sfa 56*64 fp32,
    # sfb 17*56 fp32, C and D 64*2112 bf16
    p = inputgen.make_config(1)
    assert (p.M, p.N, p.K) == (64, 2112, 7168)
    want = 64 * 7168 + 2112 * 7168 + 56 * 64 * 4 + 17 * 56 * 4 + 2 * 64 * 2112 * 2
    assert want == 16_156_384
    assert bench.algorithmic_bytes(p) == want
    assert p.flops == 2 * 64 * 2112 * 7168


def test_fp4_decode_algorithmic_bytes():
    # B at half a byte per value and its int32 [K/128][N] E8M0 scales
    p = inputgen.make_dense_fp4(64, 2112, 7168, 0, 1.0, 0.02, 0.1, False)
    want = 64 * 7168 + 2112 * 7168 // 2 + 56 * 64 * 4 + 56 * 2112 * 4 + 2 * 64 * 2112 * 2
    assert bench.algorithmic_bytes(p) == want


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


class _W:
    def __init__(self, p, name="w"):
        self.p, self.name = p, name


def test_oracle_samples_cover_every_kind_and_count_their_flops():
    # the CPU baseline is timed on a bounded sample of each workload; its rate
    # divides the sample's own algorithmic flops
    d = inputgen.make_dense(100, 256, 256, seed=1)          # small: the whole call
    fn, flops, what = bench.oracle_sample(_W(d))
    assert flops == 2.0 * 100 * 256 * 256 and what == "the whole call"
    assert fn().shape == (100, 256)
    d = inputgen.make_dense(100, 256, 1 << 13, seed=1)     # beyond 2**27 multiply-adds: 64 rows
    fn, flops, what = bench.oracle_sample(_W(d))
    assert flops == 2.0 * 64 * 256 * (1 << 13) and "rows 0-63" in what
    assert fn().shape == (64, 256)
    c = inputgen.make_contiguous(3, 256, 256, 300, seed=2)
    fn, flops, what = bench.oracle_sample(_W(c))
    bits, written = fn()
    assert written.all() and flops == 2.0 * bits.shape[0] * 256 * 256
    m = inputgen.make_masked(4, 64, 256, 256, seed=3, expected_m=32)
    fn, flops, what = bench.oracle_sample(_W(m))
    bits, written = fn()
    assert flops == 2.0 * written.sum() * 256 * 256
    k = inputgen.make_kgrouped(3, 32, 48, 300, seed=4)
    fn, flops, what = bench.oracle_sample(_W(k))
    g = int(what.split()[1])
    assert fn().shape == (1, 32, 48) and flops == 2.0 * k.counts[g] * 32 * 48
    f4 = inputgen.make_dense_fp4(16, 256, 256, 0, 1.0, 0.02, 0.1, False)
    fn, flops, what = bench.oracle_sample(_W(f4))
    assert what == "the whole call" and fn().shape == (16, 256)


def test_cpu_baseline_record():
    rec = bench.cpu_baseline(_W(inputgen.make_dense(16, 128, 128, seed=5), "tiny"), 0.05)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOPS" and rec["value"] > 0 and rec["cores"] >= 1
    assert "the whole call of tiny" in rec["sample"]
