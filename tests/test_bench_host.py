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
