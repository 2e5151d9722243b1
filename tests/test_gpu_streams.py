"""Per-stream workspaces (dg_bind_stream_workspace): decode-shape calls that
split K (fp32 partials in the workspace, and for the one-launch form its
per-tile counters) enqueued on two streams at once, each stream with its own
bound workspace, give the oracle's result bit for bit; a workspace too small
for partials gives the same result without a split."""
import numpy as np
import pytest
import torch

import inputgen
import oracle
from tests.gpu_util import bf16_bits_dev, bits_host, dev, sentinel_like

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_grouped_gemm_nt_amd as m
    m.dg_init()
    return m


# 1: partials, then the reduction kernel; 12: one launch, with the per-tile
# counters in each bound workspace
@pytest.mark.parametrize("cfg", ["1", "12"])
def test_two_streams_with_their_own_workspaces(dg, monkeypatch, cfg):
    print(f"case: two streams, bound workspaces, 64x2112x7168 split-K calls overlapping, config {cfg}", flush=True)
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    probs = [inputgen.exact_dense(64, 2112, 7168, seed=200 + i) for i in range(2)]
    ins = [(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), bf16_bits_dev(p.c)) for p in probs]
    outs = [sentinel_like((64, 2112)) for _ in probs]
    streams = [torch.cuda.Stream() for _ in probs]
    wss = [torch.empty(8 << 20, dtype=torch.uint8, device="cuda") for _ in probs]
    torch.cuda.synchronize()
    try:
        for s, w in zip(streams, wss):
            dg.dg_bind_stream_workspace(s, w)
        for _ in range(20):
            for i in range(2):
                a, sfa, b, sfb, c = ins[i]
                dg.dg_fp8_gemm_nt(a, sfa, b, sfb, c, outs[i], stream=streams[i])
        torch.cuda.synchronize()
        for i, p in enumerate(probs):
            assert np.array_equal(bits_host(outs[i]), oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c)), i
    finally:
        for s in streams:
            dg.dg_bind_stream_workspace(s, None)


def test_workspace_too_small_for_partials(dg):
    print("case: a 256-byte bound workspace (no split-K possible)", flush=True)
    p = inputgen.exact_dense(64, 2112, 7168, seed=210)
    s = torch.cuda.Stream()
    w = torch.empty(256, dtype=torch.uint8, device="cuda")
    d = sentinel_like((64, 2112))
    try:
        dg.dg_bind_stream_workspace(s, w)
        dg.dg_fp8_gemm_nt(dev(p.a), dev(p.sfa), dev(p.b), dev(p.sfb), bf16_bits_dev(p.c), d, stream=s)
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(d), oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c))
    finally:
        dg.dg_bind_stream_workspace(s, None)
