"""The launch-configuration choice, queried through dg_choose_config (host
code only, no device): the benchmark's workloads get the kernels their
measurements favour, and the forced-configuration switch acts as on the calls.

Configuration ids: 0 128x128, 1 decode (64x64 tiles, K split over
workgroups, a reduction launch), 5 256x128, 6 128x256, 7 128x256 with
power-of-two scales in the MFMA, 9 narrow (16x48 over the whole K), 11 256x256,
12 decode with the splits' hand-off inside one launch."""
import pytest

import moe_grouped_gemm_nt_amd as dg


@pytest.fixture(autouse=True)
def no_forcing(monkeypatch):
    for k in ("DG_FORCE_CONFIG", "DG_FORCE_SPLITS", "DG_SK_SPLITS"):
        monkeypatch.delenv(k, raising=False)


@pytest.mark.parametrize("form,rows,N,K,G,layout,has_c,want", [
    # decode shapes: too few 128x128 tiles for half the CUs; 56 K blocks in
    # 7 splits of 8 fill 231 of 256 CUs with 33 64x64 tiles
    ("dense", 64, 2112, 7168, 1, "nt", True, (1, 7)),
    ("dense", 64, 2112, 7168, 1, "nn", True, (1, 7)),
    ("dense", 64, 2112, 7168, 1, "fp4", True, (1, 7)),
    # 4 K blocks: one split, one launch
    ("dense", 128, 256, 512, 1, "nt", False, (1, 1)),
    # prefill: 448 256x256 tiles, under two rounds; with a C the 128x256 tile
    ("dense", 4096, 7168, 16384, 1, "nt", False, (11, 1)),
    ("dense", 4096, 7168, 16384, 1, "nt", True, (6, 1)),
    ("dense", 4096, 7168, 16384, 1, "fp4", False, (11, 1)),
    # contiguous calls keep 128-row tiles
    ("contiguous", 8704, 4096, 7168, 8, "nt", False, (6, 1)),
    # masked: 32 groups of about 128 rows: 256x128 tiles (three K blocks in
    # flight); larger groups 256x256; an FP4 B keeps 256x256
    ("masked", 128, 4096, 7168, 32, "nt", False, (5, 1)),
    ("masked", 192, 4096, 7168, 32, "nt", False, (11, 1)),
    ("masked", 128, 4096, 7168, 32, "fp4", False, (11, 1)),
    # masked, 8 groups of 16 rows: 128 tiles of 128x256 leave half the CUs idle
    ("masked", 16, 4096, 7168, 8, "nt", False, (0, 1)),
    # at most 16 rows and 16x48 tiles for half the CUs: the narrow kernel
    ("dense", 16, 7168, 2048, 1, "nt", False, (9, 1)),
    # one round either way: the split-tail estimate decides, with a 5% margin
    ("dense", 1024, 2112, 7168, 1, "nt", False, (6, 1)),
    ("dense", 512, 4096, 16384, 1, "nt", False, (6, 1)),
    ("dense", 512, 7168, 7168, 1, "nt", False, (0, 1)),
    ("dense", 768, 4096, 7168, 1, "nt", False, (0, 1)),
    # several rounds: rounds times rows loaded per K block
    ("dense", 1024, 7168, 7168, 1, "nt", False, (6, 1)),
    ("dense", 2048, 7168, 7168, 1, "nt", False, (11, 1)),
])
def test_choice(form, rows, N, K, G, layout, has_c, want):
    assert dg.dg_choose_config(form, rows, N, K, G, 256, layout, has_c) == want


def test_forced_configuration(monkeypatch):
    monkeypatch.setenv("DG_FORCE_CONFIG", "7")          # power-of-two kernel, behind the scale check
    assert dg.dg_choose_config("dense", 4096, 7168, 16384)[0] == 7
    monkeypatch.setenv("DG_FORCE_CONFIG", "11")         # forced: kept even with a C
    assert dg.dg_choose_config("dense", 4096, 7168, 16384, has_c=True)[0] == 11
    monkeypatch.setenv("DG_FORCE_CONFIG", "1")          # the decode kernel is dense-only: ignored
    assert dg.dg_choose_config("contiguous", 4096, 7168, 16384)[0] == 6
    assert dg.dg_choose_config("dense", 64, 2112, 7168)[0] == 1
    monkeypatch.setenv("DG_FORCE_SPLITS", "3")          # at most 8 K blocks per split: 7 at least
    assert dg.dg_choose_config("dense", 64, 2112, 7168) == (1, 7)
    monkeypatch.setenv("DG_FORCE_SPLITS", "14")
    assert dg.dg_choose_config("dense", 64, 2112, 7168) == (1, 14)
    monkeypatch.setenv("DG_FORCE_CONFIG", "12")         # the one-launch decode: dense only
    assert dg.dg_choose_config("dense", 64, 2112, 7168) == (12, 14)
    assert dg.dg_choose_config("dense", 512, 4096, 7168)[0] == 12
    assert dg.dg_choose_config("dense", 4096, 4096, 7168)[0] == 1    # 4096 tiles: more than its counters
    assert dg.dg_choose_config("contiguous", 4096, 7168, 16384)[0] == 6


@pytest.mark.parametrize("args", [
    ("dense", 0, 10, 128), ("dense", 8, 0, 128), ("dense", 8, 10, 100), ("dense", 8, 10, -128),
])
def test_invalid_query(args):
    with pytest.raises(dg.DGError) as e:
        dg.dg_choose_config(*args)
    assert e.value.status == -1


def test_forced_decode_or_narrow_ignored_without_k_blocks(monkeypatch):
    # K = 0 gives D = C; the decode and narrow kernels index their first K
    # block's scales, so a forced choice of them is ignored there
    for forced in ("1", "9", "12"):
        monkeypatch.setenv("DG_FORCE_CONFIG", forced)
        assert dg.dg_choose_config("dense", 64, 2112, 0)[0] not in (1, 9, 12)
        assert dg.dg_choose_config("dense", 64, 2112, 128)[0] == int(forced)
