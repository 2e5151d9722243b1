"""The seeded generator and quantiser that feed both the oracle and the GPU path."""
import numpy as np
import torch

import inputgen


def _vals(codes):
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_encode_ties_and_saturation():
    x = np.array([17.0, 19.0, 2.0 ** -10, 3 * 2.0 ** -11, 464.0, 1e6, -1e6, 448.0, 0.0], dtype=np.float32)
    got = _vals(inputgen.encode_e4m3(x))
    assert got.tolist() == [16.0, 20.0, 0.0, 2.0 ** -9, 448.0, 448.0, -448.0, 448.0, 0.0]


def test_pow2_ceil_scales():
    amax = np.array([448.0, 449.0, 224.0, 1.0, 0.0, 896.0 * 1.5], dtype=np.float32)
    s = inputgen._scales_from_amax(amax, pow2=True)
    assert s.tolist() == [1.0, 2.0, 0.5, 2.0 ** -8, 1.0, 4.0]
    s2 = inputgen._scales_from_amax(amax, pow2=False)
    assert s2[1] == np.float32(449.0) / np.float32(448.0) and s2[4] == 1.0


def test_quantize_rows_roundtrip_error_bounded():
    rng = inputgen.rng_for(0)
    x = rng.standard_normal((16, 512), dtype=np.float32)
    codes, sfa = inputgen.quantize_rows(x, pow2=True)
    assert codes.shape == (16, 512) and sfa.shape == (4, 16)
    deq = _vals(codes) * np.repeat(sfa.T, 128, axis=1)
    # e4m3 keeps 4 significant bits: relative error <= 2**-4 on normal values
    big = np.abs(x) > 0.05 * np.abs(x).max()
    assert np.all(np.abs(deq - x)[big] <= 2.0 ** -4 * np.abs(x)[big] + 1e-6)
    # the block amax lands within the top binade of the e4m3 range
    amax_code = np.abs(_vals(codes)).reshape(16, 4, 128).max(axis=2)
    assert np.all(amax_code <= 448) and np.all(amax_code > 224 - 1e-9)


def test_quantize_blocks_partial_last_block():
    rng = inputgen.rng_for(1)
    x = rng.standard_normal((200, 256), dtype=np.float32)
    x[150:] *= 100.0           # the partial block's own amax must be used
    codes, sfb = inputgen.quantize_blocks(x, pow2=True)
    assert sfb.shape == (2, 2)
    assert np.all(sfb[1] > 50 * sfb[0])
    deq = _vals(codes[128:]) * np.repeat(sfb[1], 128)[None, :]
    assert np.allclose(deq, x[128:], rtol=2.0 ** -4, atol=sfb[1].max() * 2.0 ** -9)


def test_configs_shapes_and_determinism():
    p0 = inputgen.make_config(0)
    p0b = inputgen.make_config(0)
    assert np.array_equal(p0.a, p0b.a) and np.array_equal(p0.sfb, p0b.sfb)
    assert (p0.M, p0.N, p0.K) == (128, 256, 512) and p0.c is None
    assert np.all(np.log2(p0.sfa) == np.rint(np.log2(p0.sfa)))
    p1 = inputgen.make_dense(64, 2112, 1024, seed=0, b_std=0.02, c_std=0.1)
    assert p1.sfb.shape == (17, 8) and p1.c.shape == (64, 2112)


def test_contiguous_layout_segments():
    p = inputgen.make_contiguous(8, 256, 256, 1000, seed=3)
    assert p.counts.sum() == 1000 and p.M % 128 == 0
    off = 0
    for g in range(8):
        seg = -(-int(p.counts[g]) // 128) * 128
        assert np.all(p.grouped_layout[off:off + seg] == g)
        assert np.all(p.a[off + p.counts[g]:off + seg] == 0)
        off += seg
    q = inputgen.make_contiguous(4, 256, 256, 300, seed=3, pad_id=-1)
    assert (q.grouped_layout == -1).sum() == q.M - 300


def test_masked_draws():
    p = inputgen.make_masked(6, 64, 256, 256, seed=2)
    assert p.a.shape == (6, 64, 256) and p.sfa.shape == (6, 2, 64)
    assert np.all((p.masked_m >= 0) & (p.masked_m <= 64))


def test_exact_regime_generators():
    p = inputgen.exact_dense(8, 8, 256, seed=0)
    v = _vals(p.a)
    assert np.array_equal(v, np.rint(v)) and np.abs(v).max() <= 4
    s = inputgen.exact_subnormal_dense(4, 4, 256)
    assert np.abs(_vals(s.a)).max() < 0.25
