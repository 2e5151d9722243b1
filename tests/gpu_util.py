"""Helpers shared by the GPU tests: device copies of generated problems and
the tolerance check on random data."""
import numpy as np
import torch

SENTINEL = 0xDEAD     # bf16 bit pattern left in rows the kernels must not write


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def bf16_bits_dev(x):
    return dev(np.asarray(x, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def bits_host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_f64(bits):
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def sentinel_like(shape):
    return torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16) \
        if SENTINEL < 0x8000 else \
        torch.full(shape, SENTINEL - 0x10000, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def check_tolerance(got_bits, ref_bits, what=""):
    """Element bound |d - ref| <= 8e-3 |ref| + 1e-3 rms(ref) and relative
    Frobenius error <= 2e-3, with ref the oracle's bf16 result."""
    d = bits_to_f64(got_bits).ravel()
    r = bits_to_f64(ref_bits).ravel()
    assert np.all(np.isfinite(d)), what
    rms = np.sqrt(np.mean(r * r))
    err = np.abs(d - r)
    bound = 8e-3 * np.abs(r) + 1e-3 * rms
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, f"{what}: {bad.size} elements out of bound, e.g. idx {bad[:5]} got {d[bad[:5]]} ref {r[bad[:5]]}"
    frob = np.linalg.norm(d - r) / max(np.linalg.norm(r), 1e-300)
    assert frob <= 2e-3, f"{what}: relative Frobenius error {frob}"
    return frob
