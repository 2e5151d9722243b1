"""ctypes binding and timing of the microbenchmarks in libdg_ceilings.so
(include/dg_ceilings.h): the FP8 MFMA loop rate, the memory rates workgroups
reach with the kernels' load forms, and the cost of one launch.

Every figure is timed with HIP events around a graph of launches replayed on
one stream, the way bench.py times the GEMM calls."""
from __future__ import annotations

import ctypes
import os

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CEILINGS_PATH = os.path.join(_PKG_DIR, "libdg_ceilings.so")
MFMA_FLOP = 2 * 16 * 16 * 128          # one 16x16x128 MFMA
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(CEILINGS_PATH):
            raise RuntimeError(f"{CEILINGS_PATH} is missing: build it with `python -m moe_grouped_gemm_nt_amd.build`")
        lib = ctypes.CDLL(CEILINGS_PATH)
        vp, ci, cl = ctypes.c_void_p, ctypes.c_int, ctypes.c_long
        lib.dgc_stream.argtypes = [vp, cl, ci, ci, vp, vp]
        lib.dgc_empty.argtypes = [ci, vp]
        lib.dgc_mfma.argtypes = [ci, ci, ci, vp, vp]
        lib.dgc_chase.argtypes = [vp, ci, ci, vp, vp]
        lib.dgc_fill.argtypes = [vp, cl, ci, ci, vp, vp]
        for f in (lib.dgc_stream, lib.dgc_empty, lib.dgc_mfma, lib.dgc_chase, lib.dgc_fill):
            f.restype = ci
        _lib = lib
    return _lib


def _time_graph(torch, launches, reps=3):
    """Captures the callables in `launches` into one graph on a side stream,
    replays it once untimed, then `reps` times timed; returns the best
    replay's milliseconds."""
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        for f in launches:
            f(stream.cuda_stream)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1)
        best = t if best is None else min(best, t)
    return best


def _ok(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} returned {rc}")


def measure(torch, num_cus=None):
    """Returns a dict of measured ceilings (see the keys' names)."""
    lib = load()
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {"num_cus": num_cus}

    # one launch: a graph of 200 empty kernels of num_cus workgroups
    n = 200
    ms = _time_graph(torch, [lambda s: _ok(lib.dgc_empty(num_cus, s), "dgc_empty")] * n)
    out["empty_kernel_us_per_launch"] = round(ms * 1e3 / n, 3)

    # MFMA loop: 4 waves per workgroup, 1, 2 or 4 workgroups per CU
    sink = torch.empty(4 * num_cus * 256, dtype=torch.float32, device="cuda")
    iters = 2048
    for promote in (0, 1):
        for per_cu in (1, 2, 4):
            grid = per_cu * num_cus
            ms = _time_graph(torch, [lambda s, g=grid, p=promote: _ok(
                lib.dgc_mfma(iters, g, p, ctypes.c_void_p(sink.data_ptr()), s), "dgc_mfma")], reps=3)
            flops = grid * 4 * iters * 8 * MFMA_FLOP
            out[f"mfma_fp8_{'promoted' if promote else 'chained'}_{per_cu * 4}waves_per_cu_pflops"] = \
                round(flops / (ms * 1e-3) / 1e15, 3)

    # rings for the round-trip latencies below (built first, so that the
    # streams in between evict them from every cache): one lane, dependent accesses.  Rings of random
    # cycles over 4 KiB-spaced slots: 2 MiB (fits one XCD's L2) and 1 GiB
    # (beyond every cache).
    import numpy as np
    rng = np.random.default_rng(0)

    def ring_of(nbytes):
        slots = nbytes // 4096
        perm = rng.permutation(slots)
        nxt = np.empty(slots, dtype=np.int64)
        nxt[perm] = np.roll(perm, -1)
        host = np.zeros(nbytes // 4, dtype=np.int32)
        host[np.arange(slots) * 1024] = (nxt * 1024).astype(np.int32)
        return torch.from_numpy(host).cuda()

    small, big = ring_of(2 << 20), ring_of(1 << 30)

    # memory: workgroups of 4 waves reading bytes_per_wg each.  "hbm": every
    # launch of the graph reads its own region of a 1 GiB buffer (4x the
    # last-level cache), so the bytes come from HBM; "cached": every launch
    # reads the same region, which the caches then hold.
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    isink = torch.empty(8 * num_cus, dtype=torch.int32, device="cuda")
    modes = {0: "lds15", 1: "lds31", 2: "vgpr8", 3: "vgpr16"}
    cases = [
        # (name, grid, bytes per workgroup, mode, rotate)
        ("hbm_bulk_4wg_per_cu_1MiB", 4 * num_cus, 1 << 20, 1, True),
        ("hbm_bulk_4wg_per_cu_1MiB_vgpr16", 4 * num_cus, 1 << 20, 3, True),
        ("hbm_1wg_per_cu_60KiB_lds15", num_cus, 60 << 10, 0, True),
        ("hbm_1wg_per_cu_60KiB_lds31", num_cus, 60 << 10, 1, True),
        ("hbm_1wg_per_cu_60KiB_vgpr16", num_cus, 60 << 10, 3, True),
        ("hbm_1wg_per_cu_128KiB_lds31", num_cus, 128 << 10, 1, True),
        ("hbm_2wg_per_cu_32KiB_lds31", 2 * num_cus, 32 << 10, 1, True),
        ("cached_1wg_per_cu_60KiB_lds31", num_cus, 60 << 10, 1, False),
        ("cached_1wg_per_cu_128KiB_lds31", num_cus, 128 << 10, 1, False),
    ]
    empty_us = out["empty_kernel_us_per_launch"]
    for name, grid, bpw, mode, rotate in cases:
        per = grid * bpw
        nreg = max(1, buf.numel() // per)
        n = 60 if per < (64 << 20) else 8
        base = buf.data_ptr()

        def mk(i):
            off = (i % nreg) * per if rotate else 0
            return lambda s: _ok(lib.dgc_stream(ctypes.c_void_p(base + off), bpw, grid, mode,
                                                ctypes.c_void_p(isink.data_ptr()), s), "dgc_stream")
        ms = _time_graph(torch, [mk(i) for i in range(n)])
        us = ms * 1e3 / n
        out[name] = {"us_per_launch": round(us, 3), "bytes": per,
                     "gbs": round(per / (us * 1e-6) / 1e9, 1),
                     "gbs_per_cu": round(per / (us * 1e-6) / 1e9 / num_cus, 2),
                     "gbs_beyond_empty_launch": round(per / (max(us - empty_us, 1e-3) * 1e-6) / 1e9, 1),
                     "mode": modes[mode]}
    # the tile kernels' load shape without their K-block barriers: 256
    # workgroups of eight waves streaming 64 KB blocks, 8 loads in flight per
    # wave; `share` workgroups of one XCD read the same blocks (from the L2
    # after the first), as the tiles of one XCD share A and B rows
    fsink = torch.empty(256, dtype=torch.int32, device="cuda")
    for name, share, steps in (("fill_8waves_distinct_hbm", 1, 64), ("fill_8waves_shared_by_8_per_xcd", 8, 128),
                               ("fill_8waves_shared_by_32_per_xcd", 32, 128)):
        group_bytes = steps * 65536
        assert (256 // share) * group_bytes <= buf.numel()
        n = 4
        ms = _time_graph(torch, [lambda s, sh=share, st=steps, gb=group_bytes: _ok(lib.dgc_fill(
            ctypes.c_void_p(buf.data_ptr()), gb, st, sh, ctypes.c_void_p(fsink.data_ptr()), s), "dgc_fill")] * n)
        us = ms * 1e3 / n
        filled = 256 * steps * 65536
        out[name] = {"us_per_launch": round(us, 3), "bytes_into_lds": filled,
                     "tbs": round(filled / (us * 1e-6) / 1e12, 2),
                     "gbs_per_cu": round(filled / (us * 1e-6) / 1e9 / num_cus, 1)}
    del buf
    torch.cuda.empty_cache()
    word = torch.zeros(64, dtype=torch.int32, device="cuda")
    state = torch.zeros(1, dtype=torch.int32, device="cuda")
    for name, ring, mode, steps in (("atomic_add_device_scope", word, 0, 2000), ("coherent_load_2MiB", small, 1, 2000),
                                    ("plain_load_2MiB", small, 2, 2000), ("coherent_load_1GiB", big, 1, 4000),
                                    ("plain_load_1GiB", big, 2, 4000)):
        state.zero_()
        # graphs of one launch with 1 step and with `steps` steps; each replay
        # walks on from where the last one stopped
        ms1 = _time_graph(torch, [lambda s, r=ring, m=mode: _ok(lib.dgc_chase(
            ctypes.c_void_p(r.data_ptr()), 1, m, ctypes.c_void_p(state.data_ptr()), s), "dgc_chase")])
        msn = _time_graph(torch, [lambda s, r=ring, m=mode, n=steps: _ok(lib.dgc_chase(
            ctypes.c_void_p(r.data_ptr()), n, m, ctypes.c_void_p(state.data_ptr()), s), "dgc_chase")])
        out[f"latency_ns_{name}"] = round((msn - ms1) * 1e6 / (steps - 1), 1)
    del small, big
    torch.cuda.empty_cache()
    return out
