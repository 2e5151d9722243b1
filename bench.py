"""Throughput of the FP8 block-scaled GEMM (NT) on one MI355X.

One step is one library call over one batch of synthetic inputs already
resident in HBM.  The headline workload is the dense decode shape
M=64 N=2112 K=7168 (A ~ N(0,1), B ~ N(0,0.02), 1x128 / 128x128 power-of-two
scales, bf16 C ~ N(0,0.1)); the other four workloads, the prefill problem
with K-major operands (nn, tn, tt), a K-grouped TN (MoE weight-gradient)
problem and the prefill problem with an FP4 B are reported per shape in the
same JSON line.  Inputs rotate over enough copies that successive steps
read from HBM rather than the 256 MB last-level cache; the timed launches are
replayed from a HIP graph so that host launch cost does not pace the GPU.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--shapes 1,...,13]
                       [--no-cpu-baseline] [--no-ceilings] [--no-graph]
       python bench.py --calibrate-copy   (a plain device copy of known size, for
                                           scaling HBM byte counters)
       python bench.py --ceilings         (only the microbenchmarks of libdg_ceilings.so)

Every workload carries a `roofline` block (its bound, the achieved rate per
call against the MI355X peak: 8 TB/s HBM, 5.0 PFLOP/s dense FP8) and a
`cpu_baseline`: the CPU oracle timed on the host cores on a bounded sample of
the same workload (the whole call for small ones; a few rows, groups or one K
group for the large ones, the rate taken over the sample's own flops).  The
line also carries a `ceilings` summary measured in the same run (FP8 MFMA loop
rate, HBM streaming rate, launch cost).

`roofline.traffic` comes from profiles/hbm_traffic.json (HBM bytes per launch
of the headline kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE passes, scaled by
the same counters on a plain copy); it is null when that file is absent or was
taken from kernel sources other than the current ones.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 MFMA peak (published)
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E peak (published)
MALL_BYTES = 256 << 20       # last-level (Infinity) cache to defeat between steps
HEADLINE = 2                 # 1-based shape index of the headline workload
PAGES_HEADLINE_TFLOPS = 206.0  # the pages' figure for the headline workload (H800 SXM5)

SHAPES = {
    1: ("dense_128x256x512", "mfma"),
    2: ("dense_decode_64x2112x7168", "hbm"),
    3: ("dense_prefill_4096x7168x16384", "mfma"),
    4: ("contiguous_8x4096x7168_rows8192", "mfma"),
    5: ("masked_32x256x4096x7168", "hbm"),
    # the prefill problem with K-major operands (A stored [K][M] for "t", B
    # stored [K][N] for a second "n"): same values, same flops and bytes
    6: ("dense_prefill_4096x7168x16384_nn", "mfma"),
    7: ("dense_prefill_4096x7168x16384_tn", "mfma"),
    8: ("dense_prefill_4096x7168x16384_tt", "mfma"),
    # K-grouped TN (MoE weight gradient): 8 experts, M=4096 x N=7168 per expert,
    # 8192 tokens split multinomially, fp32 D
    9: ("kgrouped_tn_8x4096x7168_tokens8192", "mfma"),
    # FP8 x FP4: the prefill problem with B in E2M1, one E8M0 scale per 32 K values
    10: ("dense_fp8xfp4_4096x7168x16384", "mfma"),
    # FP8 x FP4 at the decode shape (B half the bytes of the FP8 one)
    11: ("dense_fp8xfp4_decode_64x2112x7168", "hbm"),
    # the contiguous and masked problems (power-of-two scales) through the
    # kernels that apply the scales in the MFMA from their E8M0 codes, behind
    # the on-device scale check (not the default choice: measured slower)
    12: ("contiguous_8x4096x7168_rows8192_e8m0", "mfma"),
    13: ("masked_32x256x4096x7168_e8m0", "hbm"),
}
LAYOUT_OF = {6: "nn", 7: "tn", 8: "tt"}
PROBLEM_OF = {6: 3, 7: 3, 8: 3, 12: 4, 13: 5}   # workload index whose generated problem an entry reuses
FORCED_CONFIG = {12: "8", 13: "10"}     # kernel configuration an entry selects (DG_FORCE_CONFIG)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


KERNEL_SOURCES = ["fp8_gemm_core.h", "fp8_gemm.hip", "fp8_gemm_e8m0.hip", "dg_api.hip", "dg_internal.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
COPY_BYTES = 256 << 20


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "moe_grouped_gemm_nt_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per launch measured for `workload`, if taken from the current kernels."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("workloads", {}).get(workload)


def calibrate_copy(torch, reps=20):
    """Plain device-to-device copies of COPY_BYTES each: the reference the HBM
    byte counters are scaled by (one copy reads and writes COPY_BYTES)."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] calibration: {reps} copies of {COPY_BYTES} bytes")


def algorithmic_bytes(p) -> int:
    """Bytes that must move once: A and its scales for computed rows, all of
    B and sfb that computed rows touch, C (if any) and D for computed rows."""
    import inputgen
    KB = p.K // 128
    if isinstance(p, inputgen.Dense):
        rows = p.M
        b = p.b.nbytes + p.sfb.nbytes
        cbytes = (rows * p.N * 2) if p.c is not None else 0
        return rows * p.K + rows * KB * 4 + b + cbytes + rows * p.N * 2
    if isinstance(p, inputgen.Contiguous):
        rows = p.real_rows
        used = np.unique(p.grouped_layout[p.grouped_layout >= 0])
        b = sum(p.b[g].nbytes + p.sfb[g].nbytes for g in used)
        return rows * p.K + rows * KB * 4 + rows * 4 + b + rows * p.N * 2
    if isinstance(p, inputgen.DenseFP4):
        cbytes = (p.M * p.N * 2) if p.c is not None else 0
        return p.M * p.K + p.M * KB * 4 + p.b.nbytes + p.sfb.nbytes + cbytes + p.M * p.N * 2
    if isinstance(p, inputgen.KGrouped):
        tokens = int(p.counts.sum())
        return tokens * (p.M + p.N) + (tokens // 128 + p.G) * (p.M + p.N) * 4 + p.G * p.M * p.N * 4
    if isinstance(p, inputgen.Masked):
        m = np.minimum(np.maximum(p.masked_m, 0), p.max_m)
        rows = int(m.sum())
        b = sum(p.b[g].nbytes + p.sfb[g].nbytes for g in range(p.G) if m[g] > 0)
        return rows * p.K + rows * KB * 4 + b + rows * p.N * 2 + p.G * 4
    raise TypeError(p)


_PROBLEMS = {}      # generated problems by workload index, shared by the entries that reuse one


class Workload:
    """Device copies of one generated problem plus the launch closure."""

    def __init__(self, idx, torch, dg, copies=None):
        import inputgen
        t0 = time.time()
        if idx == 9:
            self.p = p = inputgen.make_kgrouped(8, 4096, 7168, 8192, seed=0, name=SHAPES[idx][0])
        elif idx == 10:
            self.p = p = inputgen.make_dense_fp4(4096, 7168, 16384, 0, 1.0, 0.02, None, False, SHAPES[idx][0])
        elif idx == 11:
            self.p = p = inputgen.make_dense_fp4(64, 2112, 7168, 0, 1.0, 0.02, 0.1, False, SHAPES[idx][0])
        else:
            src = PROBLEM_OF.get(idx, idx)
            if src not in _PROBLEMS:          # the layout entries reuse the prefill problem
                _PROBLEMS[src] = inputgen.make_config(src - 1, seed=0)
            self.p = p = _PROBLEMS[src]
        self.name, self.bound = SHAPES[idx]
        self.layout = LAYOUT_OF.get(idx, "nt")
        self.forced = FORCED_CONFIG.get(idx)
        self.flops = p.flops
        self.bytes = algorithmic_bytes(p)
        per_copy = p.a.nbytes + p.b.nbytes
        if copies is None:
            copies = max(1, min(64, math.ceil(2 * MALL_BYTES / per_copy)))
        self.copies = copies
        dev = torch.device("cuda")

        def up(x, dtype=None):
            t = torch.from_numpy(np.ascontiguousarray(x))
            return (t.view(dtype) if dtype is not None else t).to(dev)

        a_st = p.a if self.layout[0] == "n" else np.ascontiguousarray(p.a.T)
        b_st = p.b if self.layout[1] == "t" else np.ascontiguousarray(p.b.T)
        a, sfa, b, sfb = up(a_st), up(p.sfa), up(b_st), up(p.sfb)
        self.sets = []
        for i in range(copies):
            s = dict(a=a if i == 0 else a.clone(), sfa=sfa if i == 0 else sfa.clone(),
                     b=b if i == 0 else b.clone(), sfb=sfb if i == 0 else sfb.clone())
            if isinstance(p, (inputgen.Dense, inputgen.DenseFP4)):
                s["c"] = up(p.c.view(np.int16)).view(torch.bfloat16) if p.c is not None else None
                s["d"] = torch.empty((p.M, p.N), dtype=torch.bfloat16, device=dev)
            elif isinstance(p, inputgen.Contiguous):
                s["layout"] = up(p.grouped_layout)
                s["d"] = torch.empty((p.M, p.N), dtype=torch.bfloat16, device=dev)
            elif isinstance(p, inputgen.KGrouped):
                # fp32 D [G][M][N] is large: every copy writes the same buffer
                s["d"] = self.sets[0]["d"] if i else torch.empty((p.G, p.M, p.N), dtype=torch.float32, device=dev)
            else:
                s["masked_m"] = up(p.masked_m)
                s["d"] = torch.empty((p.G, p.max_m, p.N), dtype=torch.bfloat16, device=dev)
            self.sets.append(s)
        self.dg = dg
        self.kind = type(p).__name__
        torch.cuda.synchronize()
        log(f"[bench] {self.name}: generated and uploaded {copies} copies in {time.time() - t0:.1f}s")

    def launch(self, i):
        s = self.sets[i % self.copies]
        dg = self.dg
        # the configuration is chosen on the host at each call (and recorded
        # when a graph is captured)
        if self.forced is not None:
            os.environ["DG_FORCE_CONFIG"] = self.forced
        else:
            os.environ.pop("DG_FORCE_CONFIG", None)
        if self.kind == "Dense":
            getattr(dg, "dg_fp8_gemm_" + self.layout)(s["a"], s["sfa"], s["b"], s["sfb"], s["c"], s["d"])
        elif self.kind == "DenseFP4":
            dg.dg_fp8_fp4_gemm_nt(s["a"], s["sfa"], s["b"], s["sfb"], s["c"], s["d"])
        elif self.kind == "KGrouped":
            dg.dg_k_grouped_fp8_gemm_tn_contiguous(s["a"], s["sfa"], s["b"], s["sfb"], None, s["d"], self.p.ks)
        elif self.kind == "Contiguous":
            dg.dg_m_grouped_fp8_gemm_nt_contiguous(s["a"], s["sfa"], s["b"], s["sfb"], None, s["d"], s["layout"])
        else:
            dg.dg_m_grouped_fp8_gemm_nt_masked(s["a"], s["sfa"], s["b"], s["sfb"], None, s["d"],
                                               s["masked_m"], self.p.expected_m)


def time_workload(torch, w: Workload, steps: int, warmup: int, use_graph: bool = True, repeats=None):
    """Runs `warmup` untimed steps, then times exactly `steps` steps between a
    synchronisation on each side.  Returns (total ms, per-step ms).  With
    `repeats` (a list), the captured graph is then replayed that many more
    times, each replay timed on its own, and the per-step times are appended
    (outside the timed region, for the median and minimum)."""
    for i in range(warmup):
        w.launch(i)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                w.launch(i)
        torch.cuda.synchronize()
        graph.replay()                     # one untimed replay: first-replay set-up cost
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        start.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for i in range(steps):
                w.launch(i)
        end.record(stream)
    torch.cuda.synchronize()
    total = start.elapsed_time(end)
    if repeats is not None and graph is not None:
        for _ in range(10):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                graph.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            repeats.append(e0.elapsed_time(e1) / steps)
    return total, total / steps


def warm_gpu(torch, seconds=0.3):
    """Keeps the matrix cores busy for a fraction of a second before a workload
    is timed: the clock ramps up under load, and a workload timed right after
    the seconds of host work that generate its inputs (the GPU idle) measured
    up to 8% slower than the same configuration timed again at once."""
    try:
        from moe_grouped_gemm_nt_amd import ceilings
        lib = ceilings.load()
    except Exception as e:  # the warm-up is a courtesy to the first workload; timing stays valid without it
        log(f"[bench] no GPU warm-up: {e}")
        return
    import ctypes
    n = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(2 * n * 256, dtype=torch.float32, device="cuda")
    t0 = time.time()
    while time.time() - t0 < seconds:
        for _ in range(10):
            lib.dgc_mfma(256, 2 * n, 1, ctypes.c_void_p(sink.data_ptr()), None)
        torch.cuda.synchronize()


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        return os.cpu_count() or 1


def oracle_sample(w):
    """(callable, algorithmic flops, description) of a bounded sample of
    workload w for the CPU oracle: whole small calls; for large ones a few
    rows, a few groups or one K group, whose flops the rate is taken over."""
    import inputgen
    import oracle
    p = w.p
    small = p.M * p.N * p.K <= (1 << 27) if isinstance(p, (inputgen.Dense, inputgen.DenseFP4)) else False
    if isinstance(p, inputgen.Dense):
        rows = np.arange(p.M if small else min(p.M, 64))
        whole = len(rows) == p.M
        return (lambda: oracle.gemm_nt(p.a, p.sfa, p.b, p.sfb, p.c, rows=rows), 2.0 * len(rows) * p.N * p.K,
                "the whole call" if whole else f"rows 0-{len(rows) - 1} of {p.M} (all {p.N} columns, all of K)")
    if isinstance(p, inputgen.DenseFP4):
        rows = np.arange(p.M if small else min(p.M, 64))
        whole = len(rows) == p.M
        return (lambda: oracle.gemm_fp8_fp4_nt(p.a, p.sfa, p.b, p.sfb, p.c, rows=rows), 2.0 * len(rows) * p.N * p.K,
                "the whole call" if whole else f"rows 0-{len(rows) - 1} of {p.M} (all {p.N} columns, all of K)")
    if isinstance(p, inputgen.Contiguous):
        starts = np.concatenate([[0], np.cumsum(((p.counts + 127) // 128) * 128)])
        groups = [g for g in range(p.G) if p.counts[g] > 0][:2]
        rows = np.concatenate([np.arange(starts[g], starts[g] + min(64, p.counts[g])) for g in groups])
        return (lambda: oracle.m_grouped_contiguous(p.a, p.sfa, p.b, p.sfb, p.grouped_layout, rows=rows),
                2.0 * len(rows) * p.N * p.K, f"{len(rows)} real rows of experts {groups} (all columns, all of K)")
    if isinstance(p, inputgen.Masked):
        m = np.minimum(np.maximum(p.masked_m, 0), p.max_m)
        groups = [g for g in range(p.G) if m[g] > 0][:2]
        return (lambda: oracle.m_grouped_masked(p.a, p.sfa, p.b, p.sfb, p.masked_m, groups=groups),
                2.0 * float(m[groups].sum()) * p.N * p.K, f"groups {groups} ({int(m[groups].sum())} rows)")
    if isinstance(p, inputgen.KGrouped):
        g = int(np.argmax(p.ks > 0))
        return (lambda: oracle.k_grouped_tn(p.a, p.sfa, p.b, p.sfb, p.ks, groups=[g]),
                2.0 * float(p.counts[g]) * p.M * p.N, f"group {g} ({int(p.ks[g])} K rows)")
    raise TypeError(p)


def cpu_baseline(w, budget_s):
    """The oracle as it stands, on the host cores, timed on a bounded sample
    of workload w (repeated until budget_s has passed)."""
    fn, flops, what = oracle_sample(w)
    runs = 0
    t0 = time.perf_counter()
    while True:
        fn()
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per = el / runs
    return {"value": round(flops / per / 1e12, 6), "unit": "TFLOPS", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{what} of {w.name}: {runs} oracle runs in {el:.1f}s ({per * 1e3:.1f} ms per run, "
                      f"{flops / 1e9:.2f} GFLOP each)"}


def roofline_of(w, ms):
    """Roofline block of one workload from its measured time per call."""
    t = load_traffic(w.name)
    if w.bound == "hbm":
        achieved = w.bytes / (ms * 1e-3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
    else:
        achieved = w.flops / (ms * 1e-3) / 1e12
        peak, unit = FP8_PEAK_TFLOPS, "TFLOP/s"
    return {"bound": w.bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": int(t["hbm_bytes_per_launch"]) if t else None,
            "alg_bytes_per_call": int(w.bytes), "alg_flops_per_call": float(w.flops),
            "avg_call_us": round(ms * 1e3, 3)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--shapes", default="1,2,3,4,5,6,7,8,9,10,11,12,13", help="comma-separated 1-based workload indices")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="leave the microbenchmark summary out of the line")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a graph")
    ap.add_argument("--calibrate-copy", action="store_true", help="run only the copy used to scale byte counters")
    ap.add_argument("--ceilings", action="store_true",
                    help="run only the microbenchmarks (MFMA loop, memory rates, launch cost) and print them")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_grouped_gemm_nt_amd as dg

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    if args.ceilings:
        from moe_grouped_gemm_nt_amd import ceilings
        print(json.dumps({"ceilings": ceilings.measure(torch)}), flush=True)
        return
    dg.load()
    dg.dg_init()
    warm_gpu(torch)
    shapes = [int(s) for s in args.shapes.split(",") if s.strip()]
    if HEADLINE not in shapes:
        shapes = [HEADLINE] + shapes

    per_shape = {}
    head = None
    baselines = {}          # cpu_baseline by generated problem (entries that reuse one share it)
    for idx in shapes:
        w = Workload(idx, torch, dg)
        # generating and uploading a workload leaves the GPU idle for seconds;
        # bring the clock back up before its warm-up steps and timing
        warm_gpu(torch, 0.2)
        steps = args.steps
        if w.flops > 1e11:
            steps = max(10, min(steps, 50))         # large shapes: keep the timed region short
        reps = [] if idx == HEADLINE else None
        total_ms, ms = time_workload(torch, w, steps, args.warmup, use_graph=not args.no_graph, repeats=reps)
        tflops = w.flops / (ms * 1e-3) / 1e12
        gbs = w.bytes / (ms * 1e-3) / 1e9
        rec = {"ms_per_call": round(ms, 5), "tflops": round(tflops, 2),
               "frac_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4),
               "gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
               "bound": w.bound, "alg_bytes": int(w.bytes), "flops": float(w.flops),
               "steps": steps, "copies": w.copies, "roofline": roofline_of(w, ms)}
        if w.kind == "Contiguous":
            # the contiguous form computes every row of A, padding included:
            # the MFMA rate over the padded rows, labelled as such
            padded = 2.0 * w.p.M * w.p.N * w.p.K / (ms * 1e-3) / 1e12
            rec["tflops_padded_rows"] = {"value": round(padded, 2), "rows": int(w.p.M),
                                         "note": "2 * padded rows * N * K per call; the headline tflops counts real rows"}
        per_shape[w.name] = rec
        log(f"[bench] {w.name}: {ms * 1e3:.2f} us/call, {tflops:.1f} TFLOPS ({100 * tflops / FP8_PEAK_TFLOPS:.1f}% "
            f"of FP8 peak), {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of HBM peak)")
        if not args.no_cpu_baseline:
            src = PROBLEM_OF.get(idx, idx)
            if src not in baselines:
                baselines[src] = cpu_baseline(w, 10.0 if idx == HEADLINE else 2.0)
                log(f"[bench] {w.name}: oracle on the host, {baselines[src]['sample']}")
            rec["cpu_baseline"] = baselines[src]
        if idx == HEADLINE:
            head = (w, steps, total_ms, ms, tflops, gbs)
            if reps:
                rec["repeat_ms_per_call"] = {"replays": len(reps), "median": round(float(np.median(reps)), 6),
                                             "min": round(float(np.min(reps)), 6)}
        else:
            del w
            torch.cuda.empty_cache()

    w, steps, total_ms, ms, tflops, gbs = head
    roofline = dict(roofline_of(w, ms))
    roofline["kernel"] = ("fp8_gemm_nt_decode_kernel + splitk_reduce_kernel: the two launches of one call, "
                          "timed together (per-call time)")
    cpu = per_shape[w.name].get("cpu_baseline")
    ceil = None
    if not args.no_ceilings:
        try:
            from moe_grouped_gemm_nt_amd import ceilings
            c = ceilings.measure(torch)
            ceil = {"mfma_fp8_chained_pflops": max(v for k, v in c.items() if k.startswith("mfma_fp8_chained")),
                    "mfma_fp8_promoted_pflops": max(v for k, v in c.items() if k.startswith("mfma_fp8_promoted")),
                    "hbm_stream_gbs": max(c["hbm_bulk_4wg_per_cu_1MiB"]["gbs"], c["hbm_bulk_4wg_per_cu_1MiB_vgpr16"]["gbs"]),
                    "empty_kernel_us": c["empty_kernel_us_per_launch"],
                    "stream_15MiB_one_launch_us": c["hbm_1wg_per_cu_60KiB_lds31"]["us_per_launch"],
                    "lds_fill_l2_shared_tbs": c["fill_8waves_shared_by_8_per_xcd"]["tbs"],
                    "source": "bench.py --ceilings (libdg_ceilings.so)"}
        except Exception as e:  # the summary is context; its absence does not void the measurement
            log(f"[bench] ceilings not measured: {e}")
    line = {
        "metric": "FP8 block-scaled GEMM TFLOPS + % of MI355X dense FP8 peak, per shape",
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        # the pages' figure for this metric and workload, measured on another
        # machine (H800 SXM5): context, not a target
        "vs_baseline": round(tflops / PAGES_HEADLINE_TFLOPS, 4),
        "vs_baseline_ref": {"value": PAGES_HEADLINE_TFLOPS, "unit": "TFLOPS", "hardware": "H800 SXM5",
                            "workload": "dense 64x2112x7168", "role": "context (another machine), not a target"},
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic, seeded (numpy PCG64 seed 0), shapes and distributions of the DeepSeek-V3/R1 GEMMs",
        "config": {"workload": w.name, "M": w.p.M, "N": w.p.N, "K": w.p.K, "C": True,
                   "scales": "A 1x128, B 128x128, power-of-two fp32", "rotating_copies": w.copies,
                   "graph_replay": not args.no_graph, "frac_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "ceilings": ceil,
        "per_shape": per_shape,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
