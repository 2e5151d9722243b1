/*
 * dg_ceilings.h -- microbenchmarks of the MI355X (gfx950) limits that bound the
 * FP8 GEMM kernels of dg.h: the FP8 MFMA issue rate, the rate at which
 * workgroups pull bytes from memory, and the cost of one kernel launch.
 * Built into libdg_ceilings.so; not needed by the GEMM calls.
 *
 * All pointers are device pointers on the current HIP device, owned by the
 * caller; calls enqueue one kernel on `stream` (a hipStream_t, NULL = the null
 * stream) and return 0, -1 for invalid arguments (nothing launched) or -3 when
 * the launch fails.
 */
#ifndef DG_CEILINGS_H
#define DG_CEILINGS_H

#ifdef __cplusplus
extern "C" {
#endif

/* grid workgroups of four waves; workgroup i reads the bytes_per_wg bytes at
 * src + i * bytes_per_wg (bytes_per_wg a positive multiple of 4096), 1 KB per
 * wave load instruction.  mode 0: direct global->LDS loads (the GEMM kernels'
 * form), at most 15 outstanding per wave; 1: the same with 31; 2: 16-byte
 * loads into registers, 8 outstanding per wave; 3: the same with 16.
 * sink: int32 [grid], written by mode 0 and 1 only. */
int dgc_stream(const void* src, long bytes_per_wg, int grid, int mode, int* sink, void* stream);

/* 256 workgroups of eight waves in groups of `share` workgroups of one XCD
 * (share divides 32; workgroup i is on XCD i % 8): group g reads the steps
 * 64 KB blocks at src + g * group_bytes (steps * 65536 <= group_bytes) with
 * direct global->LDS loads, 8 in flight per wave.  The caller's buffer must
 * hold (256 / share) * group_bytes bytes.  sink: int32 [256]. */
int dgc_fill(const void* src, long group_bytes, int steps, int share, int* sink, void* stream);

/* grid workgroups of 256 threads that do nothing. */
int dgc_empty(int grid, void* stream);

/* grid workgroups of four waves; each wave issues iters x 8 back-to-back
 * 16x16x128 FP8 MFMAs (65536 flop each) on register operands.  promote != 0:
 * each MFMA starts from zero and is folded into its total with one fp32 FMA
 * per element, as the general-scale kernels do.  sink: float [grid * 256]. */
int dgc_mfma(int iters, int grid, int promote, float* sink, void* stream);

/* One lane issues iters dependent memory operations: mode 0 device-scope
 * atomic adds on ring[0]; 1 a pointer chase with device-coherent loads
 * (x = ring[x], past the XCD's L2); 2 the same chase with plain loads.  The
 * chase starts at index state[0] and leaves its last index there (mode 0
 * leaves 0), so successive launches continue along the chain.  For modes 1
 * and 2 every ring[i] must hold an index inside the caller's allocation, and
 * so must state[0].  state: int32 [1]. */
int dgc_chase(int* ring, int iters, int mode, int* state, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DG_CEILINGS_H */
