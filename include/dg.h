/*
 * dg.h -- FP8 (OCP e4m3) GEMM with fine-grained block scaling for AMD MI355X (gfx950).
 *
 * What the calls compute (DeepGEMM pages: likun.im/craft/deepgemm.html, section
 * 一 "the GEMM family", D = C + A @ B in the NT layout, and section 二, the
 * register_apis listing of the dense call and the two M-grouped MoE calls;
 * aitangshan.cn/news/1491278, "4. FP8 精度优化的核心": each block's GEMM result is
 * multiplied by that block's scale factors):
 *
 *   D[m,n] = bf16_rne( C[m,n] + sum_kb sa[kb][m] * sb[n/128][kb]
 *                                      * sum_{k in block kb} A[m,k] * B[n,k] )
 *
 * with kb running over the K/128 blocks of 128 consecutive K indices.  A and B
 * hold e4m3 codes; every product is summed in fp32 on the GPU ("fp32
 * accumulation"); each block's partial sum is multiplied by its A scale (one
 * per row per block, "1x128") and its B scale (one per 128x128 block) and added
 * to an fp32 total; C is added and the total is rounded once to bf16 (round to
 * nearest, ties to even).
 *
 * Layouts (every array row-major, every pointer a device pointer on the
 * current HIP device, owned by the caller; the library keeps no pointer after
 * the call returns):
 *   a    uint8  [M][K]            e4m3 codes, K contiguous            (16-byte aligned)
 *   sfa  float  [K/128][M]        A scales, M contiguous ("MN-major") (4-byte aligned)
 *   b    uint8  [N][K]            e4m3 codes, K contiguous ("NT")     (16-byte aligned)
 *   sfb  float  [ceil(N/128)][K/128]  B scales                        (4-byte aligned)
 *   c    bf16   [M][N]            bit patterns; NULL means C = 0; may equal d
 *   d    bf16   [M][N]            output                              (2-byte aligned)
 * K must be a multiple of 128.  The grouped forms add a leading group axis to
 * B and sfb: b [G][N][K], sfb [G][ceil(N/128)][K/128].
 *
 * Calls are asynchronous: they validate their arguments on the host, enqueue
 * one or more kernels on `stream` (a hipStream_t; NULL = the null stream) and
 * return without waiting.  Device-resident control data (grouped_layout,
 * masked_m) is read only by the kernels, so no call synchronises with the
 * device and every call may be captured in a HIP graph once dg_init() has run
 * on the device.  Faults inside a kernel surface at the caller's next
 * synchronisation, as for any HIP kernel.
 *
 * All calls on one device share its split-K workspace (fp32 partial tiles)
 * and its scale-check results, unless their stream has a workspace of its own
 * (dg_bind_stream_workspace).  Calls enqueued on one stream, or ordered across
 * streams by events, are safe; calls that may run at the same time on
 * different streams of one device race on the shared memory and must be
 * ordered by the caller, or given per-stream workspaces.
 *
 * Errors: an invalid argument returns DG_ERR_INVALID_ARG and launches nothing;
 * a shape the kernels do not handle returns DG_ERR_UNSUPPORTED; a failing HIP
 * call returns DG_ERR_HIP.  dg_last_error() then describes the failure (per
 * host thread).  No C++ exception crosses this interface.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DG_OK = 0,
  DG_ERR_INVALID_ARG = -1,
  DG_ERR_UNSUPPORTED = -2,
  DG_ERR_HIP = -3
} dg_status;

/* Dense FP8 GEMM, NT layout: D[M][N] = C + A[M][K] . B[N][K]^T with 1x128 A
 * scales and 128x128 B scales (likun.im section 一 naming: "fp8_gemm_nt";
 * aitangshan.cn usage example: a, a's scales, b, b's scales, c, out).
 * M == 0 or N == 0 is a successful no-op; K == 0 gives D = C.
 * Returns a dg_status. */
int dg_fp8_gemm_nt(const void* a, const float* sfa, const void* b, const float* sfb,
                   const void* c, void* d, int M, int N, int K, void* stream);

/* Dense FP8 GEMM with K-major operands (likun.im section 一: the family
 * fp8_gemm_{nt,nn,tn,tt}; the first letter gives A's storage, the second B's,
 * "n" for A meaning [M][K] and "t" [K][M], "t" for B meaning [N][K] and "n"
 * [K][N]).  Same arithmetic, scales (sfa [K/128][M], sfb [ceil(N/128)][K/128],
 * indexed by the logical row, column and K block whatever the storage), C and
 * D as dg_fp8_gemm_nt:
 *   nn: a [M][K] (K contiguous), b [K][N] (N contiguous)
 *   tn: a [K][M] (M contiguous), b [K][N] (N contiguous)
 *   tt: a [K][M] (M contiguous), b [N][K] (K contiguous)
 * An operand stored [K][M] needs M % 16 == 0, one stored [K][N] needs
 * N % 16 == 0; other sizes return DG_ERR_UNSUPPORTED.  Returns a dg_status. */
int dg_fp8_gemm_nn(const void* a, const float* sfa, const void* b, const float* sfb,
                   const void* c, void* d, int M, int N, int K, void* stream);
int dg_fp8_gemm_tn(const void* a, const float* sfa, const void* b, const float* sfb,
                   const void* c, void* d, int M, int N, int K, void* stream);
int dg_fp8_gemm_tt(const void* a, const float* sfa, const void* b, const float* sfb,
                   const void* c, void* d, int M, int N, int K, void* stream);

/* Dense FP8 x FP4 GEMM, NT layout (likun.im section 一: "fp8_fp4_gemm_nt";
 * section 五: packed UE8M0 scale factors, four to an int; lqnn.cn: the FP8 x
 * FP4 GEMM release):
 *   D[m,n] = bf16_rne( C[m,n] + sum_kb sa[kb][m]
 *            * sum_{k in block kb} A[m,k] * B[n,k] * 2^(e[n][k/32] - 127) )
 *   a    uint8  [M][K]       e4m3 codes (16-byte aligned); sfa float [K/128][M] as in dg_fp8_gemm_nt
 *   b    uint8  [N][K/2]     OCP E2M1 (FP4) codes, two per byte, element 2i in the
 *                            low nibble, K contiguous (16-byte aligned)
 *   sfb  int32  [K/128][N]   E8M0 scale exponents e (value 2^(e-127)), one byte per
 *                            32 K values: byte j of sfb[kb][n] scales K values
 *                            128*kb + 32*j .. +31 of row n (4-byte aligned)
 *   c, d bf16   [M][N]       as in dg_fp8_gemm_nt
 * K must be a multiple of 128.  Runs on the tile kernels (no split-K variant).
 * Returns a dg_status. */
int dg_fp8_fp4_gemm_nt(const void* a, const float* sfa, const void* b, const int32_t* sfb,
                       const void* c, void* d, int M, int N, int K, void* stream);

/* M-grouped GEMM, contiguous layout (likun.im section 二:
 * "m_grouped_..._gemm_nt_contiguous" taking grouped_layout): the rows of every
 * expert are concatenated along M.  grouped_layout is a device int32 array of
 * M entries; row m is computed with expert grouped_layout[m]'s B and sfb.
 * Rows come in aligned blocks of 128 (rows 128*i .. 128*i+127); within one
 * block every row whose id lies in [0, num_groups) must carry the same id.
 * Rows whose id lies outside [0, num_groups) (for example -1 on padding) are
 * not written.  a [M][K], sfa [K/128][M], b [num_groups][N][K],
 * sfb [num_groups][ceil(N/128)][K/128], c and d [M][N].
 * Returns a dg_status. */
int dg_m_grouped_fp8_gemm_nt_contiguous(const void* a, const float* sfa, const void* b,
                                        const float* sfb, const void* c, void* d, int M, int N,
                                        int K, int num_groups, const int32_t* grouped_layout,
                                        void* stream);

/* M-grouped GEMM, masked layout (likun.im section 二:
 * "m_grouped_..._gemm_nt_masked" taking masked_m and expected_m; zwt0204
 * DeepGEMM deep dive: the masked layout serves inference decoding).  Every
 * group g owns max_m rows; only its first min(max(masked_m[g], 0), max_m)
 * rows are computed and written, the others are left untouched.  masked_m is a
 * device int32 array of num_groups entries, read only by the kernel.
 * expected_m is a host-side hint of the typical masked_m; it only steers the
 * launch configuration and never changes which rows are computed.
 * a [G][max_m][K], sfa [G][K/128][max_m], b [G][N][K], sfb [G][ceil(N/128)][K/128],
 * c and d [G][max_m][N].  Returns a dg_status. */
int dg_m_grouped_fp8_gemm_nt_masked(const void* a, const float* sfa, const void* b,
                                    const float* sfb, const void* c, void* d, int max_m, int N,
                                    int K, int num_groups, const int32_t* masked_m,
                                    int expected_m, void* stream);

/* M-grouped FP8 x FP4 GEMMs (likun.im section 二: "m_grouped_fp8_fp4_gemm_nt_contiguous"
 * and "..._masked"): as dg_m_grouped_fp8_gemm_nt_contiguous / _masked with the
 * FP4 B of dg_fp8_fp4_gemm_nt per group: b uint8 [G][N][K/2] (packed E2M1),
 * sfb int32 [G][K/128][N] (four E8M0 exponents per int).  A, sfa, C, D,
 * grouped_layout, masked_m and expected_m exactly as in the FP8 forms.
 * Returns a dg_status. */
int dg_m_grouped_fp8_fp4_gemm_nt_contiguous(const void* a, const float* sfa, const void* b,
                                            const int32_t* sfb, const void* c, void* d, int M, int N,
                                            int K, int num_groups, const int32_t* grouped_layout,
                                            void* stream);
int dg_m_grouped_fp8_fp4_gemm_nt_masked(const void* a, const float* sfa, const void* b,
                                        const int32_t* sfb, const void* c, void* d, int max_m, int N,
                                        int K, int num_groups, const int32_t* masked_m,
                                        int expected_m, void* stream);

/* K-grouped GEMM, TN layout, for MoE weight gradients (likun.im section 一:
 * "k_grouped_fp8_gemm_tn", grouped along K for the MoE backward pass; section
 * 二: the call takes the per-group K sizes ks and the (1, 1, 128) scale
 * recipe).  Group g owns K rows k_start[g] .. k_start[g] + ks[g] - 1 of both
 * operands (k_start = running sum of ks), i.e. its tokens, and
 *   D[g][m][n] = C[g][m][n] + sum_kb sfa[kb][m] * sfb[kb][n]
 *                             * sum_{k in block kb} A[k][m] * B[k][n]
 * over the group's 128-row K blocks, accumulated in fp32 and stored in fp32.
 *   a    uint8  [K][M]   e4m3 codes, M contiguous (16-byte aligned)
 *   sfa  float  [K/128][M]   one scale per column per 128 K rows
 *   b    uint8  [K][N]   e4m3 codes, N contiguous (16-byte aligned)
 *   sfb  float  [K/128][N]   one scale per column per 128 K rows
 *   c    float  [G][M][N] or NULL (C = 0); may equal d (accumulation)
 *   d    float  [G][M][N] output (a group with ks[g] == 0 gets C, or zeros)
 *   ks   int32  [num_groups] on the HOST: each a non-negative multiple of 128
 *        (pad a group's tokens with zero rows); K = sum of ks.
 * M and N must be multiples of 16 and num_groups at most 256
 * (DG_ERR_UNSUPPORTED otherwise).  The K offsets travel in the launch's
 * arguments, so a captured graph replays the call with the ks it was captured
 * with.  Returns a dg_status. */
int dg_k_grouped_fp8_gemm_tn_contiguous(const void* a, const float* sfa, const void* b,
                                        const float* sfb, const float* c, float* d, int M, int N,
                                        int num_groups, const int32_t* ks, void* stream);

/* dg_fp8_gemm_nt without any device allocation, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, arithmetic, layouts and
 * errors as dg_fp8_gemm_nt.  Its kernels' scratch (split-K partial tiles and
 * scale-check verdicts) is a fixed 8 MiB device array per GPU, part of the
 * library's code object and held until the process ends; the call allocates
 * nothing, neither on its first use on a device nor later.  The kernel
 * configuration is chosen so that its partials fit the array; one forced
 * beyond it (DG_FORCE_SPLITS) returns DG_ERR_UNSUPPORTED.  Every call on a GPU
 * shares that GPU's array, and nothing in it needs clearing between calls
 * (every call writes what it reads; the one-launch decode configuration's
 * per-tile counters in it start at zero with the array and every call leaves
 * them at zero), but calls that may overlap on one GPU (different streams not
 * ordered by events) race on it and must be ordered by the caller.  Returns a
 * dg_status. */
int dg_fp8_gemm_nt_noalloc(const void* a, const float* sfa, const void* b, const float* sfb,
                           const void* c, void* d, int M, int N, int K, void* stream);

/* The kernel configuration the calls above would choose, as a host-side query
 * that touches no device (for tests and for callers that want to know what
 * runs).  form: 0 dense (any operand storage), 1 contiguous, 2 masked.  rows:
 * M for dense and contiguous calls, expected_m for masked ones.  ab_layout:
 * 0 nt, 1 tt (A stored [K][M]), 2 nn (B stored [K][N]), 3 tn, 4 FP4 B.
 * num_cus: the device's compute units (256 on MI355X).  has_c: nonzero when
 * the call passes a C.  Writes the configuration id to *cfg (0 128x128 tile,
 * 1 decode kernel with K split over workgroups, 2 128x64, 3 64x128, 4 128x128
 * two per CU, 5 256x128, 6 128x256, 7 and 8 128x256 and 10 256x256 with
 * power-of-two scales in the MFMA, 9 narrow 16x48 whole-K, 11 256x256, 12 the
 * decode kernel with its splits summed inside the same launch) and
 * the decode kernel's K splits to *splits (1 otherwise).  DG_FORCE_CONFIG and
 * DG_FORCE_SPLITS act as they do on the calls.  Returns DG_ERR_INVALID_ARG
 * for NULL outputs, a form outside 0-2, rows or N below 1, K negative or not
 * a multiple of 128, num_groups below 1, num_cus below 8 or ab_layout
 * outside 0-4; DG_OK otherwise. */
int dg_choose_config(int form, int rows, int N, int K, int num_groups, int num_cus, int ab_layout,
                     int has_c, int* cfg, int* splits);

/* Binds a caller-owned device workspace to a stream of the current device:
 * every later call of this library enqueued on that stream uses it in place
 * of the device's shared workspace (split-K partial tiles and scale-check
 * verdicts), so that calls running at the same time on different streams no
 * longer share scratch memory.  workspace: device memory on the current
 * device, 256-byte aligned, at least 256 bytes (the verdicts).  A workspace of
 * at least 256 + 4096 bytes also holds, after the verdicts, the 4096 bytes of
 * counters of the one-launch decode configuration, which this call clears
 * (synchronously) and every later call leaves at zero; the rest holds
 * partials, and the configuration is chosen so that they fit (a bound
 * workspace of a few hundred bytes simply means no split-K).  The caller keeps
 * the memory alive, and unused by anything else, while the binding lasts and
 * while calls enqueued with it run.  workspace NULL (or bytes 0) removes the
 * stream's binding.  The allocation-free call (dg_fp8_gemm_nt_noalloc) always
 * uses its own fixed array.  Returns DG_ERR_INVALID_ARG for a misaligned or
 * too small workspace, DG_ERR_HIP if the current device cannot be queried or
 * the counters cannot be cleared. */
int dg_bind_stream_workspace(void* stream, void* workspace, size_t bytes);

/* Host-side check of a contiguous grouped_layout held in HOST memory (M int32
 * entries) against the contract of the contiguous calls: within every aligned
 * block of 128 rows, all rows whose id lies in [0, num_groups) carry the same
 * id.  Returns DG_OK, or DG_ERR_INVALID_ARG with dg_last_error() naming the
 * first offending block.  Touches no device.
 *
 * Debug mode: with the environment variable DG_VALIDATE=1, the M-grouped calls
 * copy their device-resident grouped_layout (or masked_m) to the host on the
 * call's stream, wait for it, and apply this check (masked: every masked_m[g]
 * within [0, max_m], which the kernels would otherwise clamp) before launching
 * anything; a violation returns DG_ERR_INVALID_ARG.  It synchronises, so it is
 * for debugging only, and it is skipped while the stream is being captured. */
int dg_check_grouped_layout(const int32_t* grouped_layout, int M, int num_groups);

/* Prepares per-device state for the current HIP device (device properties and
 * the split-K workspace, allocated once and kept until the process ends).
 * Calls above do this lazily on first use; call dg_init() first when the
 * first call would otherwise happen inside HIP graph capture.
 * Returns a dg_status. */
int dg_init(void);

/* Message describing the last non-DG_OK status returned on this host thread
 * (empty string if none).  The pointer stays valid until the next call on
 * this thread. */
const char* dg_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int dg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DG_H */
