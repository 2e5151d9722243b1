// gfx950 kernels for the FP8 (e4m3) block-scaled GEMM, NT layout, and its two
// M-grouped MoE forms.
//
// Computation (likun.im DeepGEMM article, section 一: D = C + A @ B in the NT
// layout; aitangshan.cn DeepGEMM article, "4. FP8 精度优化的核心": each block's
// GEMM result is multiplied by the block's scales): for every 128-wide K
// block kb, one v_mfma_f32_16x16x128_f8f6f4 per 16x16 output sub-tile forms the
// block's partial sum in fp32 from zero; the partial is then promoted into the
// fp32 total with one FMA per element, total += partial * (sa[kb][m] * sb[n/128][kb]).
// After the last block, C is added and the total is rounded to bf16 (RNE).
//
// Work decomposition:
//   * a workgroup owns a BM x BN output tile; its waves each own a
//     (BM/WAVES_M) x (BN/WAVES_N) sub-tile held in VGPRs;
//   * A and B K-blocks stream HBM -> LDS with 16-byte coalesced loads into a
//     two-stage ring, the next stage in flight while the current one feeds
//     the MFMAs; LDS rows are 128 bytes with 16-byte chunks XOR-swizzled by
//     row so that fragment reads are free of bank conflicts;
//   * the A scales of the tile's rows for each K block travel with the stage;
//   * workgroups walk a list of work items (tile, K split); the list is split
//     into 8 contiguous ranges, one per XCD (the hardware deals workgroups to
//     the XCDs round-robin), so that tiles sharing A rows or B columns run on
//     the same XCD and meet in its L2;
//   * masked form: each workgroup builds the per-group tile counts from the
//     device-resident masked_m in LDS and walks the expert groups, skipping
//     empty ones; contiguous form: the expert of each 128-row block is read
//     from the device-resident grouped_layout;
//   * split-K (decode shapes): each split writes its fp32 partial tile to a
//     workspace and bumps a per-tile counter; the last split to arrive sums
//     the partials in split order (deterministic), runs the epilogue and
//     resets the counter to zero for the next call.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dg_internal.h"

namespace dg {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int KBLK = 128;        // K block of the scales and of one MFMA
constexpr int MAX_GROUPS_LDS = 1024;

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 h = static_cast<__bf16>(x);   // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct Shape {
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int NT = NWAVES * 64;
  static constexpr int WTM = BM / WAVES_M;      // wave tile rows
  static constexpr int WTN = BN / WAVES_N;      // wave tile cols
  static constexpr int SM = WTM / 16;           // 16-row strips per wave
  static constexpr int SN = WTN / 16;           // 16-col strips per wave
  static constexpr int A_BYTES = BM * KBLK;
  static constexpr int B_BYTES = BN * KBLK;
  static constexpr int SA_OFF = A_BYTES + B_BYTES;
  static constexpr int STAGE = A_BYTES + B_BYTES + BM * 4;
  static constexpr int A_CHUNKS = BM * 8;       // 16-byte chunks per stage
  static constexpr int B_CHUNKS = BN * 8;
  static constexpr int LA = (A_CHUNKS + NT - 1) / NT;
  static constexpr int LB = (B_CHUNKS + NT - 1) / NT;
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(WTN <= 128 && 128 % WTN == 0, "a wave's columns must sit in one 128-wide B scale block");
  static_assert(BM % 4 == 0 && BM / 4 <= NT, "A scales are staged as float4 by the first BM/4 threads");
};

// Per-work-item geometry resolved by the tile walker.
struct Item {
  int valid;
  int group;      // expert (grouped forms), 0 for dense
  int mt, nt;     // tile coordinates
  int split;      // K split index
  int tile_id;    // linear output tile id (split-K counters)
  int rows_lim;   // rows [0, rows_lim) of the operand may be computed (masked: masked_m)
};

template <int BM, int BN, int WAVES_M, int WAVES_N, int MODE>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64)
fp8_gemm_nt_kernel(Params p) {
  using S = Shape<BM, BN, WAVES_M, WAVES_N>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * S::STAGE];
  __shared__ int s_prefix[MODE == kMasked ? MAX_GROUPS_LDS + 1 : 1];
  __shared__ int s_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int KB = p.K / KBLK;
  const int NB = (p.N + 127) / 128;

  // ---- the work list ------------------------------------------------------
  int total;
  if constexpr (MODE == kMasked) {
    // exclusive prefix over groups of (m tiles * n tiles); masked_m clamped to [0, max_m]
    if (tid == 0) {
      int acc = 0;
      for (int g = 0; g < p.G; ++g) {
        int m = p.masked_m[g];
        m = m < 0 ? 0 : (m > p.rows ? p.rows : m);
        s_prefix[g] = acc;
        acc += ((m + BM - 1) / BM) * p.tiles_n;
      }
      s_prefix[p.G] = acc;
    }
    __syncthreads();
    total = s_prefix[p.G];
  } else {
    total = p.tiles_m * p.tiles_n * p.splits;
  }

  const int slots = (gridDim.x + 7) / 8;          // workgroups per XCD
  const int xcd = blockIdx.x % 8;
  const int slot = blockIdx.x / 8;
  const int per_xcd = (total + 7) / 8;
  const int w_begin = xcd * per_xcd;
  const int w_end = min(total, w_begin + per_xcd);
  int g_cur = 0;                                   // masked walker state

  for (int w = w_begin + slot; w < w_end; w += slots) {
    // ---- resolve the work item ---------------------------------------------
    Item it;
    it.valid = 1;
    it.group = 0;
    it.split = 0;
    it.rows_lim = p.rows;
    if constexpr (MODE == kMasked) {
      while (w >= s_prefix[g_cur + 1]) ++g_cur;
      const int local = w - s_prefix[g_cur];
      int m = p.masked_m[g_cur];
      m = m < 0 ? 0 : (m > p.rows ? p.rows : m);
      const int tm = (m + BM - 1) / BM;
      it.group = g_cur;
      it.mt = local % tm;
      it.nt = local / tm;
      it.rows_lim = m;
      it.tile_id = 0;
    } else {
      const int tile = w / p.splits;
      it.split = w % p.splits;
      it.tile_id = tile;
      // grouped ordering: bands of 8 m-tiles sweep across n
      constexpr int GM = 8;
      const int band = tile / (GM * p.tiles_n);
      const int first_m = band * GM;
      const int gm = min(p.tiles_m - first_m, GM);
      const int in_band = tile - band * GM * p.tiles_n;
      it.mt = first_m + in_band % gm;
      it.nt = in_band / gm;
      if constexpr (MODE == kContiguous) {
        // the expert of this 128-row block: the largest id among its rows
        // (padding rows may carry -1); all valid ids in a block agree
        if (wave == 0) {
          int best = -1;
          for (int r = lane; r < BM; r += 64) {
            const int row = it.mt * BM + r;
            if (row < p.rows) best = max(best, p.layout[row]);
          }
          for (int off = 32; off > 0; off >>= 1) best = max(best, __shfl_xor(best, off));
          if (lane == 0) s_flag = best;
        }
        __syncthreads();
        it.group = s_flag;
        __syncthreads();
        if (it.group < 0 || it.group >= p.G) continue;   // uniform across the workgroup
      }
    }

    const int m0 = it.mt * BM;
    const int n0 = it.nt * BN;
    const int kb_begin = (int)(((long long)KB * it.split) / p.splits);
    const int kb_end = (int)(((long long)KB * (it.split + 1)) / p.splits);

    // ---- operand bases -----------------------------------------------------
    const uint8_t* A = p.a;
    const float* SA = p.sfa;
    const uint8_t* B = p.b;
    const float* SB = p.sfb;
    uint16_t* D = p.d;
    const uint16_t* C = p.c;
    const int a_rows = p.rows;     // rows allocated in this A operand
    if constexpr (MODE == kMasked) {
      A += (size_t)it.group * p.rows * p.K;
      SA += (size_t)it.group * KB * p.rows;
      D += (size_t)it.group * p.rows * p.N;
      if (C) C += (size_t)it.group * p.rows * p.N;
    }
    if constexpr (MODE != kDense) {
      B += (size_t)it.group * p.N * p.K;
      SB += (size_t)it.group * NB * KB;
    }

    // ---- global -> LDS staging ---------------------------------------------
    v4i ra[S::LA], rb[S::LB];
    v4f rsa = {0.f, 0.f, 0.f, 0.f};
    auto gload = [&](int kb) {
#pragma unroll
      for (int i = 0; i < S::LA; ++i) {
        const int q = i * S::NT + tid;
        if (S::A_CHUNKS % S::NT == 0 || q < S::A_CHUNKS) {
          const int r = q >> 3, ch = q & 7;
          int grow = m0 + r;
          grow = grow < a_rows ? grow : a_rows - 1;     // rows past the end are never stored
          ra[i] = *reinterpret_cast<const v4i*>(A + (size_t)grow * p.K + (size_t)kb * KBLK + ch * 16);
        }
      }
#pragma unroll
      for (int i = 0; i < S::LB; ++i) {
        const int q = i * S::NT + tid;
        if (S::B_CHUNKS % S::NT == 0 || q < S::B_CHUNKS) {
          const int r = q >> 3, ch = q & 7;
          int gn = n0 + r;
          gn = gn < p.N ? gn : p.N - 1;
          rb[i] = *reinterpret_cast<const v4i*>(B + (size_t)gn * p.K + (size_t)kb * KBLK + ch * 16);
        }
      }
      if (tid < BM / 4) {
        const int r = m0 + tid * 4;
        const float* src = SA + (size_t)kb * a_rows;
        if (r + 3 < a_rows && ((a_rows & 3) == 0)) {
          rsa = *reinterpret_cast<const v4f*>(src + r);
        } else {
          rsa.x = src[min(r + 0, a_rows - 1)];
          rsa.y = src[min(r + 1, a_rows - 1)];
          rsa.z = src[min(r + 2, a_rows - 1)];
          rsa.w = src[min(r + 3, a_rows - 1)];
        }
      }
    };
    auto lstore = [&](int stage) {
      uint8_t* base = smem + stage * S::STAGE;
#pragma unroll
      for (int i = 0; i < S::LA; ++i) {
        const int q = i * S::NT + tid;
        if (S::A_CHUNKS % S::NT == 0 || q < S::A_CHUNKS) {
          const int r = q >> 3, ch = q & 7;
          *reinterpret_cast<v4i*>(base + r * KBLK + ((ch ^ swz(r)) << 4)) = ra[i];
        }
      }
#pragma unroll
      for (int i = 0; i < S::LB; ++i) {
        const int q = i * S::NT + tid;
        if (S::B_CHUNKS % S::NT == 0 || q < S::B_CHUNKS) {
          const int r = q >> 3, ch = q & 7;
          *reinterpret_cast<v4i*>(base + S::A_BYTES + r * KBLK + ((ch ^ swz(r)) << 4)) = rb[i];
        }
      }
      if (tid < BM / 4) *reinterpret_cast<v4f*>(base + S::SA_OFF + tid * 16) = rsa;
    };

    // ---- accumulators --------------------------------------------------------
    v4f acc[S::SM][S::SN];
#pragma unroll
    for (int i = 0; i < S::SM; ++i)
#pragma unroll
      for (int j = 0; j < S::SN; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

    const int g16 = lane >> 4;          // which 32-byte K slice of the row (operands), row quad (result)
    const int r16 = lane & 15;          // row of A / column of B within a 16-strip
    const int wrow0 = wm * S::WTM;      // wave's first row in the tile
    const int wcol0 = wn * S::WTN;
    int nb = (n0 + wcol0) / 128;
    nb = nb < NB ? nb : NB - 1;

    if (kb_begin < kb_end) {
      gload(kb_begin);
      lstore(0);
    }
    for (int kb = kb_begin; kb < kb_end; ++kb) {
      const int stage = (kb - kb_begin) & 1;
      __syncthreads();
      const bool more = kb + 1 < kb_end;
      if (more) gload(kb + 1);

      const uint8_t* base = smem + stage * S::STAGE;
      const float sb = SB[(size_t)nb * KB + kb];

      v8i bf[S::SN];
#pragma unroll
      for (int j = 0; j < S::SN; ++j) {
        const int r = wcol0 + j * 16 + r16;
        const uint8_t* rp = base + S::A_BYTES + r * KBLK;
        const int s = swz(r);
        const v4i lo = *reinterpret_cast<const v4i*>(rp + (((2 * g16) ^ s) << 4));
        const v4i hi = *reinterpret_cast<const v4i*>(rp + (((2 * g16 + 1) ^ s) << 4));
        bf[j] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
#pragma unroll
      for (int i = 0; i < S::SM; ++i) {
        const int r = wrow0 + i * 16 + r16;
        const uint8_t* rp = base + r * KBLK;
        const int s = swz(r);
        const v4i lo = *reinterpret_cast<const v4i*>(rp + (((2 * g16) ^ s) << 4));
        const v4i hi = *reinterpret_cast<const v4i*>(rp + (((2 * g16 + 1) ^ s) << 4));
        const v8i af = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        // scales of this lane's four result rows
        const v4f sa4 = *reinterpret_cast<const v4f*>(base + S::SA_OFF + (wrow0 + i * 16 + g16 * 4) * 4);
        const v4f sc = sa4 * sb;
#pragma unroll
        for (int j = 0; j < S::SN; ++j) {
          const v4f zero = {0.f, 0.f, 0.f, 0.f};
          const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], zero, 0, 0, 0, 0, 0, 0);
          acc[i][j].x = __builtin_fmaf(part.x, sc.x, acc[i][j].x);
          acc[i][j].y = __builtin_fmaf(part.y, sc.y, acc[i][j].y);
          acc[i][j].z = __builtin_fmaf(part.z, sc.z, acc[i][j].z);
          acc[i][j].w = __builtin_fmaf(part.w, sc.w, acc[i][j].w);
        }
      }
      if (more) lstore(stage ^ 1);
    }

    // ---- split-K: publish the partial, the last split reduces ----------------
    if (p.splits > 1) {
      float* ws = p.workspace + (size_t)it.tile_id * p.splits * (BM * BN);
      v4f* mine = reinterpret_cast<v4f*>(ws + (size_t)it.split * (BM * BN));
#pragma unroll
      for (int i = 0; i < S::SM; ++i)
#pragma unroll
        for (int j = 0; j < S::SN; ++j)
          mine[((wave * S::SM + i) * S::SN + j) * 64 + lane] = acc[i][j];
      __threadfence();
      __syncthreads();
      if (tid == 0) {
        const int old = atomicAdd(p.counters + it.tile_id, 1);
        s_flag = (old == p.splits - 1);
      }
      __syncthreads();
      const int last = s_flag;
      __syncthreads();
      if (!last) continue;
      __threadfence();
#pragma unroll
      for (int i = 0; i < S::SM; ++i)
#pragma unroll
        for (int j = 0; j < S::SN; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < p.splits; ++s) {
        const v4f* src = reinterpret_cast<const v4f*>(ws + (size_t)s * (BM * BN));
#pragma unroll
        for (int i = 0; i < S::SM; ++i)
#pragma unroll
          for (int j = 0; j < S::SN; ++j)
            acc[i][j] += __builtin_nontemporal_load(&src[((wave * S::SM + i) * S::SN + j) * 64 + lane]);
      }
      if (tid == 0) p.counters[it.tile_id] = 0;
    }

    // ---- epilogue: + C, round to bf16, store the rows that belong to the result
#pragma unroll
    for (int i = 0; i < S::SM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wrow0 + i * 16 + g16 * 4 + e;
        bool ok = row < it.rows_lim;
        if constexpr (MODE == kContiguous) ok = ok && p.layout[row] == it.group;
        if (!ok) continue;
#pragma unroll
        for (int j = 0; j < S::SN; ++j) {
          const int col = n0 + wcol0 + j * 16 + r16;
          if (col < p.N) {
            float v = acc[i][j][e];
            if (C) v += bf16_to_f32(C[(size_t)row * p.N + col]);
            D[(size_t)row * p.N + col] = f32_to_bf16(v);
          }
        }
      }
    }
    // the next item reuses the LDS ring
    __syncthreads();
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
hipError_t launch_cfg(int mode, const Params& p, int grid, hipStream_t stream) {
  constexpr int threads = WAVES_M * WAVES_N * 64;
  switch (mode) {
    case kDense:
      hipLaunchKernelGGL((fp8_gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, kDense>), dim3(grid), dim3(threads), 0, stream, p);
      break;
    case kContiguous:
      hipLaunchKernelGGL((fp8_gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, kContiguous>), dim3(grid), dim3(threads), 0, stream, p);
      break;
    case kMasked:
      hipLaunchKernelGGL((fp8_gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, kMasked>), dim3(grid), dim3(threads), 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

const ConfigInfo kConfigs[kNumConfigs] = {
    {128, 128, 256, "128x128_w2x2"},
    {64, 64, 256, "64x64_w1x4"},
    {256, 128, 256, "256x128_w2x2"},
    {128, 64, 256, "128x64_w2x2"},
};

}  // namespace

const ConfigInfo& config_info(int cfg) { return kConfigs[cfg]; }

hipError_t launch_gemm(int mode, int cfg, const Params& p, int grid, hipStream_t stream) {
  switch (cfg) {
    case kCfg128x128: return launch_cfg<128, 128, 2, 2>(mode, p, grid, stream);
    case kCfg64x64: return launch_cfg<64, 64, 1, 4>(mode, p, grid, stream);
    case kCfg256x128: return launch_cfg<256, 128, 2, 2>(mode, p, grid, stream);
    case kCfg128x64: return launch_cfg<128, 64, 2, 2>(mode, p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dg
