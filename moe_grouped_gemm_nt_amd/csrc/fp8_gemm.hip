// gfx950 kernels for the FP8 block-scaled GEMM, NT layout: instantiations of
// the tile kernel with fp32 promotion on the VALU (any fp32 scales), the
// decode kernel and its split-K reduction, and the launch dispatch.  The
// kernels themselves are described in fp8_gemm_core.h.
//
// Built with MFMA results in VGPRs (-amdgpu-mfma-vgpr-form), where the
// promotion FMAs read them.
#include "fp8_gemm_core.h"

namespace dg {
namespace {

// ============================================================================
// decode kernel: 64x64 tiles, K split across workgroups and across waves
// ============================================================================
constexpr int DBM = 64, DBN = 64;                 // decode tile
constexpr int DKBS = 8;                           // max K blocks per workgroup
constexpr int DSLOT = DBM * KBLK + DBN * KBLK + DBM * 4;
constexpr int DLPB = DBM / 8 + DBN / 8 + 1;       // loads per K block (one wave)
constexpr int DNPW = DKBS / 4;                    // K blocks per wave
static_assert(DBM == 64, "one 64-lane load carries the tile's row scales");
static_assert(DLPB * DNPW < 64, "outstanding loads must fit the 6-bit vmcnt");
static_assert(4 * DBM * DBN * 4 <= DKBS * DSLOT, "the wave reduction reuses the slot memory");

__global__ void __launch_bounds__(256)
fp8_gemm_nt_decode_kernel(Params p) {
  constexpr int SM = DBM / 16, SN = DBN / 16, T = SM * SN;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[DKBS * DSLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t smem_base = lds_u32(smem);
  const int KB = p.K / KBLK;
  const int NB = (p.N + 127) / 128;

  // work item: XCD-contiguous ranges of (tile, split), splits of a tile adjacent
  const int total = p.tiles_m * p.tiles_n * p.splits;
  const int per_xcd = (total + 7) / 8;
  const int w = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (blockIdx.x / 8 >= per_xcd || w >= total) return;
  const int tile = w / p.splits;
  const int split = w % p.splits;
  int mt, nt;
  tile_coords(tile, p.tiles_m, p.tiles_n, mt, nt);
  const int m0 = mt * DBM, n0 = nt * DBN;
  const int kb0 = split * p.kbs_per_split;
  const int kbs = max(0, min(p.kbs_per_split, KB - kb0));
  int nb = n0 / 128;
  nb = nb < NB ? nb : NB - 1;

  // this wave's K blocks: kb0 + wave, kb0 + wave + 4, ...
  const int nown = kbs > wave ? (kbs - wave + 3) / 4 : 0;
  float sb[DNPW];
#pragma unroll
  for (int j = 0; j < DNPW; ++j) sb[j] = p.sfb[(size_t)nb * KB + min(kb0 + wave + 4 * j, KB - 1)];

  // issue every load of this wave's blocks: A (64 rows), B (64 rows), A scales
  const int lr = lane >> 3;
#pragma unroll
  for (int j = 0; j < DNPW; ++j) {
    if (j < nown) {
      const int kb = kb0 + wave + 4 * j;
      const uint32_t slot = smem_base + (uint32_t)((wave + 4 * j) * DSLOT);
#pragma unroll
      for (int q = 0; q < DBM / 8; ++q) {
        const int r = q * 8 + lr;
        const int grow = min(m0 + r, p.rows - 1);
        dma_16(p.a + (size_t)grow * p.K + (size_t)kb * KBLK + (((lane & 7) ^ swz(r)) << 4), slot + q * 1024);
      }
#pragma unroll
      for (int q = 0; q < DBN / 8; ++q) {
        const int r = q * 8 + lr;
        const int gn = min(n0 + r, p.N - 1);
        dma_16(p.b + (size_t)gn * p.K + (size_t)kb * KBLK + (((lane & 7) ^ swz(r)) << 4),
               slot + DBM * KBLK + q * 1024);
      }
      dma_4(p.sfa + (size_t)kb * p.rows + min(m0 + lane, p.rows - 1), slot + (DBM + DBN) * KBLK);
    }
  }

  v4f acc[SM][SN];
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
  const int g16 = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int j = 0; j < DNPW; ++j) {
    if (j < nown) {
      wait_stages<DLPB, DNPW - 1>(nown - 1 - j);
      const uint8_t* base = smem + (wave + 4 * j) * DSLOT;
      const float* sa = reinterpret_cast<const float*>(base + (DBM + DBN) * KBLK);
      v4f sc[SM];
#pragma unroll
      for (int i = 0; i < SM; ++i) sc[i] = *reinterpret_cast<const v4f*>(sa + i * 16 + g16 * 4) * sb[j];
      mma_block<SM, SN>(base, 0, base + DBM * KBLK, 0, sc, acc, lane);
    }
  }

  // ---- sum the four wave totals in wave order; wave w finishes strip w ----
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  v4f* red = reinterpret_cast<v4f*>(smem);
#pragma unroll
  for (int t = 0; t < T; ++t) red[(wave * T + t) * 64 + lane] = acc[t / SN][t % SN];
  __syncthreads();
  v4f out[SN];
#pragma unroll
  for (int j = 0; j < SN; ++j) {
    const int t = wave * SN + j;
    out[j] = red[t * 64 + lane];
#pragma unroll
    for (int src = 1; src < 4; ++src) out[j] += red[(src * T + t) * 64 + lane];
  }

  if (p.splits > 1) {
    // fp32 partial, in the result layout: [tile][split][sub-tile][lane]
    if (!p.splitk_inline) {
      v4f* ws = reinterpret_cast<v4f*>(p.workspace) + ((size_t)tile * p.splits + split) * (T * 64);
#pragma unroll
      for (int j = 0; j < SN; ++j) ws[(wave * SN + j) * 64 + lane] = out[j];
      return;
    }
    // In-kernel reduction by the last split to arrive.  Partials are written
    // and read with device-scope (sc1) accesses, which are coherent across the
    // XCDs' L2 caches without flushing or invalidating them; a split's stores
    // are complete (vmcnt 0) before its arrival is counted, and the last split
    // reads them only after it has seen every arrival.
    // C of this wave's strip, fetched now so its latency hides behind the exchange
    float cpre[4][SN];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        const int row = min(m0 + wave * 16 + g16 * 4 + e, p.rows - 1), col = min(n0 + j * 16 + r16, p.N - 1);
        cpre[e][j] = p.c ? bf16_to_f32(p.c[(size_t)row * p.N + col]) : 0.f;
      }
    const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(
        p.workspace, 0, (int)(p.workspace_bytes > 0x7fffffff ? 0x7fffffff : p.workspace_bytes), 0x00020000);
    constexpr int SC1 = 0x10;     // cache-policy bits of a device-scope access
    const size_t part_base = ((size_t)tile * p.splits) * (T * 64);
#pragma unroll
    for (int j = 0; j < SN; ++j)
      __builtin_amdgcn_raw_buffer_store_b128(
          out[j], ws, (int)(((part_base + (size_t)split * (T * 64)) + (wave * SN + j) * 64 + lane) * 16), 0, SC1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __shared__ int s_last;
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(p.counters + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               p.splits - 1;
    __syncthreads();
    if (!s_last) return;
    constexpr int MAXS = 8;
#pragma unroll
    for (int j = 0; j < SN; ++j) out[j] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < p.splits; s0 += MAXS) {
      v4f part[MAXS][SN];
#pragma unroll
      for (int u = 0; u < MAXS; ++u)
        if (s0 + u < p.splits) {
#pragma unroll
          for (int j = 0; j < SN; ++j)
            part[u][j] = __builtin_amdgcn_raw_buffer_load_b128(
                ws, (int)((part_base + (size_t)(s0 + u) * (T * 64) + (wave * SN + j) * 64 + lane) * 16), 0, SC1);
        }
#pragma unroll
      for (int u = 0; u < MAXS; ++u)
        if (s0 + u < p.splits) {
#pragma unroll
          for (int j = 0; j < SN; ++j) out[j] += part[u][j];
        }
    }
    if (tid == 0) __hip_atomic_store(p.counters + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = m0 + wave * 16 + g16 * 4 + e;
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        const int col = n0 + j * 16 + r16;
        if (row < p.rows && col < p.N) p.d[(size_t)row * p.N + col] = f32_to_bf16(out[j][e] + cpre[e][j]);
      }
    }
    return;
  }
  // single split: + C, round, store
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = m0 + wave * 16 + g16 * 4 + e;
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const int col = n0 + j * 16 + r16;
      if (p.c) out[j][e] += bf16_to_f32(p.c[(size_t)min(row, p.rows - 1) * p.N + min(col, p.N - 1)]);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = m0 + wave * 16 + g16 * 4 + e;
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const int col = n0 + j * 16 + r16;
      if (row < p.rows && col < p.N) p.d[(size_t)row * p.N + col] = f32_to_bf16(out[j][e]);
    }
  }
}

// Split-K reduction of the decode kernel's partials: one 64-lane workgroup per
// (tile, 16-row strip).  Every load (all splits, C) is issued before any add so
// one memory round trip covers them; the splits are summed in split order.
__global__ void __launch_bounds__(64)
splitk_reduce_kernel(Params p) {
  constexpr int SN = DBN / 16, T = (DBM / 16) * SN;
  constexpr int MAXS = 8;                        // splits loaded per pass
  const int lane = threadIdx.x;
  const int tile = blockIdx.x / (DBM / 16);
  const int strip = blockIdx.x % (DBM / 16);
  int mt, nt;
  tile_coords(tile, p.tiles_m, p.tiles_n, mt, nt);
  const int g16 = lane >> 4, r16 = lane & 15;
  const int m0 = mt * DBM + strip * 16, n0 = nt * DBN;
  const v4f* ws = reinterpret_cast<const v4f*>(p.workspace) + (size_t)tile * p.splits * (T * 64);

  float cv[4][SN];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const int row = min(m0 + g16 * 4 + e, p.rows - 1), col = min(n0 + j * 16 + r16, p.N - 1);
      cv[e][j] = p.c ? bf16_to_f32(p.c[(size_t)row * p.N + col]) : 0.f;
    }
  v4f acc[SN];
#pragma unroll
  for (int j = 0; j < SN; ++j) acc[j] = (v4f){0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < p.splits; s0 += MAXS) {
    v4f part[MAXS][SN];
#pragma unroll
    for (int u = 0; u < MAXS; ++u) {
      if (s0 + u < p.splits) {
        const v4f* src = ws + (size_t)(s0 + u) * (T * 64);
#pragma unroll
        for (int j = 0; j < SN; ++j) part[u][j] = __builtin_nontemporal_load(&src[(strip * SN + j) * 64 + lane]);
      }
    }
#pragma unroll
    for (int u = 0; u < MAXS; ++u)
      if (s0 + u < p.splits) {
#pragma unroll
        for (int j = 0; j < SN; ++j) acc[j] += part[u][j];
      }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = m0 + g16 * 4 + e;
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const int col = n0 + j * 16 + r16;
      if (row < p.rows && col < p.N) p.d[(size_t)row * p.N + col] = f32_to_bf16(acc[j][e] + cv[e][j]);
    }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int NSLOT, int WG_PER_CU = 1>
hipError_t launch_cfg(int mode, const Params& p, int grid, hipStream_t stream) {
  constexpr int threads = WAVES_M * WAVES_N * 64;
  switch (mode) {
    case kDense:
      hipLaunchKernelGGL((fp8_gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, NSLOT, kDense, WG_PER_CU, false>), dim3(grid),
                         dim3(threads), 0, stream, p);
      break;
    case kContiguous:
      hipLaunchKernelGGL((fp8_gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, NSLOT, kContiguous, WG_PER_CU, false>),
                         dim3(grid), dim3(threads), 0, stream, p);
      break;
    case kMasked:
      hipLaunchKernelGGL((fp8_gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, NSLOT, kMasked, WG_PER_CU, false>), dim3(grid),
                         dim3(threads), 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const Params& p, hipStream_t stream) {
  const int items = p.tiles_m * p.tiles_n * p.splits;
  const int grid = ((items + 7) / 8) * 8;
  hipLaunchKernelGGL(fp8_gemm_nt_decode_kernel, dim3(grid), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1 || p.splitk_inline) return e;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(p.tiles_m * p.tiles_n * (DBM / 16)), dim3(64), 0, stream, p);
  return hipGetLastError();
}

const ConfigInfo kConfigs[kNumConfigs] = {
    {128, 128, 256, "128x128_w2x2_s4"},
    {DBM, DBN, 256, "decode_64x64_ksplit"},
    {128, 64, 256, "128x64_w2x2_s4"},
    {64, 128, 256, "64x128_w1x4_s4"},
    {128, 128, 256, "128x128_w2x2_s2_2wg"},
    {256, 128, 512, "256x128_w4x2_s3"},
    {128, 256, 512, "128x256_w2x4_s3"},
    {128, 256, 256, "e8m0_128x256_w2x2_s3"},
    {128, 256, 512, "e8m0_ws_128x256_w2x2+4_s3"},
};

}  // namespace

const ConfigInfo& config_info(int cfg) { return kConfigs[cfg]; }

hipError_t launch_gemm(int mode, int cfg, const Params& p, int grid, hipStream_t stream) {
  switch (cfg) {
    case kCfg128x128: return launch_cfg<128, 128, 2, 2, 4>(mode, p, grid, stream);
    case kCfgDecode: return mode == kDense ? launch_decode(p, stream) : hipErrorInvalidValue;
    case kCfg128x64: return launch_cfg<128, 64, 2, 2, 4>(mode, p, grid, stream);
    case kCfg64x128: return launch_cfg<64, 128, 1, 4, 4>(mode, p, grid, stream);
    case kCfg128x128x2: return launch_cfg<128, 128, 2, 2, 2, 2>(mode, p, grid, stream);
    case kCfg256x128w8: return launch_cfg<256, 128, 4, 2, 3>(mode, p, grid, stream);
    case kCfg128x256w8: return launch_cfg<128, 256, 2, 4, 3>(mode, p, grid, stream);
    case kCfgE8_128x256:
    case kCfgWs_128x256: return launch_gemm_e8m0(mode, cfg, p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dg
