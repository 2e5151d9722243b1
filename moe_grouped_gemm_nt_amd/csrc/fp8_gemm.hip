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

// ============================================================================
// narrow kernel (dense shapes with few rows): the whole K per workgroup
// ============================================================================
// A workgroup owns a 16-row x 48-column tile and the whole K, so no partial
// sums leave it and one launch does all the work.  Its four waves take the K
// blocks in turn (wave w: blocks w, w+4, ...); each wave streams its blocks
// through a private ring of NR LDS slots with direct global->LDS loads (8 rows
// of 128 bytes per instruction: A 16 rows, B 48 rows, the 16 row scales and
// the B scales of the three 16-column strips) and waits only for its own
// loads, so the K loop has no barrier.  At the end the four wave totals are
// summed through LDS in wave order, C is added and the result rounded.  The
// m-strips of one column slice get workgroup ids of one residue mod 8, so
// they run on one XCD and read B from one L2.
constexpr int NWM = 16, NWN = 48;                // tile
constexpr int NR = 4;                            // slots per wave
constexpr int NA = NWM * KBLK, NBB = NWN * KBLK; // A / B bytes per block
constexpr int NSLOTB = NA + NBB + NWM * 4 + 16;  // + row scales + strip B scales
constexpr int NLPB = NWM / 8 + NWN / 8 + 2;      // loads per block
static_assert(NLPB * NR < 64, "outstanding loads must fit the 6-bit vmcnt");

__global__ void __launch_bounds__(256)
fp8_gemm_nt_narrow_kernel(Params p) {
  constexpr int SN = NWN / 16;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * NR * NSLOTB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g16 = lane >> 4, r16 = lane & 15;
  const int strips = (p.rows + NWM - 1) / NWM;
  const int slices = (p.N + NWN - 1) / NWN;
  const int xcd = blockIdx.x % 8, k = blockIdx.x / 8;
  const int slice = (k / strips) * 8 + xcd, strip = k % strips;
  if (slice >= slices) return;
  const int m0 = strip * NWM, n0 = slice * NWN;
  const int KB = p.K / KBLK;
  const int NB = (p.N + 127) / 128;
  const uint32_t ring = lds_u32(smem) + (uint32_t)(wave * NR * NSLOTB);

  // load sources: lane l of a load instruction takes row 8q + l/8, 16-byte
  // chunk l%8 (stored at its swizzled position)
  const int lr = lane >> 3;
  const uint8_t* a_src[NWM / 8];
  const uint8_t* b_src[NWN / 8];
#pragma unroll
  for (int q = 0; q < NWM / 8; ++q) {
    const int r = q * 8 + lr;
    a_src[q] = p.a + (size_t)min(m0 + r, p.rows - 1) * p.K + (((lane & 7) ^ swz(r)) << 4);
  }
#pragma unroll
  for (int q = 0; q < NWN / 8; ++q) {
    const int r = q * 8 + lr;
    b_src[q] = p.b + (size_t)min(n0 + r, p.N - 1) * p.K + (((lane & 7) ^ swz(r)) << 4);
  }
  const float* sa_src = p.sfa + min(m0 + (lane & 15), p.rows - 1);
  const int strip_nb = min(min(n0 + 16 * min(lane, SN - 1), p.N - 1) / 128, NB - 1);
  const float* sb_src = p.sfb + (size_t)strip_nb * KB;

  const int nblk = wave < KB ? (KB - wave + 3) / 4 : 0;
  auto issue = [&](int j, int u) {
    const int kb = wave + 4 * j;
    const size_t kofs = (size_t)kb * KBLK;
    const uint32_t slot = ring + (uint32_t)(u * NSLOTB);
#pragma unroll
    for (int q = 0; q < NWM / 8; ++q) dma_16(a_src[q] + kofs, slot + q * 1024);
#pragma unroll
    for (int q = 0; q < NWN / 8; ++q) dma_16(b_src[q] + kofs, slot + NA + q * 1024);
    if (lane < 16) dma_4(sa_src + (size_t)kb * p.rows, slot + NA + NBB);
    if (lane < SN) dma_4(sb_src + kb, slot + NA + NBB + NWM * 4);
  };
  v4f acc[1][SN];
#pragma unroll
  for (int c = 0; c < SN; ++c) acc[0][c] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < NR; ++u)
    if (u < nblk) issue(u, u);
  for (int j0 = 0; j0 < nblk; j0 += NR) {
    static_for<NR>([&](auto u_const) {
      constexpr int u = decltype(u_const)::value;
      const int j = j0 + u;
      if (j < nblk) {
        wait_stages<NLPB, NR - 1>(min(NR - 1, nblk - 1 - j));
        const uint8_t* base = smem + (wave * NR + u) * NSLOTB;
        const float* sa = reinterpret_cast<const float*>(base + NA + NBB);
        v8i bf[SN];
#pragma unroll
        for (int c = 0; c < SN; ++c) bf[c] = lds_fragment(base + NA, c * 16 + r16, g16);
        const v8i af = lds_fragment(base, r16, g16);
        const v4f sr = *reinterpret_cast<const v4f*>(sa + g16 * 4);
        v4f q[SN];
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < SN; ++c)
          q[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[c], zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int c = 0; c < SN; ++c) {
          const v4f f = sr * sa[NWM + c];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[0][c][e] = __builtin_fmaf(q[c][e], f[e], acc[0][c][e]);
        }
        if (j + NR < nblk) {
          wait_vm_lgkm0<63>();                    // the slot's LDS reads have completed
          issue(j + NR, u);
        }
      }
    });
  }
  // wave totals, summed in wave order through the (now idle) slot memory
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  v4f* red = reinterpret_cast<v4f*>(smem);
  if (wave > 0) {
#pragma unroll
    for (int c = 0; c < SN; ++c) red[((wave - 1) * SN + c) * 64 + lane] = acc[0][c];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int c = 0; c < SN; ++c) acc[0][c] += red[(w * SN + c) * 64 + lane];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = m0 + 4 * g16 + e;
#pragma unroll
    for (int c = 0; c < SN; ++c) {
      const int col = n0 + 16 * c + r16;
      float v = acc[0][c][e];
      if (p.c) v += bf16_to_f32(p.c[(size_t)min(row, p.rows - 1) * p.N + min(col, p.N - 1)]);
      if (row < p.rows && col < p.N) p.d[(size_t)row * p.N + col] = f32_to_bf16(v);
    }
  }
}

hipError_t launch_narrow(const Params& p, hipStream_t stream) {
  const int strips = (p.rows + NWM - 1) / NWM;
  const int slices = (p.N + NWN - 1) / NWN;
  const int grid = 8 * strips * ((slices + 7) / 8);
  hipLaunchKernelGGL(fp8_gemm_nt_narrow_kernel, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
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
    {NWM, NWN, 256, "narrow_16x48_fullk"},
    {256, 256, 512, "e8m0_256x256_w2x4_s2"},
    {256, 256, 512, "256x256_w2x4_s2"},
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
    case kCfg256x256w8: return launch_cfg<256, 256, 2, 4, 2>(mode, p, grid, stream);
    case kCfgE8_128x256:
    case kCfgWs_128x256:
    case kCfgE8_256x256: return launch_gemm_e8m0(mode, cfg, p, grid, stream);
    case kCfgNarrow: return mode == kDense ? launch_narrow(p, stream) : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dg
