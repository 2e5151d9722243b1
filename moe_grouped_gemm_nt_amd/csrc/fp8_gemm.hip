// gfx950 kernels for the FP8 block-scaled GEMM: instantiations of the tile
// kernel with fp32 promotion on the VALU (any fp32 scales) for every form
// (dense in the four storages, M-grouped contiguous and masked, K-grouped,
// FP8 x FP4), the decode kernel (64x64 tiles with K split over workgroups, in
// any operand storage and with an FP4 B) and its split-K reduction, the
// narrow kernel, the split-tail reduction, and the launch dispatch.  The tile
// and decode kernels' structure is described in fp8_gemm_core.h.
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
constexpr int DNW = 4;                            // waves per workgroup
// one K block's slot: A rows, B rows (FP4: 64 bytes each), A row scales and,
// for an FP4 B, its packed E8M0 column scales
template <bool B4> constexpr int dslot() { return DBM * KBLK + DBN * (B4 ? KBLK / 2 : KBLK) + DBM * 4 + (B4 ? DBN * 4 : 0); }
template <bool B4> constexpr int dlpb() { return DBM / 8 + DBN / (B4 ? 16 : 8) + 1 + B4; }   // loads per K block (one wave)
constexpr int DLPB = dlpb<false>();
constexpr int DNPW = DKBS / DNW;                  // K blocks per wave
constexpr int DT = (DBM / 16) * (DBN / 16);       // 16x16 sub-tiles of the tile
constexpr int DTPW = DT / DNW;                    // sub-tiles each wave finishes
static_assert(DBM == 64, "one 64-lane load carries the tile's row scales");
static_assert(DKBS % DNW == 0 && DT % DNW == 0, "blocks and sub-tiles divide among the waves");
static_assert(DLPB * DNPW < 64, "outstanding loads must fit the 6-bit vmcnt");
static_assert(DNW * DT * 64 * 16 <= DKBS * dslot<true>(), "the wave reduction reuses the slot memory");

// One K block of the FP8 x FP4 decode tile: like mma_block, with B rows of 64
// bytes (chunk c of row r at c ^ swz4(r)), the A fragment read as K chunks g16
// and 4+g16 (the fp8 operand's K order against an FP4 operand), and each
// lane's E8M0 byte for its column and 32-K slice taken from the packed ints.
template <int SM, int SN>
__device__ __forceinline__ void mma_block_fp4(const uint8_t* a_rows, const uint8_t* b_rows, const uint32_t* bscale,
                                              const v4f (&sc)[SM], v4f (&acc)[SM][SN], int lane) {
  const int g16 = lane >> 4, r16 = lane & 15;
  v8i bf[SN], af[SM];
  int esb[SN];
#pragma unroll
  for (int j = 0; j < SN; ++j) {
    const int r = j * 16 + r16;
    const v4i q = *reinterpret_cast<const v4i*>(b_rows + r * (KBLK / 2) + ((g16 ^ swz4(r)) << 4));
    bf[j] = (v8i){q.x, q.y, q.z, q.w, 0, 0, 0, 0};
    esb[j] = (int)((bscale[r] >> (8 * g16)) & 0xFF);
  }
#pragma unroll
  for (int i = 0; i < SM; ++i) {
    const int r = i * 16 + r16;
    const uint8_t* rp = a_rows + r * KBLK;
    const v4i lo = *reinterpret_cast<const v4i*>(rp + ((g16 ^ swz(r)) << 4));
    const v4i hi = *reinterpret_cast<const v4i*>(rp + (((4 + g16) ^ swz(r)) << 4));
    af[i] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  }
  constexpr int T = SM * SN;
  constexpr int P = 4;
  v4f part[P];
#pragma unroll
  for (int t = 0; t < T + P - 1; ++t) {
    if (t < T) {
      const v4f zero = {0.f, 0.f, 0.f, 0.f};
      part[t % P] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[t / SN], bf[t % SN], zero, 0, 4, 0, 127, 0,
                                                                     esb[t % SN]);
    }
    const int u = t - (P - 1);
    if (u >= 0) {
      v4f& a = acc[u / SN][u % SN];
      const v4f& q = part[u % P];
      const v4f& c = sc[u / SN];
      a.x = __builtin_fmaf(q.x, c.x, a.x);
      a.y = __builtin_fmaf(q.y, c.y, a.y);
      a.z = __builtin_fmaf(q.z, c.z, a.z);
      a.w = __builtin_fmaf(q.w, c.w, a.w);
    }
  }
}

// One K block of the decode tile with a K-major operand (TA: A stored
// [K][M]; TB: B stored [K][N]): such an operand's block sits in LDS in the
// octet layout of kmajor_slot<64> and its fragments are gathered with the
// transposing LDS reads of kmajor_frag; the other operand is read as in
// mma_block.  a_lds / b_lds are the LDS addresses of the same rows.
template <int SM, int SN, bool TA, bool TB>
__device__ __forceinline__ void mma_block_kmajor(const uint8_t* a_rows, uint32_t a_lds, const uint8_t* b_rows,
                                                 uint32_t b_lds, const v4f (&sc)[SM], v4f (&acc)[SM][SN], int lane) {
  const int g16 = lane >> 4, r16 = lane & 15;
  v8i bf[SN], af[SM];
#pragma unroll
  for (int j = 0; j < SN; ++j)
    bf[j] = TB ? kmajor_frag<DBN>(b_lds + kmajor_frag_base<DBN>(0, lane, j & 1) + 128 * j)
               : lds_fragment(b_rows, j * 16 + r16, g16);
#pragma unroll
  for (int i = 0; i < SM; ++i)
    af[i] = TA ? kmajor_frag<DBM>(a_lds + kmajor_frag_base<DBM>(0, lane, i & 1) + 128 * i)
               : lds_fragment(a_rows, i * 16 + r16, g16);
  constexpr int T = SM * SN;
  constexpr int P = 4;
  v4f part[P];
#pragma unroll
  for (int t = 0; t < T + P - 1; ++t) {
    if (t < T) {
      const v4f zero = {0.f, 0.f, 0.f, 0.f};
      part[t % P] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[t / SN], bf[t % SN], zero, 0, 0, 0, 0, 0, 0);
    }
    const int u = t - (P - 1);
    if (u >= 0) {
      v4f& a = acc[u / SN][u % SN];
      const v4f& q = part[u % P];
      const v4f& c = sc[u / SN];
      a.x = __builtin_fmaf(q.x, c.x, a.x);
      a.y = __builtin_fmaf(q.y, c.y, a.y);
      a.z = __builtin_fmaf(q.z, c.z, a.z);
      a.w = __builtin_fmaf(q.w, c.w, a.w);
    }
  }
}

// LAYOUT: 0 nt; 1 tt (A stored [K][M]); 2 nn (B stored [K][N]); 3 tn (both);
// 4 FP8 x FP4: B holds packed FP4 (E2M1) codes with E8M0 scales per column per
// 32 K values, packed four to an int32 [K/128][N].
// One work item of the decode kernels: the (tile, split) pair's fp32 result
// over its K blocks, summed over the four waves; on return out[j] holds
// sub-tile wave*DTPW + j (lane layout of the MFMA result) and the slot memory
// is free once the workgroup has passed a barrier.
template <int LAYOUT>
__device__ __forceinline__ void decode_item(const Params& p, uint8_t* smem, int tile, int split, v4f (&out)[DTPW]) {
  constexpr bool B4 = LAYOUT == 4;
  constexpr bool TA = !B4 && (LAYOUT & 1), TB = !B4 && (LAYOUT & 2);
  constexpr int SM = DBM / 16, SN = DBN / 16, T = DT;
  constexpr int SLOT = dslot<B4>(), LPB = dlpb<B4>();
  constexpr int BROW = B4 ? KBLK / 2 : KBLK;       // bytes of a B row per K block

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t smem_base = lds_u32(smem);
  const int KB = p.K / KBLK;
  const int NB = (p.N + 127) / 128;
  int mt, nt;
  tile_coords(tile, p.tiles_m, p.tiles_n, mt, nt);
  const int m0 = mt * DBM, n0 = nt * DBN;
  const int kb0 = split * p.kbs_per_split;
  const int kbs = max(0, min(p.kbs_per_split, KB - kb0));
  int nb = n0 / 128;
  nb = nb < NB ? nb : NB - 1;

  // this wave's K blocks: kb0 + wave, kb0 + wave + DNW, ...
  const int nown = kbs > wave ? (kbs - wave + DNW - 1) / DNW : 0;
  float sb[DNPW];                 // the block's B scale (FP4: 1, the MFMA applies the E8M0 scales)
#pragma unroll
  for (int j = 0; j < DNPW; ++j)
    sb[j] = B4 || j >= nown ? 1.f : p.sfb[(size_t)nb * KB + kb0 + wave + DNW * j];   // only blocks the wave owns

  // issue every load of this wave's blocks: A (64 rows), B (64 rows), A scales.
  // B lines are read once per call (streaming policy); the other column tiles
  // read A again from the L2 (default policy)
  const int lr = lane >> 3;
#pragma unroll
  for (int j = 0; j < DNPW; ++j) {
    if (j < nown) {
      const int kb = kb0 + wave + DNW * j;
      const uint32_t slot = smem_base + (uint32_t)((wave + DNW * j) * SLOT);
      if constexpr (TA) {
        // A stored [K][M]: 128 K rows of the tile's 64 columns in octets
        // (kmajor_slot); chunks past M re-read the last 16 columns
#pragma unroll
        for (int q = 0; q < DBM / 8; ++q) {
          int kr, c;
          kmajor_slot<DBM>(64 * q + lane, kr, c);
          dma_16(p.a + (size_t)(kb * KBLK + kr) * p.rows + min(m0 + 16 * c, p.rows - 16), slot + q * 1024);
        }
      } else {
#pragma unroll
        for (int q = 0; q < DBM / 8; ++q) {
          const int r = q * 8 + lr;
          const int grow = min(m0 + r, p.rows - 1);
          dma_16(p.a + (size_t)grow * p.K + (size_t)kb * KBLK + (((lane & 7) ^ swz(r)) << 4), slot + q * 1024);
        }
      }
      if constexpr (TB) {
        // B stored [K][N], as A above
#pragma unroll
        for (int q = 0; q < DBN / 8; ++q) {
          int kr, c;
          kmajor_slot<DBN>(64 * q + lane, kr, c);
          dma_16_nt(p.b + (size_t)(kb * KBLK + kr) * p.N + min(n0 + 16 * c, p.N - 16), slot + DBM * KBLK + q * 1024);
        }
      } else if constexpr (B4) {
        // 16 rows of 64 bytes per instruction: lane l takes row 16q + l/4,
        // logical chunk (l%4) ^ swz4(row)
#pragma unroll
        for (int q = 0; q < DBN / 16; ++q) {
          const int r = q * 16 + (lane >> 2);
          const int gn = min(n0 + r, p.N - 1);
          dma_16_nt(p.b + (size_t)gn * (p.K / 2) + (size_t)kb * BROW + (((lane & 3) ^ swz4(r)) << 4),
                 slot + DBM * KBLK + q * 1024);
        }
      } else {
#pragma unroll
        for (int q = 0; q < DBN / 8; ++q) {
          const int r = q * 8 + lr;
          const int gn = min(n0 + r, p.N - 1);
          dma_16_nt(p.b + (size_t)gn * p.K + (size_t)kb * KBLK + (((lane & 7) ^ swz(r)) << 4),
                 slot + DBM * KBLK + q * 1024);
        }
      }
      dma_4(p.sfa + (size_t)kb * p.rows + min(m0 + lane, p.rows - 1), slot + DBM * KBLK + DBN * BROW);
      if constexpr (B4)   // the 64 columns' packed E8M0 scales of this K block
        dma_4(p.sfb + (size_t)kb * p.N + min(n0 + lane, p.N - 1), slot + DBM * KBLK + DBN * BROW + DBM * 4);
    }
  }

  v4f acc[SM][SN];
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
  const int g16 = lane >> 4;
#pragma unroll
  for (int j = 0; j < DNPW; ++j) {
    if (j < nown) {
      wait_stages<LPB, DNPW - 1>(nown - 1 - j);
      const uint8_t* base = smem + (wave + DNW * j) * SLOT;
      const float* sa = reinterpret_cast<const float*>(base + DBM * KBLK + DBN * BROW);
      v4f sc[SM];
#pragma unroll
      for (int i = 0; i < SM; ++i) sc[i] = *reinterpret_cast<const v4f*>(sa + i * 16 + g16 * 4) * sb[j];
      if constexpr (B4)
        mma_block_fp4<SM, SN>(base, base + DBM * KBLK,
                              reinterpret_cast<const uint32_t*>(base + DBM * KBLK + DBN * BROW + DBM * 4), sc, acc,
                              lane);
      else if constexpr (TA || TB)
        mma_block_kmajor<SM, SN, TA, TB>(base, lds_u32(base), base + DBM * KBLK, lds_u32(base + DBM * KBLK), sc, acc,
                                         lane);
      else
        mma_block<SM, SN>(base, 0, base + DBM * KBLK, 0, sc, acc, lane);
    }
  }

  // ---- sum the wave totals in wave order; wave w finishes sub-tiles
  // DTPW*w .. DTPW*w + DTPW-1 (sub-tile t: rows 16*(t/SN), columns 16*(t%SN))
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  v4f* red = reinterpret_cast<v4f*>(smem);
#pragma unroll
  for (int t = 0; t < T; ++t) red[(wave * T + t) * 64 + lane] = acc[t / SN][t % SN];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < DTPW; ++j) {
    const int t = wave * DTPW + j;
    out[j] = red[t * 64 + lane];
#pragma unroll
    for (int src = 1; src < DNW; ++src) out[j] += red[(src * T + t) * 64 + lane];
  }
}

// The lane's C values of sub-tiles wave*DTPW + j of tile (mt, nt) (zeros
// without a C).  One branch for the whole set, so that all the loads are in
// flight together (a branch per element would wait for each load).
__device__ __forceinline__ void load_c_tile(const Params& p, int mt, int nt, float (&cv)[DTPW][4]) {
  constexpr int SN = DBN / 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g16 = lane >> 4, r16 = lane & 15;
  if (p.c) {
#pragma unroll
    for (int j = 0; j < DTPW; ++j) {
      const int t = wave * DTPW + j;
      const int row0 = mt * DBM + (t / SN) * 16 + g16 * 4, col = min(nt * DBN + (t % SN) * 16 + r16, p.N - 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) cv[j][e] = bf16_to_f32(p.c[(size_t)min(row0 + e, p.rows - 1) * p.N + col]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < DTPW; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) cv[j][e] = 0.f;
  }
}

// + C (cv, from load_c_tile), round to bf16, store: the lane's sub-tiles
// wave*DTPW + j of tile (mt, nt)
__device__ __forceinline__ void store_d_tile(const Params& p, int mt, int nt, const v4f (&res)[DTPW],
                                             const float (&cv)[DTPW][4]) {
  constexpr int SN = DBN / 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g16 = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int j = 0; j < DTPW; ++j) {
      const int t = wave * DTPW + j;
      const int row = mt * DBM + (t / SN) * 16 + g16 * 4 + e, col = nt * DBN + (t % SN) * 16 + r16;
      if (row < p.rows && col < p.N) p.d[(size_t)row * p.N + col] = f32_to_bf16(res[j][e] + cv[j][e]);
    }
}

// + C, round to bf16, store: the lane's sub-tiles wave*DTPW + j of `tile`
__device__ __forceinline__ void decode_store(const Params& p, int tile, const v4f (&res)[DTPW]) {
  int mt, nt;
  tile_coords(tile, p.tiles_m, p.tiles_n, mt, nt);
  float cv[DTPW][4];
  load_c_tile(p, mt, nt, cv);
  store_d_tile(p, mt, nt, res, cv);
}

constexpr int kCoherent = 16;     // buffer-access cache policy: SC1 (device scope)
constexpr int kRawBufferWord3 = 0x00020000;   // buffer descriptor word 3: 32-bit data format, raw access
typedef unsigned v4u __attribute__((ext_vector_type(4)));

template <int LAYOUT>
__global__ void __launch_bounds__(64 * DNW)
fp8_gemm_nt_decode_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[DKBS * dslot<LAYOUT == 4>()];
  // work item: XCD-contiguous ranges of (tile, split), splits of a tile adjacent
  const int total = p.tiles_m * p.tiles_n * p.splits;
  const int per_xcd = (total + 7) / 8;
  const int w = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (blockIdx.x / 8 >= per_xcd || w >= total) return;
  const int tile = w / p.splits;
  const int split = w % p.splits;
  v4f out[DTPW];
  decode_item<LAYOUT>(p, smem, tile, split, out);
  if (p.splits > 1) {
    // fp32 partial, in the result layout [tile][split][sub-tile][lane];
    // splitk_reduce_kernel, launched next on the same stream, sums the splits.
    // The stores write through to memory (device-coherent policy), so the
    // launch ends with no dirty partial lines in the L2s to write back.
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    v4f* part = reinterpret_cast<v4f*>(p.workspace) + ((size_t)tile * p.splits + split) * (DT * 64);
    const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(part, 0, DT * 64 * 16, kRawBufferWord3);
#pragma unroll
    for (int j = 0; j < DTPW; ++j)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, out[j]), ws,
                                             (uint32_t)(((wave * DTPW + j) * 64 + lane) * 16), 0, kCoherent);
    return;
  }
  decode_store(p, tile, out);   // single split
}

// ---- one-launch decode: the split-K hand-off inside the launch ------------
// The splits of a tile hand their fp32 partials to the split that finishes
// last, inside the one launch; no workgroup waits for another.
//   * Work items (tile, split) are dealt to the workgroups as in the two-launch
//     form (XCD-contiguous ranges, the splits of a tile adjacent).
//   * Each split stores its partial with device-coherent 16-byte stores
//     (written through to memory), waits until they are complete and counts
//     itself in on the tile's counter (device-scope atomic); whichever split
//     sees the count reach the tile's split count reads the other partials
//     with device-coherent loads, so the hand-off holds wherever the splits
//     ran.  It sums the splits in split order, as splitk_reduce_kernel does
//     (bit-identical results), adds C, rounds, stores, and resets the counter.
// p.sync holds one counter per tile from kSyncTile0 on; every call leaves
// them at zero.

__device__ __forceinline__ int atomic_add_dev(int* a, int v) {
  return __hip_atomic_fetch_add(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(int* a, int v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publishes this split's partial and, for the tile's last split, completes
// the tile.  Ends with a workgroup barrier.
__device__ __forceinline__ void decode_hand_off(const Params& p, int tile, int split, const v4f (&out)[DTPW],
                                                int* s_flag) {
  constexpr int MAXS = 8;                        // partials loaded per pass
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t ws_bytes = p.workspace_bytes < 0xFFFFFFF0u ? (uint32_t)p.workspace_bytes : 0xFFFFFFF0u;
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(p.workspace, 0, ws_bytes, kRawBufferWord3);
  // byte offsets (32-bit: the host keeps every partial below 4 GiB): partial
  // [tile][split][sub-tile][lane] of 16 bytes
  const uint32_t lane_off = (uint32_t)(((wave * DTPW) * 64 + lane) * 16);
  const uint32_t tile_off = (uint32_t)tile * (uint32_t)p.splits * (uint32_t)(DT * 64 * 16);
#pragma unroll
  for (int j = 0; j < DTPW; ++j)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, out[j]), ws,
                                           tile_off + (uint32_t)split * (DT * 64 * 16) + lane_off + j * 64 * 16, 0,
                                           kCoherent);
  // the stores are complete before the workgroup counts itself in
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int* cnt = p.sync + kSyncTile0 + tile;
  if (tid == 0) *s_flag = atomic_add_dev(cnt, 1) == p.splits - 1;
  __syncthreads();
  if (*s_flag != 0) {
    // every other split has stored its partial.  C first, then the partials
    // in split order, all in flight together
    int mt, nt;
    tile_coords(tile, p.tiles_m, p.tiles_n, mt, nt);
    float cv[DTPW][4];
    load_c_tile(p, mt, nt, cv);
    v4f acc[DTPW];
#pragma unroll
    for (int j = 0; j < DTPW; ++j) acc[j] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < p.splits; s0 += MAXS) {
      v4f part[MAXS][DTPW];
#pragma unroll
      for (int u = 0; u < MAXS; ++u) {
        const int s = s0 + u;
        if (s < p.splits && s != split)
#pragma unroll
          for (int j = 0; j < DTPW; ++j)
            part[u][j] = __builtin_bit_cast(
                v4f, __builtin_amdgcn_raw_buffer_load_b128(
                         ws, tile_off + (uint32_t)s * (DT * 64 * 16) + lane_off + j * 64 * 16, 0, kCoherent));
      }
#pragma unroll
      for (int u = 0; u < MAXS; ++u) {
        const int s = s0 + u;
        if (s < p.splits)
#pragma unroll
          for (int j = 0; j < DTPW; ++j) acc[j] += s == split ? out[j] : part[u][j];
      }
    }
    store_d_tile(p, mt, nt, acc, cv);
    if (tid == 0) store_dev(cnt, 0);
  }
  __syncthreads();
}

template <int LAYOUT>
__global__ void __launch_bounds__(64 * DNW)
fp8_gemm_nt_decode_fused_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[DKBS * dslot<LAYOUT == 4>()];
  __shared__ int s_flag;
  const int total = p.tiles_m * p.tiles_n * p.splits;
  const int per_xcd = (total + 7) / 8;
  const int w = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (blockIdx.x / 8 >= per_xcd || w >= total) return;
  const int tile = w / p.splits;
  const int split = w % p.splits;
  v4f out[DTPW];
  decode_item<LAYOUT>(p, smem, tile, split, out);
  decode_hand_off(p, tile, split, out, &s_flag);
}

// Split-K reduction of the decode kernel's partials: one 64-lane workgroup per
// (tile, 16x16 sub-tile), so the small reduction spreads over many CUs.  Each
// lane issues all its loads (every split's partial, C) before any add, so one
// memory round trip covers them; the splits are summed in split order.
__global__ void __launch_bounds__(64)
splitk_reduce_kernel(Params p) {
  constexpr int SN = DBN / 16, T = (DBM / 16) * SN;
  constexpr int MAXS = 16;                       // splits loaded per pass
  const int lane = threadIdx.x;
  const int tile = blockIdx.x / T;
  const int t = blockIdx.x % T;                  // sub-tile: strip t / SN, column block t % SN
  int mt, nt;
  tile_coords(tile, p.tiles_m, p.tiles_n, mt, nt);
  const int g16 = lane >> 4, r16 = lane & 15;
  const int row0 = mt * DBM + (t / SN) * 16 + g16 * 4;
  const int col = nt * DBN + (t % SN) * 16 + r16;
  const v4f* ws = reinterpret_cast<const v4f*>(p.workspace) + (size_t)tile * p.splits * (T * 64) + t * 64 + lane;

  float cv[4] = {0.f, 0.f, 0.f, 0.f};
  if (p.c) {   // one branch for the four loads, so that they are in flight together
#pragma unroll
    for (int e = 0; e < 4; ++e) cv[e] = bf16_to_f32(p.c[(size_t)min(row0 + e, p.rows - 1) * p.N + min(col, p.N - 1)]);
  }
  v4f acc = (v4f){0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < p.splits; s0 += MAXS) {
    v4f part[MAXS];
#pragma unroll
    for (int u = 0; u < MAXS; ++u)
      if (s0 + u < p.splits) part[u] = __builtin_nontemporal_load(ws + (size_t)(s0 + u) * (T * 64));
#pragma unroll
    for (int u = 0; u < MAXS; ++u)
      if (s0 + u < p.splits) acc += part[u];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (row0 + e < p.rows && col < p.N) p.d[(size_t)(row0 + e) * p.N + col] = f32_to_bf16(acc[e] + cv[e]);
}

// Split-tail reduction of the tile kernels (dense and contiguous calls whose
// last round of items is split over K): one 256-lane workgroup per 1024
// elements of a tail item; each lane sums the sk_splits partials of four
// consecutive columns in split order (deterministic), adds C, rounds and
// stores the rows that belong to the result.  The item of (XCD x, tail index
// t) follows the tile kernel's work list: XCD x owns items x*per_xcd ..,
// whole rounds of `slots` items first, then the tail.
__global__ void __launch_bounds__(256)
splitk_tile_reduce_kernel(Params p, int bm, int bn, int slots, int contiguous) {
  const int chunks = bm * bn / 1024;
  const int b = blockIdx.x;
  const int c = b % chunks;
  const int t = (b / chunks) % p.sk_tail;
  const int x = b / chunks / p.sk_tail;
  const int total = p.tiles_m * p.tiles_n;
  const int per_xcd = (total + 7) / 8;
  const int w_begin = x * per_xcd;
  const int n_x = max(0, min(total, w_begin + per_xcd) - w_begin);
  const int full_x = n_x / slots * slots;
  if (t >= n_x - full_x) return;
  int mt, nt;
  tile_coords(w_begin + full_x + t, p.tiles_m, p.tiles_n, mt, nt);
  const int e0 = c * 1024 + threadIdx.x * 4;
  const int row = mt * bm + e0 / bn, col = nt * bn + e0 % bn;
  if (row >= p.rows) return;
  // every load (the row's expert id, the partials, C) is issued before the
  // first is used, so one memory round trip covers them all; then the
  // partials are summed in split order (deterministic), C added, and the
  // stores follow (a load after a store would wait for the store too)
  constexpr int MAXS = 16;                       // split count bound of the split tail
  const int g = contiguous ? p.layout[row] : 0;
  const v4f* part = reinterpret_cast<const v4f*>(p.workspace + ((size_t)(x * p.sk_tail + t) * p.sk_splits) * bm * bn + e0);
  v4f pv[MAXS];
#pragma unroll
  for (int s0 = 0; s0 < MAXS; ++s0)
    if (s0 < p.sk_splits) pv[s0] = __builtin_nontemporal_load(part + (size_t)s0 * (bm * bn / 4));
  float cv[4] = {0.f, 0.f, 0.f, 0.f};
  if (p.c) {
#pragma unroll
    for (int k = 0; k < 4; ++k) cv[k] = bf16_to_f32(p.c[(size_t)row * p.N + min(col + k, p.N - 1)]);
  }
  if (contiguous && (g < 0 || g >= p.G)) return;
  v4f acc = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s0 = 0; s0 < MAXS; ++s0)
    if (s0 < p.sk_splits) acc += pv[s0];
  if (p.c) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += cv[k];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (col + k < p.N) p.d[(size_t)row * p.N + col + k] = f32_to_bf16(acc[k]);
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
  // C first, then the stores (a load after a store waits for the store too)
  if (p.c) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int c = 0; c < SN; ++c)
        acc[0][c][e] += bf16_to_f32(p.c[(size_t)min(m0 + 4 * g16 + e, p.rows - 1) * p.N +
                                        min(n0 + 16 * c + r16, p.N - 1)]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = m0 + 4 * g16 + e;
#pragma unroll
    for (int c = 0; c < SN; ++c) {
      const int col = n0 + 16 * c + r16;
      if (row < p.rows && col < p.N) p.d[(size_t)row * p.N + col] = f32_to_bf16(acc[0][c][e]);
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

// Dense calls with K-major operands (nn, tn, tt) and FP8 x FP4 calls are
// compiled for the tiles the chooser gives them: 128x128 (four waves, 4-slot
// ring), 128x256 and 256x256.
template <int BM, int BN, int WAVES_M, int WAVES_N, int NSLOT, int WG_PER_CU, int LAYOUT>
hipError_t launch_dense_layout(const Params& p, int grid, hipStream_t stream) {
  constexpr bool compiled = WG_PER_CU == 1 && ((BM == 128 && BN == 128 && NSLOT == 4) ||
                                               (BM == 128 && BN == 256) || (BM == 256 && BN == 256));
  if constexpr (compiled) {
    hipLaunchKernelGGL((fp8_gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, NSLOT, kDense, WG_PER_CU, false, LAYOUT>),
                       dim3(grid), dim3(WAVES_M * WAVES_N * 64), 0, stream, p);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

// M-grouped FP8 x FP4 calls, on the same tiles.
template <int BM, int BN, int WAVES_M, int WAVES_N, int NSLOT, int WG_PER_CU, int MODE>
hipError_t launch_grouped_fp4(const Params& p, int grid, hipStream_t stream) {
  constexpr bool compiled = WG_PER_CU == 1 && ((BM == 128 && BN == 128 && NSLOT == 4) ||
                                               (BM == 128 && BN == 256) || (BM == 256 && BN == 256));
  if constexpr (compiled) {
    hipLaunchKernelGGL((fp8_gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, NSLOT, MODE, WG_PER_CU, false, 4>),
                       dim3(grid), dim3(WAVES_M * WAVES_N * 64), 0, stream, p);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int NSLOT, int WG_PER_CU = 1>
hipError_t launch_cfg(int mode, const Params& p, int grid, hipStream_t stream) {
  constexpr int threads = WAVES_M * WAVES_N * 64;
  if (mode != kDense && p.ab_layout != 0) {
    if (p.ab_layout != 4) return hipErrorInvalidValue;
    if (mode == kContiguous)
      return launch_grouped_fp4<BM, BN, WAVES_M, WAVES_N, NSLOT, WG_PER_CU, kContiguous>(p, grid, stream);
    if (mode == kMasked)
      return launch_grouped_fp4<BM, BN, WAVES_M, WAVES_N, NSLOT, WG_PER_CU, kMasked>(p, grid, stream);
    return hipErrorInvalidValue;
  }
  if (mode == kDense && p.ab_layout != 0) {
    switch (p.ab_layout) {
      case 1: return launch_dense_layout<BM, BN, WAVES_M, WAVES_N, NSLOT, WG_PER_CU, 1>(p, grid, stream);
      case 2: return launch_dense_layout<BM, BN, WAVES_M, WAVES_N, NSLOT, WG_PER_CU, 2>(p, grid, stream);
      case 3: return launch_dense_layout<BM, BN, WAVES_M, WAVES_N, NSLOT, WG_PER_CU, 3>(p, grid, stream);
      case 4: return launch_dense_layout<BM, BN, WAVES_M, WAVES_N, NSLOT, WG_PER_CU, 4>(p, grid, stream);
      default: return hipErrorInvalidValue;
    }
  }
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
  switch (p.ab_layout) {
    case 0: hipLaunchKernelGGL(fp8_gemm_nt_decode_kernel<0>, dim3(grid), dim3(64 * DNW), 0, stream, p); break;
    case 1: hipLaunchKernelGGL(fp8_gemm_nt_decode_kernel<1>, dim3(grid), dim3(64 * DNW), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(fp8_gemm_nt_decode_kernel<2>, dim3(grid), dim3(64 * DNW), 0, stream, p); break;
    case 3: hipLaunchKernelGGL(fp8_gemm_nt_decode_kernel<3>, dim3(grid), dim3(64 * DNW), 0, stream, p); break;
    case 4: hipLaunchKernelGGL(fp8_gemm_nt_decode_kernel<4>, dim3(grid), dim3(64 * DNW), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(p.tiles_m * p.tiles_n * (DBM / 16) * (DBN / 16)), dim3(64), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_fused(const Params& p, hipStream_t stream) {
  if (!p.sync || p.tiles_m * p.tiles_n > kSyncMaxTiles) return hipErrorInvalidValue;
  const int items = p.tiles_m * p.tiles_n * p.splits;
  const int grid = ((items + 7) / 8) * 8;
  switch (p.ab_layout) {
    case 0: hipLaunchKernelGGL(fp8_gemm_nt_decode_fused_kernel<0>, dim3(grid), dim3(64 * DNW), 0, stream, p); break;
    case 1: hipLaunchKernelGGL(fp8_gemm_nt_decode_fused_kernel<1>, dim3(grid), dim3(64 * DNW), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(fp8_gemm_nt_decode_fused_kernel<2>, dim3(grid), dim3(64 * DNW), 0, stream, p); break;
    case 3: hipLaunchKernelGGL(fp8_gemm_nt_decode_fused_kernel<3>, dim3(grid), dim3(64 * DNW), 0, stream, p); break;
    case 4: hipLaunchKernelGGL(fp8_gemm_nt_decode_fused_kernel<4>, dim3(grid), dim3(64 * DNW), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

const ConfigInfo kConfigs[kNumConfigs] = {
    {128, 128, 256, "128x128_w2x2_s4"},
    {DBM, DBN, 64 * DNW, "decode_64x64_ksplit"},
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
    {DBM, DBN, 64 * DNW, "decode_64x64_ksplit_one_launch"},
};

}  // namespace

const ConfigInfo& config_info(int cfg) { return kConfigs[cfg]; }

namespace {
template <int BM, int BN, int WAVES_M, int WAVES_N, int NSLOT>
hipError_t launch_kg_cfg(const KGroupedParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fp8_gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, NSLOT, kKGrouped, 1, false, 3, KGroupedParams>),
                     dim3(grid), dim3(WAVES_M * WAVES_N * 64), 0, stream, p);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_tile_reduce(int mode, int cfg, const Params& p, int grid, hipStream_t stream) {
  const ConfigInfo& ci = config_info(cfg);
  const int blocks = 8 * p.sk_tail * (ci.bm * ci.bn / 1024);
  hipLaunchKernelGGL(splitk_tile_reduce_kernel, dim3(blocks), dim3(256), 0, stream, p, ci.bm, ci.bn, grid / 8,
                     mode == kContiguous ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_kgrouped(int cfg, const KGroupedParams& p, int grid, hipStream_t stream) {
  switch (cfg) {
    case kCfg128x128: return launch_kg_cfg<128, 128, 2, 2, 4>(p, grid, stream);
    case kCfg128x256w8: return launch_kg_cfg<128, 256, 2, 4, 3>(p, grid, stream);
    case kCfg256x256w8: return launch_kg_cfg<256, 256, 2, 4, 2>(p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(int mode, int cfg, const Params& p, int grid, hipStream_t stream) {
  switch (cfg) {
    case kCfg128x128: return launch_cfg<128, 128, 2, 2, 4>(mode, p, grid, stream);
    case kCfgDecode: return mode == kDense ? launch_decode(p, stream) : hipErrorInvalidValue;
    case kCfgDecodeFused: return mode == kDense ? launch_decode_fused(p, stream) : hipErrorInvalidValue;
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
