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
// Two kernels share that per-block step:
//
// fp8_gemm_nt_kernel (prefill shapes and both grouped forms)
//   * a workgroup of four waves owns a BM x BN output tile; each wave owns a
//     (BM/WAVES_M) x (BN/WAVES_N) sub-tile held in VGPRs;
//   * A and B K-blocks travel HBM -> LDS through the direct global->LDS path
//     (global_load_lds_dwordx4: no VGPR staging) into a ring of NSLOT slots,
//     so up to NSLOT-1 K-blocks are in flight while one feeds the MFMAs; each
//     wave waits only for its own loads of the block it is about to use
//     (s_waitcnt vmcnt(n)) and a bare s_barrier publishes them; the A scales
//     of the tile's rows and each wave's B scale ride in the same slot;
//   * workgroups walk a list of work items; the list is split into 8
//     contiguous ranges, one per XCD (the hardware deals workgroups to the
//     XCDs round-robin), so that tiles sharing A rows or B columns run on the
//     same XCD and meet in its L2;
//   * masked form: each workgroup builds the per-group tile counts from the
//     device-resident masked_m in LDS and walks the expert groups, skipping
//     empty ones; contiguous form: the expert of each 128-row block is read
//     from the device-resident grouped_layout.
//
// fp8_gemm_nt_decode_kernel (dense shapes with few rows)
//   * a workgroup owns a 64x64 tile and a range of at most 8 K-blocks (a K
//     split); its four waves split those K-blocks among themselves, each wave
//     loading and consuming only its own blocks with no barrier in the K loop;
//     every load of the workgroup is issued up front, so the whole range is in
//     flight at once;
//   * the four wave totals are summed through LDS in wave order; with one
//     split the result goes through the +C / bf16 epilogue; otherwise every
//     split stores its fp32 partial to a workspace and splitk_reduce_kernel,
//     launched next on the same stream, sums the splits in split order
//     (deterministic), adds C and rounds; the kernel boundary orders the two.
//     An in-kernel alternative (selected on the host) lets the last split to
//     arrive do that sum: partials go through device-scope (sc1) stores and
//     loads, coherent across the XCDs' L2 caches without flushing or
//     invalidating them, and a per-tile arrival counter is reset to zero by
//     the last split for the next call.
//
// LDS rows are 128 bytes with 16-byte chunks XOR-swizzled by row so that the
// fragment reads of a 16-row strip are free of bank conflicts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "dg_internal.h"

namespace dg {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

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

// s_waitcnt with vmcnt <= N and all LDS reads of this wave complete
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
}

// Runtime-selected wait: vmcnt <= n * LPS for n in [0, MAXN].
template <int LPS, int MAXN>
__device__ __forceinline__ void wait_stages(int n) {
  if constexpr (MAXN >= 0) {
    if (n >= MAXN) {
      wait_vm_lgkm0<LPS * MAXN>();
      return;
    }
    wait_stages<LPS, MAXN - 1>(n);
  }
}

// Direct global->LDS loads.  Lane l's bytes land at LDS address m0 + size*l.
// Written as inline asm so that the compiler does not treat every later LDS
// read as dependent on every load in flight (it cannot tell the ring slots
// apart and would wait for all of them); the kernels wait on vmcnt themselves.
// One wait state separates the M0 write from the load that uses it.
__device__ __forceinline__ void dma_16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gptr), "s"(lds_addr) : "memory", "m0");
}
__device__ __forceinline__ void dma_4(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(gptr), "s"(lds_addr) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  // the C-style cast is an address-space cast: generic -> LDS offset
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void*)(p));
}

// barrier that does not wait for outstanding global->LDS loads; the caller has
// already waited for the ones it needs.  The empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Reads the MFMA operand fragment of one 16-row strip: lane l takes row l%16
// of the strip and the 32-byte K slice l/16 of it (logical 16-byte chunks
// 2*(l/16) and 2*(l/16)+1, stored at their swizzled positions).
__device__ __forceinline__ v8i lds_fragment(const uint8_t* rows, int r, int g16) {
  const uint8_t* rp = rows + r * KBLK;
  const int s = swz(r);
  const v4i lo = *reinterpret_cast<const v4i*>(rp + (((2 * g16) ^ s) << 4));
  const v4i hi = *reinterpret_cast<const v4i*>(rp + (((2 * g16 + 1) ^ s) << 4));
  return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// One 128-wide K block for a (16*SM) x (16*SN) wave sub-tile whose A rows
// start at row arow0 of `a_rows` and whose B rows start at row bcol0 of
// `b_rows` (both LDS, 128-byte swizzled rows).  sc[i] holds the promotion
// factors sa*sb of the lane's four result rows in strip i.
//
// Software pipeline over the sub-tiles: the MFMA of sub-tile t is issued
// before the promotion of sub-tile t-(P-1), so P-1 MFMAs are in flight while
// the VALU promotes a finished partial.
template <int SM, int SN>
__device__ __forceinline__ void mma_block(const uint8_t* a_rows, int arow0, const uint8_t* b_rows, int bcol0,
                                          const v4f (&sc)[SM], v4f (&acc)[SM][SN], int lane) {
  const int g16 = lane >> 4, r16 = lane & 15;
  v8i bf[SN], af[SM];
#pragma unroll
  for (int j = 0; j < SN; ++j) bf[j] = lds_fragment(b_rows, bcol0 + j * 16 + r16, g16);
#pragma unroll
  for (int i = 0; i < SM; ++i) af[i] = lds_fragment(a_rows, arow0 + i * 16 + r16, g16);
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

// Output tile of linear tile id `tile` in the grouped order: bands of 8
// m-tiles sweep across n, so consecutive tiles share B columns.
__device__ __forceinline__ void tile_coords(int tile, int tiles_m, int tiles_n, int& mt, int& nt) {
  constexpr int GM = 8;
  const int band = tile / (GM * tiles_n);
  const int first_m = band * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in_band = tile - band * GM * tiles_n;
  mt = first_m + in_band % gm;
  nt = in_band / gm;
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <int I, int N, class F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) { static_for_impl<0, N>(f); }

// ============================================================================
// prefill / grouped kernel
// ============================================================================
template <int BM, int BN, int WAVES_M, int WAVES_N, int NSLOT>
struct Shape {
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int NT = NWAVES * 64;
  static constexpr int WTM = BM / WAVES_M;      // wave tile rows
  static constexpr int WTN = BN / WAVES_N;      // wave tile cols
  static constexpr int SM = WTM / 16;           // 16-row strips per wave
  static constexpr int SN = WTN / 16;           // 16-col strips per wave
  static constexpr int A_BYTES = BM * KBLK;     // one slot of each region
  static constexpr int B_BYTES = BN * KBLK;
  static constexpr int RS = BM / NWAVES;        // row scales loaded per wave
  static constexpr int SA_PER_WAVE = RS + 4;    // RS row scales, this wave's B scale, pad
  static constexpr int S_BYTES = NWAVES * SA_PER_WAVE * 4;
  // LDS: [A slot 0..NSLOT-1][B slot 0..NSLOT-1][scales slot 0..NSLOT-1]
  static constexpr int B_REGION = NSLOT * A_BYTES;
  static constexpr int S_REGION = NSLOT * (A_BYTES + B_BYTES);
  static constexpr int LDS_BYTES = NSLOT * (A_BYTES + B_BYTES + S_BYTES);
  static constexpr int A_INSTR = BM / 8 / NWAVES;     // 1 KB (8 rows) per wave instruction
  static constexpr int B_INSTR = BN / 8 / NWAVES;
  static constexpr int LPS = A_INSTR + B_INSTR + 1;   // loads per wave per K block
  static_assert(NWAVES == 4 || NWAVES == 8, "four or eight waves per workgroup");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(WTN <= 128 && 128 % WTN == 0, "a wave's columns must sit in one 128-wide B scale block");
  static_assert(BM % (8 * NWAVES) == 0 && BN % (8 * NWAVES) == 0, "every wave issues the same number of loads");
  static_assert(RS % 4 == 0 && RS < 64, "row scales plus the B scale fit one 64-lane load per wave");
  static_assert((NSLOT - 1) * LPS < 64, "outstanding loads must fit the 6-bit vmcnt");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
};

// LDS accesses at an integer LDS byte address; an added constant folds into
// the instruction's offset field.
__device__ __forceinline__ v4i lds_v4i(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) v4i*>(static_cast<uintptr_t>(addr));
}
__device__ __forceinline__ v4f lds_v4f(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) v4f*>(static_cast<uintptr_t>(addr));
}
__device__ __forceinline__ float lds_f32(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) float*>(static_cast<uintptr_t>(addr));
}

// Direct global->LDS load with a uniform 64-bit base in SGPRs and a 32-bit
// per-lane byte offset.
__device__ __forceinline__ void dma_16s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int NSLOT, int MODE, int WG_PER_CU>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64, WG_PER_CU)
fp8_gemm_nt_kernel(Params p) {
  using S = Shape<BM, BN, WAVES_M, WAVES_N, NSLOT>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S::LDS_BYTES];
  __shared__ int s_prefix[MODE == kMasked ? MAX_GROUPS_LDS + 1 : 1];
  __shared__ int s_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t smem_base = lds_u32(smem);
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int KB = p.K / KBLK;
  const int NB = (p.N + 127) / 128;
  const int g16 = lane >> 4;          // K slice of the operands, row quad of the result
  const int r16 = lane & 15;          // row of A / column of B within a 16-strip
  const int wrow0 = wm * S::WTM;      // wave's first row in the tile
  const int wcol0 = wn * S::WTN;

  // per-lane LDS addresses of the fragments in slot 0 (other slots add a constant)
  uint32_t offA[S::SM][2], offB[S::SN][2], offS[S::SM];
#pragma unroll
  for (int i = 0; i < S::SM; ++i) {
    const int r = wrow0 + i * 16 + r16;
#pragma unroll
    for (int h = 0; h < 2; ++h) offA[i][h] = smem_base + r * KBLK + (((2 * g16 + h) ^ swz(r)) << 4);
    const int q = wrow0 + i * 16 + g16 * 4;     // a 4-row group never straddles a wave block
    offS[i] = smem_base + S::S_REGION + 4 * ((q / S::RS) * S::SA_PER_WAVE + q % S::RS);
  }
#pragma unroll
  for (int j = 0; j < S::SN; ++j) {
    const int r = wcol0 + j * 16 + r16;
#pragma unroll
    for (int h = 0; h < 2; ++h) offB[j][h] = smem_base + S::B_REGION + r * KBLK + (((2 * g16 + h) ^ swz(r)) << 4);
  }
  const uint32_t offSB = smem_base + S::S_REGION + 4 * (wave * S::SA_PER_WAVE + S::RS);

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
    total = p.tiles_m * p.tiles_n;
  }

  const int slots = (gridDim.x + 7) / 8;          // workgroups per XCD
  const int xcd = blockIdx.x % 8;
  const int slot_id = blockIdx.x / 8;
  const int per_xcd = (total + 7) / 8;
  const int w_begin = xcd * per_xcd;
  const int w_end = min(total, w_begin + per_xcd);
  int g_cur = 0;                                   // masked walker state

  for (int w = w_begin + slot_id; w < w_end; w += slots) {
    // ---- resolve the work item ---------------------------------------------
    int group = 0, mt, nt, rows_lim = p.rows;
    if constexpr (MODE == kMasked) {
      while (w >= s_prefix[g_cur + 1]) ++g_cur;
      const int local = w - s_prefix[g_cur];
      int m = p.masked_m[g_cur];
      m = m < 0 ? 0 : (m > p.rows ? p.rows : m);
      const int tm = (m + BM - 1) / BM;
      group = g_cur;
      mt = local % tm;             // the m-tiles of one B tile are neighbours in the list
      nt = local / tm;
      rows_lim = m;
    } else {
      tile_coords(w, p.tiles_m, p.tiles_n, mt, nt);
      if constexpr (MODE == kContiguous) {
        // the expert of this block of rows: the largest id among its rows
        // (padding rows may carry -1); all valid ids in a block agree
        if (wave == 0) {
          int best = -1;
          for (int r = lane; r < BM; r += 64) {
            const int row = mt * BM + r;
            if (row < p.rows) best = max(best, p.layout[row]);
          }
          for (int off = 32; off > 0; off >>= 1) best = max(best, __shfl_xor(best, off));
          if (lane == 0) s_flag = best;
        }
        __syncthreads();
        group = s_flag;
        __syncthreads();
        if (group < 0 || group >= p.G) continue;   // uniform across the workgroup
      }
    }

    const int m0 = mt * BM;
    const int n0 = nt * BN;
    const int kbs = KB;

    // ---- operand bases -----------------------------------------------------
    const uint8_t* A = p.a;
    const float* SA = p.sfa;
    const uint8_t* B = p.b;
    const float* SB = p.sfb;
    uint16_t* D = p.d;
    const uint16_t* C = p.c;
    const int a_rows = p.rows;     // rows allocated in this A operand
    if constexpr (MODE == kMasked) {
      A += (size_t)group * p.rows * p.K;
      SA += (size_t)group * KB * p.rows;
      D += (size_t)group * p.rows * p.N;
      if (C) C += (size_t)group * p.rows * p.N;
    }
    if constexpr (MODE != kDense) {
      B += (size_t)group * p.N * p.K;
      SB += (size_t)group * NB * KB;
    }
    int nb = (n0 + wcol0) / 128;
    nb = nb < NB ? nb : NB - 1;

    // ---- load addresses -------------------------------------------------------
    // A / B: wave instruction j covers tile rows 8*(wave + NWAVES*j) .. +7; lane l lands
    // at LDS byte 16*l of that 1 KB piece: row 8*(...) + l/8, physical chunk l%8,
    // which holds logical chunk (l%8) ^ swz(row).  Uniform bases (tile origin,
    // K block) live in SGPRs; lanes add a 32-bit offset inside the tile.
    const uint8_t* a_tile = A + (size_t)m0 * p.K;
    const uint8_t* b_tile = B + (size_t)n0 * p.K;
    uint32_t a_off[S::A_INSTR], b_off[S::B_INSTR];
#pragma unroll
    for (int j = 0; j < S::A_INSTR; ++j) {
      const int r = (wave + S::NWAVES * j) * 8 + (lane >> 3);
      const int grow = min(m0 + r, a_rows - 1);       // rows past the end are never stored
      a_off[j] = (uint32_t)((grow - m0) * p.K) + (((lane & 7) ^ swz(r)) << 4);
    }
#pragma unroll
    for (int j = 0; j < S::B_INSTR; ++j) {
      const int r = (wave + S::NWAVES * j) * 8 + (lane >> 3);
      const int gn = min(n0 + r, p.N - 1);
      b_off[j] = (uint32_t)((gn - n0) * p.K) + (((lane & 7) ^ swz(r)) << 4);
    }
    // scales: lanes < RS load row scales of rows wave*RS + lane, lane RS loads
    // this wave's B scale
    const float* s_src;
    size_t s_stride;                  // elements per K block
    if (lane < S::RS) {
      const int grow = min(m0 + wave * S::RS + lane, a_rows - 1);
      s_src = SA + grow;
      s_stride = a_rows;
    } else {
      s_src = SB + (size_t)nb * KB;
      s_stride = 1;
    }

    // issue K block i into slot u
    auto issue = [&](int i, int u) {
      const uint8_t* abase = a_tile + (size_t)i * KBLK;
      const uint8_t* bbase = b_tile + (size_t)i * KBLK;
#pragma unroll
      for (int j = 0; j < S::A_INSTR; ++j)
        dma_16s(abase, a_off[j], smem_base + u * S::A_BYTES + (wave + S::NWAVES * j) * 1024);
#pragma unroll
      for (int j = 0; j < S::B_INSTR; ++j)
        dma_16s(bbase, b_off[j], smem_base + S::B_REGION + u * S::B_BYTES + (wave + S::NWAVES * j) * 1024);
      if (lane <= S::RS)
        dma_4(s_src + (size_t)i * s_stride, smem_base + S::S_REGION + u * S::S_BYTES + wave * S::SA_PER_WAVE * 4);
    };

    v4f acc[S::SM][S::SN];
#pragma unroll
    for (int i = 0; i < S::SM; ++i)
#pragma unroll
      for (int j = 0; j < S::SN; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

    // one K block from slot u (compile-time): fragments, promotion factors, MFMAs
    auto compute = [&](auto u_const) {
      constexpr int u = decltype(u_const)::value;
      const float sb = lds_f32(offSB + u * S::S_BYTES);
      v8i bf[S::SN], af[S::SM];
      v4f sc[S::SM];
#pragma unroll
      for (int j = 0; j < S::SN; ++j) {
        const v4i lo = lds_v4i(offB[j][0] + u * S::B_BYTES);
        const v4i hi = lds_v4i(offB[j][1] + u * S::B_BYTES);
        bf[j] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
#pragma unroll
      for (int i = 0; i < S::SM; ++i) {
        const v4i lo = lds_v4i(offA[i][0] + u * S::A_BYTES);
        const v4i hi = lds_v4i(offA[i][1] + u * S::A_BYTES);
        af[i] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        sc[i] = lds_v4f(offS[i] + u * S::S_BYTES) * sb;
      }
      constexpr int T = S::SM * S::SN;
      constexpr int P = 4;
      v4f part[P];
#pragma unroll
      for (int t = 0; t < T + P - 1; ++t) {
        if (t < T) {
          const v4f zero = {0.f, 0.f, 0.f, 0.f};
          part[t % P] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[t / S::SN], bf[t % S::SN], zero,
                                                                         0, 0, 0, 0, 0, 0);
        }
        const int v = t - (P - 1);
        if (v >= 0) {
          v4f& a = acc[v / S::SN][v % S::SN];
          const v4f& q = part[v % P];
          const v4f& c = sc[v / S::SN];
          a.x = __builtin_fmaf(q.x, c.x, a.x);
          a.y = __builtin_fmaf(q.y, c.y, a.y);
          a.z = __builtin_fmaf(q.z, c.z, a.z);
          a.w = __builtin_fmaf(q.w, c.w, a.w);
        }
      }
    };

    // ---- K loop over the slot ring, unrolled by NSLOT so slots are constants --
    const bool wraps = kbs > NSLOT;
    const int pre = wraps ? NSLOT - 1 : kbs;
#pragma unroll
    for (int u = 0; u < NSLOT - 1; ++u)
      if (u < pre) issue(u, u);
    if (!wraps && kbs == NSLOT) issue(NSLOT - 1, NSLOT - 1);
    for (int i0 = 0; i0 < kbs; i0 += NSLOT) {
      static_for<NSLOT>([&](auto u_const) {
        constexpr int u = decltype(u_const)::value;
        const int i = i0 + u;
        if (i < kbs) {
          // loads issued after block i that may stay in flight
          const int after = min(kbs - 1 - i, wraps ? NSLOT - 2 : NSLOT - 1);
          wait_stages<S::LPS, NSLOT - 1>(after);
          bare_barrier();
          if (wraps && i + NSLOT - 1 < kbs) issue(i + NSLOT - 1, (u + NSLOT - 1) % NSLOT);
          compute(u_const);
        }
      });
    }

    // ---- epilogue: + C, round to bf16, store the rows that belong to the result
    // All loads (row ids, C) are issued before any store so their latencies overlap.
    bool row_ok[S::SM][4];
#pragma unroll
    for (int i = 0; i < S::SM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wrow0 + i * 16 + g16 * 4 + e;
        row_ok[i][e] = row < rows_lim;
        if constexpr (MODE == kContiguous)
          row_ok[i][e] = row_ok[i][e] && p.layout[min(row, p.rows - 1)] == group;
      }
    if (C) {
#pragma unroll
      for (int i = 0; i < S::SM; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = min(m0 + wrow0 + i * 16 + g16 * 4 + e, p.rows - 1);
#pragma unroll
          for (int j = 0; j < S::SN; ++j) {
            const int col = min(n0 + wcol0 + j * 16 + r16, p.N - 1);
            acc[i][j][e] += bf16_to_f32(C[(size_t)row * p.N + col]);
          }
        }
    }
#pragma unroll
    for (int i = 0; i < S::SM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wrow0 + i * 16 + g16 * 4 + e;
#pragma unroll
        for (int j = 0; j < S::SN; ++j) {
          const int col = n0 + wcol0 + j * 16 + r16;
          if (row_ok[i][e] && col < p.N) D[(size_t)row * p.N + col] = f32_to_bf16(acc[i][j][e]);
        }
      }
    // the next item reuses the LDS ring; nothing of this item stays in flight
    // (without this the compiler assumes a load of this item may still be
    // pending in the next item's K loop and waits for every load there)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

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
  switch (mode) {
    case kDense:
      hipLaunchKernelGGL((fp8_gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, NSLOT, kDense, WG_PER_CU>), dim3(grid), dim3(WAVES_M * WAVES_N * 64), 0,
                         stream, p);
      break;
    case kContiguous:
      hipLaunchKernelGGL((fp8_gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, NSLOT, kContiguous, WG_PER_CU>), dim3(grid), dim3(WAVES_M * WAVES_N * 64),
                         0, stream, p);
      break;
    case kMasked:
      hipLaunchKernelGGL((fp8_gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, NSLOT, kMasked, WG_PER_CU>), dim3(grid), dim3(WAVES_M * WAVES_N * 64), 0,
                         stream, p);
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
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dg
