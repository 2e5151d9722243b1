// gfx950 kernels for the FP8 (e4m3) block-scaled GEMM, NT layout, its two
// M-grouped MoE forms, the other operand storages (nn, tn, tt), the K-grouped
// TN form and FP8 x FP4.
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
// fp8_gemm_nt_kernel (prefill shapes, both M-grouped forms, the K-grouped form)
//   * a workgroup of WAVES_M x WAVES_N waves (four or eight) owns a BM x BN
//     output tile; each wave owns a (BM/WAVES_M) x (BN/WAVES_N) sub-tile held
//     in VGPRs;
//   * A and B K-blocks travel HBM -> LDS through the direct global->LDS path
//     (global_load_lds_dwordx4: no VGPR staging) into a ring of NSLOT slots,
//     so up to NSLOT-1 K-blocks are in flight while one feeds the MFMAs; each
//     wave waits only for its own loads of the block it is about to use
//     (s_waitcnt vmcnt(n)) and a bare s_barrier publishes them; the A scales
//     of the tile's rows and each wave's B scale ride in the same slot;
//   * workgroups walk a list of work items; the list is split into 8
//     contiguous ranges, one per XCD (the hardware deals workgroups to the
//     XCDs round-robin), so that tiles sharing A rows or B columns run on the
//     same XCD and meet in its L2; the items of a last, partial round may be
//     split over K (the split tail: fp32 partials that a reduction kernel
//     sums);
//   * dense and K-grouped items take their K blocks in aligned windows of
//     p.k_window blocks, each tile starting at its own offset inside every
//     window, so that the tiles of an XCD that share A rows or B columns do
//     not all request the same K block at the same time;
//   * masked form: each workgroup builds the per-group tile counts from the
//     device-resident masked_m in LDS and walks the expert groups, skipping
//     empty ones; contiguous form: the expert of each 128-row block is read
//     from the device-resident grouped_layout; waves with no valid rows skip
//     their MFMAs;
//   * template bits select K-major ("t" / second "n") operands, an FP4 (E2M1)
//     B with E8M0 scales applied by the MFMA, MFMA-applied power-of-two
//     scales, and the K-grouped form (per-column B scales, fp32 D).
//
// fp8_gemm_nt_decode_kernel (dense shapes with few rows; fp8_gemm.hip)
//   * a workgroup owns a 64x64 tile and a range of at most 8 K-blocks (a K
//     split); its four waves split those K-blocks among themselves, each wave
//     loading and consuming only its own blocks with no barrier in the K loop;
//     every load of the workgroup is issued up front, so the whole range is in
//     flight at once;
//   * the four wave totals are summed through LDS in wave order; with one
//     split the result goes through the +C / bf16 epilogue; otherwise every
//     split stores its fp32 partial to a workspace and splitk_reduce_kernel,
//     launched next on the same stream, sums the splits in split order
//     (deterministic), adds C and rounds; the kernel boundary orders the two;
//   * fp8_gemm_nt_decode_fused_kernel (opt-in) runs the same items in one
//     launch: each split publishes its partial with device-coherent stores
//     and counts itself in on its tile's counter, and the tile's last split
//     sums the partials in split order and finishes the tile.
//
// LDS rows are 128 bytes with 16-byte chunks XOR-swizzled by row so that the
// fragment reads of a 16-row strip are free of bank conflicts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "dg_internal.h"

namespace dg {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int KBLK = 128;        // K block of the scales and of one MFMA

constexpr int MAX_GROUPS_LDS = 1024;

// 16-byte chunk swizzle of a 128-byte LDS row.  It depends only on the row's
// position inside its 16-row strip, so a strip's addresses are those of strip 0
// plus a constant, and the 16 rows read by one fragment instruction hit 8
// distinct chunk positions in each half.
__device__ __forceinline__ int swz(int row) { return (row ^ ((row >> 3) & 1)) & 7; }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// FP4 rows are 64 bytes (four 16-byte chunks): chunk c of row r is stored at
// c ^ swz4(r), so the 16 rows a fragment read touches cover all 16 bank groups.
__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }

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
// (The asm writes M0 and lists it as clobbered; the compiler notes that M0 is a
// reserved register, which is expected here.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gptr), "s"(lds_addr) : "memory", "m0");
}
// The same with the streaming (non-temporal) cache policy: for lines that one
// load brings in once and nothing reads again.
__device__ __forceinline__ void dma_16_nt(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :: "v"(gptr), "s"(lds_addr) : "memory", "m0");
}
__device__ __forceinline__ void dma_4(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(gptr), "s"(lds_addr) : "memory", "m0");
}
#pragma clang diagnostic pop
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

// barrier for LDS traffic only: waits for this wave's LDS operations, not for
// its global stores (__syncthreads would also wait for every store in flight)
__device__ __forceinline__ void lds_barrier() {
  wait_vm_lgkm0<63>();
  bare_barrier();
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

// Masked form: s_prefix[g] = work items of the groups before g (their m-tiles
// of BM rows times the n-tiles), s_prefix[G] = all items, with masked_m
// clamped to [0, max_m].  Every thread of the NT-thread workgroup loads the
// masked_m of its own run of consecutive groups (all loads in flight at once,
// one memory round trip), then a workgroup-wide exclusive scan: an inclusive
// scan inside each wave by lane shuffles, the wave totals through LDS.
// Ends with a workgroup barrier; s_prefix then holds the list.
template <int BM, int NT>
__device__ __forceinline__ void masked_prefix(const Params& p, int* s_prefix, int tid) {
  constexpr int GPT = (MAX_GROUPS_LDS + NT) / NT;        // groups per thread (entries 0..G, G <= MAX_GROUPS_LDS)
  constexpr int NW = NT / 64;
  static_assert(NT % 64 == 0 && NW <= 64, "whole waves");
  __shared__ int s_wave[NW];
  int cnt[GPT];
  int local = 0;
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int g = tid * GPT + i;
    int m = g < p.G ? p.masked_m[g] : 0;
    m = m < 0 ? 0 : (m > p.rows ? p.rows : m);
    cnt[i] = ((m + BM - 1) / BM) * p.tiles_n;
    local += cnt[i];
  }
  const int lane = tid & 63, wave = tid >> 6;
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_wave[w];
  int run = before + incl - local;          // exclusive prefix of this thread's first group
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int g = tid * GPT + i;
    if (g <= p.G) s_prefix[g] = run;        // g == G receives the total
    run += cnt[i];
  }
  __syncthreads();
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

// ---- K-major ("t" / second-"n") operands ----------------------------------
// A K block of an operand stored [K][rows] (rows contiguous) is 128 K rows of
// X bytes (X = the tile's BM or BN).  In LDS it is kept in units of 8 K rows
// ("octets", X/2 16-byte slots each); inside octet o, 16-byte chunk c of K row
// r (columns 16c..16c+15) sits at slot 8*(c ^ odd(o)) + r, odd(o) = (o/4) & 1.
// The 8 rows of one chunk are then 128 contiguous bytes, and the octets that
// lanes 16..31 (48..63) read hold each chunk in the other 128-byte half of the
// 256 bytes the LDS banks cover than the octets lanes 0..15 (32..47) read, so
// a transposing read has no bank conflict.  The direct loads fill slot s of
// the block (s = 64 * instruction + lane).
template <int X>
__device__ __forceinline__ void kmajor_slot(int s, int& krow, int& chunk) {
  const int octet = s / (X / 2), rem = s % (X / 2);
  krow = 8 * octet + (rem & 7);
  chunk = (rem >> 3) ^ ((octet >> 2) & 1);
}
// ds_read_b64_tr_b8 (measured lane layout): in each group of 16 lanes, lane i
// < 8 receives byte i of the 8-byte words addressed by the group's even lanes
// 0, 2, .., 14 (in that order) and lane 8 + i byte i of the odd lanes' words.
// A fragment lane (row r = l % 16, K bytes 32*(l/16) .. +31) is gathered by four
// such reads, t = 0..3, in which lane s of the group addresses K row
// 32*(l/16) + 8t + s/2 at column row0 + 16*i + 8*(s%2) of 16-row strip i.
// With row0 a multiple of 32, strip i's address is
// kmajor_frag_base(row0, lane, i & 1) + 128*i + 8*X*t.
template <int X>
__device__ __forceinline__ uint32_t kmajor_frag_base(int row0, int lane, int parity) {
  const int odd = (lane >> 4) & 1;
  return (uint32_t)(32 * X * (lane >> 4) + 8 * (row0 + (lane & 15)) + (parity ? -128 : 128) * odd);
}
template <int X>
__device__ __forceinline__ v8i kmajor_frag(uint32_t addr) {
  typedef __attribute__((address_space(3))) v2i lds_v2i;
  const v2i q0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<lds_v2i*>(static_cast<uintptr_t>(addr)));
  const v2i q1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<lds_v2i*>(static_cast<uintptr_t>(addr + 8 * X)));
  const v2i q2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<lds_v2i*>(static_cast<uintptr_t>(addr + 16 * X)));
  const v2i q3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<lds_v2i*>(static_cast<uintptr_t>(addr + 24 * X)));
  return (v8i){q0.x, q0.y, q1.x, q1.y, q2.x, q2.y, q3.x, q3.y};
}

// ============================================================================
// prefill / grouped kernel
// ============================================================================
// CS: B scales per column per K block (the K-grouped form) instead of one per
// 128x128 block: each wave loads 64 of them per block into its own area.
// B4: B holds packed FP4 codes, 64 bytes per row per K block.
template <int BM, int BN, int WAVES_M, int WAVES_N, int NSLOT, bool CS = false, bool B4 = false>
struct Shape {
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int NT = NWAVES * 64;
  static constexpr int WTM = BM / WAVES_M;      // wave tile rows
  static constexpr int WTN = BN / WAVES_N;      // wave tile cols
  static constexpr int SM = WTM / 16;           // 16-row strips per wave
  static constexpr int SN = WTN / 16;           // 16-col strips per wave
  static constexpr int A_BYTES = BM * KBLK;     // one slot of each region
  static constexpr int B_ROW = B4 ? KBLK / 2 : KBLK;   // bytes of one B row per K block
  static constexpr int B_BYTES = BN * B_ROW;
  static constexpr int RS = BM / NWAVES;        // row scales loaded per wave
  // with 64 row scales per wave the B scale needs a load of its own
  static constexpr bool SB_SEP = RS >= 64;
  // a wave's scale area takes a whole 64-lane load (and a second one for the
  // B scale when SB_SEP), so every lane of the scale loads writes its own word
  // and the loads need no lane mask: RS row scales, then the B scale
  static constexpr int SA_PER_WAVE = SB_SEP ? 128 : 64;
  static constexpr int S_BYTES = NWAVES * SA_PER_WAVE * 4;
  // LDS: [A slot 0..NSLOT-1][B slot 0..NSLOT-1][scales slot 0..NSLOT-1]
  static constexpr int B_REGION = NSLOT * A_BYTES;
  static constexpr int S_REGION = NSLOT * (A_BYTES + B_BYTES);
  // column scales (CS): wave w's 64 floats hold columns 64*(w % (BN/64)) ..
  // +63, so column x of the tile sits at float x of the area
  static constexpr bool HAS_CS = CS;
  static constexpr int SC_BYTES = CS ? NWAVES * 256 : 0;
  static constexpr int SC_REGION = NSLOT * (A_BYTES + B_BYTES + S_BYTES);
  static constexpr int LDS_BYTES = NSLOT * (A_BYTES + B_BYTES + S_BYTES + SC_BYTES);
  static constexpr int A_INSTR = BM / 8 / NWAVES;     // 1 KB (8 rows) per wave instruction
  static constexpr int B_INSTR = B_BYTES / 1024 / NWAVES;
  static constexpr int LPS = A_INSTR + B_INSTR + 1 + SB_SEP + CS;   // loads per wave per K block
  static_assert(!CS || (BN % 64 == 0 && BN / 64 <= NWAVES), "column scales: one 64-column load per wave");
  static_assert(NWAVES == 4 || NWAVES == 8, "four or eight waves per workgroup");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert(WTN <= 128 && 128 % WTN == 0, "a wave's columns must sit in one 128-wide B scale block");
  static_assert(BM % (8 * NWAVES) == 0 && B_BYTES % (1024 * NWAVES) == 0, "every wave issues the same number of loads");
  static_assert(RS % 4 == 0 && RS <= 64, "row scales fit one 64-lane load per wave");
  static_assert((NSLOT - 1) * LPS < 64, "outstanding loads must fit the 6-bit vmcnt");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
  // strips start on a wave block boundary plus a multiple of 16 rows, so the scale
  // slot of row (16*i + x), x < 16, is that of row x plus a constant
  static_assert(WTM % RS == 0 && RS % 16 == 0, "scale addresses of strips differ by constants");
  static constexpr int strip_scale_off(int i) { return 4 * (((16 * i) / RS) * SA_PER_WAVE + (16 * i) % RS); }
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
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_16s(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}
// The same with the streaming (non-temporal) cache policy.
__device__ __forceinline__ void dma_16s_nt(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}
#pragma clang diagnostic pop

// E8M0 = false: MFMA partials promoted by fp32 FMAs (any scales).
// E8M0 = true:  every scale is a power of two, applied by the MFMA itself from
//               its E8M0 exponent; results accumulate in place (AGPRs).
// LAYOUT: bit 0 set = A is stored K-major ([K][M], M contiguous: the "t" of
//         "tn"/"tt"), bit 1 set = B is stored [K][N] (the second "n" of
//         "nn"/"tn"); clear bits are the K-contiguous "nt" operands; bit 2
//         (LAYOUT 4) = B holds packed FP4 (E2M1) codes, 64 bytes per row per K
//         block, with E8M0 scales per column per 32 K values that the MFMA
//         applies (sfb int32 [K/128][N], four scale bytes per int).
// MODE kKGrouped (PT = KGroupedParams): work items are (group, tile) pairs;
// group g's K range is k_start[g] .. k_start[g+1]-1, both operands K-major,
// B scales per column, fp32 D and C.
template <int BM, int BN, int WAVES_M, int WAVES_N, int NSLOT, int MODE, int WG_PER_CU, bool E8M0, int LAYOUT = 0,
          class PT = Params>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64, WG_PER_CU)
fp8_gemm_nt_kernel(PT p) {
  constexpr bool KG = MODE == kKGrouped;
  constexpr bool B4 = (LAYOUT & 4) != 0;    // FP8 x FP4: B packed E2M1, E8M0 scales per row per 32 K
  using S = Shape<BM, BN, WAVES_M, WAVES_N, NSLOT, KG || B4, B4>;
  constexpr bool TA = (LAYOUT & 1) != 0, TB = (LAYOUT & 2) != 0;
  static_assert(!B4 || (LAYOUT == 4 && !KG && !E8M0), "FP8 x FP4: NT storage (dense or M-grouped), fp32 promotion");
  static_assert(LAYOUT == 0 || LAYOUT == 4 || MODE == kDense || (KG && LAYOUT == 3),
                "K-major operands are supported by the dense and K-grouped forms");
  static_assert(!KG || (LAYOUT == 3 && !E8M0), "the K-grouped form reads K-major operands with fp32 promotion");
  static_assert((!TA || S::WTM % 32 == 0) && (!TB || S::WTN % 32 == 0), "K-major strips pair up in 32-row steps");
  // Path gate: the scale check kernel leaves one verdict per check workgroup;
  // the E8M0 kernel runs only if all scales are powers of two, the other
  // kernel only if not.  Every lane reads the same verdicts, so the exit is
  // uniform.
  if (p.gate_ok) {
    const int ok = (threadIdx.x & 63) < kCheckWGs ? p.gate_ok[threadIdx.x & 63] : 1;
    const bool all_pow2 = __builtin_amdgcn_ballot_w64(ok == 0) == 0;
    if (all_pow2 != E8M0) return;
  }
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S::LDS_BYTES];
  __shared__ int s_prefix[MODE == kMasked ? MAX_GROUPS_LDS + 1 : 1];
  // contiguous form: 128-row blocks per tile (segments are 128-row aligned)
  constexpr int CBLK = BM >= 256 ? BM / 128 : 1;
  static_assert(CBLK <= 2, "at most two expert blocks per tile");
  __shared__ int s_group[CBLK];

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

  // per-lane LDS addresses of the fragments of strip 0 in slot 0; strip i and
  // slot u add the constants 2048*i and u*region bytes (the swizzle repeats
  // every 16 rows)
  // (a K-major operand: the bases of the lane's transposing reads for even and
  // for odd strips, see kmajor_frag_base)
  uint32_t offA0[2], offB0[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // The fp8 operand of the 16x16x128 MFMA holds, in lane group g = l/16,
    // K bytes 16g..16g+15 in its low four dwords and 64+16g..64+16g+15 in the
    // high four (measured against the FP4 operand, whose lane group s holds K
    // 32s..32s+31).  Two fp8 operands only need the same K order, so the fp8 x
    // fp8 kernels read chunks 2g and 2g+1; against an FP4 B, A reads chunks g
    // and 4+g.
    offA0[h] = smem_base + (TA ? kmajor_frag_base<BM>(wrow0, lane, h)
                               : (wrow0 + r16) * KBLK + (((B4 ? 4 * h + g16 : 2 * g16 + h) ^ swz(r16)) << 4));
    // FP4 B: a 64-byte row per K block, the lane's 16 bytes (32 codes) at chunk
    // g16 of its column, chunks XOR-swizzled by (row / 4) % 4
    offB0[h] = smem_base + S::B_REGION + (TB ? kmajor_frag_base<BN>(wcol0, lane, h)
                                          : B4 ? (wcol0 + r16) * S::B_ROW + ((g16 ^ swz4(r16)) << 4)
                                               : (wcol0 + r16) * KBLK + (((2 * g16 + h) ^ swz(r16)) << 4));
  }
  // row scales of the lane's four result rows in strip 0 (strip i adds strip_scale_off(i))
  const uint32_t offS0 = smem_base + S::S_REGION +
                         4 * (((wrow0 + g16 * 4) / S::RS) * S::SA_PER_WAVE + (wrow0 + g16 * 4) % S::RS);
  const uint32_t offSB = smem_base + S::S_REGION + 4 * (wave * S::SA_PER_WAVE + S::RS);
  // K-grouped: column scale of the lane's column in strip 0 (strip j adds 64 bytes)
  const uint32_t offSC = smem_base + S::SC_REGION + 4 * (wcol0 + r16);
  // scale of the lane's MFMA operand row (row 16*i + l%16 of the wave tile) in strip 0
  const uint32_t offR0 = smem_base + S::S_REGION +
                         4 * (((wrow0 + r16) / S::RS) * S::SA_PER_WAVE + (wrow0 + r16) % S::RS);

  // ---- the work list ------------------------------------------------------
  int total;
  if constexpr (MODE == kMasked) {
    // exclusive prefix over groups of (m tiles * n tiles); masked_m clamped to [0, max_m]
    masked_prefix<BM, S::NT>(p, s_prefix, tid);
    total = s_prefix[p.G];
  } else if constexpr (KG) {
    total = p.G * p.tiles_m * p.tiles_n;
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

  // Split tail (dense and 128-row contiguous calls, p.sk_splits > 1): the
  // XCD's items that do not fill a last round of its workgroups are each
  // split into sk_splits K ranges, one per workgroup; those write fp32
  // partial tiles and splitk_tile_reduce_kernel, launched next, sums them.
  // (not compiled into the 256x256 tile, whose registers are full and whose
  // calls rarely leave a tail worth splitting)
  constexpr bool SKOK = (MODE == kDense || (MODE == kContiguous && CBLK == 1)) && !E8M0 && BM * BN <= 128 * 256;
  const int n_x = max(0, w_end - w_begin);
  const int sk_s = SKOK ? p.sk_splits : 1;
  const int full_x = sk_s > 1 ? n_x / slots * slots : n_x;      // items of whole rounds
  const int units_x = full_x + (n_x - full_x) * sk_s;

  // A contiguous tile whose two 128-row blocks belong to two experts is
  // visited twice, once per expert (pass 0, 1); each visit stores only the
  // rows of its own expert.  The second visit is a repeat of the same item
  // rather than an inner loop, so the K loop keeps a single copy.
  int pass = 0;
  for (int it = slot_id; it < units_x;) {
    // ---- resolve the work item ---------------------------------------------
    int w = w_begin + it, split = -1, tail_idx = 0;
    if (it >= full_x) {
      tail_idx = (it - full_x) / sk_s;
      w = w_begin + full_x + tail_idx;
      split = (it - full_x) % sk_s;
    }
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
      if constexpr (KG) {
        const int per_group = p.tiles_m * p.tiles_n;
        group = w / per_group;
        tile_coords(w - group * per_group, p.tiles_m, p.tiles_n, mt, nt);
      } else {
        tile_coords(w, p.tiles_m, p.tiles_n, mt, nt);
      }
      if constexpr (MODE == kContiguous) {
        // the expert of each 128-row block of the tile: the largest valid id
        // among its rows; ids outside [0, G) (padding, conventionally -1) count
        // as -1, so that they never hide the block's valid rows.  All valid ids
        // in a block agree.
        if (wave < CBLK) {
          int best = -1;
          for (int r = lane; r < BM / CBLK; r += 64) {
            const int row = mt * BM + wave * (BM / CBLK) + r;
            if (row < p.rows) {
              const int id = p.layout[row];
              best = max(best, id >= 0 && id < p.G ? id : -1);
            }
          }
          for (int off = 32; off > 0; off >>= 1) best = max(best, __shfl_xor(best, off));
          if (lane == 0) s_group[wave] = best;
        }
        lds_barrier();
        const int g0 = s_group[0], g1 = s_group[CBLK - 1];
        lds_barrier();
        const bool v0 = g0 >= 0 && g0 < p.G, v1 = g1 >= 0 && g1 < p.G;
        group = pass == 0 && v0 ? g0 : g1;
        if (pass == 0 && v0 && v1 && g0 != g1) {
          pass = 1;                        // visit this tile again for g1
        } else {
          pass = 0;
          it += slots;
        }
        if (!v0 && !v1) continue;          // uniform across the workgroup (the reduction skips
                                           // such rows, so a split unit need not write)
      } else {
        it += slots;
      }
    }
    if constexpr (MODE == kMasked) it += slots;

    const int m0 = mt * BM;
    const int n0 = nt * BN;
    int kbs = KB, kb0 = 0;          // this item's K blocks (K-grouped: the group's; split: its range)
    if constexpr (KG) {
      kb0 = p.k_start[group] / KBLK;
      kbs = p.k_start[group + 1] / KBLK - kb0;
    }
    if (split >= 0) {
      kb0 = split * KB / sk_s;
      kbs = (split + 1) * KB / sk_s - kb0;
    }

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
    if constexpr (MODE == kContiguous || MODE == kMasked) {
      if constexpr (B4) {                 // packed FP4 rows and int32 [K/128][N] E8M0 scales per group
        B += (size_t)group * p.N * (p.K / 2);
        SB += (size_t)group * KB * p.N;
      } else {
        B += (size_t)group * p.N * p.K;
        SB += (size_t)group * NB * KB;
      }
    }
    float* D32 = nullptr;
    const float* C32 = nullptr;
    if constexpr (KG) {
      // the group's first K row of A [K][M] and B [K][N] and of the scales
      A += (size_t)kb0 * KBLK * a_rows;
      B += (size_t)kb0 * KBLK * p.N;
      SA += (size_t)kb0 * a_rows;
      SB += (size_t)kb0 * p.N;          // column scales [K/128][N]
      D32 = p.d32 + (size_t)group * a_rows * p.N;
      if (p.c32) C32 = p.c32 + (size_t)group * a_rows * p.N;
    }
    if (SKOK && split >= 0) {
      // a split's K range: its first K block of A, B and their scales
      A += TA ? (size_t)kb0 * KBLK * a_rows : (size_t)kb0 * KBLK;
      B += TB ? (size_t)kb0 * KBLK * p.N : (size_t)kb0 * S::B_ROW;
      SA += (size_t)kb0 * a_rows;
      // B scales: FP4 int32 [K/128][N]; otherwise [NB][KB], block nb's row at nb*KB
      SB += B4 ? (size_t)kb0 * p.N : (size_t)kb0;
    }
    int nb = (KG || B4) ? 0 : (n0 + wcol0) / 128;
    nb = nb < NB ? nb : NB - 1;

    // ---- load addresses -------------------------------------------------------
    // A / B: wave instruction j covers tile rows 8*(wave + NWAVES*j) .. +7; lane l lands
    // at LDS byte 16*l of that 1 KB piece: row 8*(...) + l/8, physical chunk l%8,
    // which holds logical chunk (l%8) ^ swz(row).  Uniform bases (tile origin,
    // K block) live in SGPRs; lanes add a 32-bit offset inside the tile.
    // A K-major operand's tile starts at column m0 (n0) of its [K][rows] array
    // and a K block advances 128 of its rows; chunks of columns past the valid
    // ones re-read the last valid 16 columns (rows_lim and N are multiples of
    // 16 for such operands), whose results are never stored.
    const uint8_t* a_tile = TA ? A + m0 : A + (size_t)m0 * p.K;
    const uint8_t* b_tile = TB ? B + n0 : B + (size_t)n0 * (p.K / KBLK) * S::B_ROW;
    const size_t a_kstep = TA ? (size_t)KBLK * a_rows : KBLK;
    const size_t b_kstep = TB ? (size_t)KBLK * p.N : S::B_ROW;
    uint32_t a_off[S::A_INSTR], b_off[S::B_INSTR];
#pragma unroll
    for (int j = 0; j < S::A_INSTR; ++j) {
      if constexpr (TA) {
        int kr, c;
        kmajor_slot<BM>(64 * (wave + S::NWAVES * j) + lane, kr, c);
        a_off[j] = (uint32_t)(kr * a_rows + (min(m0 + 16 * c, rows_lim - 16) - m0));
      } else {
        const int r = (wave + S::NWAVES * j) * 8 + (lane >> 3);
        // rows past the valid ones (the end of A, or of a masked group's rows) are
        // never stored: they re-read the last valid row, whose lines the L1 holds
        const int grow = min(m0 + r, rows_lim - 1);
        a_off[j] = (uint32_t)((grow - m0) * p.K) + (((lane & 7) ^ swz(r)) << 4);
      }
    }
#pragma unroll
    for (int j = 0; j < S::B_INSTR; ++j) {
      if constexpr (B4) {
        // FP4 B: instruction j covers tile rows 16*(wave + NWAVES*j) .. +15, four
        // 16-byte chunks each; lane l loads row .. + l/4, logical chunk (l%4) ^ swz4
        const int r = (wave + S::NWAVES * j) * 16 + (lane >> 2);
        const int gn = min(n0 + r, p.N - 1);
        b_off[j] = (uint32_t)((gn - n0) * (p.K / 2)) + (((lane & 3) ^ swz4(r)) << 4);
      } else if constexpr (TB) {
        int kr, c;
        kmajor_slot<BN>(64 * (wave + S::NWAVES * j) + lane, kr, c);
        b_off[j] = (uint32_t)(kr * p.N + (min(n0 + 16 * c, p.N - 16) - n0));
      } else {
        const int r = (wave + S::NWAVES * j) * 8 + (lane >> 3);
        const int gn = min(n0 + r, p.N - 1);
        b_off[j] = (uint32_t)((gn - n0) * p.K) + (((lane & 7) ^ swz(r)) << 4);
      }
    }
    // scales: lanes < RS load row scales of rows wave*RS + lane, the other lanes
    // (or a separate load when RS is 64) this wave's B scale
    const float* s_src;
    size_t s_stride;                  // elements per K block
    const float* sb_src = SB + (size_t)nb * KB;
    if (lane < S::RS) {
      const int grow = min(m0 + wave * S::RS + lane, rows_lim - 1);
      s_src = SA + grow;
      s_stride = a_rows;
    } else {
      s_src = SB + (size_t)nb * KB;
      s_stride = 1;
    }
    // K-grouped: this wave's 64 column scales of each K block
    const float* sc_src = SB + min(n0 + 64 * (wave % (BN / 64)) + lane, p.N - 1);

    // K order: with a window of W = p.k_window blocks (a power of two), the
    // blocks of each aligned window are taken starting at offset (mt + nt) mod W
    // of that window; blocks after the last whole window stay in order.  Tiles
    // next to each other in a round then fetch different blocks of a window at
    // the same time, and each finds the blocks its neighbours fetched earlier in
    // the L2.  The summation order depends on the tile's position alone, so
    // results are the same from call to call.
    const int kwm0 = p.k_window > 1 ? p.k_window - 1 : 0;
    const int kwm = (kwm0 & (kwm0 + 1)) == 0 ? kwm0 : 0;       // window mask (in order unless W = 2^n)
    const int kwin = __builtin_amdgcn_readfirstlane((mt + nt) & kwm);
    const int kfull = kbs & ~kwm;                                // blocks in whole windows

    // the k-th load instruction (k < LPS) of the item's i-th K block into slot u
    auto issue_one = [&](int k, int i, int u) {
      i = __builtin_amdgcn_readfirstlane(i < kfull ? (i & ~kwm) | ((i + kwin) & kwm) : i);
      if (S::HAS_CS && k == S::LPS - 1) {
        dma_4(sc_src + (size_t)i * p.N, smem_base + S::SC_REGION + u * S::SC_BYTES + wave * 256);
      } else if (k < S::A_INSTR) {
        dma_16s(a_tile + i * a_kstep, a_off[k], smem_base + u * S::A_BYTES + (wave + S::NWAVES * k) * 1024);
      } else if (k < S::A_INSTR + S::B_INSTR) {
        const int j = k - S::A_INSTR;
        // a masked group's B columns go to one item per m-tile of the group
        // (one for groups of up to BM rows): streaming policy; elsewhere the
        // other row tiles read them again from the L2
        if constexpr (MODE == kMasked)
          dma_16s_nt(b_tile + i * b_kstep, b_off[j],
                     smem_base + S::B_REGION + u * S::B_BYTES + (wave + S::NWAVES * j) * 1024);
        else
          dma_16s(b_tile + i * b_kstep, b_off[j],
                  smem_base + S::B_REGION + u * S::B_BYTES + (wave + S::NWAVES * j) * 1024);
      } else if (!S::SB_SEP || k == S::A_INSTR + S::B_INSTR) {
        // lanes past RS load the B scale (lane RS's copy is the one read)
        dma_4(s_src + (size_t)i * s_stride, smem_base + S::S_REGION + u * S::S_BYTES + wave * S::SA_PER_WAVE * 4);
      } else {
        // every lane loads the B scale; lane 0's copy is the one read
        dma_4(sb_src + i, smem_base + S::S_REGION + u * S::S_BYTES + (wave * S::SA_PER_WAVE + S::RS) * 4);
      }
    };
    auto issue = [&](int i, int u) {
#pragma unroll
      for (int k = 0; k < S::LPS; ++k) issue_one(k, i, u);
    };

    v4f acc[S::SM][S::SN];

    // one K block from slot u (compile-time): fragments, promotion factors, MFMAs.
    // The loads of block `next` into slot next_u are spread between the MFMAs so
    // the vector-memory queue drains while the matrix cores run.
    // sma_const: the A strips computed (all of them, or the first half when
    // the wave's valid rows fit in them)
    auto compute = [&](auto u_const, int next, int next_u, float live, auto sma_const) {
      constexpr int u = decltype(u_const)::value;
      constexpr int SMA = decltype(sma_const)::value;
      // the block's B scale (K-grouped: 1, the per-column scales enter below)
      const float sb = (KG || B4) ? live : lds_f32(offSB + u * S::S_BYTES) * live;
      auto frag = [&](uint32_t lo_addr, uint32_t hi_addr) {
        const v4i lo = lds_v4i(lo_addr), hi = lds_v4i(hi_addr);
        return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      };
      // fragments of 16-row strip i of A / 16-column strip j of B in slot u
      auto fragA = [&](int i) {
        if constexpr (TA) return kmajor_frag<BM>(offA0[i & 1] + i * 128 + u * S::A_BYTES);
        else return frag(offA0[0] + i * 2048 + u * S::A_BYTES, offA0[1] + i * 2048 + u * S::A_BYTES);
      };
      auto fragB = [&](int j) {
        if constexpr (B4) {
          const v4i q = lds_v4i(offB0[0] + j * 16 * S::B_ROW + u * S::B_BYTES);
          return (v8i){q.x, q.y, q.z, q.w, 0, 0, 0, 0};   // FP4 operands use the low four dwords
        }
        if constexpr (TB) return kmajor_frag<BN>(offB0[j & 1] + j * 128 + u * S::B_BYTES);
        else return frag(offB0[0] + j * 2048 + u * S::B_BYTES, offB0[1] + j * 2048 + u * S::B_BYTES);
      };
      constexpr int T = SMA * S::SN;
      constexpr int STRIDE = T / S::LPS > 0 ? T / S::LPS : 1;
      static_assert(!E8M0 || SMA == S::SM, "the MFMA-scaled path computes every strip");
      if constexpr (E8M0) {
        // scale exponents: the biased fp32 exponent of 2^e is its E8M0 code;
        // lane l scales A row l%16 of the strip and B column l%16.  All A strips
        // stay in registers; B strips are read one column ahead of their MFMAs.
        const int eb = (int)(__float_as_uint(sb) >> 23);
        v8i af[S::SM];
        int ea[S::SM];
#pragma unroll
        for (int i = 0; i < S::SM; ++i) {
          af[i] = fragA(i);
          ea[i] = (int)(__float_as_uint(lds_f32(offR0 + S::strip_scale_off(i) + u * S::S_BYTES)) >> 23);
        }
        v8i bcur = fragB(0);
#pragma unroll
        for (int j = 0; j < S::SN; ++j) {
          v8i bnext = bcur;
          if (j + 1 < S::SN)
            bnext = fragB(j + 1);
#pragma unroll
          for (int i = 0; i < S::SM; ++i) {
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bcur, acc[i][j], 0, 0, 0, ea[i],
                                                                         0, eb);
            const int t = j * S::SM + i;
            if (t % STRIDE == 0 && t / STRIDE < S::LPS) issue_one(t / STRIDE, next, next_u);
          }
          bcur = bnext;
          __builtin_amdgcn_sched_barrier(0);
        }
        return;
      }
      v8i bf[S::SN], af[S::SM];
      v4f sc[S::SM];
#pragma unroll
      for (int j = 0; j < S::SN; ++j)
        bf[j] = fragB(j);
      float sbc[S::SN];               // K-grouped: the lane's column scale in each column strip
      int esb[S::SN];                 // FP4 B: E8M0 scale of the lane's column and 32-K slice
#pragma unroll
      for (int j = 0; j < S::SN; ++j) {
        sbc[j] = KG ? lds_f32(offSC + j * 64 + u * S::SC_BYTES) : 1.f;
        esb[j] = B4 ? (int)((__float_as_uint(lds_f32(offSC + j * 64 + u * S::SC_BYTES)) >> (8 * g16)) & 0xFF) : 0;
      }
      // A strips are read one strip ahead of their MFMAs, which bounds the live
      // A fragments to two
      auto load_strip = [&](int i) {
        af[i] = fragA(i);
        sc[i] = lds_v4f(offS0 + S::strip_scale_off(i) + u * S::S_BYTES) * sb;
      };
      load_strip(0);
      // P partials in flight: MFMA t's promotion runs after MFMA t+P-1 has
      // issued, so its FMAs need no wait states for the MFMA result and can
      // issue while the matrix core runs the later MFMAs (P = 4 measured 2-4%
      // faster than 2 on the NT and FP4 prefill shapes; the K-major layouts
      // keep 2, where 4 spills registers; the dense nt 256x256 tile, whose
      // schedule interleaves each MFMA with four FMAs below, takes 3: 0.3-1.2%
      // faster than 4 there)
      constexpr bool INTERLEAVED = MODE == kDense && LAYOUT == 0 && !E8M0 && S::SM * S::SN >= 32;
      constexpr int P = INTERLEAVED ? 3 : (LAYOUT == 0 || LAYOUT == 4) ? 4 : 2;
      v4f part[P];
#pragma unroll
      for (int t = 0; t < T + P - 1; ++t) {
        if (t < T) {
          if (t % S::SN == 0 && t / S::SN + 1 < SMA) {
            // keep the scheduler from hoisting every strip's reads to the top
            // (the 256x256 tile; the eight-wave nt tiles of 64x64 wave tiles
            // take the same per-strip regions for the hints below)
            constexpr bool WIDE = S::SM * S::SN >= 32;
            constexpr bool NT8 = S::NWAVES == 8 && LAYOUT == 0 && !E8M0 && !KG;
            if constexpr (WIDE || NT8) {
              // the strip just scheduled issues each MFMA followed by four
              // promotion FMAs, rather than its FMAs in one run ahead of its
              // MFMAs: dense nt and nn 256x256 (prefill 1.4-1.6% faster) and the
              // eight-wave nt 128x256 and 256x128 tiles (contiguous 2-4%
              // faster, masked unchanged); the FP4, K-major-A and K-grouped
              // kernels measured no gain or a loss
              if constexpr (WIDE ? MODE == kDense && (LAYOUT == 0 || LAYOUT == 2) && !E8M0 : NT8) {
                if (t > 0) {
                  __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // the next strip's LDS reads
#pragma unroll
                  for (int q = 0; q < S::SN; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // four VALU
                  }
                }
              }
              __builtin_amdgcn_sched_barrier(0);
            }
            load_strip(t / S::SN + 1);
          }
          const v4f zero = {0.f, 0.f, 0.f, 0.f};
          if constexpr (B4)   // B format FP4 (E2M1), its E8M0 scale per lane; A unscaled (2^0)
            part[t % P] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[t / S::SN], bf[t % S::SN], zero,
                                                                           0, 4, 0, 127, 0, esb[t % S::SN]);
          else
            part[t % P] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[t / S::SN], bf[t % S::SN], zero,
                                                                           0, 0, 0, 0, 0, 0);
          // spread the LPS loads of the next block over the first MFMAs
          if (t % STRIDE == 0 && t / STRIDE < S::LPS) issue_one(t / STRIDE, next, next_u);
        }
        const int v = t - (P - 1);
        if (v >= 0) {
          v4f& a = acc[v / S::SN][v % S::SN];
          const v4f& q = part[v % P];
          const v4f c = KG ? sc[v / S::SN] * sbc[v % S::SN] : sc[v / S::SN];
          a.x = __builtin_fmaf(q.x, c.x, a.x);
          a.y = __builtin_fmaf(q.y, c.y, a.y);
          a.z = __builtin_fmaf(q.z, c.z, a.z);
          a.w = __builtin_fmaf(q.w, c.w, a.w);
        }
      }
      // with fewer MFMAs than loads (half the strips of a small wave tile) the
      // rest of the next block's loads follow the MFMAs
      if constexpr (T < S::LPS) {
#pragma unroll
        for (int k = T; k < S::LPS; ++k) issue_one(k, next, next_u);
      }
      // nothing of the next block is hoisted into this one (bounds live fragments)
      __builtin_amdgcn_sched_barrier(0);
    };

    // ---- K loop over the slot ring, unrolled by NSLOT so slots are constants --
    // Every step issues the loads of block i+NSLOT-1, clamped to the last
    // block: past the end the copy lands in the slot just consumed, which no
    // later block of this item reads.  The schedule is then the same at every
    // step (NSLOT-2 blocks in flight behind the one awaited) with no branch
    // between the MFMAs, which would keep the accumulators from being updated
    // in place.
    if (kbs > 0) {
#pragma unroll
      for (int u = 0; u < NSLOT - 1; ++u) issue(min(u, kbs - 1), u);
    }
#pragma unroll
    for (int i = 0; i < S::SM; ++i)
#pragma unroll
      for (int j = 0; j < S::SN; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

    // A wave whose rows all lie past the item's valid rows (a masked group's
    // last m-tile, the end of A) only issues its share of the loads and meets
    // the barriers: its MFMAs would produce nothing that is stored, and
    // skipping them frees its SIMD for the wave sharing it.
    const bool idle = __builtin_amdgcn_readfirstlane(m0 + wrow0 >= rows_lim ? 1 : 0) != 0;
    if (idle) {
      const int steps = E8M0 ? kbs : (kbs + NSLOT - 1) / NSLOT * NSLOT;
      for (int i = 0; i < steps; ++i) {
        wait_vm_lgkm0<(NSLOT - 2) * S::LPS>();
        bare_barrier();
        issue(min(i + NSLOT - 1, kbs - 1), (i + NSLOT - 1) % NSLOT);
      }
    } else if constexpr (E8M0) {
      for (int i0 = 0; i0 < kbs; i0 += NSLOT) {
        static_for<NSLOT>([&](auto u_const) {
          constexpr int u = decltype(u_const)::value;
          const int i = i0 + u;
          if (i < kbs) {
            wait_vm_lgkm0<(NSLOT - 2) * S::LPS>();
            bare_barrier();
            compute(u_const, min(i + NSLOT - 1, kbs - 1), (u + NSLOT - 1) % NSLOT, 1.f,
                    std::integral_constant<int, S::SM>{});
          }
        });
      }
    } else {
      // The fp32-promotion path runs a whole number of ring turns: a step past
      // the last block recomputes a copy of it (the clamped loads put one in
      // its slot) and promotes it with a zero factor.  Every step is then the
      // same straight-line code, which keeps the VGPR accumulators in place.
      const int steps = (kbs + NSLOT - 1) / NSLOT * NSLOT;
      auto run = [&](auto sma_const) {
        for (int i0 = 0; i0 < steps; i0 += NSLOT) {
          static_for<NSLOT>([&](auto u_const) {
            constexpr int u = decltype(u_const)::value;
            const int i = i0 + u;
            wait_vm_lgkm0<(NSLOT - 2) * S::LPS>();
            bare_barrier();
            compute(u_const, min(i + NSLOT - 1, kbs - 1), (u + NSLOT - 1) % NSLOT, i < kbs ? 1.f : 0.f, sma_const);
          });
        }
      };
      // masked groups: a wave whose valid rows fit in its first half of strips
      // computes only those (its other strips' results are never stored)
      if constexpr (MODE == kMasked && S::SM % 2 == 0) {
        const bool half = __builtin_amdgcn_readfirstlane(rows_lim - (m0 + wrow0) <= S::WTM / 2 ? 1 : 0) != 0;
        if (half) run(std::integral_constant<int, S::SM / 2>{});
        else run(std::integral_constant<int, S::SM>{});
      } else {
        run(std::integral_constant<int, S::SM>{});
      }
    }

    // ---- epilogue: round to bf16, store the rows that belong to the result
    // One element at a time in accumulator order (i, j, e): each accumulator
    // tuple is consumed whole, which keeps register pressure low enough that
    // the accumulators are never split or spilled around the K loop.
    // Contiguous: the lane's rows (strip i, quad row e: bit 4i+e) that belong
    // to this item's expert, read from grouped_layout once, all loads together.
    static_assert(S::SM * 4 <= 32, "row mask bits");
    uint32_t row_ok = ~0u;
    if constexpr (MODE == kContiguous) {
      int ids[S::SM * 4];
#pragma unroll
      for (int q = 0; q < S::SM * 4; ++q)
        ids[q] = p.layout[min(m0 + wrow0 + (q / 4) * 16 + g16 * 4 + q % 4, p.rows - 1)];
      row_ok = 0;
#pragma unroll
      for (int q = 0; q < S::SM * 4; ++q) row_ok |= (ids[q] == group ? 1u : 0u) << q;
    }
    // C is read a strip at a time, strip i+1 before the stores of strip i: a
    // load issued after a store can only be waited for together with that
    // store (one in-order count covers both), so reading C element by element
    // between the stores would wait for every earlier store.  The 256x256
    // tile and the MFMA-scaled kernels have no registers for the two strip
    // buffers and read C per element.
    const bool split_unit = SKOK && split >= 0;
    const bool c_in = !split_unit && (KG ? C32 != nullptr : C != nullptr);
    constexpr bool C_PIPE = BM * BN <= 128 * 256 && !E8M0;
    float cv[2][S::SN * 4];
    auto c_at = [&](int row, int col) {
      const size_t off = (size_t)min(row, p.rows - 1) * p.N + min(col, p.N - 1);
      return KG ? C32[off] : bf16_to_f32(C[off]);
    };
    auto load_c = [&](int i, float (&dst)[S::SN * 4]) {
#pragma unroll
      for (int j = 0; j < S::SN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[j * 4 + e] = c_at(m0 + wrow0 + i * 16 + g16 * 4 + e, n0 + wcol0 + j * 16 + r16);
    };
    if (C_PIPE && c_in) load_c(0, cv[0]);
#pragma unroll
    for (int i = 0; i < S::SM; ++i) {
      if (C_PIPE && c_in && i + 1 < S::SM) load_c(i + 1, cv[(i + 1) % 2]);
#pragma unroll
      for (int j = 0; j < S::SN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + wrow0 + i * 16 + g16 * 4 + e;
          const int col = n0 + wcol0 + j * 16 + r16;
          float v = acc[i][j][e];
          if (split_unit) {
            // split unit: the fp32 partial, row-major [BM][BN], to the
            // workspace slot of (XCD, tail item, split)
            p.workspace[((size_t)(xcd * p.sk_tail + tail_idx) * sk_s + split) * (BM * BN) +
                        (wrow0 + i * 16 + g16 * 4 + e) * BN + wcol0 + j * 16 + r16] = v;
          } else {
            if (c_in) v += C_PIPE ? cv[i % 2][j * 4 + e] : c_at(row, col);
            if constexpr (KG) {
              // fp32 result + C: no rounding beyond the fp32 accumulation
              if (row < rows_lim && col < p.N) D32[(size_t)row * p.N + col] = v;
            } else {
              if (row < rows_lim && col < p.N && ((row_ok >> (i * 4 + e)) & 1))
                D[(size_t)row * p.N + col] = f32_to_bf16(v);
            }
          }
        }
    }
    // The next item reuses the LDS ring once every wave is past its K loop.
    // The epilogue's stores stay in flight while the next item's first loads
    // are issued: a wait for "at most n operations outstanding" in its K loop
    // still covers the block it needs, because loads complete in issue order
    // and stores only add to the count.
    lds_barrier();
  }
}

}  // namespace
}  // namespace dg
