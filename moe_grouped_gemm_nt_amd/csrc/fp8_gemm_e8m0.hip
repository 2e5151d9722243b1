// gfx950 kernels for the FP8 block-scaled GEMM, NT layout, when every scale is
// a power of two: the MFMA applies the scales from their E8M0 exponents and
// accumulates in place, so there is no fp32 promotion on the VALU and the
// accumulators can live in AGPRs, which allows 64x128 wave tiles.  Also the
// scale check that gates between this path and the general one.
//
// Built without -amdgpu-mfma-vgpr-form, so MFMA accumulators go to AGPRs.
#include "fp8_gemm_core.h"

namespace dg {
namespace {

// Wave-specialised power-of-two kernel.  A workgroup owns a BM x BN tile and
// runs two sets of WAVES_M*WAVES_N waves on each SIMD pair:
//   * MFMA waves own a wave tile each and only read LDS and issue MFMAs; the
//     scales enter the MFMA as E8M0 exponents and the accumulators stay in
//     AGPRs, updated in place;
//   * loader waves issue the direct global->LDS loads of the slot ring (each
//     mirrors one MFMA wave: that wave's share of the A/B rows, its rows'
//     scales and its B scale) and wait for them.
// A wave blocked on a full vector-memory queue cannot issue anything else, so
// keeping the loads out of the MFMA waves keeps the matrix cores fed.  One
// s_barrier per K block hands a landed slot to the MFMA waves and a consumed
// one back to the loaders; one more after the last block lets the loaders
// start the next tile's loads while the MFMA waves run the epilogue.
template <int BM, int BN, int WAVES_M, int WAVES_N, int NSLOT, int MODE>
__global__ void __launch_bounds__(2 * WAVES_M * WAVES_N * 64, 1)
fp8_gemm_nt_ws_kernel(Params p) {
  using S = Shape<BM, BN, WAVES_M, WAVES_N, NSLOT>;
  if (p.gate_ok) {
    const int ok = (threadIdx.x & 63) < kCheckWGs ? p.gate_ok[threadIdx.x & 63] : 1;
    if (__builtin_amdgcn_ballot_w64(ok == 0) != 0) return;   // some scale is not a power of two
  }
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S::LDS_BYTES];
  __shared__ int s_prefix[MODE == kMasked ? MAX_GROUPS_LDS + 1 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool loader = wave >= S::NWAVES;
  const int cw = loader ? wave - S::NWAVES : wave;   // the MFMA wave this wave is or serves
  const uint32_t smem_base = lds_u32(smem);
  const int wm = cw / WAVES_N;
  const int wn = cw % WAVES_N;
  const int KB = p.K / KBLK;
  const int NB = (p.N + 127) / 128;
  const int g16 = lane >> 4;
  const int r16 = lane & 15;
  const int wrow0 = wm * S::WTM;
  const int wcol0 = wn * S::WTN;

  // MFMA waves: fragment addresses of strip 0 in slot 0 (strip i adds 2048*i)
  uint32_t offA0[2], offB0[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    offA0[h] = smem_base + (wrow0 + r16) * KBLK + (((2 * g16 + h) ^ swz(r16)) << 4);
    offB0[h] = smem_base + S::B_REGION + (wcol0 + r16) * KBLK + (((2 * g16 + h) ^ swz(r16)) << 4);
  }
  const uint32_t offSB = smem_base + S::S_REGION + 4 * (cw * S::SA_PER_WAVE + S::RS);
  const uint32_t offR0 = smem_base + S::S_REGION +
                         4 * (((wrow0 + r16) / S::RS) * S::SA_PER_WAVE + (wrow0 + r16) % S::RS);

  int total;
  if constexpr (MODE == kMasked) {
    masked_prefix<BM, 2 * S::NT>(p, s_prefix, tid);     // MFMA and loader waves together
    total = s_prefix[p.G];
  } else {
    total = p.tiles_m * p.tiles_n;
  }

  const int slots = (gridDim.x + 7) / 8;
  const int xcd = blockIdx.x % 8;
  const int slot_id = blockIdx.x / 8;
  const int per_xcd = (total + 7) / 8;
  const int w_begin = xcd * per_xcd;
  const int w_end = min(total, w_begin + per_xcd);
  int g_cur = 0;

  for (int w = w_begin + slot_id; w < w_end; w += slots) {
    int group = 0, mt, nt, rows_lim = p.rows;
    if constexpr (MODE == kMasked) {
      while (w >= s_prefix[g_cur + 1]) ++g_cur;
      const int local = w - s_prefix[g_cur];
      int m = p.masked_m[g_cur];
      m = m < 0 ? 0 : (m > p.rows ? p.rows : m);
      const int tm = (m + BM - 1) / BM;
      group = g_cur;
      mt = local % tm;
      nt = local / tm;
      rows_lim = m;
    } else {
      tile_coords(w, p.tiles_m, p.tiles_n, mt, nt);
      if constexpr (MODE == kContiguous) {
        // every wave finds the block's expert itself (largest valid id among
        // its rows; ids outside [0, G), conventionally -1 on padding rows,
        // count as -1), so no workgroup sync is needed
        int best = -1;
        for (int r = lane; r < BM; r += 64) {
          const int row = mt * BM + r;
          if (row < p.rows) {
            const int id = p.layout[row];
            best = max(best, id >= 0 && id < p.G ? id : -1);
          }
        }
        for (int off = 32; off > 0; off >>= 1) best = max(best, __shfl_xor(best, off));
        group = __builtin_amdgcn_readfirstlane(best);
        if (group < 0 || group >= p.G) continue;   // the same for every wave
      }
    }

    const int m0 = mt * BM;
    const int n0 = nt * BN;
    const int kbs = KB;
    const uint8_t* A = p.a;
    const float* SA = p.sfa;
    const uint8_t* B = p.b;
    const float* SB = p.sfb;
    uint16_t* D = p.d;
    const uint16_t* C = p.c;
    const int a_rows = p.rows;
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

    if (loader) {
      // ---- loader wave: the loads MFMA wave cw would issue -------------------
      const uint8_t* a_tile = A + (size_t)m0 * p.K;
      const uint8_t* b_tile = B + (size_t)n0 * p.K;
      uint32_t a_off[S::A_INSTR], b_off[S::B_INSTR];
#pragma unroll
      for (int j = 0; j < S::A_INSTR; ++j) {
        const int r = (cw + S::NWAVES * j) * 8 + (lane >> 3);
        const int grow = min(m0 + r, rows_lim - 1);   // rows past the valid ones are never stored
        a_off[j] = (uint32_t)((grow - m0) * p.K) + (((lane & 7) ^ swz(r)) << 4);
      }
#pragma unroll
      for (int j = 0; j < S::B_INSTR; ++j) {
        const int r = (cw + S::NWAVES * j) * 8 + (lane >> 3);
        const int gn = min(n0 + r, p.N - 1);
        b_off[j] = (uint32_t)((gn - n0) * p.K) + (((lane & 7) ^ swz(r)) << 4);
      }
      int nb = (n0 + wcol0) / 128;
      nb = nb < NB ? nb : NB - 1;
      const float* sb_src = SB + (size_t)nb * KB;
      const float* s_src;
      size_t s_stride;
      if (lane < S::RS) {
        s_src = SA + min(m0 + cw * S::RS + lane, rows_lim - 1);
        s_stride = a_rows;
      } else {
        s_src = sb_src;
        s_stride = 1;
      }
      auto issue = [&](int i, int u) {
#pragma unroll
        for (int k = 0; k < S::A_INSTR; ++k)
          dma_16s(a_tile + (size_t)i * KBLK, a_off[k], smem_base + u * S::A_BYTES + (cw + S::NWAVES * k) * 1024);
#pragma unroll
        for (int k = 0; k < S::B_INSTR; ++k)
          dma_16s(b_tile + (size_t)i * KBLK, b_off[k],
                  smem_base + S::B_REGION + u * S::B_BYTES + (cw + S::NWAVES * k) * 1024);
        // every lane writes its own word of the wave's scale area (lanes past RS
        // load the B scale), so the scale loads need no lane mask
        dma_4(s_src + (size_t)i * s_stride, smem_base + S::S_REGION + u * S::S_BYTES + cw * S::SA_PER_WAVE * 4);
        if (S::SB_SEP)
          dma_4(sb_src + i, smem_base + S::S_REGION + u * S::S_BYTES + (cw * S::SA_PER_WAVE + S::RS) * 4);
      };
#pragma unroll
      for (int u = 0; u < NSLOT - 1; ++u)
        if (u < kbs) issue(u, u);
      int u_next = NSLOT - 1;                   // slot of block i + NSLOT - 1
      for (int i = 0; i < kbs; ++i) {
        // block i has landed once at most min(kbs-1-i, NSLOT-2) later blocks are in flight
        wait_stages<S::LPS, NSLOT - 2>(min(kbs - 1 - i, NSLOT - 2));
        bare_barrier();                         // slot of block i -> MFMA waves; slot of i-1 free
        if (i + NSLOT - 1 < kbs) issue(i + NSLOT - 1, u_next);
        u_next = u_next + 1 == NSLOT ? 0 : u_next + 1;
      }
      bare_barrier();                           // the MFMA waves are done with the ring
      continue;
    }

    // ---- MFMA wave -------------------------------------------------------------
    v4f acc[S::SM][S::SN];
#pragma unroll
    for (int i = 0; i < S::SM; ++i)
#pragma unroll
      for (int j = 0; j < S::SN; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

    auto frag = [&](uint32_t lo_addr, uint32_t hi_addr) {
      const v4i lo = lds_v4i(lo_addr), hi = lds_v4i(hi_addr);
      return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    };
    // one K block from slot u: the E8M0 code of a positive normal power of two
    // is its biased fp32 exponent; lane l scales A row l%16 and B column l%16
    auto compute = [&](auto u_const) {
      constexpr int u = decltype(u_const)::value;
      const int eb = (int)(__float_as_uint(lds_f32(offSB + u * S::S_BYTES)) >> 23);
      v8i af[S::SM];
      int ea[S::SM];
#pragma unroll
      for (int i = 0; i < S::SM; ++i) {
        af[i] = frag(offA0[0] + i * 2048 + u * S::A_BYTES, offA0[1] + i * 2048 + u * S::A_BYTES);
        ea[i] = (int)(__float_as_uint(lds_f32(offR0 + S::strip_scale_off(i) + u * S::S_BYTES)) >> 23);
      }
      v8i bcur = frag(offB0[0] + u * S::B_BYTES, offB0[1] + u * S::B_BYTES);
#pragma unroll
      for (int j = 0; j < S::SN; ++j) {
        v8i bnext = bcur;
        if (j + 1 < S::SN)
          bnext = frag(offB0[0] + (j + 1) * 2048 + u * S::B_BYTES, offB0[1] + (j + 1) * 2048 + u * S::B_BYTES);
#pragma unroll
        for (int i = 0; i < S::SM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bcur, acc[i][j], 0, 0, 0, ea[i], 0, eb);
        bcur = bnext;
      }
    };
    for (int i0 = 0; i0 < kbs; i0 += NSLOT) {
      static_for<NSLOT>([&](auto u_const) {
        if (i0 + decltype(u_const)::value < kbs) {
          bare_barrier();                       // block i0+u has landed in slot u
          compute(u_const);
        }
      });
    }
    // every fragment read has returned (the MFMAs consumed them); release the ring
    bare_barrier();

    // epilogue: + C, round to bf16, store the rows that belong to the result,
    // one element at a time in accumulator order
#pragma unroll
    for (int i = 0; i < S::SM; ++i)
#pragma unroll
      for (int j = 0; j < S::SN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + wrow0 + i * 16 + g16 * 4 + e;
          const int col = n0 + wcol0 + j * 16 + r16;
          float v = acc[i][j][e];
          if (C) v += bf16_to_f32(C[(size_t)min(row, p.rows - 1) * p.N + min(col, p.N - 1)]);
          if (row < rows_lim && col < p.N &&
              (MODE != kContiguous || p.layout[min(row, p.rows - 1)] == group))
            D[(size_t)row * p.N + col] = f32_to_bf16(v);
        }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int NSLOT>
hipError_t launch_ws(int mode, const Params& p, int grid, hipStream_t stream) {
  constexpr int threads = 2 * WAVES_M * WAVES_N * 64;
  switch (mode) {
    case kDense:
      hipLaunchKernelGGL((fp8_gemm_nt_ws_kernel<BM, BN, WAVES_M, WAVES_N, NSLOT, kDense>), dim3(grid), dim3(threads),
                         0, stream, p);
      break;
    case kContiguous:
      hipLaunchKernelGGL((fp8_gemm_nt_ws_kernel<BM, BN, WAVES_M, WAVES_N, NSLOT, kContiguous>), dim3(grid),
                         dim3(threads), 0, stream, p);
      break;
    case kMasked:
      hipLaunchKernelGGL((fp8_gemm_nt_ws_kernel<BM, BN, WAVES_M, WAVES_N, NSLOT, kMasked>), dim3(grid), dim3(threads),
                         0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}


template <int BM, int BN, int WAVES_M, int WAVES_N, int NSLOT>
hipError_t launch_e8(int mode, const Params& p, int grid, hipStream_t stream) {
  constexpr int threads = WAVES_M * WAVES_N * 64;
  static_assert(threads == 256 || threads == 512, "four or eight waves");
  switch (mode) {
    case kDense:
      hipLaunchKernelGGL((fp8_gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, NSLOT, kDense, 1, true>), dim3(grid),
                         dim3(threads), 0, stream, p);
      break;
    case kContiguous:
      hipLaunchKernelGGL((fp8_gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, NSLOT, kContiguous, 1, true>), dim3(grid),
                         dim3(threads), 0, stream, p);
      break;
    case kMasked:
      hipLaunchKernelGGL((fp8_gemm_nt_kernel<BM, BN, WAVES_M, WAVES_N, NSLOT, kMasked, 1, true>), dim3(grid),
                         dim3(threads), 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// One verdict per workgroup: 1 if every scale the workgroup looked at is a
// positive normal power of two (fp32 mantissa zero, biased exponent 1..254,
// which is then exactly the scale's E8M0 code), else 0.  Zero, negative,
// subnormal, non-power-of-two and non-finite scales all fail.  Every
// workgroup writes its verdict, so the buffer needs no clearing.  Scales are
// read 16 bytes per lane where the array is 16-byte aligned, with four loads
// in flight per lane.
__device__ __forceinline__ bool e8m0_exact(uint32_t bits) {
  const uint32_t ex = bits >> 23;     // the sign bit is included: negative values fail
  return (bits & 0x7FFFFFu) == 0 && ex >= 1 && ex <= 254;
}

__device__ __forceinline__ bool check_scales(const float* __restrict__ s, size_t n) {
  bool good = true;
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nthreads = (size_t)gridDim.x * blockDim.x;
  size_t head = 0;
  if ((reinterpret_cast<uintptr_t>(s) & 15) == 0) {
    const size_t n4 = n / 4;
    const float4* s4 = reinterpret_cast<const float4*>(s);
    size_t i = tid;
    for (; i + 3 * nthreads < n4; i += 4 * nthreads) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = s4[i + u * nthreads];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        good = good && e8m0_exact(__float_as_uint(v[u].x)) && e8m0_exact(__float_as_uint(v[u].y)) &&
               e8m0_exact(__float_as_uint(v[u].z)) && e8m0_exact(__float_as_uint(v[u].w));
    }
    for (; i < n4; i += nthreads) {
      const float4 v = s4[i];
      good = good && e8m0_exact(__float_as_uint(v.x)) && e8m0_exact(__float_as_uint(v.y)) &&
             e8m0_exact(__float_as_uint(v.z)) && e8m0_exact(__float_as_uint(v.w));
    }
    head = n4 * 4;
  }
  for (size_t i = head + tid; i < n; i += nthreads) good = good && e8m0_exact(__float_as_uint(s[i]));
  return good;
}

__global__ void __launch_bounds__(256) scale_check_kernel(const float* __restrict__ sfa, size_t na,
                                                          const float* __restrict__ sfb, size_t nb,
                                                          int32_t* __restrict__ verdicts) {
  const bool good = check_scales(sfa, na) && check_scales(sfb, nb);
  const int all = __syncthreads_and(good ? 1 : 0);
  if (threadIdx.x == 0) verdicts[blockIdx.x] = all ? 1 : 0;
}

}  // namespace

hipError_t launch_scale_check(const float* sfa, size_t na, const float* sfb, size_t nb, int32_t* verdicts,
                              hipStream_t stream) {
  hipLaunchKernelGGL(scale_check_kernel, dim3(kCheckWGs), dim3(256), 0, stream, sfa, na, sfb, nb, verdicts);
  return hipGetLastError();
}

hipError_t launch_gemm_e8m0(int mode, int cfg, const Params& p, int grid, hipStream_t stream) {
  switch (cfg) {
    case kCfgE8_128x256: return launch_e8<128, 256, 2, 2, 3>(mode, p, grid, stream);
    case kCfgE8_256x256: return launch_e8<256, 256, 2, 4, 2>(mode, p, grid, stream);
    case kCfgWs_128x256: return launch_ws<128, 256, 2, 2, 3>(mode, p, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dg
