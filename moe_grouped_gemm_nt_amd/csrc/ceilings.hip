// Microbenchmarks of the two ceilings the GEMM kernels run into on gfx950:
// the FP8 MFMA issue rate (operands already in registers) and the rate at
// which workgroups pull bytes from memory, with the load forms the kernels
// use.  Also an empty kernel, for the cost of one launch.  Built into its own
// library (libdg_ceilings.so); nothing of the GEMM path depends on it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dg_ceilings.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void*)(p));
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 64 lanes x 16 bytes straight into LDS (lane l's bytes at m0 + 16*l)
__device__ __forceinline__ void dma_16(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Each workgroup (four waves) reads bytes_per_wg consecutive bytes starting at
// src + blockIdx.x * bytes_per_wg; wave w reads the w-th quarter, 1 KB per
// load instruction, at most INFLIGHT loads outstanding.  DIRECT: global->LDS
// loads into a private ring of INFLIGHT+1 one-KB slots per wave (no slot is
// the target of two loads in flight); otherwise 16-byte loads into VGPRs,
// folded into one word so that none is dead.
template <bool DIRECT, int INFLIGHT>
__global__ void __launch_bounds__(256) stream_kernel(const uint8_t* __restrict__ src, long bytes_per_wg,
                                                     int* __restrict__ sink) {
  constexpr int RING = INFLIGHT + 1;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[DIRECT ? 4 * RING * 1024 : 4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long quarter = bytes_per_wg / 4;
  const int n = (int)(quarter / 1024);
  const uint8_t* base = src + (long)blockIdx.x * bytes_per_wg + (long)wave * quarter + lane * 16;
  if constexpr (DIRECT) {
    const uint32_t r0 = lds_addr(ring) + (uint32_t)(wave * RING * 1024);
    int i = 0;
    for (; i < n && i < INFLIGHT; ++i) dma_16(base + (long)i * 1024, r0 + (uint32_t)(i % RING) * 1024);
    for (; i < n; ++i) {
      wait_vm<INFLIGHT - 1>();
      dma_16(base + (long)i * 1024, r0 + (uint32_t)(i % RING) * 1024);
    }
    wait_vm<0>();
    if (threadIdx.x == 0) sink[blockIdx.x] = n;
  } else {
    v4i acc = {0, 0, 0, 0};
    int i = 0;
    for (; i + INFLIGHT <= n; i += INFLIGHT) {
      v4i v[INFLIGHT];
#pragma unroll
      for (int u = 0; u < INFLIGHT; ++u) v[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(base + (long)(i + u) * 1024));
#pragma unroll
      for (int u = 0; u < INFLIGHT; ++u) acc ^= v[u];
    }
    for (; i < n; ++i) acc ^= __builtin_nontemporal_load(reinterpret_cast<const v4i*>(base + (long)i * 1024));
    const int x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x7fffffff) sink[blockIdx.x] = x;   // practically never taken; keeps the loads live
  }
}

// 256 workgroups of eight waves, the tile kernels' shape.  The workgroups of
// one XCD (blockIdx % 8) form groups of `share` (32 / share groups per XCD);
// group g reads the `steps` 64 KB blocks at src + g * group_bytes, each block
// 64 direct global->LDS loads of 1 KB spread over the waves (8 each), 8
// loads in flight per wave and no barrier: with share > 1 most of the bytes
// come from the L2, which the group's workgroups share as a tile kernel's
// workgroups share A and B rows.
__global__ void __launch_bounds__(512) fill_kernel(const uint8_t* __restrict__ src, long group_bytes, int steps,
                                                   int share, int* __restrict__ sink) {
  constexpr int INFL = 8, RING = INFL + 1;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[8 * RING * 1024];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = (blockIdx.x % 8) * (32 / share) + (blockIdx.x / 8) / share;
  const uint8_t* base = src + (long)group * group_bytes + lane * 16;
  const uint32_t r0 = lds_addr(ring) + (uint32_t)(wave * RING * 1024);
  const int n = steps * 8;
  auto addr = [&](int i) { return base + (long)((i / 8) * 64 + wave * 8 + i % 8) * 1024; };
  int i = 0;
  for (; i < n && i < INFL; ++i) dma_16(addr(i), r0 + (uint32_t)(i % RING) * 1024);
  for (; i < n; ++i) {
    wait_vm<INFL - 1>();
    dma_16(addr(i), r0 + (uint32_t)(i % RING) * 1024);
  }
  wait_vm<0>();
  if (threadIdx.x == 0) sink[blockIdx.x] = n;
}

__global__ void __launch_bounds__(256) empty_kernel() {}

// Back-to-back 16x16x128 FP8 MFMAs on register operands, eight independent
// accumulators per wave.  PROMOTE: each MFMA starts from zero and its result is
// folded into the total with one fp32 FMA per element, as the general-scale
// GEMM kernels do.
template <bool PROMOTE>
__global__ void __launch_bounds__(256) mfma_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const v8i a = {lane * 0x01010101, 0x38383838, lane, 0x30303030, 0x3c3c3c3c, lane ^ 5, 0x34343434, 0x3a3a3a3a};
  const v8i b0 = {0x38383838, lane * 0x01000100, 0x36363636, lane, 0x3c3c3c3c, 0x32323232, lane ^ 9, 0x38383838};
  // a different B operand per chain, so that no two MFMAs compute the same thing
  v8i b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = b0 ^ (v8i){j, j << 8, j, j << 16, j, j << 8, j, j << 24};
  v4f acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = (v4f){0.f, 0.f, 0.f, 0.f};
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  const float f = 0.5f + 0.001f * lane;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (PROMOTE) {
        const v4f q = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[j], zero, 0, 0, 0, 0, 0, 0);
        acc[j].x = __builtin_fmaf(q.x, f, acc[j].x);
        acc[j].y = __builtin_fmaf(q.y, f, acc[j].y);
        acc[j].z = __builtin_fmaf(q.z, f, acc[j].z);
        acc[j].w = __builtin_fmaf(q.w, f, acc[j].w);
      } else {
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[j], acc[j], 0, 0, 0, 0, 0, 0);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j].x + acc[j].y + acc[j].z + acc[j].w;
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// One lane issues `iters` dependent memory operations, each waiting for the
// one before: the round-trip latency of that kind of access.  mode 0: device-
// scope atomic add on ring[0]; 1: pointer chase x = ring[x] with device-
// coherent loads (sc1); 2: the same chase with plain vector loads.  The chase
// starts at state[0] and leaves its last index there, so that successive
// launches walk on along the chain rather than over lines already cached; the
// caller fills `ring` (every entry an index inside it), and with it chooses
// the footprint and so the level of the memory hierarchy that answers.  The
// loads are written as asm that waits for its own result, so that they stay
// vector loads (a uniform address would otherwise become a scalar load).
__global__ void __launch_bounds__(64) chase_kernel(int* __restrict__ ring, int iters, int mode,
                                                   int* __restrict__ state) {
  if (threadIdx.x != 0) return;
  int x = state[0];
  if (mode == 0) {
    for (int i = 0; i < iters; ++i) x += __hip_atomic_fetch_add(ring, 1 + (x & 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (mode == 1) {
    for (int i = 0; i < iters; ++i)
      asm volatile("global_load_dword %0, %1, off sc1\n\ts_waitcnt vmcnt(0)" : "=v"(x) : "v"(ring + x) : "memory");
  } else {
    for (int i = 0; i < iters; ++i)
      asm volatile("global_load_dword %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(x) : "v"(ring + x) : "memory");
  }
  state[0] = mode == 0 ? 0 : x;
}

}  // namespace

extern "C" int dgc_stream(const void* src, long bytes_per_wg, int grid, int mode, int* sink, void* stream) {
  if (!src || !sink || grid < 1 || bytes_per_wg < 4096 || bytes_per_wg % 4096 != 0 || mode < 0 || mode > 3)
    return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* p = static_cast<const uint8_t*>(src);
  switch (mode) {
    case 0: hipLaunchKernelGGL((stream_kernel<true, 15>), dim3(grid), dim3(256), 0, s, p, bytes_per_wg, sink); break;
    case 1: hipLaunchKernelGGL((stream_kernel<true, 31>), dim3(grid), dim3(256), 0, s, p, bytes_per_wg, sink); break;
    case 2: hipLaunchKernelGGL((stream_kernel<false, 8>), dim3(grid), dim3(256), 0, s, p, bytes_per_wg, sink); break;
    case 3: hipLaunchKernelGGL((stream_kernel<false, 16>), dim3(grid), dim3(256), 0, s, p, bytes_per_wg, sink); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int dgc_fill(const void* src, long group_bytes, int steps, int share, int* sink, void* stream) {
  if (!src || !sink || steps < 1 || share < 1 || share > 32 || 32 % share != 0 ||
      (long)steps * 65536 > group_bytes)
    return -1;
  hipLaunchKernelGGL(fill_kernel, dim3(256), dim3(512), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(src), group_bytes, steps, share, sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int dgc_empty(int grid, void* stream) {
  if (grid < 1) return -1;
  hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int dgc_mfma(int iters, int grid, int promote, float* sink, void* stream) {
  if (!sink || grid < 1 || iters < 1) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (promote)
    hipLaunchKernelGGL(mfma_kernel<true>, dim3(grid), dim3(256), 0, s, iters, sink);
  else
    hipLaunchKernelGGL(mfma_kernel<false>, dim3(grid), dim3(256), 0, s, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int dgc_chase(int* ring, int iters, int mode, int* state, void* stream) {
  if (!ring || !state || iters < 1 || mode < 0 || mode > 2) return -1;
  hipLaunchKernelGGL(chase_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), ring, iters, mode, state);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
