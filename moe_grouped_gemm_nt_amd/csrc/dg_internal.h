// Internal interface between the host entry points (dg_api.hip) and the
// gfx950 kernels (fp8_gemm.hip).  Not installed, not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// kKGrouped: groups along K (each group's tokens), both operands K-major, fp32 D.
enum Mode : int { kDense = 0, kContiguous = 1, kMasked = 2, kKGrouped = 3 };

// Everything one launch needs.  Row counts and strides are in elements.
struct Params {
  const uint8_t* a;        // e4m3 codes
  const float* sfa;        // [KB][rows] (masked: [G][KB][max_m])
  const uint8_t* b;        // e4m3 codes [N][K] (grouped: [G][N][K])
  const float* sfb;        // [NB][KB] (grouped: [G][NB][KB])
  const uint16_t* c;       // bf16 bits or nullptr
  uint16_t* d;             // bf16 bits
  const int32_t* layout;   // contiguous: expert id per row
  const int32_t* masked_m; // masked: valid rows per group
  float* workspace;        // split-K partial tiles (fp32)
  size_t workspace_bytes;
  const int32_t* gate_ok;  // scale check verdicts (kernel path gate), or nullptr for no gate
  int rows;                // dense/contiguous: M; masked: max_m
  int N;
  int K;
  int G;                   // groups (1 for dense)
  int tiles_m;             // ceil(rows / BM)
  int tiles_n;             // ceil(N / BN)
  int splits;              // split-K factor (>= 1; decode kernel only)
  int kbs_per_split;       // K blocks per split (decode kernel only)
  int ab_layout;           // dense: bit 0 = A stored [K][M], bit 1 = B stored [K][N] (0 = nt),
                           // 4 = B packed FP4 (E2M1) with E8M0 scales, sfb int32 [K/128][N]
  int sk_splits;           // tile kernels: > 1 splits each XCD's tail items over K into this many parts
  int sk_tail;             // tail items per XCD reserved in the workspace (partial index stride)
  int k_window;            // tile kernels: K blocks taken in aligned windows of this many (a power of
                           // two; <= 1 = in order), each tile at its own offset in every window
  float* d32;              // K-grouped: fp32 D [G][M][N]
  const float* c32;        // K-grouped: fp32 C [G][M][N] or nullptr
  int* sync;               // one-launch decode: kSyncInts counters, zero before and after every call
};

// Counters of the one-launch decode kernel: kSyncTile0 reserved, then one per
// 64x64 tile.
constexpr int kSyncInts = 1024;
constexpr int kSyncTile0 = 16;
constexpr int kSyncMaxTiles = kSyncInts - kSyncTile0;

// The K-grouped form carries its groups' K offsets in the launch arguments,
// so a captured graph replays with the offsets of the captured call.
constexpr int kMaxKGroups = 256;
struct KGroupedParams : Params {
  int k_start[kMaxKGroups + 1];   // group g owns K rows k_start[g] .. k_start[g+1]-1 (multiples of 128)
};

// Tile configurations compiled into the library.
enum Config : int {
  kCfg128x128 = 0,   // 128x128 tile, 4 waves of 64x64, 4-slot ring: large GEMMs
  kCfgDecode = 1,    // dense only: 64x64 tile, K split over workgroups (<= 8 blocks each) and waves
  kCfg128x64 = 2,    // 128x64 tile, 4 waves of 64x32, 4-slot ring
  kCfg64x128 = 3,    // 64x128 tile, 4 waves of 64x32, 4-slot ring
  kCfg128x128x2 = 4, // 128x128 tile, 2-slot ring, two workgroups per CU
  kCfg256x128w8 = 5, // 256x128 tile, 8 waves of 64x64, 3-slot ring
  kCfg128x256w8 = 6, // 128x256 tile, 8 waves of 64x64, 3-slot ring
  kCfgE8_128x256 = 7, // power-of-two scales only: 128x256 tile, 4 waves of 64x128, 3-slot ring
  kCfgWs_128x256 = 8, // power-of-two scales only: as 7 plus 4 loader waves (wave-specialised)
  kCfgNarrow = 9,     // dense only: 16x48 tile over the whole K, per-wave LDS rings, no split-K
  kCfgE8_256x256 = 10, // power-of-two scales only: 256x256 tile, 8 waves of 128x64, 2-slot ring
  kCfg256x256w8 = 11, // 256x256 tile, 8 waves of 128x64, 2-slot ring (fp32 promotion)
  kCfgDecodeFused = 12, // dense only: the decode tile with the split-K hand-off inside the launch
  kNumConfigs
};

struct ConfigInfo {
  int bm, bn, threads;
  const char* name;
};

const ConfigInfo& config_info(int cfg);

// Enqueues the kernel(s) for `mode` with configuration `cfg` on `stream`.
// `grid` is the number of workgroups of the tile kernel, which walks its tiles
// persistently when grid is smaller than the tile count; the decode
// configuration sizes its own grid from tiles and splits.
hipError_t launch_gemm(int mode, int cfg, const Params& p, int grid, hipStream_t stream);
// Sums the split-tail partial tiles of a tile-kernel launch (p.sk_splits > 1)
// into D; grid is the tile kernel's grid.
hipError_t launch_tile_reduce(int mode, int cfg, const Params& p, int grid, hipStream_t stream);
// K-grouped TN launch on configuration cfg (128x128, 128x256 or 256x256 tiles).
hipError_t launch_kgrouped(int cfg, const KGroupedParams& p, int grid, hipStream_t stream);

// Power-of-two-scale kernels (fp8_gemm_e8m0.hip).  Launched with a gate
// (Params::gate_ok) after launch_scale_check, beside the general kernel with
// the same gate: exactly one of the two does the work.
hipError_t launch_gemm_e8m0(int mode, int cfg, const Params& p, int grid, hipStream_t stream);

// Writes kCheckWGs verdicts (int32, 1 = every scale in sfa[0..na) and
// sfb[0..nb) is a positive normal power of two).
constexpr int kCheckWGs = 64;
hipError_t launch_scale_check(const float* sfa, size_t na, const float* sfb, size_t nb, int32_t* verdicts,
                              hipStream_t stream);

}  // namespace dg
