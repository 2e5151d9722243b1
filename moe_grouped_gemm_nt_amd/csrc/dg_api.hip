// Host side of the C ABI declared in include/dg.h: argument validation,
// launch-configuration choice, per-device state and error reporting.
//
// Configuration choice (the pages' host heuristics pick a kernel layout and
// launch shape per problem; prefill and decode shapes get different kernels,
// zwt0204 DeepGEMM deep dive, "它的核心思路" point 2):
//   * dense NT shapes with at most 16 rows take the narrow kernel (16x48 tiles
//     over the whole K, one launch) when its tiles occupy at least half the
//     CUs or K is at most 16 blocks;
//   * dense shapes (any operand storage, FP8 or FP4 B) with fewer 128x128
//     tiles than half the CUs take the 64x64 decode tile with K split across
//     workgroups (one split up to 8 K blocks, else enough splits of 4 to 8
//     blocks to fill the chip) and a split-K reduction kernel, as long as the
//     splits fit in about two rounds of the chip and in the workspace;
//   * otherwise the fp32-promotion tile kernel: dense, contiguous and
//     K-grouped calls take the tile (256x256, 128x256 or 128x128) that
//     minimises the rounds of the chip times the rows loaded per K block
//     (128-row tiles for contiguous calls), and where 128x128 and 128x256
//     both fit in one round, an estimate of the split tail's loads and fp32
//     partials decides between them; masked calls the largest tile that
//     still gives every CU one, counting m-tiles per group; 128x256 rather
//     than 256x256 when the call has a C; a last partial round of items is
//     split over K where the tile allows (the split tail); dense and
//     K-grouped items on the 256x256 tile take their K blocks in windows of 4
//     (k_window_for);
//   * the power-of-two kernels (scales applied inside the MFMA) are selected
//     with DG_FORCE_CONFIG; they run behind a scale check that leaves its
//     verdicts on the device, beside the general kernel, and exactly one of
//     the two does the work.  On this hardware these shapes are bound by the
//     loads, not the promotion, so they are not the default.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dg.h"
#include "dg_internal.h"

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

constexpr int kMaxDevices = 64;
constexpr size_t kWorkspaceBytes = size_t(64) << 20;    // split-K partial tiles

// Control memory of a call besides its split-K partials: the scale-check
// verdicts, then the one-launch decode kernel's counters (zero at set-up; every
// call of that kernel leaves them at zero).
constexpr size_t kVerdictBytes = 256;
constexpr size_t kSyncBytes = sizeof(int32_t) * dg::kSyncInts;
static_assert(dg::kCheckWGs * sizeof(int32_t) <= kVerdictBytes, "verdicts fit their area");

struct DeviceState {
  std::atomic<bool> ready{false};   // set once, with release order, after the fields below
  int num_cus = 0;
  float* workspace = nullptr;
  int32_t* verdicts = nullptr;    // scale check results, dg::kCheckWGs entries
  int32_t* sync = nullptr;        // dg::kSyncInts counters
};

DeviceState g_dev[kMaxDevices];

std::mutex g_mu;

int get_device_state(DeviceState** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DG_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DG_ERR_UNSUPPORTED, "device index %d out of range", dev);
  DeviceState& st = g_dev[dev];
  if (!st.ready.load(std::memory_order_acquire)) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!st.ready.load(std::memory_order_relaxed)) {
      hipDeviceProp_t prop;
      e = hipGetDeviceProperties(&prop, dev);
      if (e != hipSuccess) return fail(DG_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
      if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(DG_ERR_UNSUPPORTED, "device %d is %s; the kernels are built for gfx950 only", dev, prop.gcnArchName);
      float* ws = nullptr;
      int32_t* verdicts = nullptr;
      e = hipMalloc(&ws, kWorkspaceBytes);
      if (e != hipSuccess) return fail(DG_ERR_HIP, "hipMalloc(workspace): %s", hipGetErrorString(e));
      e = hipMalloc(&verdicts, kVerdictBytes + kSyncBytes);
      if (e == hipSuccess) e = hipMemset(verdicts, 0, kVerdictBytes + kSyncBytes);
      if (e == hipSuccess) e = hipDeviceSynchronize();
      if (e != hipSuccess) {
        // nothing is kept from a failed set-up; the next call tries again
        (void)hipFree(ws);
        if (verdicts) (void)hipFree(verdicts);
        return fail(DG_ERR_HIP, "control memory set-up: %s", hipGetErrorString(e));
      }
      st.num_cus = prop.multiProcessorCount;
      st.workspace = ws;
      st.verdicts = verdicts;
      st.sync = verdicts + kVerdictBytes / sizeof(int32_t);
      st.ready.store(true, std::memory_order_release);
    }
  }
  *out = &st;
  return DG_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_common(const void* a, const float* sfa, const void* b, const float* sfb, const void* c,
                 void* d, int M, int N, int K) {
  if (!a || !sfa || !b || !sfb || !d) return fail(DG_ERR_INVALID_ARG, "a, sfa, b, sfb and d must not be NULL");
  if (M < 0 || N < 0 || K < 0) return fail(DG_ERR_INVALID_ARG, "negative size (M=%d N=%d K=%d)", M, N, K);
  if (K % 128 != 0) return fail(DG_ERR_INVALID_ARG, "K=%d is not a multiple of 128", K);
  if (!aligned(a, 16) || !aligned(b, 16)) return fail(DG_ERR_INVALID_ARG, "a and b must be 16-byte aligned");
  if (!aligned(sfa, 4) || !aligned(sfb, 4)) return fail(DG_ERR_INVALID_ARG, "sfa and sfb must be 4-byte aligned");
  if (!aligned(d, 2) || (c && !aligned(c, 2))) return fail(DG_ERR_INVALID_ARG, "c and d must be 2-byte aligned");
  return DG_OK;
}

// The contiguous layout's contract on host data: in every aligned block of
// 128 rows, all rows whose id lies in [0, G) carry the same id.
int check_layout_host(const int32_t* layout, int M, int G) {
  for (int b = 0; b * 128 < M; ++b) {
    int id = -1;
    for (int r = b * 128; r < M && r < (b + 1) * 128; ++r) {
      const int v = layout[r];
      if (v < 0 || v >= G) continue;
      if (id >= 0 && v != id)
        return fail(DG_ERR_INVALID_ARG,
                    "grouped_layout: rows %d..%d (one 128-row block) hold experts %d and %d; a block may hold one",
                    b * 128, std::min(M, (b + 1) * 128) - 1, id, v);
      id = v;
    }
  }
  return DG_OK;
}

// DG_VALIDATE=1: copies device control data to the host (on the call's
// stream, then waits for it) and checks it before anything is launched.  A
// debugging aid: it synchronises, so it is skipped while the stream is being
// captured into a graph.
bool validate_on(hipStream_t stream) {
  const char* v = std::getenv("DG_VALIDATE");
  if (!v || !*v || *v == '0') return false;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return false;
  return cs == hipStreamCaptureStatusNone;
}

int copy_to_host(std::vector<int32_t>& dst, const int32_t* src, int n, hipStream_t stream) {
  dst.assign((size_t)n, 0);
  hipError_t e = hipMemcpyAsync(dst.data(), src, sizeof(int32_t) * (size_t)n, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(DG_ERR_HIP, "DG_VALIDATE: reading device data: %s", hipGetErrorString(e));
  return DG_OK;
}

int validate_layout(const int32_t* layout, int M, int G, hipStream_t stream) {
  if (!validate_on(stream)) return DG_OK;
  std::vector<int32_t> h;
  int s = copy_to_host(h, layout, M, stream);
  return s != DG_OK ? s : check_layout_host(h.data(), M, G);
}

int validate_masked(const int32_t* masked_m, int G, int max_m, hipStream_t stream) {
  if (!validate_on(stream)) return DG_OK;
  std::vector<int32_t> h;
  int s = copy_to_host(h, masked_m, G, stream);
  if (s != DG_OK) return s;
  for (int g = 0; g < G; ++g)
    if (h[g] < 0 || h[g] > max_m)
      return fail(DG_ERR_INVALID_ARG, "masked_m[%d] = %d lies outside [0, max_m = %d] (the kernels would clamp it)", g,
                  h[g], max_m);
  return DG_OK;
}

struct Choice {
  int cfg;
  int splits;
  int kbs;        // K blocks per split (decode configuration)
  int gated_cfg;  // >= 0: power-of-two kernel run beside cfg behind the scale check
};

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  return v && *v ? std::atoi(v) : dflt;
}

// K-block window of the tile kernels (Params::k_window).  Dense and K-grouped
// items on the 256x256 tile take their K blocks in windows of 4, each tile at
// its own offset in the window: measured 2% faster on the 4096x7168x16384 NT
// prefill problem, 5-7% with K-major operands and on the K-grouped problem,
// 4-5% at 2048x7168x7168 and 8192^3.  The smaller tiles keep the plain order
// (128x128 measured 2-4% slower with windows, 128x256 within 1.3% either way),
// and so do the M-grouped forms (contiguous 1% slower, masked no faster).
// DG_K_WINDOW sets the window of every dense and K-grouped tile (1 = plain
// order; a power of two up to 16).
int k_window_for(int mode, int cfg) {
  if (mode != dg::kDense && mode != dg::kKGrouped) return 1;
  const int w = env_int("DG_K_WINDOW", 0);
  if (w >= 1 && w <= 16 && (w & (w - 1)) == 0) return w;
  return cfg == dg::kCfg256x256w8 ? 4 : 1;
}

// The decode kernel runs one workgroup per CU; with a long K its splits (at
// most 8 K blocks each) can need several rounds of the chip, and measured
// beyond about two and a quarter rounds the tile kernels (with their split
// tail) were faster.  Its fp32 partials must also fit the workspace.
bool decode_fits(long long tiles64, int KB, int num_cus, size_t ws_bytes) {
  const long long wgs = tiles64 * ((KB + 7) / 8);
  return wgs <= 2LL * num_cus + num_cus / 4 && wgs * 64 * 64 * (long long)sizeof(float) <= (long long)ws_bytes;
}

// Estimated time (µs) of a call whose tiles all fit in one round of the chip,
// with the split tail of plan_split_tail: each CU loads (BM+BN) rows of 128
// bytes for each of its KB/sk K blocks at the per-CU rate the tile kernels
// measure (about 35 GB/s with the split tail, 40 GB/s without, when some CUs
// stay idle), and the sk fp32 partial tiles are written and read back at
// about 5 TB/s.
double split_tail_us(long long tiles, int bm, int bn, int KB, int num_cus, size_t ws_bytes) {
  const long long slots = num_cus / 8;
  const long long tail = (tiles + 7) / 8;        // items of the fullest XCD
  long long sk = tail > 0 ? slots / tail : 1;
  sk = std::min<long long>({sk, 16, (long long)KB});
  while (sk > 1 && 8 * tail * sk * bm * bn * (long long)sizeof(float) > (long long)ws_bytes) --sk;
  if (sk < 2) sk = 1;
  const double load = (double)KB / (double)sk * (bm + bn) * 128.0 / (sk > 1 ? 35e3 : 40e3);
  const double partials = sk > 1 ? 2.0 * (double)sk * tiles * bm * bn * sizeof(float) / 5e6 : 0.0;
  return load + partials;
}

// rows: rows computed per group (dense: M; contiguous: M; masked: expected rows per group)
// ab_layout: 0 nt; 1-3 a K-major operand (tt, nn, tn); 4 an FP4 B.  The
// other layouts are read by the 128x128, 128x256 and 256x256 tile kernels and
// the decode kernel only.
// ws_bytes: the split-K workspace the call may use.
Choice choose(int mode, int rows, int N, int K, int groups, int num_cus, int ab_layout, size_t ws_bytes) {
  Choice ch{dg::kCfg128x128x2, 1, 0, -1};
  const bool kmajor = ab_layout != 0;
  const int KB = K / 128;
  const long long tiles128 = (long long)((rows + 127) / 128) * ((N + 127) / 128);
  if (!kmajor && mode == dg::kDense && rows <= 16 && KB > 0 && ((N + 47) / 48 >= num_cus / 2 || KB <= 16)) {
    // one 16-row strip and enough 16x48 tiles to occupy half the chip, or a
    // K short enough that one launch beats a split and its reduction (1 or 16
    // rows, N 2112, K 2048: 4.4-4.9 us against 7.2-7.5): whole-K tiles, one
    // launch, nothing crosses workgroups
    ch.cfg = dg::kCfgNarrow;
  } else if (mode == dg::kDense && KB > 0 && 2 * tiles128 < num_cus &&
             decode_fits(((long long)(rows + 63) / 64) * ((N + 63) / 64), KB, num_cus, ws_bytes)) {
    // too few tiles to occupy half the chip (decode shapes): 64x64 tiles; split
    // K so that the workgroups fill the chip while each split keeps at most 8
    // K blocks, all of them in flight at once, and at least 4
    ch.cfg = dg::kCfgDecode;
    const int tiles = ((rows + 63) / 64) * ((N + 63) / 64);
    int splits = (KB + 7) / 8;
    const int fill = num_cus / (tiles > 0 ? tiles : 1);
    // up to 8 K blocks one split does the call in one launch, which measured
    // faster than any split count (the reduction is a second launch); beyond,
    // splits of fewer than 4 blocks measured slower than fewer, longer ones
    // (the partials to reduce grow with the split count)
    const int cap = KB / 4;
    if (KB > 8 && fill > splits) splits = fill < cap ? fill : cap;
    ch.splits = splits;
  } else {
    // Tile kernels: per K block a CU loads (BM+BN)*128 bytes for BM*BN/256
    // MFMAs, and the loads bound these kernels, so bigger tiles run faster.
    // Contiguous calls stay at 128-row tiles: a 256-row tile that spans two
    // experts' segments runs once per expert, and on the measured expert
    // mixes that costs more than the larger tile saves.  Masked calls take the
    // largest tile that still gives every CU a tile (128x128 below that, with
    // the deepest ring): every group rounds up to its own m-tiles, and groups
    // expected to hold fewer than 128 rows keep 128-row tiles (measured on
    // 32 groups of 4-64 rows: 128x256 tiles 4-5% faster than the others).
    const bool masked = mode == dg::kMasked;
    const long long g = masked ? groups : 1;
    const long long tiles256 = g * (((long long)rows + 255) / 256) * ((N + 255) / 256);
    const long long tiles128x256 = g * (((long long)rows + 127) / 128) * ((N + 255) / 256);
    if (mode == dg::kDense || mode == dg::kContiguous) {
      // Dense and contiguous: the tiles are bound by the bytes each CU loads per K block,
      // BM+BN rows of 128 bytes, so a call costs about its rounds of the chip
      // times that; a partial round of large tiles beats more rounds of small
      // ones (measured on 256-2048 x 2112-7168 x 7168: within 5% of the best
      // forced configuration, where filling every CU first cost up to 1.4x).
      const long long tiles128 = (((long long)rows + 127) / 128) * ((N + 127) / 128);
      auto cost = [&](long long tiles, int edge) { return ((tiles + num_cus - 1) / num_cus) * edge; };
      const long long c256 = cost(tiles256, 512), c128x256 = cost(tiles128x256, 384), c128 = cost(tiles128, 256);
      // (contiguous calls keep 128-row tiles: see above)
      if (mode == dg::kDense && c256 <= c128x256 && c256 <= c128) ch.cfg = dg::kCfg256x256w8;
      else if (tiles128 <= num_cus && KB > 0)
        // one round either way: the split tail divides K over the idle CUs,
        // so the larger tile's fewer bytes per output count against its larger
        // partials.  The larger tile is taken only when the estimate gives it
        // a 5% margin: closer than that the measured order went either way,
        // while beyond it the larger tile measured faster (128x256 against
        // 128x128: 1024x2112x7168 38.7 against 43.0 us, 384x4096x16384 46.7
        // against 54.3, 512x4096x16384 57.3 against 59.2).
        ch.cfg = split_tail_us(tiles128x256, 128, 256, KB, num_cus, ws_bytes) <
                         0.95 * split_tail_us(tiles128, 128, 128, KB, num_cus, ws_bytes)
                     ? dg::kCfg128x256w8 : dg::kCfg128x128;
      else if (c128x256 <= c128) ch.cfg = dg::kCfg128x256w8;
      else ch.cfg = dg::kCfg128x128;
    } else if (mode != dg::kContiguous && !(masked && rows < 128) && tiles256 >= num_cus) {
      // masked groups of 128 to 191 expected rows: 256x128 tiles (three
      // K blocks in the ring instead of two, and rows idle in 64-row wave
      // rows past a group's end) measured 4% faster than 256x256 at 32
      // groups of 0-256 rows (N 4096, K 7168), the same at 128-256 rows, and
      // slower for larger groups (FP8 B only: no FP4 build of that tile)
      const long long tiles256x128 = g * (((long long)rows + 255) / 256) * ((N + 127) / 128);
      ch.cfg = masked && rows < 192 && ab_layout == 0 && tiles256x128 >= num_cus ? dg::kCfg256x128w8
                                                                                    : dg::kCfg256x256w8;
    } else if (tiles128x256 >= num_cus) {
      ch.cfg = dg::kCfg128x256w8;
    } else {
      ch.cfg = dg::kCfg128x128;
    }
  }
  // DG_FORCE_CONFIG picks a configuration; a power-of-two one runs behind the
  // scale check, beside the general 128x128 kernel.
  const int forced = env_int("DG_FORCE_CONFIG", -1);
  const bool forced_decode = forced == dg::kCfgDecode || forced == dg::kCfgDecodeFused;
  const bool forced_ok = !kmajor || forced == dg::kCfg128x128 || forced == dg::kCfg128x256w8 ||
                         forced == dg::kCfg256x256w8 || forced_decode;
  // (the decode and narrow kernels are dense-only and need a K block: with
  // K = 0 a forced choice of them is ignored)
  if (forced >= 0 && forced < dg::kNumConfigs && forced_ok &&
      ((!forced_decode && forced != dg::kCfgNarrow) || (mode == dg::kDense && KB > 0))) {
    if (forced == dg::kCfgE8_128x256 || forced == dg::kCfgWs_128x256 || forced == dg::kCfgE8_256x256) {
      ch.cfg = dg::kCfg128x128x2;
      ch.gated_cfg = forced;
    } else {
      ch.cfg = forced;
      ch.gated_cfg = -1;
    }
  }
  const bool is_decode = ch.cfg == dg::kCfgDecode || ch.cfg == dg::kCfgDecodeFused;
  if (is_decode || ch.cfg == dg::kCfgNarrow) ch.gated_cfg = -1;
  if (is_decode) {
    const int fs = env_int("DG_FORCE_SPLITS", 0);
    if (fs > 0) ch.splits = fs;
    if (ch.splits < (KB + 7) / 8) ch.splits = (KB + 7) / 8;   // at most 8 K blocks per split
    if (ch.splits > KB) ch.splits = KB > 0 ? KB : 1;
    ch.kbs = (KB + ch.splits - 1) / ch.splits;
    ch.splits = ch.kbs > 0 ? (KB + ch.kbs - 1) / ch.kbs : 1;  // no empty splits
    // the one-launch form (DG_FORCE_CONFIG 12) needs a counter per tile; it
    // measured slower than the two launches on the decode shapes (its last
    // split reduces the whole tile through one CU, where the reduction
    // kernel spreads it over the chip), so it is not the default
    const long long tiles64 = ((long long)(rows + 63) / 64) * ((N + 63) / 64);
    if (ch.cfg == dg::kCfgDecodeFused && tiles64 > dg::kSyncMaxTiles) ch.cfg = dg::kCfgDecode;
  } else {
    ch.splits = 1;
  }
  return ch;
}

// Fills the tile counts of p for configuration cfg and returns its grid (0 on
// error).  The tile kernels walk their work list persistently: masked grids,
// and both grids of a gated pair (one of which exits at once), hold only as
// many workgroups as are resident on the chip together.
int plan(int mode, int cfg, dg::Params& p, int num_cus, bool gated) {
  const dg::ConfigInfo& ci = dg::config_info(cfg);
  p.tiles_m = (p.rows + ci.bm - 1) / ci.bm;
  p.tiles_n = (p.N + ci.bn - 1) / ci.bn;
  long long items;
  // one workgroup per CU, except the two-workgroup 128x128 configuration
  const long long resident = (long long)num_cus * (cfg == dg::kCfg128x128x2 ? 2 : 1);
  if (mode == dg::kMasked) {
    items = (long long)p.G * p.tiles_m * p.tiles_n;     // upper bound; the kernel walks the real list
    if (items > resident) items = resident;
  } else {
    items = (long long)p.tiles_m * p.tiles_n * p.splits;
    if (gated && items > resident) items = resident;
  }
  if (items > (1LL << 30)) {
    fail(DG_ERR_UNSUPPORTED, "problem too large (%lld work items)", items);
    return 0;
  }
  return (int)(((items + 7) / 8) * 8);
}

// Split tail: with a persistent grid of one workgroup per resident slot, the
// items of an XCD that do not fill a last round are split over K so that the
// round's workgroups all take a part (dense and 128-row contiguous calls on
// tiles up to 128x256; the tile kernel writes fp32 partials that
// splitk_tile_reduce_kernel sums).  Returns the grid (0 = no split tail) and
// sets p.sk_splits / p.sk_tail.
int plan_split_tail(int mode, int cfg, dg::Params& p, int num_cus, size_t ws_bytes) {
  const dg::ConfigInfo& ci = dg::config_info(cfg);
  p.sk_splits = 1;
  p.sk_tail = 0;
  if (mode == dg::kMasked || ci.bm * ci.bn > 128 * 256) return 0;
  if (mode == dg::kContiguous && ci.bm > 128) return 0;
  if (cfg == dg::kCfgDecode || cfg == dg::kCfgDecodeFused || cfg == dg::kCfgNarrow || cfg == dg::kCfgE8_128x256 || cfg == dg::kCfgWs_128x256 ||
      cfg == dg::kCfgE8_256x256)
    return 0;
  const int KB = p.K / 128;
  const int resident = num_cus * (cfg == dg::kCfg128x128x2 ? 2 : 1);
  const int grid = resident / 8 * 8;
  const int slots = grid / 8;
  const long long total = (long long)p.tiles_m * p.tiles_n;
  const long long per_xcd = (total + 7) / 8;
  int tail = 0;
  for (int x = 0; x < 8; ++x) {
    long long n_x = total - x * per_xcd;
    n_x = n_x < 0 ? 0 : (n_x > per_xcd ? per_xcd : n_x);
    tail = std::max(tail, (int)(n_x % slots));
  }
  if (tail == 0) return 0;
  int sk = slots / tail;
  const int forced = env_int("DG_SK_SPLITS", -1);
  if (forced == 0) return 0;
  if (forced > 0) sk = forced;
  if (sk > KB) sk = KB;
  if (sk > 16) sk = 16;
  while (sk > 1 && 8LL * tail * sk * ci.bm * ci.bn * (long long)sizeof(float) > (long long)ws_bytes) --sk;
  if (sk < 2) return 0;
  p.sk_splits = sk;
  p.sk_tail = tail;
  return grid;
}

// The choice for one call: choose(), then with a C the 128x256 tile in place
// of the 256x256 one: it reads C a strip ahead of its stores, while the
// 256x256 tile must read it per element between them.
Choice choose_call(int mode, int rows, int N, int K, int groups, int num_cus, int ab_layout, bool has_c,
                   size_t ws_bytes) {
  Choice ch = choose(mode, rows, N, K, groups, num_cus, ab_layout, ws_bytes);
  if (ch.cfg == dg::kCfg256x256w8 && has_c && env_int("DG_FORCE_CONFIG", -1) < 0) ch.cfg = dg::kCfg128x256w8;
  return ch;
}

// What a call runs with: the device's compute units and the scratch memory
// its kernels may use (split-K partials, scale-check verdicts).
struct Resources {
  int num_cus;
  float* workspace;
  size_t ws_bytes;
  int32_t* verdicts;     // dg::kCheckWGs entries
  int32_t* sync;         // dg::kSyncInts zeroed counters, or nullptr (no one-launch decode)
};


int launch_with(int mode, dg::Params& p, int rows_hint, hipStream_t stream, const Resources& r) {
  if ((long long)p.N * 256 * 2 >= (1LL << 31)) return fail(DG_ERR_UNSUPPORTED, "N=%d is too large", p.N);
  Choice ch = choose_call(mode, rows_hint, p.N, p.K, p.G, r.num_cus, p.ab_layout, p.c != nullptr, r.ws_bytes);
  p.splits = ch.splits;
  p.kbs_per_split = ch.kbs;
  p.workspace = r.workspace;
  p.workspace_bytes = r.ws_bytes;
  p.sync = r.sync;
  // the one-launch form needs the counters and addresses its partials with
  // 32-bit offsets; otherwise the two launches
  if (ch.cfg == dg::kCfgDecodeFused &&
      (!p.sync || ((long long)(p.rows + 63) / 64) * ((p.N + 63) / 64) * ch.splits * 64 * 64 * 4 >= (1LL << 32)))
    ch.cfg = dg::kCfgDecode;
  p.gate_ok = nullptr;
  const dg::ConfigInfo& ci = dg::config_info(ch.cfg);
  int grid = plan(mode, ch.cfg, p, r.num_cus, ch.gated_cfg >= 0);
  if (grid == 0) return DG_ERR_UNSUPPORTED;
  p.sk_splits = 1;
  p.sk_tail = 0;
  p.k_window = k_window_for(mode, ch.cfg);
  if (ch.gated_cfg < 0 && ch.splits == 1) {
    const int sk_grid = plan_split_tail(mode, ch.cfg, p, r.num_cus, r.ws_bytes);
    if (sk_grid > 0) grid = sk_grid;
  }
  if (ch.splits > 1) {
    const long long need = (long long)p.tiles_m * p.tiles_n * ch.splits * ci.bm * ci.bn * (long long)sizeof(float);
    if (need > (long long)r.ws_bytes)
      return fail(DG_ERR_UNSUPPORTED, "split-K workspace of %lld bytes exceeds the %zu available", need, r.ws_bytes);
  }
  hipError_t e = hipSuccess;
  if (ch.gated_cfg >= 0) {
    dg::Params pe = p;
    const int grid_e = plan(mode, ch.gated_cfg, pe, r.num_cus, true);
    if (grid_e == 0) return DG_ERR_UNSUPPORTED;
    const int KB = p.K / 128;
    const int NB = (p.N + 127) / 128;
    const size_t na = (size_t)KB * p.rows * (mode == dg::kMasked ? p.G : 1);
    const size_t nb = (size_t)NB * KB * (mode == dg::kDense ? 1 : p.G);
    p.gate_ok = pe.gate_ok = r.verdicts;
    if (env_int("DG_LOG", 0))
      std::fprintf(stderr, "[dg] mode=%d rows=%d N=%d K=%d G=%d gated cfg=%s grid=%d | cfg=%s grid=%d\n", mode,
                   p.rows, p.N, p.K, p.G, dg::config_info(ch.gated_cfg).name, grid_e, ci.name, grid);
    e = dg::launch_scale_check(p.sfa, na, p.sfb, nb, r.verdicts, stream);
    if (e == hipSuccess) e = dg::launch_gemm(mode, ch.gated_cfg, pe, grid_e, stream);
  } else if (env_int("DG_LOG", 0)) {
    std::fprintf(stderr, "[dg] mode=%d rows=%d N=%d K=%d G=%d cfg=%s splits=%d kbs=%d grid=%d tail_splits=%d\n",
                 mode, p.rows, p.N, p.K, p.G, ci.name, p.splits, p.kbs_per_split, grid, p.sk_splits);
  }
  if (e == hipSuccess) e = dg::launch_gemm(mode, ch.cfg, p, grid, stream);
  if (e == hipSuccess && p.sk_splits > 1) e = dg::launch_tile_reduce(mode, ch.cfg, p, grid, stream);
  if (e != hipSuccess) return fail(DG_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return DG_OK;
}

// Caller-supplied workspaces bound to streams (dg_bind_stream_workspace):
// calls enqueued on a bound stream of that device use it in place of the
// device's shared workspace.
constexpr size_t kBoundVerdictBytes = kVerdictBytes;   // the first bytes of a bound workspace hold the verdicts
struct Binding {
  int dev;
  hipStream_t stream;
  uint8_t* ptr;
  size_t bytes;
};
std::vector<Binding> g_bindings;
std::mutex g_bind_mu;
std::atomic<int> g_nbind{0};        // bindings in g_bindings (read without the lock)

bool find_binding(int dev, hipStream_t stream, Binding* out) {
  std::lock_guard<std::mutex> lock(g_bind_mu);
  for (const Binding& b : g_bindings)
    if (b.dev == dev && b.stream == stream) {
      *out = b;
      return true;
    }
  return false;
}

int launch(int mode, dg::Params& p, int rows_hint, hipStream_t stream) {
  DeviceState* st = nullptr;
  int s = get_device_state(&st);
  if (s != DG_OK) return s;
  Resources r{st->num_cus, st->workspace, kWorkspaceBytes, st->verdicts, st->sync};
  int dev = 0;
  Binding b;
  if (g_nbind.load(std::memory_order_acquire) > 0 && hipGetDevice(&dev) == hipSuccess && find_binding(dev, stream, &b)) {
    // [verdicts][counters, if the workspace holds more than them][partials]
    const bool has_sync = b.bytes >= kBoundVerdictBytes + kSyncBytes;
    const size_t ctl = kBoundVerdictBytes + (has_sync ? kSyncBytes : 0);
    r.verdicts = reinterpret_cast<int32_t*>(b.ptr);
    r.sync = has_sync ? reinterpret_cast<int32_t*>(b.ptr + kBoundVerdictBytes) : nullptr;
    r.workspace = reinterpret_cast<float*>(b.ptr + ctl);
    r.ws_bytes = b.bytes - ctl;
  }
  return launch_with(mode, p, rows_hint, stream, r);
}

}  // namespace

extern "C" int dg_fp8_gemm_nt(const void* a, const float* sfa, const void* b, const float* sfb,
                              const void* c, void* d, int M, int N, int K, void* stream) {
  int s = check_common(a, sfa, b, sfb, c, d, M, N, K);
  if (s != DG_OK) return s;
  if (M == 0 || N == 0) return DG_OK;
  dg::Params p{};
  p.a = static_cast<const uint8_t*>(a);
  p.sfa = sfa;
  p.b = static_cast<const uint8_t*>(b);
  p.sfb = sfb;
  p.c = static_cast<const uint16_t*>(c);
  p.d = static_cast<uint16_t*>(d);
  p.rows = M;
  p.N = N;
  p.K = K;
  p.G = 1;
  return launch(dg::kDense, p, M, static_cast<hipStream_t>(stream));
}

namespace {
// Dense call with K-major operands: layout bit 0 = A is [K][M], bit 1 = B is [K][N].
int dense_kmajor(const void* a, const float* sfa, const void* b, const float* sfb, const void* c, void* d,
                 int M, int N, int K, int layout, void* stream) {
  int s = check_common(a, sfa, b, sfb, c, d, M, N, K);
  if (s != DG_OK) return s;
  if ((layout & 1) && M % 16 != 0)
    return fail(DG_ERR_UNSUPPORTED, "A stored [K][M] needs M %% 16 == 0 (M=%d)", M);
  if ((layout & 2) && N % 16 != 0)
    return fail(DG_ERR_UNSUPPORTED, "B stored [K][N] needs N %% 16 == 0 (N=%d)", N);
  if (M == 0 || N == 0) return DG_OK;
  dg::Params p{};
  p.a = static_cast<const uint8_t*>(a);
  p.sfa = sfa;
  p.b = static_cast<const uint8_t*>(b);
  p.sfb = sfb;
  p.c = static_cast<const uint16_t*>(c);
  p.d = static_cast<uint16_t*>(d);
  p.rows = M;
  p.N = N;
  p.K = K;
  p.G = 1;
  p.ab_layout = layout;
  return launch(dg::kDense, p, M, static_cast<hipStream_t>(stream));
}
}  // namespace

extern "C" int dg_fp8_fp4_gemm_nt(const void* a, const float* sfa, const void* b, const int32_t* sfb,
                                  const void* c, void* d, int M, int N, int K, void* stream) {
  // b holds K/2 bytes per row; the common checks see the same pointers
  int s = check_common(a, sfa, b, reinterpret_cast<const float*>(sfb), c, d, M, N, K);
  if (s != DG_OK) return s;
  if (M == 0 || N == 0) return DG_OK;
  dg::Params p{};
  p.a = static_cast<const uint8_t*>(a);
  p.sfa = sfa;
  p.b = static_cast<const uint8_t*>(b);
  p.sfb = reinterpret_cast<const float*>(sfb);   // copied as raw words by the kernel
  p.c = static_cast<const uint16_t*>(c);
  p.d = static_cast<uint16_t*>(d);
  p.rows = M;
  p.N = N;
  p.K = K;
  p.G = 1;
  p.ab_layout = 4;
  return launch(dg::kDense, p, M, static_cast<hipStream_t>(stream));
}

extern "C" int dg_fp8_gemm_nn(const void* a, const float* sfa, const void* b, const float* sfb,
                              const void* c, void* d, int M, int N, int K, void* stream) {
  return dense_kmajor(a, sfa, b, sfb, c, d, M, N, K, 2, stream);
}

extern "C" int dg_fp8_gemm_tn(const void* a, const float* sfa, const void* b, const float* sfb,
                              const void* c, void* d, int M, int N, int K, void* stream) {
  return dense_kmajor(a, sfa, b, sfb, c, d, M, N, K, 3, stream);
}

extern "C" int dg_fp8_gemm_tt(const void* a, const float* sfa, const void* b, const float* sfb,
                              const void* c, void* d, int M, int N, int K, void* stream) {
  return dense_kmajor(a, sfa, b, sfb, c, d, M, N, K, 1, stream);
}

extern "C" int dg_k_grouped_fp8_gemm_tn_contiguous(const void* a, const float* sfa, const void* b,
                                                   const float* sfb, const float* c, float* d, int M, int N,
                                                   int num_groups, const int32_t* ks, void* stream) {
  if (!a || !sfa || !b || !sfb || !d || !ks)
    return fail(DG_ERR_INVALID_ARG, "a, sfa, b, sfb, d and ks must not be NULL");
  if (M < 0 || N < 0) return fail(DG_ERR_INVALID_ARG, "negative size (M=%d N=%d)", M, N);
  if (num_groups < 1) return fail(DG_ERR_INVALID_ARG, "num_groups=%d must be at least 1", num_groups);
  if (num_groups > dg::kMaxKGroups)
    return fail(DG_ERR_UNSUPPORTED, "num_groups=%d exceeds %d", num_groups, dg::kMaxKGroups);
  if (!aligned(a, 16) || !aligned(b, 16)) return fail(DG_ERR_INVALID_ARG, "a and b must be 16-byte aligned");
  if (!aligned(sfa, 4) || !aligned(sfb, 4) || !aligned(d, 4) || (c && !aligned(c, 4)))
    return fail(DG_ERR_INVALID_ARG, "sfa, sfb, c and d must be 4-byte aligned");
  dg::KGroupedParams p{};
  long long K = 0;
  for (int g = 0; g < num_groups; ++g) {
    if (ks[g] < 0 || ks[g] % 128 != 0)
      return fail(DG_ERR_INVALID_ARG, "ks[%d]=%d is not a non-negative multiple of 128", g, ks[g]);
    p.k_start[g] = (int)K;
    K += ks[g];
    if (K > (1LL << 30)) return fail(DG_ERR_UNSUPPORTED, "total K of %lld is too large", K);
  }
  p.k_start[num_groups] = (int)K;
  if (M % 16 != 0 || N % 16 != 0)
    return fail(DG_ERR_UNSUPPORTED, "the K-major operands need M and N multiples of 16 (M=%d N=%d)", M, N);
  if (M == 0 || N == 0) return DG_OK;
  DeviceState* st = nullptr;
  int s = get_device_state(&st);
  if (s != DG_OK) return s;
  if ((long long)N * 256 * 2 >= (1LL << 31)) return fail(DG_ERR_UNSUPPORTED, "N=%d is too large", N);
  p.a = static_cast<const uint8_t*>(a);
  p.sfa = sfa;
  p.b = static_cast<const uint8_t*>(b);
  p.sfb = sfb;
  p.d32 = d;
  p.c32 = c;
  p.rows = M;
  p.N = N;
  p.K = (int)K;
  p.G = num_groups;
  p.splits = 1;
  // the tile by rounds of the chip times the rows loaded per K block, as for
  // dense calls; with a C the 256x256 tile is left out: it reads C per element
  // between its stores, while the smaller tiles read it a strip ahead
  const long long t256 = (long long)num_groups * ((M + 255) / 256) * ((N + 255) / 256);
  const long long t128x256 = (long long)num_groups * ((M + 127) / 128) * ((N + 255) / 256);
  const long long t128 = (long long)num_groups * ((M + 127) / 128) * ((N + 127) / 128);
  auto cost = [&](long long tiles, int edge) { return ((tiles + st->num_cus - 1) / st->num_cus) * edge; };
  const long long c256 = cost(t256, 512), c128x256 = cost(t128x256, 384), c128 = cost(t128, 256);
  int cfg = !c && c256 <= c128x256 && c256 <= c128 ? dg::kCfg256x256w8
            : c128x256 <= c128                    ? dg::kCfg128x256w8
                                                  : dg::kCfg128x128;
  const int forced = env_int("DG_FORCE_CONFIG", -1);
  if (forced == dg::kCfg128x128 || forced == dg::kCfg128x256w8 || forced == dg::kCfg256x256w8) cfg = forced;
  const dg::ConfigInfo& ci = dg::config_info(cfg);
  p.k_window = k_window_for(dg::kKGrouped, cfg);
  p.tiles_m = (M + ci.bm - 1) / ci.bm;
  p.tiles_n = (N + ci.bn - 1) / ci.bn;
  const long long items = (long long)num_groups * p.tiles_m * p.tiles_n;
  if (items > (1LL << 30)) return fail(DG_ERR_UNSUPPORTED, "problem too large (%lld work items)", items);
  const int grid = (int)(((items + 7) / 8) * 8);
  if (env_int("DG_LOG", 0))
    std::fprintf(stderr, "[dg] k-grouped M=%d N=%d K=%lld G=%d cfg=%s grid=%d\n", M, N, K, num_groups, ci.name, grid);
  hipError_t e = dg::launch_kgrouped(cfg, p, grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DG_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
  return DG_OK;
}

namespace {
// M-grouped calls; ab_layout 0 = FP8 B [G][N][K] with fp32 128x128 scales,
// 4 = FP4 B [G][N][K/2] with packed E8M0 scales [G][K/128][N].
int grouped_contiguous(const void* a, const float* sfa, const void* b, const float* sfb, const void* c, void* d,
                       int M, int N, int K, int num_groups, const int32_t* grouped_layout, int ab_layout,
                       void* stream) {
  int s = check_common(a, sfa, b, sfb, c, d, M, N, K);
  if (s != DG_OK) return s;
  if (num_groups < 1) return fail(DG_ERR_INVALID_ARG, "num_groups=%d must be at least 1", num_groups);
  if (!grouped_layout) return fail(DG_ERR_INVALID_ARG, "grouped_layout must not be NULL");
  if (!aligned(grouped_layout, 4)) return fail(DG_ERR_INVALID_ARG, "grouped_layout must be 4-byte aligned");
  if (M == 0 || N == 0) return DG_OK;
  s = validate_layout(grouped_layout, M, num_groups, static_cast<hipStream_t>(stream));
  if (s != DG_OK) return s;
  dg::Params p{};
  p.a = static_cast<const uint8_t*>(a);
  p.sfa = sfa;
  p.b = static_cast<const uint8_t*>(b);
  p.sfb = sfb;
  p.c = static_cast<const uint16_t*>(c);
  p.d = static_cast<uint16_t*>(d);
  p.layout = grouped_layout;
  p.rows = M;
  p.N = N;
  p.K = K;
  p.G = num_groups;
  p.ab_layout = ab_layout;
  return launch(dg::kContiguous, p, M, static_cast<hipStream_t>(stream));
}

int grouped_masked(const void* a, const float* sfa, const void* b, const float* sfb, const void* c, void* d,
                   int max_m, int N, int K, int num_groups, const int32_t* masked_m, int expected_m, int ab_layout,
                   void* stream) {
  int s = check_common(a, sfa, b, sfb, c, d, max_m, N, K);
  if (s != DG_OK) return s;
  if (num_groups < 1) return fail(DG_ERR_INVALID_ARG, "num_groups=%d must be at least 1", num_groups);
  if (num_groups > 1024) return fail(DG_ERR_UNSUPPORTED, "num_groups=%d exceeds 1024", num_groups);
  if (!masked_m) return fail(DG_ERR_INVALID_ARG, "masked_m must not be NULL");
  if (!aligned(masked_m, 4)) return fail(DG_ERR_INVALID_ARG, "masked_m must be 4-byte aligned");
  if (expected_m < 0) return fail(DG_ERR_INVALID_ARG, "expected_m=%d must not be negative", expected_m);
  if (max_m == 0 || N == 0) return DG_OK;
  s = validate_masked(masked_m, num_groups, max_m, static_cast<hipStream_t>(stream));
  if (s != DG_OK) return s;
  dg::Params p{};
  p.a = static_cast<const uint8_t*>(a);
  p.sfa = sfa;
  p.b = static_cast<const uint8_t*>(b);
  p.sfb = sfb;
  p.c = static_cast<const uint16_t*>(c);
  p.d = static_cast<uint16_t*>(d);
  p.masked_m = masked_m;
  p.rows = max_m;
  p.N = N;
  p.K = K;
  p.G = num_groups;
  p.ab_layout = ab_layout;
  return launch(dg::kMasked, p, expected_m > 0 ? expected_m : max_m, static_cast<hipStream_t>(stream));
}
}  // namespace

extern "C" int dg_m_grouped_fp8_gemm_nt_contiguous(const void* a, const float* sfa, const void* b,
                                                   const float* sfb, const void* c, void* d, int M,
                                                   int N, int K, int num_groups,
                                                   const int32_t* grouped_layout, void* stream) {
  return grouped_contiguous(a, sfa, b, sfb, c, d, M, N, K, num_groups, grouped_layout, 0, stream);
}

extern "C" int dg_m_grouped_fp8_gemm_nt_masked(const void* a, const float* sfa, const void* b,
                                               const float* sfb, const void* c, void* d, int max_m,
                                               int N, int K, int num_groups, const int32_t* masked_m,
                                               int expected_m, void* stream) {
  return grouped_masked(a, sfa, b, sfb, c, d, max_m, N, K, num_groups, masked_m, expected_m, 0, stream);
}

extern "C" int dg_m_grouped_fp8_fp4_gemm_nt_contiguous(const void* a, const float* sfa, const void* b,
                                                       const int32_t* sfb, const void* c, void* d, int M,
                                                       int N, int K, int num_groups,
                                                       const int32_t* grouped_layout, void* stream) {
  return grouped_contiguous(a, sfa, b, reinterpret_cast<const float*>(sfb), c, d, M, N, K, num_groups,
                            grouped_layout, 4, stream);
}

extern "C" int dg_m_grouped_fp8_fp4_gemm_nt_masked(const void* a, const float* sfa, const void* b,
                                                   const int32_t* sfb, const void* c, void* d, int max_m,
                                                   int N, int K, int num_groups, const int32_t* masked_m,
                                                   int expected_m, void* stream) {
  return grouped_masked(a, sfa, b, reinterpret_cast<const float*>(sfb), c, d, max_m, N, K, num_groups, masked_m,
                        expected_m, 4, stream);
}

extern "C" int dg_choose_config(int form, int rows, int N, int K, int num_groups, int num_cus, int ab_layout,
                                int has_c, int* cfg, int* splits) {
  if (!cfg || !splits) return fail(DG_ERR_INVALID_ARG, "cfg and splits must not be NULL");
  if (form < dg::kDense || form > dg::kMasked) return fail(DG_ERR_INVALID_ARG, "form=%d is not 0, 1 or 2", form);
  if (rows < 1 || N < 1 || K < 0 || K % 128 != 0 || num_groups < 1 || num_cus < 8 || ab_layout < 0 || ab_layout > 4)
    return fail(DG_ERR_INVALID_ARG, "invalid query (rows=%d N=%d K=%d num_groups=%d num_cus=%d ab_layout=%d)", rows,
                N, K, num_groups, num_cus, ab_layout);
  const Choice ch = choose_call(form, rows, N, K, num_groups, num_cus, ab_layout, has_c != 0, kWorkspaceBytes);
  *cfg = ch.gated_cfg >= 0 ? ch.gated_cfg : ch.cfg;
  *splits = ch.splits;
  return DG_OK;
}

// ---- the allocation-free call ------------------------------------------------
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid it): the kernels' scratch
// (scale-check verdicts, then split-K partials) lives in a file-scope device
// array.  In host code `scratch` names a host-side stand-in, not a device
// address; the device address is taken once per device with
// hipGetSymbolAddress and only that address is handed to kernels.
namespace dg_noalloc {
constexpr size_t kScratchBytes = size_t(8) << 20;   // per device, held until the process ends
// [verdicts][one-launch decode counters][partials]; the array starts zeroed
// (static storage) and every call leaves the counters at zero
constexpr size_t kCtlBytes = kVerdictBytes + kSyncBytes;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

struct State {
  std::atomic<bool> ready{false};
  int num_cus = 0;
  uint8_t* ptr = nullptr;       // this device's copy of scratch
};
State g_state[kMaxDevices];
std::mutex g_mu;

int get_state(State** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DG_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DG_ERR_UNSUPPORTED, "device index %d out of range", dev);
  State& st = g_state[dev];
  if (!st.ready.load(std::memory_order_acquire)) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!st.ready.load(std::memory_order_relaxed)) {
      hipDeviceProp_t prop;
      e = hipGetDeviceProperties(&prop, dev);
      if (e != hipSuccess) return fail(DG_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
      if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(DG_ERR_UNSUPPORTED, "device %d is %s; the kernels are built for gfx950 only", dev, prop.gcnArchName);
      void* ptr = nullptr;
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));    // with this device current
      if (e != hipSuccess || !ptr) return fail(DG_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      st.num_cus = prop.multiProcessorCount;
      st.ptr = static_cast<uint8_t*>(ptr);
      st.ready.store(true, std::memory_order_release);
    }
  }
  *out = &st;
  return DG_OK;
}
}  // namespace dg_noalloc

extern "C" int dg_fp8_gemm_nt_noalloc(const void* a, const float* sfa, const void* b, const float* sfb,
                                      const void* c, void* d, int M, int N, int K, void* stream) {
  int s = check_common(a, sfa, b, sfb, c, d, M, N, K);
  if (s != DG_OK) return s;
  if (M == 0 || N == 0) return DG_OK;
  dg_noalloc::State* st = nullptr;
  s = dg_noalloc::get_state(&st);
  if (s != DG_OK) return s;
  dg::Params p{};
  p.a = static_cast<const uint8_t*>(a);
  p.sfa = sfa;
  p.b = static_cast<const uint8_t*>(b);
  p.sfb = sfb;
  p.c = static_cast<const uint16_t*>(c);
  p.d = static_cast<uint16_t*>(d);
  p.rows = M;
  p.N = N;
  p.K = K;
  p.G = 1;
  // the chooser keeps split-K partials within the scratch; a configuration
  // forced beyond it (DG_FORCE_SPLITS) is refused with DG_ERR_UNSUPPORTED
  const Resources r{st->num_cus, reinterpret_cast<float*>(st->ptr + dg_noalloc::kCtlBytes),
                    dg_noalloc::kScratchBytes - dg_noalloc::kCtlBytes, reinterpret_cast<int32_t*>(st->ptr),
                    reinterpret_cast<int32_t*>(st->ptr + kVerdictBytes)};
  return launch_with(dg::kDense, p, M, static_cast<hipStream_t>(stream), r);
}

extern "C" int dg_bind_stream_workspace(void* stream, void* workspace, size_t bytes) {
  if (workspace && !aligned(workspace, 256))
    return fail(DG_ERR_INVALID_ARG, "the workspace must be 256-byte aligned");
  if (workspace && bytes < kBoundVerdictBytes)
    return fail(DG_ERR_INVALID_ARG, "a workspace of %zu bytes is smaller than the %zu the verdicts need", bytes,
                kBoundVerdictBytes);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DG_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (workspace && bytes >= kBoundVerdictBytes + kSyncBytes) {
    // the one-launch decode kernel's counters start at zero
    e = hipMemset(static_cast<uint8_t*>(workspace) + kBoundVerdictBytes, 0, kSyncBytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail(DG_ERR_HIP, "clearing the workspace's counters: %s", hipGetErrorString(e));
  }
  std::lock_guard<std::mutex> lock(g_bind_mu);
  for (size_t i = 0; i < g_bindings.size(); ++i)
    if (g_bindings[i].dev == dev && g_bindings[i].stream == st) {
      g_bindings.erase(g_bindings.begin() + (long)i);
      break;
    }
  if (workspace && bytes > 0) g_bindings.push_back(Binding{dev, st, static_cast<uint8_t*>(workspace), bytes});
  g_nbind.store((int)g_bindings.size(), std::memory_order_release);
  return DG_OK;
}

extern "C" int dg_check_grouped_layout(const int32_t* grouped_layout, int M, int num_groups) {
  if (!grouped_layout && M > 0) return fail(DG_ERR_INVALID_ARG, "grouped_layout must not be NULL");
  if (M < 0 || num_groups < 1) return fail(DG_ERR_INVALID_ARG, "M=%d num_groups=%d", M, num_groups);
  return check_layout_host(grouped_layout, M, num_groups);
}

extern "C" int dg_init(void) {
  DeviceState* st = nullptr;
  return get_device_state(&st);
}

extern "C" const char* dg_last_error(void) { return g_err.c_str(); }

extern "C" int dg_version(void) { return 100; }
