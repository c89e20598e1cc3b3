// Host side of the C ABI: argument checks, the NVFP4 packer, the host
// quantizers and kernel selection.  No HIP call happens before every check
// has passed, so all error paths run on machines without a GPU.
#include "skinny.h"
#include "internal.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstring>
#include <thread>
#include <vector>

using namespace skinny;

namespace {

constexpr int kMaxK = 1 << 20;
constexpr int kMaxN = 1 << 24;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(int M, int K, int N) {
  if (M < 1 || M > SKINNY_MAX_M) return SKINNY_ESHAPE;
  if (K < 16 || K % 16 != 0 || K > kMaxK) return SKINNY_ESHAPE;
  if (N < 1 || N > kMaxN) return SKINNY_ESHAPE;
  return SKINNY_OK;
}

// ---- E2M1 / E4M3FN encoders (round to nearest, ties to the even code) ------
// Positive magnitudes of E2M1 codes 0..7.
const double kE2m1Mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

int e2m1_code(double v) {
  const int sign = std::signbit(v) ? 8 : 0;
  const double a = std::fabs(v);
  int i = 0;  // smallest i with a <= midpoint(i, i+1), else 7
  while (i < 7 && a > 0.5 * (kE2m1Mag[i] + kE2m1Mag[i + 1])) ++i;
  if (i < 7 && a == 0.5 * (kE2m1Mag[i] + kE2m1Mag[i + 1]) && (i & 1)) ++i;
  return sign | i;
}

double e4m3_value(int code) {  // code 0..126 (positive, finite)
  const int e = (code >> 3) & 15, m = code & 7;
  return e == 0 ? std::ldexp(static_cast<double>(m), -9) : std::ldexp(1.0 + m / 8.0, e - 7);
}

struct E4m3Table {
  double mid[126];  // midpoint between codes i and i+1
  E4m3Table() {
    for (int i = 0; i < 126; ++i) mid[i] = 0.5 * (e4m3_value(i) + e4m3_value(i + 1));
  }
};
const E4m3Table& e4m3_table() {
  static const E4m3Table t;
  return t;
}

int e4m3_code(double v) {
  const int sign = std::signbit(v) ? 0x80 : 0;
  const double a = std::fabs(v);
  const double* mid = e4m3_table().mid;
  int lo = 0, hi = 126;  // find smallest i in [0,126] with a <= mid[i] (126 = saturate)
  while (lo < hi) {
    const int md = (lo + hi) / 2;
    if (a <= mid[md]) hi = md; else lo = md + 1;
  }
  int i = lo;
  if (i < 126 && a == mid[i] && (i & 1)) ++i;
  return sign | i;
}

// Host worker threads for the quantizers: the machine's hardware threads, at most 16.
int host_threads() {
  const unsigned hw = std::thread::hardware_concurrency();
  return static_cast<int>(std::max(1u, std::min(hw, 16u)));
}

// Runs fn(thread_index, begin, end) over [0, count) split into contiguous ranges.
template <typename Fn>
void parallel_for(int count, Fn fn) {
  const int nt = std::max(1, std::min(host_threads(), count));
  std::vector<std::thread> pool;
  for (int t = 0; t < nt; ++t) {
    const int b = static_cast<int>(static_cast<long long>(count) * t / nt);
    const int e = static_cast<int>(static_cast<long long>(count) * (t + 1) / nt);
    pool.emplace_back(fn, t, b, e);
  }
  for (auto& th : pool) th.join();
}

int launch_status(hipError_t e) { return e == hipSuccess ? SKINNY_OK : SKINNY_EHIP; }

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// Kernel choice made by the library when the caller does not pick one.  The
// rules follow timings of every choice on the decode shapes and on one rank's
// share of them under 4-way tensor parallelism, at M = 1, 4 and 8:
//
// NVFP4 at M = 1 (GEMV, and the lm_head with its argmax: on the 151936-column
// vocabulary the GEMV reads at 6.95 TB/s against 6.5 TB/s for the streaming
// engine): VALU engine, whole K per workgroup, two tiles per workgroup when
// there are few tiles (N <= 6144), else one.  With few tiles and K beyond 16
// spans (a K split either way), four tiles of two spans per workgroup
// instead: with the split added inside the kernel, the 17408 x 5120 down
// projection took 10.40-10.43 us so against 10.65-10.72 us for two tiles of
// six spans (three-way split).  NVFP4 at M = 2 without argmax
// takes the same choice when there are few tiles (N <= 6144): on the
// 17408 x 5120 down projection it took 12.7 us against 13.7 us for the MFMA
// engine, and 6.0 against 6.5-6.7 us on one rank's 4-way share of up and
// down; with more tiles (up, gate+up) and on the lm_head the MFMA and
// streaming engines were faster.  FP8 at M <= 2: its VALU engine,
// whole K per workgroup, two tiles only when 2 * K spans <= 16 and N <= 6144
// (on qkv and o_proj one tile of 10 or 12 units was within 0.03 us of the
// fastest choice at M = 1, 0.3 to 0.6 us ahead of the MFMA engine, and about
// 0.1 to 0.2 us ahead at M = 2; at M = 4 the MFMA engine is faster).
//
// Other NVFP4 calls: the streaming engine when there are enough column tiles
// to keep the CUs busy with whole tiles (N >= 8192) and all of x fits in LDS
// (K <= 9216): one workgroup per CU of about N / 3200 wavefronts (4 to 12),
// which gives each wavefront about one tile on the MLP shapes and a few on a
// vocabulary.  With fewer tiles a wavefront per tile is too little
// parallelism, so the one-unit-per-wavefront MFMA engine is used instead,
// like FP8:
//   - up to four rows and K <= 8192: whole K per workgroup (two tiles per
//     workgroup when K and N are short), except NVFP4 with few tiles and
//     K of at least 5 spans, which takes the short choice below;
//   - otherwise four tiles per workgroup and the fewest K spans per workgroup
//     that keep the K split at most nine ways (the x slice a workgroup stages
//     in LDS grows with M and with its spans; short workgroups keep it small).
// The largest S (K spans per workgroup) from `s_max` down for which the
// choice is supported (its LDS copy of x fits), with the K split evened out.
template <typename Fits>
LaunchCfg fit_spans(int engine, int ct, int ku, int s_max, Fits fits) {
  for (int s0 = std::max(1, s_max); s0 >= 1; --s0) {
    const int ksplit = (ku + s0 - 1) / s0;
    const int s = (ku + ksplit - 1) / ksplit;
    const LaunchCfg c{engine, ct, ct * s, ksplit};
    if (fits(c)) return c;
  }
  return LaunchCfg{engine, ct, ct, ku};
}

template <typename Fits>
LaunchCfg pick_whole_k_cfg(int engine, int ct, int ku, Fits fits) {
  return fit_spans(engine, ct, ku, std::min(ku, kMaxWaves / ct), fits);
}

template <typename Fits>
LaunchCfg pick_short_cfg(int ku, int nt, Fits fits) {
  constexpr int kMaxSplit = 9;
  const int ct = nt >= 4 ? 4 : (nt >= 2 ? 2 : 1);
  return fit_spans(1, ct, ku, std::min((ku + kMaxSplit - 1) / kMaxSplit, kMaxWaves / ct), fits);
}

// One-unit-per-wavefront MFMA choice (NVFP4 without streaming, and FP8);
// ku counts K spans of `unit_k`.
template <typename Fits>
LaunchCfg pick_oneshot_cfg(int M, int K, int ku, int nt, Fits fits) {
  if (M <= 4 && K <= 8192) return pick_whole_k_cfg(1, 2 * ku <= kMaxWaves && nt <= 512 ? 2 : 1, ku, fits);
  return pick_short_cfg(ku, nt, fits);
}

// Streaming choice: one workgroup per CU of about nt / 200 wavefronts, 4 to
// 6 up to 4096 tiles and 4 to 12 beyond.  On the 2176 tiles of gate+up, six
// wavefronts (all 256 CUs, one or two tiles each) against eleven (198 CUs,
// one tile each) took 18.87-18.92 us against 19.40-19.99 us at M = 8,
// 18.21-18.87 against 18.40-19.68 us at M = 5..7 and the same within noise at
// M = 2 and 4 (and the SwiGLU pair at M = 8 18.84-18.87 against 19.48 us);
// the 2374 tiles of one rank's lm_head took the same with 6 or 12, and the
// whole vocabulary (9496 tiles) 73.3-73.4 us with 12 against 77.1 with 6.
bool pick_stream_cfg(int M, int K, int N, bool argmax, LaunchCfg* out) {
  const int nt = (N + kTileCols - 1) / kTileCols;
  if (nt < 512) return false;
  const LaunchCfg c{2, 1, std::min(nt <= 4096 ? 6 : 12, std::max(4, (nt + 199) / 200)), 1};
  if (!nvfp4_cfg_supported(c, M, K, argmax)) return false;
  *out = c;
  return true;
}

LaunchCfg default_nvfp4_cfg(int M, int K, int N, bool argmax, bool swiglu = false) {
  const Geometry g = nvfp4_geometry(K, N);
  auto fits = [&](const LaunchCfg& c) { return nvfp4_cfg_supported(c, M, K, argmax); };
  // One tile of whole K per workgroup, balanced over the CUs when the tiles
  // do not divide evenly (BalancedLayout), with three or four whole tiles per
  // CU.  On MI355X at K = 5120: 1088 tiles took 10.11 against 10.28 us at
  // M = 1 and 11.04 against 11.23 us (streaming engine) at M = 2, 832 tiles
  // 8.17 against 8.30 and 9.21 against 10.34 us; with one or two whole tiles
  // per CU (400 and 576 tiles) it was up to 0.24 us slower.
  BalancedLayout bal;
  const int cus = device_cu_count();
  if (M <= 2 && !argmax && !swiglu && g.nt > 384 && g.ku <= kMaxWaves && g.nt / cus >= 3 &&
      nvfp4_balanced_layout(g.nt, g.ku, cus, &bal))
    return LaunchCfg{3, 1, g.ku, 1};
  if (M == 1 && !argmax && g.nt <= 384 && g.ku > kMaxWaves) return fit_spans(0, 4, g.ku, 2, fits);
  // With at most 384 tiles and K of at least 5 spans, MFMA workgroups of four
  // tiles of one span each (pick_short_cfg), added inside the kernel, spread
  // the bytes over every CU, where whole-K workgroups leave CUs idle or
  // unevenly loaded and each busy CU's time grows with K.  On MI355X (one
  // box, same runs), M = 3 / 4: 128 tiles at K = 5120 5.12 / 5.24 us against
  // 6.53 / 6.81 us whole-K; 272 tiles (one rank's up share) 6.39 / 6.53
  // against 6.89 / 7.15; 384 tiles 6.72 / 6.91 against 7.33 / 7.58; 320 tiles
  // at K = 4352 (one rank's down share) 6.85 / 6.97 against 7.22 / 7.48; 256
  // tiles at K = 8192 6.82 / 6.97 against 8.48 / 8.85.  At 480 tiles it tied,
  // and at K = 2048 (2 spans) it lost by 0.5-0.7 us.  At M = 2 it won with at
  // most half a tile per CU (128 tiles: 5.07 against 6.12 us for the VALU
  // engine) or K of at least 8 spans (256 tiles at K = 8192: 6.71 against
  // 7.41), and tied or lost by up to 0.13 us at 272 to 384 tiles and K = 5120
  // or 4352.
  if (!argmax && !swiglu && g.ku >= 5 && g.nt <= 384 &&
      (M == 3 || M == 4 || (M == 2 && (2 * g.nt <= cus || (g.ku >= 8 && g.nt <= cus)))))
    return pick_short_cfg(g.ku, g.nt, fits);
  if (M == 1 || (M == 2 && !argmax && g.nt <= 384)) return pick_whole_k_cfg(0, g.nt <= 384 ? 2 : 1, g.ku, fits);
  LaunchCfg c;
  if (pick_stream_cfg(M, K, N, argmax, &c)) return c;
  return pick_oneshot_cfg(M, K, g.ku, g.nt, fits);
}

LaunchCfg default_fp8_cfg(int M, int K, int N) {
  const int ku = (K + 511) / 512, nt = (N + 15) / 16;
  auto fits = [&](const LaunchCfg& c) { return fp8_cfg_supported(c, M, K); };
  // Whole-K workgroups of one tile load the CUs unevenly when there are
  // between one and two tiles per CU, and leave CUs idle below one per CU,
  // where each busy CU's time grows with its K.  There the MFMA engine with
  // two tiles of two units per workgroup and a K split added inside the
  // kernel reads x once per two tiles and spreads the work evenly.  On MI355X,
  // packed codes, K = 6144 (12 units): 320 tiles (o_proj, 5120 columns)
  // M = 2 / 3 / 4 7.89 / 8.10 / 8.34 us against 8.28 / 9.09 / 9.51 us whole-K
  // (canonical M = 4 8.43-8.60 against 10.24 us); 352 to 416 tiles gained
  // 0.1-0.55 us from M = 3 on but lost at M = 2; 256 and 448 tiles, and
  // K = 1536, lost at every M.  K = 5120 (10 units): 32 / 64 / 112 tiles
  // gained 0.6-0.9 / 0.6-0.8 / 0.2 us at M = 3 and 4, 32 and 64 tiles 0.2-0.3
  // us at M = 2; 160 tiles tied and 224 lost.  K = 4096 (8 units) lost from
  // 64 tiles on.
  const int cus = device_cu_count();
  const bool uneven =
      nt > cus ? ku >= 8 && (M >= 3 ? 4 * nt < 7 * cus : M == 2 && 4 * nt <= 5 * cus)
               : ku >= 10 && (M >= 3 ? 2 * nt <= cus : M == 2 && 4 * nt <= cus);
  if (uneven && M <= 4) {
    const LaunchCfg c{1, 2, 4, (ku + 1) / 2};
    if (fits(c)) return c;
  }
  // M <= 2: the VALU engine, whole K per workgroup (two tiles per workgroup
  // only when both fit whole: 2 * ku <= 16 and few tiles).
  if (M <= 2) return pick_whole_k_cfg(0, 2 * ku <= kMaxWaves && nt <= 384 ? 2 : 1, ku, fits);
  return pick_oneshot_cfg(M, K, ku, nt, fits);
}

// A SwiGLU pair of F columns each packs to swiglu_packed_cols(F) <= kMaxN columns.
int swiglu_shape(int M, int K, int F) {
  if (F < 1 || F > kMaxN / 2) return SKINNY_ESHAPE;
  return check_shape(M, K, F);
}

int nvfp4_common_checks(const void* w_packed, const uint16_t* x, const void* out, int M, int K, int N) {
  if (!w_packed || !x || !out) return SKINNY_EINVAL;
  int s = check_shape(M, K, N);
  if (s) return s;
  if (!aligned(w_packed, 16) || !aligned(x, 16)) return SKINNY_EALIGN;
  return SKINNY_OK;
}

int check_workspace(const void* ws, size_t have, size_t need) {
  if (need == 0) return SKINNY_OK;
  if (!ws) return SKINNY_EINVAL;
  if (!aligned(ws, 16)) return SKINNY_EALIGN;
  if (have < need) return SKINNY_ESIZE;
  return SKINNY_OK;
}

}  // namespace

namespace skinny {

// Cached per device; calls from several host threads may race to fill an
// entry, and each stores the same value.
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

Geometry nvfp4_geometry(int K, int N) {
  Geometry g;
  g.ku = (K + kUnitK - 1) / kUnitK;
  g.nt = (N + kTileCols - 1) / kTileCols;
  g.units_bytes = static_cast<size_t>(g.nt) * g.ku * kUnitBytes;
  g.total_bytes = kHeaderBytes + g.units_bytes;
  return g;
}

bool nvfp4_balanced_layout(int nt, int ku, int cus, BalancedLayout* out) {
  if (cus < 1 || nt % cus == 0 || nt / cus > 4) return false;
  const int rest = nt % cus;
  const int cap = std::min(cus, kMaxSyncGroups);
  for (int spans = 1; spans <= ku; ++spans) {
    const int splits = (ku + spans - 1) / spans;
    if (static_cast<long>(rest) * splits <= cap) {
      *out = BalancedLayout{nt - rest, spans, splits};
      return true;
    }
  }
  return false;
}

bool nvfp4_uses_xsplit(const LaunchCfg& cfg, int N, bool plain_epilogue) {
  const int nt = (N + kTileCols - 1) / kTileCols;
  // The reduction's buffer offsets, up to (ksplit + 16) blocks of at most
  // 8 rows x ct tiles of fp32, stay far inside an int.
  const int64_t reach = static_cast<int64_t>(cfg.ksplit + 16) * 8 * cfg.ct * kTileCols * 4;
  return (cfg.engine == 0 || cfg.engine == 1) && cfg.ksplit > 1 && plain_epilogue &&
         (nt + cfg.ct - 1) / cfg.ct <= kMaxSyncGroups && reach < (int64_t{1} << 30);
}

// Partial sums of a K split: fp32, ksplit x M x (the tiles' columns) for the
// M real rows, laid out [split][m][n] for the split reduction kernel or in one
// [m][column] block per (tile group, split) for the in-kernel reduction; the
// size covers both.  Argmax candidates: one 64-bit key per row for each
// workgroup of the GEMM kernel (no split) or each column block of the split
// reduction.
WorkspaceLayout nvfp4_workspace_layout(const LaunchCfg& cfg, int M, int K, int N, bool argmax) {
  const Geometry g = nvfp4_geometry(K, N);
  WorkspaceLayout w{};
  if (cfg.engine == 3) {  // the balanced GEMV's split tiles: at most kMaxSyncGroups blocks of M x 16
    w.sync_bytes = kSyncBytes;
    w.part_off = kSyncBytes;
    w.part_bytes = static_cast<size_t>(kMaxSyncGroups) * M * kTileCols * 4;
    w.total = align256(w.part_off + w.part_bytes);
    return w;
  }
  if (!argmax && cfg.ksplit == 1) return w;
  size_t off = kSyncBytes;
  w.sync_bytes = kSyncBytes;
  if (argmax) {
    const size_t groups = cfg.engine == 2 ? kMaxStreamGroups
                          : cfg.ksplit > 1 ? finalize_groups(N) : (g.nt + cfg.ct - 1) / cfg.ct;
    w.keys_off = off;
    w.keys_bytes = groups * M * 8;
    off = align256(off + w.keys_bytes);
  }
  if (cfg.ksplit > 1) {
    const size_t cols = std::max(static_cast<size_t>(N),
                                 static_cast<size_t>((g.nt + cfg.ct - 1) / cfg.ct) * cfg.ct * kTileCols);
    w.part_off = off;
    w.part_bytes = static_cast<size_t>(cfg.ksplit) * M * cols * 4;
    off = align256(off + w.part_bytes);
  }
  w.total = off;
  return w;
}

// The MFMA engine adds its K splits inside the kernel (as nvfp4_uses_xsplit)
// when the tile groups fit the arrival counters; the VALU engine's splits go
// to the split reduction kernel.
bool fp8_uses_xsplit(const LaunchCfg& cfg, int N) {
  const int nt = (N + kTileCols - 1) / kTileCols;
  const int64_t reach = static_cast<int64_t>(cfg.ksplit + 16) * 8 * cfg.ct * kTileCols * 4;
  return cfg.engine == 1 && cfg.ksplit > 1 && (nt + cfg.ct - 1) / cfg.ct <= kMaxSyncGroups &&
         reach < (int64_t{1} << 30);
}

// Partial sums of a K split: fp32, ksplit x M x (the tiles' columns), laid
// out [split][m][n] for the split reduction kernel or in one [m][column] block
// per (tile group, split) for the in-kernel reduction; the size covers both.
WorkspaceLayout fp8_workspace_layout(const LaunchCfg& cfg, int M, int K, int N) {
  (void)K;
  WorkspaceLayout w{};
  if (cfg.ksplit == 1) return w;
  const int nt = (N + kTileCols - 1) / kTileCols;
  const size_t cols = std::max(static_cast<size_t>(N), static_cast<size_t>((nt + cfg.ct - 1) / cfg.ct) * cfg.ct * kTileCols);
  size_t off = kSyncBytes;
  w.sync_bytes = kSyncBytes;
  w.part_off = off;
  w.part_bytes = static_cast<size_t>(cfg.ksplit) * M * cols * 4;
  off = align256(off + w.part_bytes);
  w.total = off;
  return w;
}

}  // namespace skinny

extern "C" {

const char* skinny_strerror(int status) {
  switch (status) {
    case SKINNY_OK: return "ok";
    case SKINNY_EINVAL: return "invalid argument (null pointer or bad value)";
    case SKINNY_ESHAPE: return "unsupported shape (M in 1..8, K % 16 == 0, N >= 1)";
    case SKINNY_EALIGN: return "device pointer not aligned";
    case SKINNY_ESIZE: return "buffer or workspace too small";
    case SKINNY_EHIP: return "HIP runtime or launch error";
    case SKINNY_EFORMAT: return "bad format (NaN scale byte or bad blob)";
    default: return "unknown status";
  }
}

size_t skinny_workspace_bytes_config(int op, int M, int K, int N, int engine, int ct, int nw, int ksplit) {
  if (check_shape(M, K, N)) return 0;
  const LaunchCfg c{engine, ct, nw, ksplit};
  switch (op) {
    case 0: return nvfp4_cfg_supported(c, M, K, false) ? nvfp4_workspace_layout(c, M, K, N, false).total : 0;
    case 1: return fp8_cfg_supported(c, M, K) ? fp8_workspace_layout(c, M, K, N).total : 0;
    case 2: return nvfp4_cfg_supported(c, M, K, true) ? nvfp4_workspace_layout(c, M, K, N, true).total : 0;
    case 3:
      return swiglu_shape(M, K, N) == SKINNY_OK && c.engine != 3 && nvfp4_cfg_supported(c, M, K, false)
                 ? nvfp4_workspace_layout(c, M, K, swiglu_packed_cols(N), false).total
                 : 0;
    default: return 0;
  }
}

int skinny_config_supported(int op, int M, int K, int N, int engine, int ct, int nw, int ksplit) {
  if (check_shape(M, K, N)) return 0;
  const LaunchCfg c{engine, ct, nw, ksplit};
  switch (op) {
    case 0: return nvfp4_cfg_supported(c, M, K, false) ? 1 : 0;
    case 1: return fp8_cfg_supported(c, M, K) ? 1 : 0;
    case 2: return nvfp4_cfg_supported(c, M, K, true) ? 1 : 0;
    case 3: return swiglu_shape(M, K, N) == SKINNY_OK && c.engine != 3 && nvfp4_cfg_supported(c, M, K, false) ? 1 : 0;
    default: return 0;
  }
}

int skinny_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!buf || !sink) return SKINNY_EINVAL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return SKINNY_EALIGN;
  if (bytes < 9216 || bytes / 9216 >= (static_cast<size_t>(1) << 31)) return SKINNY_ESIZE;
  return launch_status(launch_read_probe(buf, bytes, sink, stream));
}

int skinny_read_probe_pattern(const void* buf, size_t bytes, int pattern, int a, int b, uint32_t* sink,
                              size_t* bytes_read, hipStream_t stream) {
  if (!buf || !sink) return SKINNY_EINVAL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return SKINNY_EALIGN;
  size_t block = 0, groups = 0, read = 0;
  switch (pattern) {
    case 0: case 1: case 2:
      if (a < 1 || a > kMaxWaves) return SKINNY_EINVAL;
      block = pattern == 0 ? 9216 : pattern == 1 ? 4096 : 18432;
      read = bytes / block * block;
      groups = (bytes / block + a - 1) / a;
      break;
    case 3:
      if (a < 1 || a > kMaxWaves) return SKINNY_EINVAL;
      block = static_cast<size_t>(a) * kUnitBytes;   // one tile of a spans
      read = bytes / block * block;
      groups = bytes / block;
      break;
    case 4: case 5: case 6:
      if (a < 1 || a > 65535 || b < 1 || b > kMaxWaves) return SKINNY_EINVAL;
      block = kUnitBytes;
      read = bytes / block * block;
      groups = static_cast<size_t>(a);
      break;
    default:
      return SKINNY_EINVAL;
  }
  if (read == 0 || groups >= (static_cast<size_t>(1) << 31)) return SKINNY_ESIZE;
  if (bytes_read) *bytes_read = read;
  return launch_status(launch_read_probe_pattern(buf, bytes, pattern, a, b, sink, stream));
}

int skinny_default_config(int op, int M, int K, int N, int* engine, int* ct, int* nw, int* ksplit) {
  if (!engine || !ct || !nw || !ksplit) return SKINNY_EINVAL;
  if (op < 0 || op > 3) return SKINNY_EINVAL;
  if (op == 3 ? swiglu_shape(M, K, N) : check_shape(M, K, N)) return SKINNY_ESHAPE;
  const LaunchCfg c = op == 1   ? default_fp8_cfg(M, K, N)
                      : op == 3 ? default_nvfp4_cfg(M, K, swiglu_packed_cols(N), false, true)
                                : default_nvfp4_cfg(M, K, N, op == 2);
  *engine = c.engine;
  *ct = c.ct;
  *nw = c.nw;
  *ksplit = c.ksplit;
  return SKINNY_OK;
}

size_t skinny_workspace_bytes(int op, int M, int K, int N) {
  if (check_shape(M, K, N)) return 0;
  switch (op) {
    case 0: return nvfp4_workspace_layout(default_nvfp4_cfg(M, K, N, false), M, K, N, false).total;
    case 1: return fp8_workspace_layout(default_fp8_cfg(M, K, N), M, K, N).total;
    case 2: return nvfp4_workspace_layout(default_nvfp4_cfg(M, K, N, true), M, K, N, true).total;
    case 3: {
      if (swiglu_shape(M, K, N)) return 0;
      const int Np = swiglu_packed_cols(N);
      return nvfp4_workspace_layout(default_nvfp4_cfg(M, K, Np, false, true), M, K, Np, false).total;
    }
    default: return 0;
  }
}

}  // extern "C"

namespace {

static_assert(offsetof(Nvfp4Header, g) == kGOffset && offsetof(Nvfp4Header, g2) == kG2Offset,
              "header field offsets");

bool has_nan_scale(const uint8_t* scales, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if ((scales[i] & 0x7F) == 0x7F) return true;
  return false;
}

// Writes the header and the span-major units of canonical codes [N][K/2] and
// scales [N][K/16] into blob (geo.total_bytes, zeroed here first).
void write_blob(const uint8_t* codes, const uint8_t* scales, int K, int N, float g, float g2, uint32_t kind,
                int F, uint8_t* blob) {
  const Geometry geo = nvfp4_geometry(K, N);
  std::memset(blob, 0, geo.total_bytes);
  Nvfp4Header h{};
  h.magic = kBlobMagic;
  h.version = kBlobVersion;
  h.K = K;
  h.N = N;
  h.ku = geo.ku;
  h.nt = geo.nt;
  h.unit_bytes = kUnitBytes;
  h.g = g;
  h.units_off = kHeaderBytes;
  h.units_bytes = geo.units_bytes;
  h.g2 = g2;
  h.kind = kind;
  h.F = static_cast<uint32_t>(F);
  std::memcpy(blob, &h, sizeof(h));

  const size_t row_codes = K / 2, row_scales = K / 16;
  for (int t = 0; t < geo.nt; ++t) {
    for (int u = 0; u < geo.ku; ++u) {
      uint8_t* unit = blob + kHeaderBytes + (static_cast<size_t>(u) * geo.nt + t) * kUnitBytes;
      uint8_t* svec = unit + kChunksPerUnit * kChunkBytes;
      for (int lane = 0; lane < 64; ++lane) {
        const int grp = lane >> 4, c = lane & 15;
        const int n = t * kTileCols + c;
        if (n >= N) continue;
        for (int j = 0; j < kChunksPerUnit; ++j) {
          const int k0 = u * kUnitK + j * kChunkK + grp * 32;  // this lane's 32-K run
          if (k0 >= K) break;                                  // K % 16 == 0: runs end on blocks
          uint8_t* dst = unit + j * kChunkBytes + lane * 16;
          for (int i = 0; i < 16 && k0 + 2 * i < K; ++i)
            dst[i] = codes[static_cast<size_t>(n) * row_codes + (k0 + 2 * i) / 2];
          for (int half = 0; half < 2 && k0 + 16 * half < K; ++half)
            svec[lane * 16 + 2 * j + half] = scales[static_cast<size_t>(n) * row_scales + (k0 + 16 * half) / 16];
        }
      }
    }
  }
}

}  // namespace

extern "C" {

int nvfp4_pack(const uint8_t* codes, const uint8_t* scales, float gscale, int K, int N,
               void* out, size_t* out_bytes) {
  if (!codes || !scales || !out_bytes) return SKINNY_EINVAL;
  if (K < 16 || K % 16 != 0 || K > kMaxK || N < 1 || N > kMaxN) return SKINNY_ESHAPE;
  if (!std::isfinite(gscale) || gscale < 0.0f) return SKINNY_EINVAL;
  const Geometry geo = nvfp4_geometry(K, N);
  if (!out) {
    *out_bytes = geo.total_bytes;
    return SKINNY_OK;
  }
  if (*out_bytes < geo.total_bytes) return SKINNY_ESIZE;
  if (has_nan_scale(scales, static_cast<size_t>(N) * (K / 16))) return SKINNY_EFORMAT;
  write_blob(codes, scales, K, N, gscale, gscale, kKindPlain, 0, static_cast<uint8_t*>(out));
  *out_bytes = geo.total_bytes;
  return SKINNY_OK;
}

int nvfp4_pack_swiglu(const uint8_t* gate_codes, const uint8_t* gate_scales, float gate_g,
                      const uint8_t* up_codes, const uint8_t* up_scales, float up_g, int K, int F,
                      void* out, size_t* out_bytes) {
  if (!gate_codes || !gate_scales || !up_codes || !up_scales || !out_bytes) return SKINNY_EINVAL;
  if (K < 16 || K % 16 != 0 || K > kMaxK || F < 1 || F > kMaxN / 2) return SKINNY_ESHAPE;
  if (!std::isfinite(gate_g) || gate_g < 0.0f || !std::isfinite(up_g) || up_g < 0.0f) return SKINNY_EINVAL;
  const int N = swiglu_packed_cols(F);
  const Geometry geo = nvfp4_geometry(K, N);
  if (!out) {
    *out_bytes = geo.total_bytes;
    return SKINNY_OK;
  }
  if (*out_bytes < geo.total_bytes) return SKINNY_ESIZE;
  const size_t row_codes = K / 2, row_scales = K / 16;
  if (has_nan_scale(gate_scales, static_cast<size_t>(F) * row_scales) ||
      has_nan_scale(up_scales, static_cast<size_t>(F) * row_scales))
    return SKINNY_EFORMAT;
  // Canonical arrays of the interleaved N columns: packed column 16t + c is
  // gate column 8t + c (c < 8) or up column 8t + c - 8, zero past F.
  std::vector<uint8_t> codes(static_cast<size_t>(N) * row_codes, 0), scales(static_cast<size_t>(N) * row_scales, 0);
  for (int n = 0; n < N; ++n) {
    const int c = n % kTileCols, f = (n / kTileCols) * 8 + (c & 7);
    if (f >= F) continue;
    const uint8_t* sc = c < 8 ? gate_codes : up_codes;
    const uint8_t* ss = c < 8 ? gate_scales : up_scales;
    std::memcpy(codes.data() + static_cast<size_t>(n) * row_codes, sc + static_cast<size_t>(f) * row_codes, row_codes);
    std::memcpy(scales.data() + static_cast<size_t>(n) * row_scales, ss + static_cast<size_t>(f) * row_scales,
                row_scales);
  }
  write_blob(codes.data(), scales.data(), K, N, gate_g, up_g, kKindSwiglu, F, static_cast<uint8_t*>(out));
  *out_bytes = geo.total_bytes;
  return SKINNY_OK;
}

size_t fp8_packed_bytes(int K, int N) {
  const size_t ku = (K + kFp8PackK - 1) / kFp8PackK, nt = (N + kTileCols - 1) / kTileCols;
  return kHeaderBytes + ku * nt * kFp8UnitBytes;
}

int fp8_pack(const uint8_t* codes, int K, int N, void* out, size_t* out_bytes) {
  if (!codes || !out_bytes) return SKINNY_EINVAL;
  if (K < 16 || K % 16 != 0 || K > kMaxK || N < 1 || N > kMaxN) return SKINNY_ESHAPE;
  const size_t total = fp8_packed_bytes(K, N);
  if (!out) {
    *out_bytes = total;
    return SKINNY_OK;
  }
  if (*out_bytes < total) return SKINNY_ESIZE;
  const int ku = (K + kFp8PackK - 1) / kFp8PackK, nt = (N + kTileCols - 1) / kTileCols;
  uint8_t* blob = static_cast<uint8_t*>(out);
  std::memset(blob, 0, total);
  Fp8Header h{};
  h.magic = kFp8BlobMagic;
  h.version = kFp8BlobVersion;
  h.K = K;
  h.N = N;
  h.ku = ku;
  h.nt = nt;
  h.unit_bytes = kFp8UnitBytes;
  h.units_off = kHeaderBytes;
  h.units_bytes = total - kHeaderBytes;
  std::memcpy(blob, &h, sizeof(h));
  // Piece q = 2j + h of unit (t, u), lane l = 16grp + c: 16 codes of column
  // 16t + 8(c % 2) + c / 2 from K = 512u + 128j + 32grp + 16h on (K % 16 ==
  // 0: a run is all in or all out of range).
  parallel_for(nt, [&](int, int t0, int t1) {
    for (int t = t0; t < t1; ++t)
      for (int u = 0; u < ku; ++u) {
        uint8_t* unit = blob + kHeaderBytes + (static_cast<size_t>(u) * nt + t) * kFp8UnitBytes;
        for (int q = 0; q < 8; ++q)
          for (int lane = 0; lane < 64; ++lane) {
            const int n = t * kTileCols + 8 * (lane & 1) + ((lane & 15) >> 1);
            const int k = u * kFp8PackK + (q >> 1) * 128 + (lane >> 4) * 32 + (q & 1) * 16;
            if (n < N && k < K)
              std::memcpy(unit + q * 1024 + lane * 16, codes + static_cast<size_t>(n) * K + k, 16);
          }
      }
  });
  *out_bytes = total;
  return SKINNY_OK;
}

int nvfp4_quantize(const float* w, int K, int N, uint8_t* codes, uint8_t* scales, float* g_out) {
  if (!w || !codes || !scales || !g_out) return SKINNY_EINVAL;
  if (K < 16 || K % 16 != 0 || K > kMaxK || N < 1 || N > kMaxN) return SKINNY_ESHAPE;
  const size_t total = static_cast<size_t>(K) * N;
  std::vector<double> part_amax(host_threads(), 0.0);
  std::vector<char> part_bad(part_amax.size(), 0);
  parallel_for(K, [&](int t, int k0, int k1) {
    double a = 0.0;
    for (size_t i = static_cast<size_t>(k0) * N; i < static_cast<size_t>(k1) * N; ++i) {
      const float v = w[i];
      if (!std::isfinite(v)) { part_bad[t] = 1; return; }
      a = std::fmax(a, std::fabs(static_cast<double>(v)));
    }
    part_amax[t] = a;
  });
  double amax = 0.0;
  for (size_t t = 0; t < part_amax.size(); ++t) {
    if (part_bad[t]) return SKINNY_EINVAL;
    amax = std::fmax(amax, part_amax[t]);
  }
  const float g = static_cast<float>(amax / (6.0 * 448.0));
  *g_out = g;
  const size_t row_codes = K / 2, row_scales = K / 16;
  std::memset(codes, 0, row_codes * N);
  std::memset(scales, 0, row_scales * N);
  if (g == 0.0f) return SKINNY_OK;
  const double gd = g;
  // One 16-row K block at a time, every column of it (rows of w are contiguous in n).
  parallel_for(K / 16, [&](int, int b0, int b1) {
    std::vector<double> bmax(N), denom(N);
    for (int b = b0; b < b1; ++b) {
      const float* rows = w + static_cast<size_t>(b) * 16 * N;
      std::fill(bmax.begin(), bmax.end(), 0.0);
      for (int i = 0; i < 16; ++i)
        for (int n = 0; n < N; ++n)
          bmax[n] = std::fmax(bmax[n], std::fabs(static_cast<double>(rows[static_cast<size_t>(i) * N + n])));
      for (int n = 0; n < N; ++n) {
        const int sc = e4m3_code((bmax[n] / 6.0) / gd);
        scales[static_cast<size_t>(n) * row_scales + b] = static_cast<uint8_t>(sc);
        denom[n] = e4m3_value(sc & 0x7F) * gd;
      }
      for (int i = 0; i < 8; ++i) {
        const float* lo_row = rows + static_cast<size_t>(2 * i) * N;
        const float* hi_row = lo_row + N;
        for (int n = 0; n < N; ++n) {
          if (denom[n] == 0.0) continue;
          const int lo = e2m1_code(static_cast<double>(lo_row[n]) / denom[n]);
          const int hi = e2m1_code(static_cast<double>(hi_row[n]) / denom[n]);
          codes[static_cast<size_t>(n) * row_codes + b * 8 + i] = static_cast<uint8_t>(lo | (hi << 4));
        }
      }
    }
  });
  return SKINNY_OK;
}

int fp8_quantize(const float* w, int K, int N, uint8_t* codes, float* scales) {
  if (!w || !codes || !scales) return SKINNY_EINVAL;
  if (K < 1 || K > kMaxK || N < 1 || N > kMaxN) return SKINNY_ESHAPE;
  std::vector<char> part_bad(host_threads(), 0);
  parallel_for(K, [&](int t, int k0, int k1) {
    for (size_t i = static_cast<size_t>(k0) * N; i < static_cast<size_t>(k1) * N; ++i)
      if (!std::isfinite(w[i])) { part_bad[t] = 1; return; }
  });
  for (char bad : part_bad)
    if (bad) return SKINNY_EINVAL;
  const int KB = (K + 127) / 128, NB = (N + 127) / 128;
  std::memset(codes, 0, static_cast<size_t>(K) * N);
  // One 128-row K block at a time, every column block of it.
  parallel_for(KB, [&](int, int kb0, int kb1) {
    std::vector<double> bmax(NB);
    for (int kb = kb0; kb < kb1; ++kb) {
      const int k1 = std::min(K, kb * 128 + 128);
      std::fill(bmax.begin(), bmax.end(), 0.0);
      for (int k = kb * 128; k < k1; ++k)
        for (int n = 0; n < N; ++n)
          bmax[n / 128] = std::fmax(bmax[n / 128], std::fabs(static_cast<double>(w[static_cast<size_t>(k) * N + n])));
      for (int nb = 0; nb < NB; ++nb) scales[static_cast<size_t>(nb) * KB + kb] = static_cast<float>(bmax[nb] / 448.0);
      for (int k = kb * 128; k < k1; ++k)
        for (int n = 0; n < N; ++n) {
          const double Sd = scales[static_cast<size_t>(n / 128) * KB + kb];
          if (Sd == 0.0) continue;
          codes[static_cast<size_t>(n) * K + k] =
              static_cast<uint8_t>(e4m3_code(static_cast<double>(w[static_cast<size_t>(k) * N + n]) / Sd));
        }
    }
  });
  return SKINNY_OK;
}

int nvfp4_gemm_config(const void* w_packed, const uint16_t* x, uint16_t* y, int M, int K, int N,
                      void* workspace, size_t workspace_bytes, hipStream_t stream,
                      int engine, int ct, int nw, int ksplit) {
  int s = nvfp4_common_checks(w_packed, x, y, M, K, N);
  if (s) return s;
  if (!aligned(y, 16)) return SKINNY_EALIGN;
  const LaunchCfg cfg{engine, ct, nw, ksplit};
  if (!nvfp4_cfg_supported(cfg, M, K, false)) return SKINNY_EINVAL;
  s = check_workspace(workspace, workspace_bytes, nvfp4_workspace_layout(cfg, M, K, N, false).total);
  if (s) return s;
  return launch_status(launch_nvfp4(static_cast<const uint8_t*>(w_packed), x, y, M, K, N, cfg,
                                    nullptr, workspace, stream));
}

}  // extern "C"

namespace skinny {

int nvfp4_gemm_host_checks(const void* w_packed, const uint16_t* x, const uint16_t* y, int M, int K, int N,
                           size_t* workspace_need) {
  int s = nvfp4_common_checks(w_packed, x, y, M, K, N);
  if (s) return s;
  if (!aligned(y, 16)) return SKINNY_EALIGN;
  *workspace_need = nvfp4_workspace_layout(default_nvfp4_cfg(M, K, N, false), M, K, N, false).total;
  return SKINNY_OK;
}

}  // namespace skinny

extern "C" {

int nvfp4_gemm(const void* w_packed, const uint16_t* x, uint16_t* y, int M, int K, int N,
               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int s = check_shape(M, K, N);
  if (s) return s;
  const LaunchCfg c = default_nvfp4_cfg(M, K, N, false);
  return nvfp4_gemm_config(w_packed, x, y, M, K, N, workspace, workspace_bytes, stream, c.engine, c.ct,
                           c.nw, c.ksplit);
}

int fp8_gemm_config(const uint8_t* w, const float* block_scales, const uint16_t* x, uint16_t* y,
                    int M, int K, int N, void* workspace, size_t workspace_bytes,
                    hipStream_t stream, int engine, int ct, int nw, int ksplit) {
  if (!w || !block_scales || !x || !y) return SKINNY_EINVAL;
  int s = check_shape(M, K, N);
  if (s) return s;
  if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 16) || !aligned(block_scales, 4))
    return SKINNY_EALIGN;
  const LaunchCfg cfg{engine, ct, nw, ksplit};
  if (!fp8_cfg_supported(cfg, M, K)) return SKINNY_EINVAL;
  s = check_workspace(workspace, workspace_bytes, fp8_workspace_layout(cfg, M, K, N).total);
  if (s) return s;
  return launch_status(launch_fp8(w, block_scales, x, y, M, K, N, cfg, workspace, stream));
}

int fp8_gemm_packed_config(const void* w_packed, const float* block_scales, const uint16_t* x, uint16_t* y,
                           int M, int K, int N, void* workspace, size_t workspace_bytes, hipStream_t stream,
                           int engine, int ct, int nw, int ksplit) {
  if (!w_packed || !block_scales || !x || !y) return SKINNY_EINVAL;
  int s = check_shape(M, K, N);
  if (s) return s;
  if (!aligned(w_packed, 16) || !aligned(x, 16) || !aligned(y, 16) || !aligned(block_scales, 4))
    return SKINNY_EALIGN;
  const LaunchCfg cfg{engine, ct, nw, ksplit};
  if (!fp8_cfg_supported(cfg, M, K)) return SKINNY_EINVAL;
  s = check_workspace(workspace, workspace_bytes, fp8_workspace_layout(cfg, M, K, N).total);
  if (s) return s;
  return launch_status(launch_fp8(static_cast<const uint8_t*>(w_packed), block_scales, x, y, M, K, N, cfg,
                                  workspace, stream, true));
}

int fp8_gemm_packed(const void* w_packed, const float* block_scales, const uint16_t* x, uint16_t* y, int M,
                    int K, int N, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int s = check_shape(M, K, N);
  if (s) return s;
  const LaunchCfg c = default_fp8_cfg(M, K, N);
  return fp8_gemm_packed_config(w_packed, block_scales, x, y, M, K, N, workspace, workspace_bytes, stream,
                                c.engine, c.ct, c.nw, c.ksplit);
}

int fp8_gemm(const uint8_t* w, const float* block_scales, const uint16_t* x, uint16_t* y,
             int M, int K, int N, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int s = check_shape(M, K, N);
  if (s) return s;
  const LaunchCfg c = default_fp8_cfg(M, K, N);
  return fp8_gemm_config(w, block_scales, x, y, M, K, N, workspace, workspace_bytes, stream,
                         c.engine, c.ct, c.nw, c.ksplit);
}

int nvfp4_gemm_swiglu_config(const void* w_packed, const uint16_t* x, uint16_t* h, int M, int K, int F,
                             void* workspace, size_t workspace_bytes, hipStream_t stream, int engine, int ct,
                             int nw, int ksplit) {
  int s = swiglu_shape(M, K, F);
  if (s) return s;
  s = nvfp4_common_checks(w_packed, x, h, M, K, F);
  if (s) return s;
  if (!aligned(h, 16)) return SKINNY_EALIGN;
  const int N = swiglu_packed_cols(F);
  const LaunchCfg cfg{engine, ct, nw, ksplit};
  if (cfg.engine == 3 || !nvfp4_cfg_supported(cfg, M, K, false)) return SKINNY_EINVAL;  // 3: plain epilogue only
  s = check_workspace(workspace, workspace_bytes, nvfp4_workspace_layout(cfg, M, K, N, false).total);
  if (s) return s;
  return launch_status(launch_nvfp4(static_cast<const uint8_t*>(w_packed), x, h, M, K, N, cfg, nullptr,
                                    workspace, stream, F));
}

int nvfp4_gemm_swiglu(const void* w_packed, const uint16_t* x, uint16_t* h, int M, int K, int F,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int s = swiglu_shape(M, K, F);
  if (s) return s;
  const LaunchCfg c = default_nvfp4_cfg(M, K, swiglu_packed_cols(F), false, true);
  return nvfp4_gemm_swiglu_config(w_packed, x, h, M, K, F, workspace, workspace_bytes, stream, c.engine, c.ct,
                                  c.nw, c.ksplit);
}

int lm_head_gemm_argmax_config(const void* w_packed, const uint16_t* x, int32_t* idx,
                               uint16_t* logits, int M, int K, int N, void* workspace,
                               size_t workspace_bytes, hipStream_t stream, int engine, int ct,
                               int nw, int ksplit) {
  int s = nvfp4_common_checks(w_packed, x, idx, M, K, N);
  if (s) return s;
  if (!aligned(idx, 4) || (logits && !aligned(logits, 16))) return SKINNY_EALIGN;
  const LaunchCfg cfg{engine, ct, nw, ksplit};
  if (!nvfp4_cfg_supported(cfg, M, K, true)) return SKINNY_EINVAL;
  s = check_workspace(workspace, workspace_bytes, nvfp4_workspace_layout(cfg, M, K, N, true).total);
  if (s) return s;
  return launch_status(launch_nvfp4(static_cast<const uint8_t*>(w_packed), x, logits, M, K, N, cfg,
                                    idx, workspace, stream));
}

int lm_head_verify_greedy_config(const void* w_packed, const uint16_t* x, const int32_t* drafts,
                                 int32_t* idx, int32_t* result, int M, int K, int N, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream, int engine, int ct, int nw,
                                 int ksplit) {
  int s = nvfp4_common_checks(w_packed, x, idx, M, K, N);
  if (s) return s;
  if (!result || (M > 1 && !drafts)) return SKINNY_EINVAL;
  if (!aligned(idx, 4) || !aligned(result, 4) || (drafts && !aligned(drafts, 4))) return SKINNY_EALIGN;
  const LaunchCfg cfg{engine, ct, nw, ksplit};
  if (!nvfp4_cfg_supported(cfg, M, K, true)) return SKINNY_EINVAL;
  s = check_workspace(workspace, workspace_bytes, nvfp4_workspace_layout(cfg, M, K, N, true).total);
  if (s) return s;
  return launch_status(launch_nvfp4(static_cast<const uint8_t*>(w_packed), x, nullptr, M, K, N, cfg, idx,
                                    workspace, stream, 0, drafts, result));
}

int lm_head_verify_greedy(const void* w_packed, const uint16_t* x, const int32_t* drafts, int32_t* idx,
                          int32_t* result, int M, int K, int N, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  int s = check_shape(M, K, N);
  if (s) return s;
  const LaunchCfg c = default_nvfp4_cfg(M, K, N, true);
  return lm_head_verify_greedy_config(w_packed, x, drafts, idx, result, M, K, N, workspace, workspace_bytes,
                                      stream, c.engine, c.ct, c.nw, c.ksplit);
}

// Host-side checks and workspace need of one layer of a mixed-allocation
// table, exactly those of the call the layer maps to (so that a table is
// rejected before anything is enqueued).
static int layer_check(const skinny_layer& l, const uint16_t* x, const uint16_t* y, int M, size_t* need) {
  switch (l.kind) {
    case SKINNY_LAYER_NVFP4: {
      int s = nvfp4_common_checks(l.weights, x, y, M, l.K, l.N);
      if (s) return s;
      if (!aligned(y, 16)) return SKINNY_EALIGN;
      *need = nvfp4_workspace_layout(default_nvfp4_cfg(M, l.K, l.N, false), M, l.K, l.N, false).total;
      return SKINNY_OK;
    }
    case SKINNY_LAYER_FP8:
    case SKINNY_LAYER_FP8_PACKED: {
      if (!l.weights || !l.scales || !x || !y) return SKINNY_EINVAL;
      int s = check_shape(M, l.K, l.N);
      if (s) return s;
      if (!aligned(l.weights, 16) || !aligned(x, 16) || !aligned(y, 16) || !aligned(l.scales, 4))
        return SKINNY_EALIGN;
      *need = fp8_workspace_layout(default_fp8_cfg(M, l.K, l.N), M, l.K, l.N).total;
      return SKINNY_OK;
    }
    case SKINNY_LAYER_SWIGLU: {
      int s = swiglu_shape(M, l.K, l.N);
      if (s) return s;
      s = nvfp4_common_checks(l.weights, x, y, M, l.K, l.N);
      if (s) return s;
      if (!aligned(y, 16)) return SKINNY_EALIGN;
      const int Np = swiglu_packed_cols(l.N);
      *need = nvfp4_workspace_layout(default_nvfp4_cfg(M, l.K, Np, false, true), M, l.K, Np, false).total;
      return SKINNY_OK;
    }
    default:
      return SKINNY_EINVAL;
  }
}

size_t skinny_layers_workspace_bytes(const skinny_layer* layers, int n, int M) {
  if (!layers || n < 1) return 0;
  size_t most = 0;
  const uint16_t* fake = reinterpret_cast<const uint16_t*>(static_cast<uintptr_t>(256));  // aligned stand-in
  for (int i = 0; i < n; ++i) {
    skinny_layer l = layers[i];
    if (!l.weights) l.weights = fake;
    if ((l.kind == SKINNY_LAYER_FP8 || l.kind == SKINNY_LAYER_FP8_PACKED) && !l.scales)
      l.scales = reinterpret_cast<const float*>(fake);
    size_t need = 0;
    if (layer_check(l, fake, fake, M, &need) != SKINNY_OK) return 0;
    most = std::max(most, need);
  }
  return most;
}

int skinny_layers_run(const skinny_layer* layers, int n, const uint16_t* const* x, uint16_t* const* y, int M,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!layers || !x || !y || n < 1) return SKINNY_EINVAL;
  for (int i = 0; i < n; ++i) {
    size_t need = 0;
    int s = layer_check(layers[i], x[i], y[i], M, &need);
    if (s) return s;
    s = check_workspace(workspace, workspace_bytes, need);
    if (s) return s;
  }
  for (int i = 0; i < n; ++i) {
    const skinny_layer& l = layers[i];
    int s = SKINNY_OK;
    if (l.kind == SKINNY_LAYER_NVFP4)
      s = nvfp4_gemm(l.weights, x[i], y[i], M, l.K, l.N, workspace, workspace_bytes, stream);
    else if (l.kind == SKINNY_LAYER_FP8)
      s = fp8_gemm(static_cast<const uint8_t*>(l.weights), l.scales, x[i], y[i], M, l.K, l.N, workspace,
                   workspace_bytes, stream);
    else if (l.kind == SKINNY_LAYER_FP8_PACKED)
      s = fp8_gemm_packed(l.weights, l.scales, x[i], y[i], M, l.K, l.N, workspace, workspace_bytes, stream);
    else
      s = nvfp4_gemm_swiglu(l.weights, x[i], y[i], M, l.K, l.N, workspace, workspace_bytes, stream);
    if (s) return s;  // only a launch error can get here
  }
  return SKINNY_OK;
}

int lm_head_gemm_argmax(const void* w_packed, const uint16_t* x, int32_t* idx, uint16_t* logits,
                        int M, int K, int N, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  int s = check_shape(M, K, N);
  if (s) return s;
  const LaunchCfg c = default_nvfp4_cfg(M, K, N, true);
  return lm_head_gemm_argmax_config(w_packed, x, idx, logits, M, K, N, workspace, workspace_bytes,
                                    stream, c.engine, c.ct, c.nw, c.ksplit);
}

}  // extern "C"
