// Host side of the fp8 rowwise-scaled grouped GEMM C ABI: argument checks,
// launch planning (tile configuration, tails, grid) and dispatch.
//
// Contracts follow MSLK pull request 471 ("Back the FP8 rowwise grouped GEMM ops
// with FlyDSL on ROCm"): the op refuses what it cannot compute instead of
// silently ignoring it (commits on strided outputs and on preshuffle refusals),
// a zero-length contraction returns a zeroed output (commit on zero-length
// reductions), and no benchmarking ever happens inside a call -- a fixed
// selector picks the tile (commit on the autotune policy).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "fp8gg.h"
#include "fp8gg_internal.h"

namespace {

thread_local std::string g_last_error;

fp8gg_status fail(fp8gg_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fp8gg_status ok() {
  g_last_error.clear();
  return FP8GG_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  const void* p;
  int64_t bytes;
  const char* name;
};

bool overlap(const Range& a, const Range& b) {
  if (a.bytes <= 0 || b.bytes <= 0 || !a.p || !b.p) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + static_cast<uintptr_t>(b.bytes) && b0 < a0 + static_cast<uintptr_t>(a.bytes);
}

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

// Packed layouts put the groups one after another along M (total rows M); slab
// layouts give each group M rows (total rows G * M).
bool packed(int layout) { return layout == FP8GG_LAYOUT_STACKED || layout == FP8GG_LAYOUT_OFFSETS; }
bool ragged(int layout) { return layout == FP8GG_LAYOUT_N_OFFSETS || layout == FP8GG_LAYOUT_K_OFFSETS; }
// Rows of Y: the n_offsets layout puts the groups side by side along N.
int64_t total_rows(int layout, int64_t G, int64_t M) {
  return packed(layout) || layout == FP8GG_LAYOUT_N_OFFSETS ? M : G * M;
}

// Element counts of each operand of a call (for size and aliasing checks).
struct Extents {
  int64_t x, w, xs, ws, y;
};
Extents extents(int layout, int64_t G, int64_t M, int64_t N, int64_t K) {
  const int64_t rows = total_rows(layout, G, M);
  switch (layout) {
    case FP8GG_LAYOUT_N_OFFSETS: return {G * M * K, N * K, G * M, N, rows * N};
    case FP8GG_LAYOUT_K_OFFSETS: return {M * K, N * K, G * M, G * N, rows * N};
    default: {
      const int64_t xrows = packed(layout) ? M : G * M;
      return {xrows * K, G * N * K, xrows, G * N, rows * N};
    }
  }
}

// Shape checks shared by plan() and the entry points.
fp8gg_status check_shape(int layout, int preshuffled, int64_t G, int64_t M, int64_t N, int64_t K) {
  if (layout < FP8GG_LAYOUT_STACKED || layout > FP8GG_LAYOUT_K_OFFSETS)
    return fail(FP8GG_ERR_INVALID_ARGUMENT, "unknown layout %d", layout);
  if (preshuffled && ragged(layout))
    return fail(FP8GG_ERR_UNSUPPORTED_SHAPE,
                "pre-shuffled weights interleave N and K across the whole matrix; the n_offsets and k_offsets "
                "layouts partition those axes, so they take plain weights only");
  if (G < 0 || M < 0 || N < 0 || K < 0)
    return fail(FP8GG_ERR_INVALID_ARGUMENT, "negative size (G=%lld M=%lld N=%lld K=%lld)", (long long)G,
                (long long)M, (long long)N, (long long)K);
  if (K % 16 != 0)
    return fail(FP8GG_ERR_UNSUPPORTED_SHAPE, "K=%lld must be a multiple of 16", (long long)K);
  if (N % 8 != 0)
    return fail(FP8GG_ERR_UNSUPPORTED_SHAPE, "N=%lld must be a multiple of 8", (long long)N);
  if (preshuffled && (N % FP8GG_SHUFFLE_N != 0 || K % FP8GG_SHUFFLE_K != 0))
    return fail(FP8GG_ERR_UNSUPPORTED_SHAPE,
                "pre-shuffled weights need N %% %d == 0 and K %% %d == 0 (N=%lld K=%lld)", FP8GG_SHUFFLE_N,
                FP8GG_SHUFFLE_K, (long long)N, (long long)K);
  const int64_t lim = (int64_t(1) << 31) - 256;
  if (K > lim || N > lim || M > lim || G > lim)
    return fail(FP8GG_ERR_UNSUPPORTED_SHAPE, "a dimension exceeds 2^31-256");
  if (!packed(layout) && G * M > lim)
    return fail(FP8GG_ERR_UNSUPPORTED_SHAPE, "G*M exceeds 2^31-256 (G times the slab height)");
  // Every tensor's byte count (and so every 64-bit offset the kernels form) stays
  // far below overflow; 2^48 bytes is beyond any device memory.
  const int64_t rows = total_rows(layout, G, M);
  const int64_t cap = int64_t(1) << 48;
  auto too_big = [](int64_t a, int64_t b) { return a > 0 && b > (int64_t(1) << 48) / a; };
  const int64_t xrows = layout == FP8GG_LAYOUT_K_OFFSETS ? M : (packed(layout) ? M : G * M);
  const int64_t wrows = ragged(layout) ? N : G * N;
  if (too_big(xrows, K) || too_big(G, N) || (wrows > 0 && too_big(wrows, K)) || too_big(rows, 2 * N) ||
      G * M > cap / 4)
    return fail(FP8GG_ERR_UNSUPPORTED_SHAPE, "a tensor would exceed 2^48 bytes (G=%lld M=%lld N=%lld K=%lld)",
                (long long)G, (long long)M, (long long)N, (long long)K);
  return FP8GG_OK;
}

// Fixed selector (measured on MI355X; no benchmarking inside a call).  The key is
// the rows one group contributes on average -- total_M normalised by G for the
// packed layouts, the slab height otherwise -- because a tile only ever sees one
// group.
// Compute units the selector plans for (MI355X).  Only a heuristic: the persistent
// grid itself is sized from the device at launch.
constexpr int64_t kPlanCus = 256;

// The ragged layouts (n_offsets, k_offsets) run one tile per workgroup on the
// configurations compiled for them (2, 7, 9, 18, 21, 28), keyed on the slab
// height and, for n_offsets, on the columns a group owns on average.
bool ragged_config(int cfg) { return cfg == 2 || cfg == 7 || cfg == 9 || cfg == 18 || cfg == 21 || cfg == 28; }

int select_ragged(int layout, int64_t G, int64_t M, int64_t N) {
  const int64_t cols = layout == FP8GG_LAYOUT_N_OFFSETS && G > 0 ? (N + G - 1) / G : N;
  if (M >= 256 && cols >= 256) {
    // 256x256 tiles, unless 192x256 tiles still make a single round of the compute
    // units (bounded from the host: n_offsets column tiles <= ceil(N/256) + G - 1):
    // then the smaller tiles put more units to work.  Measured on 8 slabs of 512
    // rows, N = 16384: 198 tiles of 192x256 in 90.5 us against 132 of 256x256 in
    // 101.1 us; with several rounds (k_offsets, 1792 tiles) 256x256 stays ahead.
    const int64_t ub = (N + 255) / 256 + G - 1;
    const int64_t col_tiles = layout == FP8GG_LAYOUT_N_OFFSETS ? (ub < N ? ub : N) : G * ((N + 255) / 256);
    return ((M + 191) / 192) * col_tiles <= kPlanCus ? 28 : 7;
  }
  if (M >= 128) return 9;
  if (M >= 48) return 2;
  return cols <= 64 ? 21 : 18;
}

int select_config(int layout, int preshuffled, int64_t G, int64_t M, int64_t N, int64_t K) {
  (void)K;
  if (ragged(layout)) return select_ragged(layout, G, M, N);
  const int64_t per_group = packed(layout) ? (G > 0 ? (M + G - 1) / G : M) : M;
  const bool slab_with_padding = layout == FP8GG_LAYOUT_PADDED;
  // Calls with at least 256 rows per group whose tiles are all in use (every
  // layout but padded) run 256x256 tiles on the persistent grid (the last round as
  // quarter tiles); with 256 to 511 rows per group this measured 8% faster than
  // 128x256 tiles (down projection, M = 2048).
  if (!slab_with_padding && per_group >= 256) return preshuffled ? 26 : 16;
  if (preshuffled) {
    // The same tiles as for plain W, reading pre-shuffled blocks.
    if (per_group >= 512) {
      const int64_t tiles = G * ((M + 255) / 256) * ((N + 255) / 256);
      return tiles >= 2 * kPlanCus ? 25 : 4;
    }
    if (per_group >= 128) return 4;
    if (per_group >= 48) return 5;
    if (per_group <= 2) return 27;
    return 6;
  }
  if (per_group >= 512) {
    // Padded: 256x256 tiles unless they make fewer than two waves (padding tiles
    // retire at once, so the busy ones are fewer still); then 128x256.
    const int64_t tiles = G * ((M + 255) / 256) * ((N + 255) / 256);
    return tiles >= 2 * kPlanCus ? 7 : 9;
  }
  if (per_group >= 128) return 9;                  // 128x256, K stage 128
  if (per_group >= 48) return 2;
  // Small M: the weights stream from HBM once, so what matters is how many bytes
  // each compute unit keeps in flight.  Fewer rows than groups: few groups hold
  // rows, so each group's weights are spread over many workgroups (32 columns each,
  // K split over 4 waves, straight to registers).  Otherwise 32-row tiles with a
  // deep LDS pipeline: 32 x 64 for at most two rows per group, 32 x 128 with four
  // 128-byte stages above (3.4% faster than three stages at 32 rows per group,
  // level at 4).
  const int64_t rows = total_rows(layout, G, M);
  if (rows < G) return 15;
  if (per_group <= 2) return 21;
  return 20;
}

// Compute units of the current device (the persistent grid), cached per device.
int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  cache[dev] = cus;
  return cus;
}

fp8gg_status make_plan(int layout, int preshuffled, int64_t G, int64_t M, int64_t N, int64_t K,
                       fp8gg_plan* p) {
  std::memset(p, 0, sizeof *p);
  p->config_id = -1;
  fp8gg_status st = check_shape(layout, preshuffled, G, M, N, K);
  if (st != FP8GG_OK) return st;
  const int64_t rows = total_rows(layout, G, M);
  if (rows == 0 || N == 0) return FP8GG_OK;  // empty output: nothing to launch
  if (K == 0) {
    p->zero_fill = 1;
    return FP8GG_OK;
  }
  if (G == 0) return FP8GG_OK;  // packed rows that belong to no group are left untouched

  int cfg = select_config(layout, preshuffled, G, M, N, K);
  if (cfg < 0)
    return fail(FP8GG_ERR_UNSUPPORTED_SHAPE, "no kernel configuration for this call (preshuffled=%d)", preshuffled);
  const int forced = env_int("FP8GG_CONFIG", -1);
  if (forced >= 0) {
    if (forced >= fp8gg::kNumConfigs || fp8gg::is_preshuffled(fp8gg::kConfigs[forced]) != (preshuffled != 0))
      return fail(FP8GG_ERR_INVALID_ARGUMENT, "FP8GG_CONFIG=%d does not name a usable configuration", forced);
    cfg = forced;
  }
  if ((layout == FP8GG_LAYOUT_PADDED || ragged(layout)) && fp8gg::kConfigs[cfg].kind == fp8gg::kKindPersistent)
    cfg = fp8gg::kConfigs[cfg].twin;   // the persistent schedule covers the packed and batched layouts
  if (ragged(layout) && !ragged_config(cfg))
    return fail(FP8GG_ERR_INVALID_ARGUMENT, "configuration %d is not built for the n_offsets/k_offsets layouts", cfg);
  const fp8gg::KernelConfig& c = fp8gg::kConfigs[cfg];
  p->config_id = cfg;
  p->BM = c.BM;
  p->BN = c.BN;
  p->BK = c.BK;
  p->threads = c.WM * c.WN * 64;
  p->stages = c.stages;
  p->k_tail = (K % c.BK) != 0;
  p->n_tail = (N % c.BN) != 0;
  p->n_tiles = (N + c.BN - 1) / c.BN;
  if (packed(layout)) {
    // Sum over groups of ceil(M_g / BM) <= ceil(total_M / BM) + G - 1, and each
    // tile holds at least one row.
    int64_t ub = (M + c.BM - 1) / c.BM + G - 1;
    p->m_tiles = ub < M ? ub : M;
    p->grid = p->m_tiles * p->n_tiles;
    p->persistent = c.kind == fp8gg::kKindPersistent ? 1 : 0;
  } else if (layout == FP8GG_LAYOUT_N_OFFSETS) {
    // Column tiles over the groups' ranges: sum of ceil(N_g / BN) <= ceil(N / BN)
    // + G - 1, and each tile holds at least one column.
    const int64_t ub = (N + c.BN - 1) / c.BN + G - 1;
    p->n_tiles = ub < N ? ub : N;
    p->m_tiles = (M + c.BM - 1) / c.BM;
    p->grid = p->m_tiles * p->n_tiles;
  } else if (layout == FP8GG_LAYOUT_K_OFFSETS) {
    // Group slices are device-side: the last stage of every slice is masked.
    p->k_tail = 1;
    p->m_tiles = (M + c.BM - 1) / c.BM;
    p->grid = p->m_tiles * p->n_tiles * G;
  } else if (layout == FP8GG_LAYOUT_BATCHED) {
    // Every group is a full slab: exactly G * ceil(M / BM) tiles.
    p->m_tiles = G * ((M + c.BM - 1) / c.BM);
    p->grid = p->m_tiles * p->n_tiles;
    p->persistent = c.kind == fp8gg::kKindPersistent ? 1 : 0;
  } else {
    p->m_tiles = (M + c.BM - 1) / c.BM;
    p->grid = p->m_tiles * p->n_tiles * G;
  }
  p->lds_bytes = fp8gg::lds_bytes(c);
  // The ragged kernel runs two-stage tiles on an asymmetric ring: two X slots,
  // three W slots (W copied two stages ahead).
  if (ragged(layout) && c.kind == fp8gg::kKindLds && c.stages == 2) p->lds_bytes = (2 * c.BM + 3 * c.BN) * c.BK;
  if (p->grid > 0x7FFFFFFFLL)
    return fail(FP8GG_ERR_UNSUPPORTED_SHAPE, "grid of %lld workgroups exceeds the launch limit",
                (long long)p->grid);
  return FP8GG_OK;
}

// meta: M_sizes or zero_start_index_M (int64), offsets (int32), none (batched).
fp8gg_status run(int layout, int preshuffled, const uint8_t* XQ, const uint8_t* WQ, const float* xs,
                 const float* ws, const void* meta, uint16_t* Y, int64_t G, int64_t M, int64_t N, int64_t K,
                 int zeroing, void* stream) {
  fp8gg_plan p;
  fp8gg_status st = make_plan(layout, preshuffled, G, M, N, K, &p);
  if (st != FP8GG_OK) return st;
  const int64_t rows = total_rows(layout, G, M);
  if (rows == 0 || N == 0) return ok();
  if (!Y) return fail(FP8GG_ERR_INVALID_ARGUMENT, "Y is null");
  if (!aligned(Y, 16)) return fail(FP8GG_ERR_INVALID_ARGUMENT, "Y must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.zero_fill) {
    hipError_t e = fp8gg::launch_zero_fill(Y, rows * N, s);
    if (e != hipSuccess) return fail(FP8GG_ERR_HIP, "zero fill launch failed: %s", hipGetErrorString(e));
    return ok();
  }
  if (p.config_id < 0) return ok();
  const bool has_meta = layout != FP8GG_LAYOUT_BATCHED;
  const bool int32_meta = layout == FP8GG_LAYOUT_OFFSETS || ragged(layout);
  const int64_t meta_elem = int32_meta ? 4 : 8;
  if (!XQ || !WQ || !xs || !ws || (has_meta && !meta))
    return fail(FP8GG_ERR_INVALID_ARGUMENT, "null input pointer (XQ=%p WQ=%p x_scale=%p w_scale=%p meta=%p)",
                (const void*)XQ, (const void*)WQ, (const void*)xs, (const void*)ws, meta);
  if (!aligned(XQ, 16) || !aligned(WQ, 16) || !aligned(ws, 16))
    return fail(FP8GG_ERR_INVALID_ARGUMENT, "XQ, WQ and w_scale must be 16-byte aligned");
  if (!aligned(xs, 4) || (has_meta && !aligned(meta, meta_elem)))
    return fail(FP8GG_ERR_INVALID_ARGUMENT, "x_scale must be 4-byte and the metadata %d-byte aligned",
                (int)meta_elem);
  const Extents ext = extents(layout, G, M, N, K);
  const Range out{Y, ext.y * 2, "Y"};
  const Range ins[] = {{XQ, ext.x, "XQ"},
                       {WQ, ext.w, "WQ"},
                       {xs, ext.xs * 4, "x_scale"},
                       {ws, ext.ws * 4, "w_scale"},
                       {has_meta ? meta : nullptr, G * meta_elem, "metadata"}};
  for (const Range& r : ins)
    if (overlap(out, r)) return fail(FP8GG_ERR_INVALID_ARGUMENT, "Y overlaps %s", r.name);

  fp8gg::GemmArgs a{};
  a.X = XQ;
  a.W = WQ;
  a.xs = xs;
  a.ws = ws;
  a.meta = layout == FP8GG_LAYOUT_STACKED || layout == FP8GG_LAYOUT_PADDED ? static_cast<const int64_t*>(meta)
                                                                             : nullptr;
  a.offs = int32_meta ? static_cast<const int32_t*>(meta) : nullptr;
  a.Y = Y;
  a.G = G;
  a.M = M;
  a.N = N;
  a.K = K;
  a.m_tiles = p.m_tiles;
  a.n_tiles = p.n_tiles;
  a.zeroing = layout == FP8GG_LAYOUT_PADDED && zeroing ? 1 : 0;
  {
    // Tile order across the XCDs (performance only; results do not depend on it):
    // the padded layout's data-parallel grid gives each XCD a contiguous share of
    // its tiles, so that the XCD holds whole groups (measured 2% faster on the
    // padded tails workload; no gain on the stacked workloads), and so does the
    // n_offsets grid, with its row tiles fastest, so that the row tiles reading one
    // column tile of W run on one XCD (85.4-85.8 against 91.1-91.3 us on the
    // n_offsets workload; XCD order with column tiles fastest: 88.1-88.3).  Not k_offsets:
    // its groups, whose K slices differ in length, would each land on one XCD
    // (285 against 137 us).  FP8GG_XCD overrides for measurements (0 = plain order).
    const fp8gg::KernelConfig& c0 = fp8gg::kConfigs[p.config_id];
    const int xg = (layout == FP8GG_LAYOUT_PADDED && c0.kind == fp8gg::kKindLds && c0.BM >= 128) ||
                           layout == FP8GG_LAYOUT_N_OFFSETS
                       ? 1
                       : 0;
    a.xcd_group = env_int("FP8GG_XCD", xg) ? 1 : 0;
  }
  a.skip_dead = env_int("FP8GG_SKIP_DEAD", 1) ? 1 : 0;
  if (env_int("FP8GG_LOG", 0))
    std::fprintf(stderr,
                 "[fp8gg] layout=%d pre=%d G=%lld M=%lld N=%lld K=%lld -> cfg=%d tile=%dx%dx%d thr=%d st=%d "
                 "ktail=%d ntail=%d grid=%lld (m_tiles=%lld n_tiles=%lld) persistent=%d\n",
                 layout, preshuffled, (long long)G, (long long)M, (long long)N, (long long)K, p.config_id, p.BM,
                 p.BN, p.BK, p.threads, p.stages, p.k_tail, p.n_tail, (long long)p.grid, (long long)p.m_tiles,
                 (long long)p.n_tiles, p.persistent);
  const fp8gg::KernelConfig& cfg = fp8gg::kConfigs[p.config_id];
  hipError_t e;
  if (ragged(layout)) {
    e = fp8gg::launch_gemm_ragged(layout, p.config_id, p.k_tail != 0, a, p.grid, s);
  } else if (cfg.kind == fp8gg::kKindPersistent) {
    // One persistent workgroup per compute unit.  For tuning and tests,
    // FP8GG_TAIL_GRID overrides the grid and FP8GG_TAIL the remainder mode
    // (0 automatic, 1 whole tiles, 2 quarter tiles).
    const int forced_grid = env_int("FP8GG_TAIL_GRID", 0);
    const int P = forced_grid > 0 ? forced_grid : device_cus();
    const int tail_mode = env_int("FP8GG_TAIL", 0);
    if (tail_mode < 0 || tail_mode > 2) return fail(FP8GG_ERR_INVALID_ARGUMENT, "FP8GG_TAIL=%d is not 0, 1 or 2", tail_mode);
    if (env_int("FP8GG_LOG", 0)) std::fprintf(stderr, "[fp8gg] persistent grid %d, tail mode %d\n", P, tail_mode);
    e = fp8gg::launch_gemm_persistent(layout, p.config_id, p.k_tail != 0, a, P, tail_mode, s);
  } else {
    e = fp8gg::launch_gemm(layout, p.config_id, p.k_tail != 0, a, p.grid, s);
  }
  if (e != hipSuccess) return fail(FP8GG_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

fp8gg_status f8f8bf16_rowwise_grouped_stacked(const uint8_t* XQ, const uint8_t* WQ, const float* x_scale,
                                              const float* w_scale, const int64_t* M_sizes, uint16_t* Y,
                                              int64_t G, int64_t total_M, int64_t N, int64_t K, void* stream) {
  return run(FP8GG_LAYOUT_STACKED, 0, XQ, WQ, x_scale, w_scale, M_sizes, Y, G, total_M, N, K, 0, stream);
}

fp8gg_status f8f8bf16_rowwise_grouped_dynamic(const uint8_t* XQ, const uint8_t* WQ, const float* x_scale,
                                              const float* w_scale, const int64_t* zero_start_index_M,
                                              uint16_t* Y, int64_t G, int64_t expected_m, int64_t N, int64_t K,
                                              int zeroing_output_tensor, void* stream) {
  return run(FP8GG_LAYOUT_PADDED, 0, XQ, WQ, x_scale, w_scale, zero_start_index_M, Y, G, expected_m, N, K,
             zeroing_output_tensor, stream);
}

fp8gg_status f8f8bf16_rowwise_grouped_stacked_preshuffle(const uint8_t* XQ, const uint8_t* WQs,
                                                         const float* x_scale, const float* w_scale,
                                                         const int64_t* M_sizes, uint16_t* Y, int64_t G,
                                                         int64_t total_M, int64_t N, int64_t K, void* stream) {
  return run(FP8GG_LAYOUT_STACKED, 1, XQ, WQs, x_scale, w_scale, M_sizes, Y, G, total_M, N, K, 0, stream);
}

fp8gg_status f8f8bf16_rowwise_grouped_dynamic_preshuffle(const uint8_t* XQ, const uint8_t* WQs,
                                                         const float* x_scale, const float* w_scale,
                                                         const int64_t* zero_start_index_M, uint16_t* Y,
                                                         int64_t G, int64_t expected_m, int64_t N, int64_t K,
                                                         int zeroing_output_tensor, void* stream) {
  return run(FP8GG_LAYOUT_PADDED, 1, XQ, WQs, x_scale, w_scale, zero_start_index_M, Y, G, expected_m, N, K,
             zeroing_output_tensor, stream);
}

fp8gg_status f8f8bf16_rowwise_grouped_offsets(const uint8_t* XQ, const uint8_t* WQ, const float* x_scale,
                                              const float* w_scale, const int32_t* offsets, uint16_t* Y,
                                              int64_t G, int64_t total_M, int64_t N, int64_t K, void* stream) {
  return run(FP8GG_LAYOUT_OFFSETS, 0, XQ, WQ, x_scale, w_scale, offsets, Y, G, total_M, N, K, 0, stream);
}

fp8gg_status f8f8bf16_rowwise_grouped_offsets_preshuffle(const uint8_t* XQ, const uint8_t* WQs,
                                                         const float* x_scale, const float* w_scale,
                                                         const int32_t* offsets, uint16_t* Y, int64_t G,
                                                         int64_t total_M, int64_t N, int64_t K, void* stream) {
  return run(FP8GG_LAYOUT_OFFSETS, 1, XQ, WQs, x_scale, w_scale, offsets, Y, G, total_M, N, K, 0, stream);
}

fp8gg_status f8f8bf16_rowwise_grouped_batched(const uint8_t* XQ, const uint8_t* WQ, const float* x_scale,
                                              const float* w_scale, uint16_t* Y, int64_t G, int64_t M, int64_t N,
                                              int64_t K, void* stream) {
  return run(FP8GG_LAYOUT_BATCHED, 0, XQ, WQ, x_scale, w_scale, nullptr, Y, G, M, N, K, 0, stream);
}

fp8gg_status f8f8bf16_rowwise_grouped_batched_preshuffle(const uint8_t* XQ, const uint8_t* WQs,
                                                         const float* x_scale, const float* w_scale, uint16_t* Y,
                                                         int64_t G, int64_t M, int64_t N, int64_t K,
                                                         void* stream) {
  return run(FP8GG_LAYOUT_BATCHED, 1, XQ, WQs, x_scale, w_scale, nullptr, Y, G, M, N, K, 0, stream);
}

fp8gg_status f8f8bf16_rowwise_grouped_n_offsets(const uint8_t* XQ, const uint8_t* WQ, const float* x_scale,
                                                const float* w_scale, const int32_t* n_offsets, uint16_t* Y,
                                                int64_t G, int64_t M, int64_t N, int64_t K, void* stream) {
  return run(FP8GG_LAYOUT_N_OFFSETS, 0, XQ, WQ, x_scale, w_scale, n_offsets, Y, G, M, N, K, 0, stream);
}

fp8gg_status f8f8bf16_rowwise_grouped_k_offsets(const uint8_t* XQ, const uint8_t* WQ, const float* x_scale,
                                                const float* w_scale, const int32_t* k_offsets, uint16_t* Y,
                                                int64_t G, int64_t M, int64_t N, int64_t K, void* stream) {
  return run(FP8GG_LAYOUT_K_OFFSETS, 0, XQ, WQ, x_scale, w_scale, k_offsets, Y, G, M, N, K, 0, stream);
}

// Block-scaled GEMM: stacked (meta = int64 M_sizes, M = total_M), padded (meta =
// int64 zero_start_index_M, M = expected_m, zeroing flag), offsets (meta = int32
// inclusive prefix, M = total_M) or batched (no meta, M = slab height) layout.
static fp8gg_status groupwise(int layout, int preshuffled, const uint8_t* XQ, const uint8_t* WQ,
                              const float* x_scale, const float* w_scale, const void* meta, uint16_t* Y, int64_t G,
                              int64_t M, int64_t N, int64_t K, int zeroing, void* stream) {
  constexpr int64_t B = 128;   // scale block along K and along N (whole pre-shuffle blocks too)
  const bool padded = layout == FP8GG_LAYOUT_PADDED;
  const bool slabs = padded || layout == FP8GG_LAYOUT_BATCHED;
  const bool has_meta = layout != FP8GG_LAYOUT_BATCHED;
  const int64_t meta_elem = layout == FP8GG_LAYOUT_OFFSETS ? 4 : 8;
  fp8gg_status st = check_shape(layout, preshuffled, G, M, N, K);
  if (st != FP8GG_OK) return st;
  if (K % B != 0 || N % B != 0)
    return fail(FP8GG_ERR_UNSUPPORTED_SHAPE,
                "block scaling needs K and N to be whole numbers of %lld-wide scale blocks (N=%lld K=%lld)",
                (long long)B, (long long)N, (long long)K);
  const int64_t rows = slabs ? G * M : M;
  if (rows == 0 || N == 0) return ok();
  if (!Y) return fail(FP8GG_ERR_INVALID_ARGUMENT, "Y is null");
  if (!aligned(Y, 16)) return fail(FP8GG_ERR_INVALID_ARGUMENT, "Y must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (K == 0) {
    hipError_t e = fp8gg::launch_zero_fill(Y, rows * N, s);
    if (e != hipSuccess) return fail(FP8GG_ERR_HIP, "zero fill launch failed: %s", hipGetErrorString(e));
    return ok();
  }
  if (G == 0) return ok();
  if (!XQ || !WQ || !x_scale || !w_scale || (has_meta && !meta))
    return fail(FP8GG_ERR_INVALID_ARGUMENT, "null input pointer");
  if (!aligned(XQ, 16) || !aligned(WQ, 16) || !aligned(x_scale, 4) || !aligned(w_scale, 4) ||
      (has_meta && !aligned(meta, meta_elem)))
    return fail(FP8GG_ERR_INVALID_ARGUMENT,
                "XQ and WQ must be 16-byte, x_scale and w_scale 4-byte and the row metadata %d-byte aligned",
                (int)meta_elem);
  const Range out{Y, rows * N * 2, "Y"};
  const Range ins[] = {{XQ, rows * K, "XQ"},
                       {WQ, G * N * K, "WQ"},
                       {x_scale, rows * (K / B) * 4, "x_scale"},
                       {w_scale, G * (N / B) * (K / B) * 4, "w_scale"},
                       {has_meta ? meta : nullptr, G * meta_elem, "row metadata"}};
  for (const Range& r : ins)
    if (overlap(out, r)) return fail(FP8GG_ERR_INVALID_ARGUMENT, "Y overlaps %s", r.name);

  // 128 x 256 tiles, on the persistent grid (stacked layout only) from 256 rows per
  // group on average, as for rowwise scaling; one per workgroup from 64; 32 x 128
  // tiles below.  FP8GG_BS_CONFIG (0, 1 or 2) forces one for tests and tuning.
  const int64_t per_group = slabs ? M : (M + G - 1) / G;
  int cfg = (!padded && per_group >= 256) ? fp8gg::kBlockscalePersistent : (per_group >= 64 ? 0 : 1);
  const int forced = env_int("FP8GG_BS_CONFIG", -1);
  if (forced >= 0) {
    if (forced > 2 || (padded && forced == fp8gg::kBlockscalePersistent))
      return fail(FP8GG_ERR_INVALID_ARGUMENT, "FP8GG_BS_CONFIG=%d is not a configuration of this layout", forced);
    cfg = forced;
  }
  const int64_t BM = fp8gg::kBlockscaleTileM[cfg], BN = fp8gg::kBlockscaleTileN[cfg];
  fp8gg::GemmArgs a{};
  a.X = XQ;
  a.W = WQ;
  a.xs = x_scale;
  a.ws = w_scale;
  a.meta = layout == FP8GG_LAYOUT_STACKED || padded ? static_cast<const int64_t*>(meta) : nullptr;
  a.offs = layout == FP8GG_LAYOUT_OFFSETS ? static_cast<const int32_t*>(meta) : nullptr;
  a.Y = Y;
  a.G = G;
  a.M = M;
  a.N = N;
  a.K = K;
  if (padded) {
    a.m_tiles = (M + BM - 1) / BM;
  } else if (layout == FP8GG_LAYOUT_BATCHED) {
    a.m_tiles = G * ((M + BM - 1) / BM);   // exactly: every group a full slab
  } else {
    const int64_t ub = (M + BM - 1) / BM + G - 1;
    a.m_tiles = ub < M ? ub : M;
  }
  a.n_tiles = (N + BN - 1) / BN;
  a.zeroing = padded && zeroing ? 1 : 0;
  // The padded layout's 128x256 grid in XCD order, as for rowwise scaling (each XCD
  // holds whole groups: 79.3-80.0 against 81.8-82.6 us on the padded block-scaled
  // workload, HBM reads of each group's W no longer repeated on every XCD).
  // FP8GG_XCD overrides for measurements.
  a.xcd_group = env_int("FP8GG_XCD", padded && cfg == 0 ? 1 : 0) ? 1 : 0;
  // persistent: one workgroup per compute unit (FP8GG_TAIL_GRID overrides it for tests)
  const int forced_grid = env_int("FP8GG_TAIL_GRID", 0);
  const int64_t grid = cfg == fp8gg::kBlockscalePersistent ? (forced_grid > 0 ? forced_grid : device_cus())
                                                           : a.m_tiles * a.n_tiles * (padded ? G : 1);
  if (grid > 0x7FFFFFFFLL)
    return fail(FP8GG_ERR_UNSUPPORTED_SHAPE, "grid of %lld workgroups exceeds the launch limit", (long long)grid);
  if (env_int("FP8GG_LOG", 0))
    std::fprintf(stderr, "[fp8gg] groupwise layout=%d G=%lld M=%lld N=%lld K=%lld -> cfg=%d tile=%lldx%lld grid=%lld\n",
                 layout, (long long)G, (long long)M, (long long)N, (long long)K, cfg, (long long)BM, (long long)BN,
                 (long long)grid);
  hipError_t e = fp8gg::launch_gemm_blockscale(layout, cfg, preshuffled != 0, a, grid, s);
  if (e != hipSuccess) return fail(FP8GG_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

fp8gg_status f8f8bf16_groupwise_grouped_stacked(const uint8_t* XQ, const uint8_t* WQ, const float* x_scale,
                                                const float* w_scale, const int64_t* M_sizes, uint16_t* Y, int64_t G,
                                                int64_t total_M, int64_t N, int64_t K, void* stream) {
  return groupwise(FP8GG_LAYOUT_STACKED, 0, XQ, WQ, x_scale, w_scale, M_sizes, Y, G, total_M, N, K, 0, stream);
}

fp8gg_status f8f8bf16_groupwise_grouped_stacked_preshuffle(const uint8_t* XQ, const uint8_t* WQs, const float* x_scale,
                                                           const float* w_scale, const int64_t* M_sizes, uint16_t* Y,
                                                           int64_t G, int64_t total_M, int64_t N, int64_t K,
                                                           void* stream) {
  return groupwise(FP8GG_LAYOUT_STACKED, 1, XQ, WQs, x_scale, w_scale, M_sizes, Y, G, total_M, N, K, 0, stream);
}

fp8gg_status f8f8bf16_groupwise_grouped_offsets(const uint8_t* XQ, const uint8_t* WQ, const float* x_scale,
                                                const float* w_scale, const int32_t* offsets, uint16_t* Y, int64_t G,
                                                int64_t total_M, int64_t N, int64_t K, void* stream) {
  return groupwise(FP8GG_LAYOUT_OFFSETS, 0, XQ, WQ, x_scale, w_scale, offsets, Y, G, total_M, N, K, 0, stream);
}

fp8gg_status f8f8bf16_groupwise_grouped_offsets_preshuffle(const uint8_t* XQ, const uint8_t* WQs,
                                                           const float* x_scale, const float* w_scale,
                                                           const int32_t* offsets, uint16_t* Y, int64_t G,
                                                           int64_t total_M, int64_t N, int64_t K, void* stream) {
  return groupwise(FP8GG_LAYOUT_OFFSETS, 1, XQ, WQs, x_scale, w_scale, offsets, Y, G, total_M, N, K, 0, stream);
}

fp8gg_status f8f8bf16_groupwise_grouped_batched(const uint8_t* XQ, const uint8_t* WQ, const float* x_scale,
                                                const float* w_scale, uint16_t* Y, int64_t G, int64_t M, int64_t N,
                                                int64_t K, void* stream) {
  return groupwise(FP8GG_LAYOUT_BATCHED, 0, XQ, WQ, x_scale, w_scale, nullptr, Y, G, M, N, K, 0, stream);
}

fp8gg_status f8f8bf16_groupwise_grouped_batched_preshuffle(const uint8_t* XQ, const uint8_t* WQs,
                                                           const float* x_scale, const float* w_scale, uint16_t* Y,
                                                           int64_t G, int64_t M, int64_t N, int64_t K, void* stream) {
  return groupwise(FP8GG_LAYOUT_BATCHED, 1, XQ, WQs, x_scale, w_scale, nullptr, Y, G, M, N, K, 0, stream);
}

fp8gg_status f8f8bf16_groupwise_grouped_dynamic(const uint8_t* XQ, const uint8_t* WQ, const float* x_scale,
                                                const float* w_scale, const int64_t* zero_start_index_M, uint16_t* Y,
                                                int64_t G, int64_t expected_m, int64_t N, int64_t K,
                                                int zeroing_output_tensor, void* stream) {
  return groupwise(FP8GG_LAYOUT_PADDED, 0, XQ, WQ, x_scale, w_scale, zero_start_index_M, Y, G, expected_m, N, K,
                   zeroing_output_tensor, stream);
}

fp8gg_status f8f8bf16_groupwise_grouped_dynamic_preshuffle(const uint8_t* XQ, const uint8_t* WQs,
                                                           const float* x_scale, const float* w_scale,
                                                           const int64_t* zero_start_index_M, uint16_t* Y, int64_t G,
                                                           int64_t expected_m, int64_t N, int64_t K,
                                                           int zeroing_output_tensor, void* stream) {
  return groupwise(FP8GG_LAYOUT_PADDED, 1, XQ, WQs, x_scale, w_scale, zero_start_index_M, Y, G, expected_m, N, K,
                   zeroing_output_tensor, stream);
}

fp8gg_status f8f8bf16_quantize_rowwise(const uint16_t* X, uint8_t* XQ, float* x_scale, int64_t rows, int64_t K,
                                       void* stream) {
  if (rows < 0 || K < 0)
    return fail(FP8GG_ERR_INVALID_ARGUMENT, "negative size (rows=%lld K=%lld)", (long long)rows, (long long)K);
  if (K % 8 != 0) return fail(FP8GG_ERR_UNSUPPORTED_SHAPE, "K=%lld must be a multiple of 8", (long long)K);
  const int64_t lim = (int64_t(1) << 31) - 256;
  if (rows > lim || K > lim || (rows > 0 && K > (int64_t(1) << 47) / rows))
    return fail(FP8GG_ERR_UNSUPPORTED_SHAPE, "rows=%lld K=%lld is too large", (long long)rows, (long long)K);
  if (rows == 0) return ok();
  if (!x_scale || (K > 0 && (!X || !XQ)))
    return fail(FP8GG_ERR_INVALID_ARGUMENT, "null pointer (X=%p XQ=%p x_scale=%p)", (const void*)X, (const void*)XQ,
                (const void*)x_scale);
  if (!aligned(X, 16) || !aligned(XQ, 8) || !aligned(x_scale, 4))
    return fail(FP8GG_ERR_INVALID_ARGUMENT, "X must be 16-byte, XQ 8-byte and x_scale 4-byte aligned");
  const Range x{X, rows * K * 2, "X"}, q{XQ, rows * K, "XQ"}, sc{x_scale, rows * 4, "x_scale"};
  if (overlap(q, x) || overlap(sc, x) || overlap(q, sc))
    return fail(FP8GG_ERR_INVALID_ARGUMENT, "X, XQ and x_scale must not overlap");
  hipError_t e = fp8gg::launch_quantize_rowwise(X, XQ, x_scale, rows, K, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FP8GG_ERR_HIP, "quantize launch failed: %s", hipGetErrorString(e));
  return ok();
}

fp8gg_status f8f8bf16_shuffle_b(const uint8_t* WQ, uint8_t* WQs, int64_t G, int64_t N, int64_t K,
                                void* stream) {
  fp8gg_status st = check_shape(FP8GG_LAYOUT_STACKED, 1, G, 0, N, K);
  if (st != FP8GG_OK) return st;
  const int64_t bytes = G * N * K;
  if (bytes == 0) return ok();
  if (!WQ || !WQs) return fail(FP8GG_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned(WQ, 16) || !aligned(WQs, 16))
    return fail(FP8GG_ERR_INVALID_ARGUMENT, "WQ and WQs must be 16-byte aligned");
  if (overlap(Range{WQ, bytes, "WQ"}, Range{WQs, bytes, "WQs"}))
    return fail(FP8GG_ERR_INVALID_ARGUMENT, "WQs overlaps WQ");
  hipError_t e = fp8gg::launch_shuffle_b(WQ, WQs, G, N, K, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FP8GG_ERR_HIP, "shuffle launch failed: %s", hipGetErrorString(e));
  return ok();
}

const char* f8f8bf16_last_error(void) { return g_last_error.c_str(); }

fp8gg_status f8f8bf16_plan(int layout, int preshuffled, int64_t G, int64_t M, int64_t N, int64_t K,
                           fp8gg_plan* out) {
  if (!out) return fail(FP8GG_ERR_INVALID_ARGUMENT, "out is null");
  fp8gg_status st = make_plan(layout, preshuffled, G, M, N, K, out);
  if (st == FP8GG_OK) ok();
  return st;
}

int32_t f8f8bf16_num_configs(void) { return fp8gg::kNumConfigs; }

}  // extern "C"
