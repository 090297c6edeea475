// Device kernels of the fp8 (e4m3fn) rowwise-scaled grouped GEMM for gfx950.
//
// Method (MSLK pull request 471, "Back the FP8 rowwise grouped GEMM ops with
// FlyDSL on ROCm"):
//   * rowwise scales are constant along K, so the K loop accumulates the raw fp8
//     products and one epilogue applies x_scale[m] * w_scale[g, n] (Design notes,
//     scaling-scheme paragraph);
//   * only the step that finds a tile's group differs between layouts; loads,
//     K loop and epilogue are shared (Design notes, the paragraph on serving every
//     layout from one kernel);
//   * stacked layout: the host launches an upper bound of M tiles and each tile
//     finds its group from the device-side row counts or retires (commit on
//     self-retiring tiles); offsets layout: the same walk over an int32 inclusive
//     prefix (commit adding the offsets layout); padded layout: the group is a grid
//     coordinate and the row base a multiple of expected_m (commit adding the
//     padded layout); batched layout: every group a full slab, so the group and
//     row base are arithmetic (commit adding the batched layout); n_offsets: the
//     groups partition W's rows, found from the N-tile index; k_offsets: the groups
//     slice K, the group is a grid coordinate and the trip count a run-time value
//     (commits adding the 3D-2D and 2D-2D forms);
//   * block scaling: each K block's partial sum is scaled inside the K loop (first
//     commit of the list, on the two scaling schemes);
//   * K-tail: K need only be a multiple of 16 bytes; chunks past K read as zero
//     (commit on the K-tail variant); N-tail: W rows past N are not used and stores
//     past N are dropped, predicated on the last column of each store (commits on
//     the N-tail variant and on store predicates).
//
// gfx950 mapping (this file's own design):
//   * fp8 MFMA v_mfma_f32_32x32x64_f8f6f4 (fp32 accumulate).  W is the MFMA "A"
//     operand (MFMA rows = output columns n) and X the "B" operand (MFMA columns =
//     output rows m), so each lane's accumulators cover consecutive output columns
//     of one row and the epilogue stores 16-byte vectors.
//   * X and W tiles of BK = 64 or 128 K-bytes per stage are copied global -> LDS
//     with global_load_lds_dwordx4 (no staging registers), 2 to 4 stages deep.
//   * LDS rows are BK bytes, XOR-swizzled per row (lds_swz) so that the MFMA
//     operand reads (consecutive rows at one logical chunk) are bank-conflict free;
//     pre-shuffled W arrives as whole 2 KB operand blocks and needs no swizzle.
//   * W rows are placed in LDS in "MFMA order": LDS row 32*fn + rho of a wave's
//     slice holds the output column that MFMA row rho of block fn produces in the
//     chosen lane -> column map, so the loads do the permutation for free.
//   * Large stacked calls run on a persistent grid (one workgroup per compute
//     unit) whose partial last round runs as quarter tiles (gg_persistent_kernel);
//     small-M calls use 32-row tiles with a deep ring, or stream W straight into
//     registers (gg_skinny_kernel).
//   * After its K loop a tile stores its output through the then idle LDS ring, so
//     each store instruction covers whole rows (LdsTile::store_shuffled); only the
//     persistent kernel's quarter tiles store straight from registers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8gg_internal.h"

namespace fp8gg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

// Sixteen zero bytes.  K-tail chunks at or past K are fetched from here, so the
// last K tile is zero-padded without a masked load.
__device__ __attribute__((aligned(64))) const uint8_t g_zero16[64] = {0};

// ---------------------------------------------------------------------------
// Small device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ v16f mfma_32x32x64_fp8(const v8i& a, const v8i& b, const v16f& c) {
  // cbsz = blgp = 0 selects fp8 e4m3 for both operands; zero scale operands give the
  // plain (unscaled) product.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // v_cvt_pk_bf16_f32: round to nearest even.
  const __bf16 l = (__bf16)lo;
  const __bf16 h = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}

// s_waitcnt immediate with only the vector-memory counter constrained to <= n
// (gfx9 encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt (bits
// 6:4) and lgkmcnt (bits 11:8) left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

__device__ __forceinline__ void wait_vmcnt_le(int n) {
  // The instruction takes an immediate: a switch over the counts the kernels use
  // (every count a compile-time constant folds to one instruction).
  switch (n) {
#define FP8GG_WAIT_CASE(k) \
  case k: __builtin_amdgcn_s_waitcnt(vmcnt_imm(k)); break;
    FP8GG_WAIT_CASE(1) FP8GG_WAIT_CASE(2) FP8GG_WAIT_CASE(3) FP8GG_WAIT_CASE(4) FP8GG_WAIT_CASE(5)
    FP8GG_WAIT_CASE(6) FP8GG_WAIT_CASE(7) FP8GG_WAIT_CASE(8) FP8GG_WAIT_CASE(9) FP8GG_WAIT_CASE(10)
    FP8GG_WAIT_CASE(11) FP8GG_WAIT_CASE(12) FP8GG_WAIT_CASE(13) FP8GG_WAIT_CASE(14) FP8GG_WAIT_CASE(15)
    FP8GG_WAIT_CASE(16) FP8GG_WAIT_CASE(18) FP8GG_WAIT_CASE(20) FP8GG_WAIT_CASE(24) FP8GG_WAIT_CASE(30)
    FP8GG_WAIT_CASE(32) FP8GG_WAIT_CASE(36) FP8GG_WAIT_CASE(40) FP8GG_WAIT_CASE(42) FP8GG_WAIT_CASE(48)
#undef FP8GG_WAIT_CASE
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;  // 0, or a count not listed: wait for all
  }
}

// LDS rows are BK bytes (BK/16 chunks of 16 bytes); chunk c of row p is stored at
// chunk c ^ lds_swz<BK>(p).  gfx950 serves a ds_read_b128 sixteen lanes (256 bytes,
// 64 banks) at a time, and rows p and p + 256/BK share banks, so XOR-ing with
// (p / (256/BK)) mod (BK/16) spreads the 16 consecutive rows that 16 lanes read at
// one logical chunk over all 16 bank groups.
template <int BK>
__device__ __forceinline__ int lds_swz(int p) { return (p / (256 / BK)) & (BK / 16 - 1); }

// One 16-byte-per-lane copy from global memory straight into LDS: lane l's 16 bytes
// land at LDS byte lds_base + 16*l.  lds_base is wave-uniform by construction; the
// readfirstlane states it, so that it always reaches M0 through a scalar register
// even where the compiler cannot prove the uniformity itself.  Written as inline
// assembly so that the compiler's wait-count pass does not track it: the pass
// cannot tell LDS slots apart when the slot index is a run-time value and would
// otherwise drain every copy in flight before each LDS read.  The callers order
// copies and reads themselves (wait_vmcnt_le, then a workgroup barrier).
__device__ __forceinline__ void copy16_to_lds(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory");
}

// Same with the non-temporal hint, for data that one workgroup reads once (the
// weights of a small-M call): it streams past the caches instead of displacing
// what other workgroups reuse.
__device__ __forceinline__ void copy16_to_lds_stream(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory");
}

// Same, 4 bytes per lane: lane l's 4 bytes land at LDS byte lds_base + 4*l.
__device__ __forceinline__ void copy4_to_lds(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Group resolution: the only layout-dependent step.
// ---------------------------------------------------------------------------

struct Tile {
  int64_t g;
  int64_t row_base;   // first row of the tile (row index into X / xs / Y)
  int64_t row_end;    // rows [row_base, row_end) are computed
  int64_t zero_end;   // rows [row_end, zero_end) are written as zero
};

// Metadata of groups g0 .. g0+7 (indices past G read group G-1 and are ignored by
// the callers).  A whole block of eight in bounds is read as one struct, which the
// compiler turns into a single scalar load.
template <typename T>
struct alignas(8) Meta8 {
  T v[8];
};
template <typename T>
__device__ __forceinline__ void load_meta8(const T* meta, int64_t g0, int64_t G, int64_t (&out)[8]) {
  if (g0 + 8 <= G) {
    const Meta8<T> c = *reinterpret_cast<const Meta8<T>*>(meta + g0);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = c.v[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = meta[g0 + i < G ? g0 + i : G - 1];
  }
}

// Row ends of groups g0 .. g0+7 of a packed layout, given the end s0 of group
// g0 - 1, clamped so that any metadata stays in bounds: stacked, from int64 row
// counts (negative -> 0, cumulative end -> M); offsets, from the int32 inclusive
// prefix (an end below the previous one -> empty group, past M -> M).  Groups past
// G end where the last one did.
template <int LAYOUT>
__device__ __forceinline__ void packed_ends8(const GemmArgs& a, int64_t g0, int64_t s0, int64_t (&end)[8]) {
  int64_t v[8];
  if constexpr (LAYOUT == kOffsets) load_meta8(a.offs, g0, a.G, v);
  else load_meta8(a.meta, g0, a.G, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int64_t e;
    if constexpr (LAYOUT == kOffsets) e = v[i] > s0 ? v[i] : s0;
    else e = s0 + (v[i] > 0 ? v[i] : 0);
    e = e > a.M ? a.M : e;
    e = g0 + i < a.G ? e : s0;
    end[i] = e;
    s0 = e;
  }
}

// Packed layouts (stacked, offsets): walk the groups with a running row prefix and
// tile prefix.  Each block of eight groups is fetched, and its row ends and tile
// counts are computed, before the search looks at any of them: a call pays one
// memory round trip per eight groups before its first operand load (a search that
// could stop early would let the compiler fetch the metadata one entry at a time,
// each behind a wait).  Batched: every group is a full slab of M rows, so the
// group and row base are arithmetic (no metadata).
template <int LAYOUT, int BM>
__device__ __forceinline__ bool resolve_packed(const GemmArgs& a, int64_t m_tile, Tile& t) {
  if constexpr (LAYOUT == kBatched) {
    const int64_t per = (a.M + BM - 1) / BM;
    if (per == 0 || m_tile >= a.G * per) return false;
    t.g = m_tile / per;
    t.row_base = t.g * a.M + (m_tile % per) * BM;
    t.row_end = t.g * a.M + a.M;
    t.zero_end = t.row_end;
    return true;
  }
  int64_t start = 0, tiles_before = 0;
  for (int64_t g0 = 0; g0 < a.G; g0 += 8) {
    int64_t end[8], tiles[8];
    packed_ends8<LAYOUT>(a, g0, start, end);
    int64_t s0 = start;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      tiles[i] = (end[i] - s0 + BM - 1) / BM;
      s0 = end[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (m_tile < tiles_before + tiles[i]) {
        t.g = g0 + i;
        t.row_base = start + (m_tile - tiles_before) * BM;
        t.row_end = end[i];
        t.zero_end = end[i];
        return true;
      }
      tiles_before += tiles[i];
      start = end[i];
    }
  }
  return false;
}

// Padded: the group is a grid coordinate; slab g spans rows [g*M, (g+1)*M).
template <int BM>
__device__ __forceinline__ bool resolve_padded(const GemmArgs& a, int64_t g, int64_t m_tile, Tile& t) {
  int64_t valid = a.meta[g];
  valid = valid < 0 ? 0 : (valid > a.M ? a.M : valid);
  const int64_t slab = g * a.M;
  t.g = g;
  t.row_base = slab + m_tile * BM;
  t.row_end = slab + valid;
  t.zero_end = a.zeroing ? slab + a.M : slab + valid;
  return t.row_base < t.zero_end;
}

// Writes zeros into rows [r0, r1) x columns [c0, c1) of Y (16-byte vectors).
template <int NT>
__device__ __forceinline__ void zero_rect(uint16_t* Y, int64_t N, int64_t r0, int64_t r1,
                                          int64_t c0, int64_t c1) {
  const int64_t vec_per_row = (c1 - c0) / 8;  // c0, c1 are multiples of 8
  const int64_t total = (r1 - r0) * vec_per_row;
  const v4i z = {0, 0, 0, 0};
  for (int64_t i = threadIdx.x; i < total; i += NT) {
    const int64_t r = r0 + i / vec_per_row;
    const int64_t c = c0 + (i % vec_per_row) * 8;
    *(v4i*)(Y + r * N + c) = z;
  }
}

// Ragged layouts ([MSLK-471] commits adding the 3D-2D and 2D-2D forms of the
// grouped mm): the groups partition W's rows, i.e. the output columns
// (n_offsets: X [G, M, K], W [N, K], Y [M, N], w_scale [N]), or slice K
// (k_offsets: X [M, K], W [N, K], Y [G, M, N], w_scale [G, N]).  Rows are numbered
// in the [G * M] space of x_scale; X and Y rows are that number minus a
// per-layout shift.
struct RaggedTile : Tile {
  int64_t x_delta;   // X row = row - x_delta
  int64_t y_delta;   // Y row = row - y_delta
  int64_t k0;        // first K byte of the group's slice (X and W rows)
  int64_t klen;      // K bytes of the slice
  int64_t n0;        // first output column of the tile
  int64_t col_end;   // columns [n0, col_end) belong to the tile's group
  int64_t w_off;     // byte offset of the group's first W row
  int64_t ws_off;    // index of the group's first w_scale entry
};

// Accessors that give the plain layouts' fixed answers for a Tile and the
// tile's own for a RaggedTile, so LdsTile serves both with no cost to the former.
template <typename TT>
struct IsRagged {
  static constexpr bool value = false;
};
template <>
struct IsRagged<RaggedTile> {
  static constexpr bool value = true;
};
__device__ __forceinline__ int64_t tile_x_delta(const Tile&) { return 0; }
__device__ __forceinline__ int64_t tile_x_delta(const RaggedTile& t) { return t.x_delta; }
__device__ __forceinline__ int64_t tile_y_delta(const Tile&) { return 0; }
__device__ __forceinline__ int64_t tile_y_delta(const RaggedTile& t) { return t.y_delta; }
__device__ __forceinline__ int64_t tile_k0(const Tile&) { return 0; }
__device__ __forceinline__ int64_t tile_k0(const RaggedTile& t) { return t.k0; }
__device__ __forceinline__ int64_t tile_col_end(const GemmArgs& a, const Tile&) { return a.N; }
__device__ __forceinline__ int64_t tile_col_end(const GemmArgs&, const RaggedTile& t) { return t.col_end; }
__device__ __forceinline__ int64_t tile_w_off(const GemmArgs& a, const Tile& t) { return t.g * a.N * a.K; }
__device__ __forceinline__ int64_t tile_w_off(const GemmArgs&, const RaggedTile& t) { return t.w_off; }
__device__ __forceinline__ int64_t tile_ws_off(const GemmArgs& a, const Tile& t) { return t.g * a.N; }
__device__ __forceinline__ int64_t tile_ws_off(const GemmArgs&, const RaggedTile& t) { return t.ws_off; }

// Ends of groups g0 .. g0+7 of an int32 inclusive prefix, given the end s0 of
// group g0 - 1: an end below its predecessor gives an empty group, ends are cut at
// `limit`, groups past G end where the last one did.
__device__ __forceinline__ void prefix_ends8(const int32_t* offs, int64_t G, int64_t g0, int64_t s0,
                                             int64_t limit, int64_t (&end)[8]) {
  int64_t v[8];
  load_meta8(offs, g0, G, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int64_t e = v[i] > s0 ? v[i] : s0;
    e = e > limit ? limit : e;
    e = g0 + i < G ? e : s0;
    end[i] = e;
    s0 = e;
  }
}

// n_offsets: workgroup b takes column tile b % n_tiles (counted over the groups'
// column ranges, BN per tile, an upper bound of them launched) and row tile
// b / n_tiles of the group's slab; with the XCD order (xcd_group) the row tile
// runs fastest instead, so that the row tiles sharing a column tile's W are
// consecutive and, within an XCD's contiguous share, share its L2.
template <int BM, int BN>
__device__ __forceinline__ bool resolve_n_offsets(const GemmArgs& a, int64_t b, RaggedTile& t) {
  const int64_t n_tile = a.xcd_group ? b / a.m_tiles : b % a.n_tiles;
  const int64_t m_tile = a.xcd_group ? b % a.m_tiles : b / a.n_tiles;
  int64_t start = 0, tiles_before = 0;
  for (int64_t g0 = 0; g0 < a.G; g0 += 8) {
    int64_t end[8], tiles[8];
    prefix_ends8(a.offs, a.G, g0, start, a.N, end);
    int64_t s0 = start;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      tiles[i] = (end[i] - s0 + BN - 1) / BN;
      s0 = end[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (n_tile < tiles_before + tiles[i]) {
        const int64_t g = g0 + i;
        t.g = g;
        t.row_base = g * a.M + m_tile * BM;
        t.row_end = g * a.M + a.M;
        t.zero_end = t.row_end;
        t.x_delta = 0;
        t.y_delta = g * a.M;
        t.k0 = 0;
        t.klen = a.K;
        t.n0 = start + (n_tile - tiles_before) * BN;
        t.col_end = end[i];
        t.w_off = 0;
        t.ws_off = 0;
        return t.row_base < t.row_end;
      }
      tiles_before += tiles[i];
      start = end[i];
    }
  }
  return false;
}

// k_offsets: the group is the slowest grid coordinate; its K slice is
// [end of g - 1, end of g) of the prefix, each end rounded down to a multiple of
// 16 bytes (the slices must be 16-byte aligned; rounding keeps any other value in
// bounds).
template <int BM, int BN>
__device__ __forceinline__ bool resolve_k_offsets(const GemmArgs& a, int64_t b, RaggedTile& t) {
  const int64_t n_tile = b % a.n_tiles;
  const int64_t rest = b / a.n_tiles;
  const int64_t m_tile = rest % a.m_tiles;
  const int64_t g = rest / a.m_tiles;
  if (g >= a.G) return false;
  int64_t start = 0, ks = 0, ke = 0;
  for (int64_t g0 = 0; g0 <= g; g0 += 8) {
    int64_t end[8];
    prefix_ends8(a.offs, a.G, g0, start, a.K, end);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (g0 + i == g) {
        ks = i == 0 ? start : end[i - 1];
        ke = end[i];
      }
    }
    start = end[7];
  }
  ks &= ~(int64_t)15;
  ke &= ~(int64_t)15;
  t.g = g;
  t.row_base = g * a.M + m_tile * BM;
  t.row_end = g * a.M + a.M;
  t.zero_end = t.row_end;
  t.x_delta = g * a.M;
  t.y_delta = 0;
  t.k0 = ks;
  t.klen = ke - ks;
  t.n0 = n_tile * BN;
  t.col_end = a.N;
  t.w_off = 0;
  t.ws_off = g * a.N;
  return t.row_base < t.row_end;
}

// Tile order across the XCDs.  MI355X dispatches consecutive workgroups of a grid
// to its eight XCDs in turn, and each XCD has its own L2, so workgroup w runs on
// XCD w % 8.  xcd_slot only reorders work (every tile is still computed by one
// workgroup in the same K order, so results do not depend on it): of a grid of P
// workgroups, XCD x runs workgroups x, x + 8, ..., ceil((P - x) / 8) of them, and
// xcd_slot gives them the contiguous positions that follow those of XCDs
// 0 .. x-1 (a permutation of [0, P) for any P), so that the workgroups running
// together on one XCD share operands.
__device__ __forceinline__ int64_t xcd_slot(int64_t w, int64_t P) {
  const int64_t x = w % 8, q = P / 8, r = P % 8;
  return x * q + (x < r ? x : r) + w / 8;
}

// ---------------------------------------------------------------------------
// The grouped GEMM with both operands staged through LDS (plain or pre-shuffled W)
// ---------------------------------------------------------------------------
//
// LdsTile holds everything one workgroup needs to compute one BM x BN output tile
// over a range of K stages: the per-thread copy descriptors, the LDS pipeline, the
// MFMA loop and the scaled epilogue.  The data-parallel kernel runs one tile per
// workgroup; the persistent kernel runs a sequence of whole tiles, then quarter
// tiles, per workgroup.

// PRE: W comes pre-shuffled (f8f8bf16_shuffle_b's layout): each 32-row, 64-byte-K
// block of W is 2048 contiguous bytes already in MFMA-operand order, so a stage's W
// copy is a linear copy of whole blocks and its fragments read with no swizzle.
template <int BM, int BN, int BK, int WM, int WN, int STAGES, bool KTAIL, bool PRE = false, bool W_AHEAD = false>
struct LdsTile {
  static constexpr int BM_ = BM, BN_ = BN, STAGES_ = STAGES;
  static constexpr int NT = WM * WN * 64;
  static constexpr int CPR = BK / 16;          // 16-byte chunks per LDS row
  static constexpr int KS = BK / 64;           // MFMA K steps per stage
  static constexpr int TM = BM / WM;           // wave tile along M (rows of X)
  static constexpr int TN = BN / WN;           // wave tile along N (columns of Y)
  static constexpr int FM = TM / 32;           // 32x32 MFMA blocks per wave along M
  static constexpr int FN = TN / 32;           // ... along N
  static constexpr int A_CHUNKS = BM * BK / 16;
  static constexpr int B_CHUNKS = BN * BK / 16;
  static constexpr int A_LOADS = (A_CHUNKS + NT - 1) / NT;
  static constexpr int B_LOADS = (B_CHUNKS + NT - 1) / NT;
  static constexpr int A_BYTES = BM * BK;
  static constexpr int STAGE_BYTES = (BM + BN) * BK;
  // W_AHEAD on a two-stage tile: an asymmetric ring, X in SA = 2 slots and W in
  // SB = 3 slots (a 256x256 tile fills the 160 KiB exactly), so that W is copied
  // two stages ahead and X one.  The same copies, reads and K order as the
  // symmetric ring, only issued earlier: results are bit-identical.
  static constexpr bool ASYM = W_AHEAD && STAGES == 2;
  static constexpr int SA = STAGES, SB = ASYM ? 3 : STAGES;
  static constexpr int B_BYTES = BN * BK;
  static constexpr int SMEM_BYTES = ASYM ? SA * A_BYTES + SB * B_BYTES : STAGES * STAGE_BYTES;
  static constexpr int ACC_FLOATS = FM * FN * 16;   // accumulator floats per thread
  // 32-row tiles serve small M: every byte of W is read by one workgroup only.
  static constexpr bool STREAM_W = BM <= 32;
  // Copies per thread per stage when every wave issues the same number (the
  // persistent kernel requires it).
  static constexpr int LOADS_PER_STAGE = A_LOADS + B_LOADS;
  static constexpr bool EVEN_LOADS = A_CHUNKS % NT == 0 && B_CHUNKS % NT == 0;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(A_CHUNKS % 64 == 0 && B_CHUNKS % 64 == 0, "tile rows must be a multiple of 16");
  static_assert(BK == 64 || BK == 128, "BK is 64 or 128");
  static_assert(STAGES >= 2, "at least two LDS stages");

  typedef v16f Acc[FM][FN];
  typedef v4i Packed[FM][FN][2];   // bf16 outputs, eight columns per vector (see scale())

  // First of the 16 consecutive tile columns that lane (h, r32) holds in block fn.
  // Plain W rows are placed in LDS so that a lane's columns run on across blocks;
  // pre-shuffled blocks are in MFMA order within each 32-column block.
  __device__ __forceinline__ int col_of(int fn) const {
    return wn * TN + (PRE ? 32 * fn + 16 * h : 16 * FN * h + 16 * fn);
  }

  uint8_t* smem;
  int tid, lane, wave, wm, wn, h, r32;
  // Whether any of this wave's TM rows belongs to the tile's group.  A wave whose
  // rows all lie past the group (a sparse last tile of a group) reads no fragments
  // and issues no MFMAs: its outputs are never stored.  Wave-uniform.
  bool rows_live;
  int loads_per_stage, a_loads, b_loads;
  const uint8_t* a_src[A_LOADS];
  int a_kc[A_LOADS];
  const uint8_t* b_src[B_LOADS];
  int b_kc[B_LOADS];

  __device__ __forceinline__ void init(uint8_t* smem_) {
    smem = smem_;
    tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    wm = wave / WN;
    wn = wave % WN;
    h = lane >> 5;
    r32 = lane & 31;
    // Loads this thread issues per stage (the vmcnt unit of one stage); waves whose
    // chunk range ends inside a partial round issue fewer.
    a_loads = 0;
    b_loads = 0;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) a_loads += (A_CHUNKS % NT == 0 || i * NT + wave * 64 < A_CHUNKS);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) b_loads += (B_CHUNKS % NT == 0 || i * NT + wave * 64 < B_CHUNKS);
    loads_per_stage = a_loads + b_loads;
  }

  // Copy descriptors (global source at k = 0) for the tile at rows t, columns n0.
  // Chunk q of a stage (16 bytes) lands at LDS byte 16*q: row p = q / CPR, physical
  // chunk q % CPR, which holds logical chunk (q % CPR) ^ lds_swz<BK>(p).
  template <typename TT>
  __device__ __forceinline__ void setup(const GemmArgs& a, const TT& t, int64_t n0) {
    static_assert(!(IsRagged<TT>::value && PRE), "pre-shuffled W only where a group owns a whole [N, K]");
    const int64_t K = a.K;
    const int64_t k0 = tile_k0(t);
    const int64_t xd = tile_x_delta(t);
    rows_live = !a.skip_dead || t.row_end - t.row_base > (int64_t)wm * TM;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int q = i * NT + tid;
      const int p = (q / CPR) % BM;
      const int c = (q % CPR) ^ lds_swz<BK>(p);
      int64_t row = t.row_base + p;
      row = row < t.row_end ? row : t.row_end - 1;   // rows past the group: any valid row, result dropped
      a_src[i] = a.X + (row - xd) * K + k0 + c * 16;
      a_kc[i] = c * 16;
    }
    if constexpr (PRE) {
      // A stage is BN/32 N blocks x KS K blocks of 2048 bytes, copied linearly:
      // chunk q is byte 16*(q % 128) of stage block q / 128 = (N block j, K block ks).
      const int64_t nbn = a.N / 32, nbk = K / 64;
#pragma unroll
      for (int i = 0; i < B_LOADS; ++i) {
        const int q = i * NT + tid;
        const int bq = (q / 128) % (BN / 32 * KS);
        const int j = bq / KS, ks = bq % KS;
        int64_t nb = n0 / 32 + j;
        nb = nb < nbn ? nb : nbn - 1;                   // blocks past N: result dropped
        b_src[i] = a.W + ((t.g * nbn + nb) * nbk + ks) * 2048 + (q % 128) * 16;
        b_kc[i] = ks * 64;
      }
      return;
    }
    const uint8_t* Wg = a.W + tile_w_off(a, t) + k0;
    const int64_t cend = tile_col_end(a, t);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int q = i * NT + tid;
      const int p = (q / CPR) % BN;
      const int c = (q % CPR) ^ lds_swz<BK>(p);
      // MFMA order: LDS row p = wn_*TN + 32*fn + rho holds output column
      // wn_*TN + h*16*FN + 16*fn + 4*j + tt, rho = 8*j + 4*h + tt.
      const int wn_ = p / TN;
      const int pp = p % TN;
      const int fn = pp >> 5;
      const int rho = pp & 31;
      const int nl = wn_ * TN + ((rho >> 2) & 1) * 16 * FN + 16 * fn + 4 * (rho >> 3) + (rho & 3);
      int64_t n = n0 + nl;
      n = n < cend ? n : cend - 1;                      // columns past the group: result dropped
      b_src[i] = Wg + n * K + c * 16;
      b_kc[i] = c * 16;
    }
  }

  // Copies of K stage kt into LDS slot `slot`; on the last stage (KTAIL) chunks at
  // or past K are read from the zero page.
  __device__ __forceinline__ void issue(int kt, int slot, int nk, int64_t K) {
    uint8_t* sbase = smem + slot * STAGE_BYTES;
    issue_a(kt, sbase, nk, K);
    issue_b(kt, sbase + A_BYTES, nk, K);
  }
  __device__ __forceinline__ uint8_t* aslot(int i) const { return smem + (ASYM ? i * A_BYTES : i * STAGE_BYTES); }
  __device__ __forceinline__ uint8_t* bslot(int i) const {
    return ASYM ? smem + SA * A_BYTES + i * B_BYTES : smem + i * STAGE_BYTES + A_BYTES;
  }
  __device__ __forceinline__ void issue_a(int kt, uint8_t* sbase, int nk, int64_t K) {
    const int64_t koff = (int64_t)kt * BK;
    const bool last = KTAIL && (kt == nk - 1);
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      if (A_CHUNKS % NT == 0 || i * NT + wave * 64 < A_CHUNKS) {
        const uint8_t* src = a_src[i] + koff;
        if (last && koff + a_kc[i] >= K) src = g_zero16;
        copy16_to_lds(src, lds_addr(sbase + (i * NT + wave * 64) * 16));
      }
    }
  }
  __device__ __forceinline__ void issue_b(int kt, uint8_t* sbase, int nk, int64_t K) {
    const int64_t koff = (int64_t)kt * BK;
    const bool last = KTAIL && (kt == nk - 1);
    const int64_t bkoff = PRE ? (int64_t)kt * KS * 2048 : koff;   // pre-shuffled: KS blocks per stage
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      if (B_CHUNKS % NT == 0 || i * NT + wave * 64 < B_CHUNKS) {
        const uint8_t* src = b_src[i] + bkoff;
        if (last && koff + b_kc[i] >= K) src = g_zero16;
        if (STREAM_W) copy16_to_lds_stream(src, lds_addr(sbase + (i * NT + wave * 64) * 16));
        else copy16_to_lds(src, lds_addr(sbase + (i * NT + wave * 64) * 16));
      }
    }
  }

  // MFMA operands of the stage in LDS slot `slot`: for MFMA step ks, lane (h, r32)
  // takes row r32 of each 32-row block, bytes [64*ks + 32h, +32) (logical chunks
  // 4ks + 2h and 4ks + 2h + 1).
  __device__ __forceinline__ void read_frags(int slot, v8i (&xf)[KS][FM], v8i (&wf)[KS][FN]) const {
    read_frags_at(smem + slot * STAGE_BYTES, smem + slot * STAGE_BYTES + A_BYTES, xf, wf);
  }
  __device__ __forceinline__ void read_frags_at(const uint8_t* sA, const uint8_t* sB, v8i (&xf)[KS][FM],
                                                v8i (&wf)[KS][FN]) const {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int p = wm * TM + 32 * fm + r32;
        const int sw = lds_swz<BK>(p);
        const v4i lo = *(const v4i*)(sA + p * BK + (((4 * ks + 2 * h) ^ sw) * 16));
        const v4i hi = *(const v4i*)(sA + p * BK + (((4 * ks + 2 * h + 1) ^ sw) * 16));
        xf[ks][fm] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        v4i lo, hi;
        if constexpr (PRE) {
          // Block layout: bytes 16*lane of the first 1024 hold the lane's first 16
          // operand bytes, of the second 1024 its last 16.
          const uint8_t* blk = sB + ((wn * FN + fn) * KS + ks) * 2048;
          lo = *(const v4i*)(blk + lane * 16);
          hi = *(const v4i*)(blk + 1024 + lane * 16);
        } else {
          const int p = wn * TN + 32 * fn + r32;
          const int sw = lds_swz<BK>(p);
          lo = *(const v4i*)(sB + p * BK + (((4 * ks + 2 * h) ^ sw) * 16));
          hi = *(const v4i*)(sB + p * BK + (((4 * ks + 2 * h + 1) ^ sw) * 16));
        }
        wf[ks][fn] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      }
    }
  }

  // acc += the tile's products over K stages [kb, ke).  Every thread of the
  // workgroup must call it; it starts by waiting until the workgroup has finished
  // reading LDS from any previous call, so LdsTile can be reused tile after tile.
  // Issues the first STAGES - 1 stages of K range [kb, ke).  It starts with a
  // workgroup barrier: every wave must be done reading LDS (from a previous tile)
  // before the copies overwrite it.
  __device__ __forceinline__ void prologue(int kb, int ke, int nk, int64_t K) {
    block_barrier();
    if constexpr (ASYM) {
      // W of stages kb and kb + 1, X of stage kb (W first: it comes from further away)
      if (kb < ke) {
        issue_b(kb, bslot(0), nk, K);
        issue_a(kb, aslot(0), nk, K);
      }
      if (kb + 1 < ke) issue_b(kb + 1, bslot(1), nk, K);
      return;
    }
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (kb + s < ke) issue(kb + s, s, nk, K);
  }

  // acc += the tile's products over K stages [kb, ke), whose first STAGES - 1
  // stages prologue() has issued.  Every thread of the workgroup must call it.
  __device__ __forceinline__ void mainloop(int kb, int ke, int nk, int64_t K, Acc& acc) {
    if constexpr (ASYM) {
      for (int kt = kb; kt < ke; ++kt) {
        const int j = kt - kb;
        // Outstanding, oldest first: ..., X(kt), W(kt + 1) (issued one step ago, W
        // only while kt + 1 < ke).  Leaving W(kt + 1)'s loads outstanding means X(kt)
        // and the older W(kt) have landed.
        if (kt + 1 < ke) wait_vmcnt_le(b_loads);
        else wait_vmcnt_le(0);
        block_barrier();
        // the slots refilled here were last read at step j - 1, which every wave has left
        if (kt + 1 < ke) issue_a(kt + 1, aslot((j + 1) % SA), nk, K);
        if (kt + 2 < ke) issue_b(kt + 2, bslot((j + 2) % SB), nk, K);
        if (rows_live) {
          v8i xf[KS][FM], wf[KS][FN];
          read_frags_at(aslot(j % SA), bslot(j % SB), xf, wf);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
              for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma_32x32x64_fp8(wf[ks][fn], xf[ks][fm], acc[fm][fn]);
        }
      }
      return;
    }
    for (int kt = kb; kt < ke; ++kt) {
      const int j = kt - kb;
      // Stage kt has landed once at most (stages issued after it) loads of this
      // thread are outstanding (vector memory operations complete in order, so
      // any younger stores only make the wait stricter); the barrier then makes
      // every thread's copies visible and frees the slot that the next issue
      // overwrites.
      const int ahead = ke - 1 - kt;
      if (ahead >= STAGES - 2) wait_vmcnt_le((STAGES - 2) * loads_per_stage);
      else wait_vmcnt_le(0);
      block_barrier();
      if (kt + STAGES - 1 < ke) issue(kt + STAGES - 1, (j + STAGES - 1) % STAGES, nk, K);
      if (rows_live) {
        v8i xf[KS][FM], wf[KS][FN];
        read_frags(j % STAGES, xf, wf);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = mfma_32x32x64_fp8(wf[ks][fn], xf[ks][fm], acc[fm][fn]);
      }
    }
  }

  __device__ __forceinline__ void run(int kb, int ke, int nk, int64_t K, Acc& acc) {
    prologue(kb, ke, nk, K);
    mainloop(kb, ke, nk, K, acc);
  }

  // The epilogue, y = bf16((acc * x_scale[m]) * w_scale[g, n]) under row and
  // column masks, in two halves: scale() loads the scales and turns the
  // accumulators into packed bf16 pairs, store() (or store_shuffled()) writes them
  // (and writes rows [row_end, zero_end) as zero).  Lane (h, r32) holds, for block (fm, fn), slot
  // i = 4*j + tt, output row wm*TM + 32*fm + r32 and column col0 + 16*fn + i; pair
  // q of Packed[fm][fn] holds slots 2q and 2q + 1.

  template <typename TT>
  __device__ __forceinline__ void scale(const GemmArgs& a, const TT& t, int64_t n0, const Acc& acc,
                                        Packed& pk) const {
    const int64_t cend = tile_col_end(a, t);
    const float* wsg = a.ws + tile_ws_off(a, t);
    float wsv[16 * FN];
#pragma unroll
    for (int v = 0; v < 4 * FN; ++v) {
      const int64_t c = n0 + col_of(v / 4) + 4 * (v % 4);
      if constexpr (IsRagged<TT>::value) {
        // a group's columns may start anywhere: scalar loads, each masked
#pragma unroll
        for (int e = 0; e < 4; ++e) wsv[4 * v + e] = c + e < cend ? wsg[c + e] : 0.f;
      } else {
        v4f w4 = {0.f, 0.f, 0.f, 0.f};
        if (c < cend) w4 = *(const v4f*)(wsg + c);
        wsv[4 * v + 0] = w4.x;
        wsv[4 * v + 1] = w4.y;
        wsv[4 * v + 2] = w4.z;
        wsv[4 * v + 3] = w4.w;
      }
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int64_t m = t.row_base + wm * TM + 32 * fm + r32;
      const float xsv = m < t.row_end ? a.xs[m] : 0.f;   // rows past the group are never stored
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint32_t q[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 8 * half + 2 * e;
            q[e] = pack_bf16x2((acc[fm][fn][i] * xsv) * wsv[16 * fn + i],
                               (acc[fm][fn][i + 1] * xsv) * wsv[16 * fn + i + 1]);
          }
          pk[fm][fn][half] = v4i{(int)q[0], (int)q[1], (int)q[2], (int)q[3]};
        }
    }
  }

  template <typename TT>
  __device__ __forceinline__ void store(const GemmArgs& a, const TT& t, int64_t n0, const Packed& pk) const {
    const int64_t N = a.N;
    const int64_t cend = tile_col_end(a, t);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int64_t m = t.row_base + wm * TM + 32 * fm + r32;
      if (m < t.row_end) {
        uint16_t* yrow = a.Y + (m - tile_y_delta(t)) * N;
#pragma unroll
        for (int s = 0; s < 2 * FN; ++s) {           // 8 columns per 16-byte store
          const int64_t c = n0 + col_of(s >> 1) + 8 * (s & 1);
          if constexpr (IsRagged<TT>::value) {
            // A group's columns may start or end inside a vector: such vectors are
            // stored column by column, each column up to the group's end.
            if ((c & 7) == 0 && c + 8 <= cend) {
              *(v4i*)(yrow + c) = pk[fm][s >> 1][s & 1];
            } else if (c < cend) {
              const v4i v = pk[fm][s >> 1][s & 1];
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (c + e < cend) yrow[c + e] = (uint16_t)((uint32_t)v[e >> 1] >> (16 * (e & 1)));
            }
          } else {
            if (c < cend) *(v4i*)(yrow + c) = pk[fm][s >> 1][s & 1];
          }
        }
      } else if (m < t.zero_end) {
        uint16_t* yrow = a.Y + m * N;
#pragma unroll
        for (int s = 0; s < 2 * FN; ++s) {
          const int64_t c = n0 + col_of(s >> 1) + 8 * (s & 1);
          if (c < N) *(v4i*)(yrow + c) = v4i{0, 0, 0, 0};
        }
      }
    }
  }

  // The same stores through LDS, for kernels whose LDS ring is idle after the K
  // loop (one tile per workgroup).  The packed tile is written to LDS in its MFMA
  // layout (row r at a stride of BN bf16, 16-byte chunk c stored at c ^ (r mod 16),
  // which keeps the column-wise writes and the row-wise reads free of bank
  // conflicts) and read back row by row, so that each global store instruction
  // covers whole rows of the tile (consecutive lanes, consecutive 16 bytes) instead
  // of 16-byte pieces of 32 rows: HBM sees whole cache lines.  Row and column masks
  // as in store().
  static constexpr int CHUNKS_PER_ROW = BN / 8;
  static constexpr int SHUF_MASK = (CHUNKS_PER_ROW < 16 ? CHUNKS_PER_ROW : 16) - 1;
  template <typename TT>
  __device__ __forceinline__ void store_shuffled(const GemmArgs& a, const TT& t, int64_t n0,
                                                 const Packed& pk) const {
    static_assert(BM * BN * 2 <= SMEM_BYTES, "the output tile fits the LDS ring");
    block_barrier();   // every wave is done reading the ring's last stage
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int r = wm * TM + 32 * fm + r32;
#pragma unroll
      for (int s = 0; s < 2 * FN; ++s) {
        const int chunk = (col_of(s >> 1) + 8 * (s & 1)) / 8;
        *(v4i*)(smem + (r * CHUNKS_PER_ROW + (chunk ^ (r & SHUF_MASK))) * 16) = pk[fm][s >> 1][s & 1];
      }
    }
    block_barrier();
    const int64_t N = a.N;
    const int64_t cend = tile_col_end(a, t);
#pragma unroll 4
    for (int q = tid; q < BM * CHUNKS_PER_ROW; q += NT) {
      const int r = q / CHUNKS_PER_ROW;
      const int chunk = q % CHUNKS_PER_ROW;
      const int64_t m = t.row_base + r;
      const int64_t c = n0 + 8 * chunk;
      if (m >= t.zero_end) continue;
      v4i v = {0, 0, 0, 0};
      if (m < t.row_end) v = *(const v4i*)(smem + (r * CHUNKS_PER_ROW + (chunk ^ (r & SHUF_MASK))) * 16);
      uint16_t* yrow = a.Y + (m - tile_y_delta(t)) * N;
      if constexpr (IsRagged<TT>::value) {
        if ((c & 7) == 0 && c + 8 <= cend) {
          *(v4i*)(yrow + c) = v;
        } else if (c < cend) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (c + e < cend) yrow[c + e] = (uint16_t)((uint32_t)v[e >> 1] >> (16 * (e & 1)));
        }
      } else {
        if (c < cend) *(v4i*)(yrow + c) = v;
      }
    }
  }

  template <typename TT>
  __device__ __forceinline__ void epilogue_shuffled(const GemmArgs& a, const TT& t, int64_t n0,
                                                    const Acc& acc) const {
    Packed pk;
    scale(a, t, n0, acc, pk);
    store_shuffled(a, t, n0, pk);
  }

  template <typename TT>
  __device__ __forceinline__ void epilogue(const GemmArgs& a, const TT& t, int64_t n0, const Acc& acc) const {
    Packed pk;
    scale(a, t, n0, acc, pk);
    store(a, t, n0, pk);
  }
};

// Data-parallel kernel: one output tile per workgroup, whole K.
template <int LAYOUT, int BM, int BN, int BK, int WM, int WN, int STAGES, bool KTAIL, bool PRE>
__global__ void __launch_bounds__(WM * WN * 64)
gg_lds_kernel(GemmArgs a) {
  typedef LdsTile<BM, BN, BK, WM, WN, STAGES, KTAIL, PRE> E;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[E::SMEM_BYTES];

  // xcd_group: each XCD takes a contiguous share of the tile order
  const int64_t bid = a.xcd_group ? xcd_slot(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
  const int64_t n_tile = bid % a.n_tiles;
  const int64_t rest = bid / a.n_tiles;
  Tile t;
  if (LAYOUT == kPadded) {
    if (!resolve_padded<BM>(a, rest / a.m_tiles, rest % a.m_tiles, t)) return;
  } else {
    if (!resolve_packed<LAYOUT, BM>(a, rest, t)) return;
  }
  const int64_t n0 = n_tile * BN;
  if (t.row_base >= t.row_end) {
    // Entirely padding (padded layout with zeroing): no K loop.
    const int64_t tile_row_end = t.row_base + BM;
    const int64_t r1 = tile_row_end < t.zero_end ? tile_row_end : t.zero_end;
    const int64_t c1 = n0 + BN < a.N ? n0 + BN : a.N;
    zero_rect<E::NT>(a.Y, a.N, t.row_base, r1, n0, c1);
    return;
  }
  E e;
  e.init(smem);
  e.setup(a, t, n0);
  typename E::Acc acc;
#pragma unroll
  for (int i = 0; i < E::FM; ++i)
#pragma unroll
    for (int j = 0; j < E::FN; ++j) acc[i][j] = v16f{0};
  const int nk = (int)((a.K + BK - 1) / BK);
  e.run(0, nk, nk, a.K, acc);
  e.epilogue_shuffled(a, t, n0, acc);
}

// Ragged layouts (n_offsets, k_offsets): one tile per workgroup, both operands
// through LDS, plain W only.  The K loop runs over the tile's group slice, whose
// length is only known on the device (k_offsets), so the trip count is a runtime
// value and the tail mask is keyed on the slice's own end.
template <int LAYOUT, int BM, int BN, int BK, int WM, int WN, int STAGES, bool KTAIL>
__global__ void __launch_bounds__(WM * WN * 64)
gg_ragged_kernel(GemmArgs a) {
  // W two stages ahead: the ragged calls measured 8.8% (n_offsets) and 3.8%
  // (k_offsets) faster with it; the packed calls' 256x256 tiles were level or slower.
  typedef LdsTile<BM, BN, BK, WM, WN, STAGES, KTAIL, false, true> E;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[E::SMEM_BYTES];
  RaggedTile t;
  // xcd_group: each XCD takes a contiguous share of the tile order
  const int64_t bid = a.xcd_group ? xcd_slot(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
  if constexpr (LAYOUT == kNOffsets) {
    if (!resolve_n_offsets<BM, BN>(a, bid, t)) return;
  } else {
    if (!resolve_k_offsets<BM, BN>(a, bid, t)) return;
  }
  E e;
  e.init(smem);
  e.setup(a, t, t.n0);
  typename E::Acc acc;
#pragma unroll
  for (int i = 0; i < E::FM; ++i)
#pragma unroll
    for (int j = 0; j < E::FN; ++j) acc[i][j] = v16f{0};
  const int nk = (int)((t.klen + BK - 1) / BK);
  e.run(0, nk, nk, t.klen, acc);
  e.epilogue_shuffled(a, t, t.n0, acc);
}

// Number of M tiles over all groups of a packed layout, with the resolver's clamping.
template <int LAYOUT, int BM>
__device__ __forceinline__ int64_t count_m_tiles(const GemmArgs& a) {
  if constexpr (LAYOUT == kBatched) return a.G * ((a.M + BM - 1) / BM);
  int64_t start = 0, tiles = 0;
  for (int64_t g0 = 0; g0 < a.G; g0 += 8) {
    int64_t end[8];
    packed_ends8<LAYOUT>(a, g0, start, end);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      tiles += (end[i] - start + BM - 1) / BM;
      start = end[i];
    }
  }
  return tiles;
}

// Persistent kernel (packed layouts: stacked, offsets, batched).
//
// A grid of P workgroups, one per compute unit, walks the T output tiles in
// data-parallel order: workgroup w computes whole tiles w, w + P, ..., each with
// its own prologue and the coalesced store through the then idle LDS ring.  When T
// is not a multiple of P, the rem = T % P tiles of the last round would keep
// P - rem compute units idle for a whole tile.  When 4 * rem <= 2 * P those tiles
// are computed as quarter tiles instead, (BM/2) x (BN/2) each: quarter q of
// remainder tile i is quarter number 4i + q, and workgroup w computes quarters w,
// w + P, ... once its whole tiles are done (quarters past the group's rows or past
// N are skipped).  A quarter copies half the operand bytes of a whole tile and
// takes about 0.3 of its time, so the last round costs 0.3 (one round of quarters)
// or 0.6 (two) of a whole tile instead of 1.  Each output element is computed by
// one workgroup in the same K order as in the data-parallel kernel, so the result
// is bitwise that of the data-parallel kernel whatever the grid.
//
// tail_mode: 0 chooses quarters by the rule above, 1 never uses them, 2 always
// does when rem > 0.
template <int LAYOUT, int BM, int BN, int BK, int WM, int WN, int STAGES, bool KTAIL, bool PRE>
__global__ void __launch_bounds__(WM * WN * 64)
gg_persistent_kernel(GemmArgs a, int tail_mode) {
  typedef LdsTile<BM, BN, BK, WM, WN, STAGES, KTAIL, PRE> E;
  // Quarter tiles reuse the LDS ring with as many stages as fit (at most 8).
  constexpr int Q_STAGE_BYTES = (BM + BN) / 2 * BK;
  constexpr int Q_STAGES = E::SMEM_BYTES / Q_STAGE_BYTES < 8 ? E::SMEM_BYTES / Q_STAGE_BYTES : 8;
  typedef LdsTile<BM / 2, BN / 2, BK, WM, WN, Q_STAGES, KTAIL, PRE> Q;
  static_assert(Q::SMEM_BYTES <= E::SMEM_BYTES, "quarter tiles reuse the LDS ring");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[E::SMEM_BYTES];

  const int64_t P = gridDim.x;
  const int64_t w = blockIdx.x;
  const int nk = (int)((a.K + BK - 1) / BK);
  const int64_t T = count_m_tiles<LAYOUT, BM>(a) * a.n_tiles;
  const int64_t rem = tail_quarters(T, P, tail_mode) ? T % P : 0;
  const int64_t whole = T - rem;

  for (int64_t tile = w; tile < whole; tile += P) {
    Tile t;
    resolve_packed<LAYOUT, BM>(a, tile / a.n_tiles, t);
    const int64_t n0 = (tile % a.n_tiles) * BN;
    E e;
    e.init(smem);
    e.setup(a, t, n0);
    typename E::Acc acc;
#pragma unroll
    for (int i = 0; i < E::FM; ++i)
#pragma unroll
      for (int j = 0; j < E::FN; ++j) acc[i][j] = v16f{0};
    e.run(0, nk, nk, a.K, acc);   // starts with a barrier: the ring is free to reuse
    e.epilogue_shuffled(a, t, n0, acc);
  }

  for (int64_t qn = w; qn < 4 * rem; qn += P) {
    const int64_t tile = whole + qn / 4;
    const int q = (int)(qn % 4);
    Tile t;
    resolve_packed<LAYOUT, BM>(a, tile / a.n_tiles, t);
    t.row_base += (q >> 1) * (BM / 2);
    const int64_t n0 = (tile % a.n_tiles) * BN + (q & 1) * (BN / 2);
    if (t.row_base >= t.row_end || n0 >= a.N) continue;
    Q e;
    e.init(smem);
    e.setup(a, t, n0);
    typename Q::Acc acc;
#pragma unroll
    for (int i = 0; i < Q::FM; ++i)
#pragma unroll
      for (int j = 0; j < Q::FN; ++j) acc[i][j] = v16f{0};
    e.run(0, nk, nk, a.K, acc);     // starts with a barrier: the ring is free to reuse
    e.epilogue(a, t, n0, acc);
  }
}

// ---------------------------------------------------------------------------
// Block (groupwise) scaling, stacked layout
// ---------------------------------------------------------------------------
//
// One scale per (128 x 128) block of W[g] and per (row, 128-byte K block) of X
// ([MSLK-471], first commit of the list: block scaling scales each block's partial
// sum inside the K loop).  The K stage is one scale block (BK = 128): the stage's
// MFMAs accumulate into a zeroed partial tile, which is then added to the running
// accumulator as acc += partial * (x_scale[m, kb] * w_scale[g, n / 128, kb]).
// The stage's scales travel with its operand copies: x_scale of the tile's rows
// and w_scale of its column blocks are copied into an LDS slot of the same ring
// index (one 4-byte copy per lane, one per wave, the waves past the block into a
// dummy word), so the stage's wait and barrier cover them too.  The epilogue only
// rounds and stores.  K and N are whole numbers of blocks (checked on the host).
// PRE: W comes pre-shuffled (f8f8bf16_shuffle_b) and is read through the same tile
// as in the rowwise kernels; a lane's 16 columns still lie in one 128-column block.
// Floats per LDS scale slot for a block-scaled tile of BM rows: the tile's x_scale
// column (slack past BM) and then its W block scales.
template <int BM>
struct BlockscaleSlots {
  static constexpr int SCX = BM > 64 ? BM : 64;
  static constexpr int SC = SCX + 64;
};

// One block-scaled output tile (rows of t, columns n0 .. n0 + BN): the K loop over
// 128-byte scale blocks and the coalesced store.  sc holds E::STAGES_ scale slots
// of BlockscaleSlots<BM>::SC floats.  Starts with a workgroup barrier, so that a
// workgroup can run tile after tile over the same LDS.
template <typename E>
__device__ __forceinline__ void blockscale_tile(E& e, const GemmArgs& a, const Tile& t, int64_t n0, float* sc,
                                                float* sc_dummy) {
  constexpr int BK = 128, BM = E::BM_, BN = E::BN_, STAGES = E::STAGES_;
  constexpr int SCX = BlockscaleSlots<BM>::SCX, SC = BlockscaleSlots<BM>::SC;
  constexpr int L = E::LOADS_PER_STAGE + 1;
  static_assert(E::EVEN_LOADS, "the stage wait counts assume equal copies per wave");
  static_assert(SCX / 64 + 1 <= E::NT / 64, "one scale copy per wave");
  static_assert(BN % 128 == 0 && E::TN % 16 == 0, "a lane's 16 columns lie in one block");
  block_barrier();   // the previous tile of this workgroup may still read the ring
  e.setup(a, t, n0);
  const int nkb = (int)(a.K / BK);
  const int64_t nbn = a.N / 128;

  // This thread's scale source at K block 0 (one float further per block).
  const float* ssrc;
  int sdst;                                // 0..: offset in the slot; -1: the dummy word
  if (e.wave < SCX / 64) {
    int r = e.wave * 64 + e.lane;
    r = r < BM ? r : BM - 1;
    int64_t row = t.row_base + r;
    row = row < t.row_end ? row : t.row_end - 1;   // rows past the group: any valid row
    ssrc = a.xs + row * nkb;
    sdst = e.wave * 64;
  } else if (e.wave == SCX / 64) {
    int64_t j = n0 / 128 + (e.lane < BN / 128 ? e.lane : BN / 128 - 1);
    j = j < nbn ? j : nbn - 1;                     // blocks past N: never used
    ssrc = a.ws + (t.g * nbn + j) * nkb;
    sdst = SCX;
  } else {
    ssrc = a.xs + t.row_base * nkb;
    sdst = -1;
  }
  auto issue = [&](int kt) {
    const int slot = kt % STAGES;
    e.issue(kt, slot, nkb, a.K);
    copy4_to_lds(ssrc + kt, lds_addr(sdst >= 0 ? sc + slot * SC + sdst : sc_dummy));
  };

  typename E::Acc acc;
#pragma unroll
  for (int i = 0; i < E::FM; ++i)
#pragma unroll
    for (int j = 0; j < E::FN; ++j) acc[i][j] = v16f{0};

#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nkb) issue(s);
  for (int kt = 0; kt < nkb; ++kt) {
    // stage kt (operands and scales) has landed once only the younger stages'
    // copies are outstanding; the barrier publishes it and frees the slot reused below
    if (nkb - 1 - kt >= STAGES - 2) wait_vmcnt_le((STAGES - 2) * L);
    else wait_vmcnt_le(0);
    block_barrier();
    if (kt + STAGES - 1 < nkb) issue(kt + STAGES - 1);
    const int slot = kt % STAGES;
    // the stage's block scales first: their LDS latency hides under the fragment reads
    float xsv[E::FM], wsv[E::FN];
#pragma unroll
    for (int fm = 0; fm < E::FM; ++fm) xsv[fm] = sc[slot * SC + e.wm * E::TM + 32 * fm + e.r32];
#pragma unroll
    for (int fn = 0; fn < E::FN; ++fn) wsv[fn] = sc[slot * SC + SCX + e.col_of(fn) / 128];
    v8i xf[E::KS][E::FM], wf[E::KS][E::FN];
    e.read_frags(slot, xf, wf);
    // block b's MFMAs, then block b - 1's scaling, so that the vector unit works on
    // one partial while the matrix unit fills the next
    constexpr int NB = E::FM * E::FN;
    v16f part[NB];
#pragma unroll
    for (int b = 0; b <= NB; ++b) {
      if (b < NB) {
        const int fm = b / E::FN, fn = b % E::FN;
        part[b] = mfma_32x32x64_fp8(wf[0][fn], xf[0][fm], v16f{0});
#pragma unroll
        for (int ks = 1; ks < E::KS; ++ks) part[b] = mfma_32x32x64_fp8(wf[ks][fn], xf[ks][fm], part[b]);
      }
      if (b > 0) {
        const int fm = (b - 1) / E::FN, fn = (b - 1) % E::FN;
        const float f = xsv[fm] * wsv[fn];
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[fm][fn][i] = __builtin_fmaf(part[b - 1][i], f, acc[fm][fn][i]);
      }
    }
  }

  typename E::Packed pk;
#pragma unroll
  for (int fm = 0; fm < E::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < E::FN; ++fn)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint32_t q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 8 * half + 2 * j;
          q[j] = pack_bf16x2(acc[fm][fn][i], acc[fm][fn][i + 1]);
        }
        pk[fm][fn][half] = v4i{(int)q[0], (int)q[1], (int)q[2], (int)q[3]};
      }
  e.store_shuffled(a, t, n0, pk);
}

// One tile per workgroup; the packed layouts (stacked, offsets, batched: the
// group from the row metadata or the slab arithmetic), or padded (the group from
// the grid, rows past the slab's valid count zeroed under the zeroing flag,
// whole-padding tiles written as zeros without a K loop).
template <int LAYOUT, int BM, int BN, int WM, int WN, int STAGES, bool PRE>
__global__ void __launch_bounds__(WM * WN * 64)
gg_blockscale_kernel(GemmArgs a) {
  typedef LdsTile<BM, BN, 128, WM, WN, STAGES, false, PRE> E;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[E::SMEM_BYTES];
  __shared__ __attribute__((aligned(16))) float sc[STAGES * BlockscaleSlots<BM>::SC];
  __shared__ __attribute__((aligned(16))) float sc_dummy[64];
  // xcd_group: each XCD takes a contiguous share of the tile order
  const int64_t bid = a.xcd_group ? xcd_slot(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
  const int64_t n0 = (bid % a.n_tiles) * BN;
  const int64_t rest = bid / a.n_tiles;
  Tile t;
  if constexpr (LAYOUT == kPadded) {
    if (!resolve_padded<BM>(a, rest / a.m_tiles, rest % a.m_tiles, t)) return;
    if (t.row_base >= t.row_end) {
      const int64_t tile_row_end = t.row_base + BM;
      const int64_t r1 = tile_row_end < t.zero_end ? tile_row_end : t.zero_end;
      const int64_t c1 = n0 + BN < a.N ? n0 + BN : a.N;
      zero_rect<E::NT>(a.Y, a.N, t.row_base, r1, n0, c1);
      return;
    }
  } else {
    if (!resolve_packed<LAYOUT, BM>(a, rest, t)) return;
  }
  E e;
  e.init(smem);
  blockscale_tile(e, a, t, n0, sc, sc_dummy);
}

// The same on a persistent grid (one workgroup per compute unit): whole tiles w,
// w + P, ..., then, when the last round is partial, its tiles as (BM/2) x (BN/2)
// quarter tiles by the rule of the rowwise persistent kernel (tail_quarters), so a
// partial round costs a fraction of a tile.  No pipelining across tiles.
template <int LAYOUT, int BM, int BN, int WM, int WN, int STAGES, bool PRE>
__global__ void __launch_bounds__(WM * WN * 64)
gg_blockscale_persistent_kernel(GemmArgs a) {
  typedef LdsTile<BM, BN, 128, WM, WN, STAGES, false, PRE> E;
  constexpr int Q_STAGE_BYTES = (BM + BN) / 2 * 128;
  constexpr int Q_STAGES = E::SMEM_BYTES / Q_STAGE_BYTES < 8 ? E::SMEM_BYTES / Q_STAGE_BYTES : 8;
  typedef LdsTile<BM / 2, BN / 2, 128, WM, WN, Q_STAGES, false, PRE> Q;
  static_assert(Q::SMEM_BYTES <= E::SMEM_BYTES, "quarter tiles reuse the LDS ring");
  constexpr int SC_FLOATS = STAGES * BlockscaleSlots<BM>::SC > Q_STAGES * BlockscaleSlots<BM / 2>::SC
                                ? STAGES * BlockscaleSlots<BM>::SC
                                : Q_STAGES * BlockscaleSlots<BM / 2>::SC;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[E::SMEM_BYTES];
  __shared__ __attribute__((aligned(16))) float sc[SC_FLOATS];
  __shared__ __attribute__((aligned(16))) float sc_dummy[64];

  const int64_t P = gridDim.x;
  const int64_t w = blockIdx.x;
  const int64_t T = count_m_tiles<LAYOUT, BM>(a) * a.n_tiles;
  const int64_t rem = tail_quarters(T, P, 0) ? T % P : 0;
  const int64_t whole = T - rem;
  for (int64_t tile = w; tile < whole; tile += P) {
    Tile t;
    resolve_packed<LAYOUT, BM>(a, tile / a.n_tiles, t);
    E e;
    e.init(smem);
    blockscale_tile(e, a, t, (tile % a.n_tiles) * BN, sc, sc_dummy);
  }
  for (int64_t qn = w; qn < 4 * rem; qn += P) {
    const int64_t tile = whole + qn / 4;
    const int q = (int)(qn % 4);
    Tile t;
    resolve_packed<LAYOUT, BM>(a, tile / a.n_tiles, t);
    t.row_base += (q >> 1) * (BM / 2);
    const int64_t n0 = (tile % a.n_tiles) * BN + (q & 1) * (BN / 2);
    if (t.row_base >= t.row_end || n0 >= a.N) continue;
    Q e;
    e.init(smem);
    blockscale_tile(e, a, t, n0, sc, sc_dummy);
  }
}

// ---------------------------------------------------------------------------
// Pre-shuffled W
// ---------------------------------------------------------------------------
//
// Layout of the pre-shuffled weights (also declared with f8f8bf16_shuffle_b): for
// group g, 32-row block nb and 64-byte K block kb, the 2048 bytes at
// ((g * N/32 + nb) * K/64 + kb) * 2048 hold the MFMA A operand of one 32x32x64
// step, lane l's 32 bytes split into halves: bytes [16*l, +16) and
// [1024 + 16*l, +16) hold W[g, 32*nb + perm32(l % 32), 64*kb + 32*(l / 32) .. +16)
// and the next 16 bytes, with perm32(r) = 16*((r >> 2) & 1) + 4*(r >> 3) + (r & 3).
// A block is one contiguous 2 KB copy; its halves read back from LDS with no bank
// conflicts; and perm32 puts W rows in MFMA order, so lane (h, r32) accumulates
// the 16 consecutive output columns 32*nb + 16*h .. +16.  The K blocks of one
// 32-row block follow each other, so a row block's K stream is contiguous.

__device__ __forceinline__ int perm32(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

__global__ void __launch_bounds__(256) shuffle_b_kernel(const v4i* __restrict__ W, v4i* __restrict__ Ws,
                                                        int64_t G, int64_t N, int64_t K) {
  // One 16-byte output chunk per iteration: chunk o of block blk is half
  // (o % 128) / 64, lane o % 64 of the block's 2048 bytes.
  const int64_t nb_n = N / 32, nb_k = K / 64;
  const int64_t total = G * N * K / 16;
  for (int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x; o < total; o += (int64_t)gridDim.x * 256) {
    const int64_t blk = o / 128;
    const int within = (int)(o % 128);
    const int half = within >> 6;
    const int lane = within & 63;
    const int64_t kb = blk % nb_k;
    const int64_t gnb = blk / nb_k;         // g * N/32 + nb
    const int64_t g = gnb / nb_n;
    const int64_t nb = gnb % nb_n;
    const int64_t row = nb * 32 + perm32(lane & 31);
    const int64_t col = kb * 64 + (lane >> 5) * 32 + half * 16;
    Ws[o] = W[((g * N + row) * K + col) / 16];
  }
}

// ---------------------------------------------------------------------------
// Small per-group M: stream W straight into registers, split K across waves
// ---------------------------------------------------------------------------
//
// For a few rows per group the call is bound by reading W once from HBM, so the
// work is spread over many workgroups: one per (group, 32 output columns, BM rows
// of X), with the four waves of a workgroup splitting K.  Each wave keeps D MFMA
// steps of W and X fragments in flight in a register ring (W rows are read in the
// MFMA A-operand layout directly from the row-major weights; X rows come from L2).
// The four partial sums are added through LDS in a fixed order (deterministic).
// A lane's accumulators are then 4-column runs of natural-order W rows; the
// epilogue pairs lanes 32 apart with permlane32_swap to form 16-byte stores.

template <int LAYOUT, int BM, int D, bool KTAIL>
__global__ void __launch_bounds__(256)
gg_skinny_kernel(GemmArgs a) {
  constexpr int FM = BM / 32;
  constexpr int WAVES = 4;
  static_assert(BM % 32 == 0, "BM must be a multiple of 32");

  __shared__ __attribute__((aligned(16))) float red[(WAVES - 1) * FM * 16 * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int64_t bid = blockIdx.x;
  const int64_t n_tile = bid % a.n_tiles;
  const int64_t rest = bid / a.n_tiles;
  Tile t;
  if (LAYOUT == kPadded) {
    if (!resolve_padded<BM>(a, rest / a.m_tiles, rest % a.m_tiles, t)) return;
  } else {
    if (!resolve_packed<LAYOUT, BM>(a, rest, t)) return;
  }
  const int64_t N = a.N;
  const int64_t K = a.K;
  const int64_t n0 = n_tile * 32;
  const int64_t tile_row_end = t.row_base + BM;
  if (t.row_base >= t.row_end) {
    const int64_t r1 = tile_row_end < t.zero_end ? tile_row_end : t.zero_end;
    const int64_t c1 = n0 + 32 < N ? n0 + 32 : N;
    zero_rect<256>(a.Y, N, t.row_base, r1, n0, c1);
    return;
  }

  const int h = lane >> 5;
  const int r32 = lane & 31;

  // The epilogue's scales are fetched now so that their latency hides under the K loop.
  const float* wsg = a.ws + t.g * N;
  float wsv[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t c = n0 + 8 * j + 4 * h;
    v4f w4 = {0.f, 0.f, 0.f, 0.f};
    if (c < N) w4 = *(const v4f*)(wsg + c);
    wsv[j][0] = w4.x;
    wsv[j][1] = w4.y;
    wsv[j][2] = w4.z;
    wsv[j][3] = w4.w;
  }
  float xsv[FM];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int64_t m = t.row_base + 32 * fm + r32;
    xsv[fm] = m < t.row_end ? a.xs[m] : 0.f;
  }

  int64_t wrow = n0 + r32;
  wrow = wrow < N ? wrow : N - 1;                         // columns past N: result dropped
  const uint8_t* wsrc = a.W + (t.g * N + wrow) * K + 32 * h;
  const uint8_t* xsrc[FM];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    int64_t row = t.row_base + 32 * fm + r32;
    row = row < t.row_end ? row : t.row_end - 1;          // rows past the group: result dropped
    xsrc[fm] = a.X + row * K + 32 * h;
  }

  const int nk = (int)((K + 63) / 64);
  const int per = (nk + WAVES - 1) / WAVES;
  const int kb = wave * per;
  const int ke = kb + per < nk ? kb + per : nk;

  // 32 bytes of one row at K step kt (two 16-byte chunks; chunks at or past K read 0).
  auto load32 = [&](const uint8_t* src, int kt) -> v8i {
    const int64_t ko = (int64_t)kt * 64;
    const v4i* p0 = (const v4i*)(src + ko);
    v4i lo, hi;
    if (!KTAIL || ko + 64 <= K) {
      lo = p0[0];
      hi = p0[1];
    } else {
      const v4i z = {0, 0, 0, 0};
      lo = (ko + 32 * h < K) ? p0[0] : z;
      hi = (ko + 32 * h + 16 < K) ? p0[1] : z;
    }
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  };

  v16f acc[FM];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) acc[fm] = v16f{0};
  v8i wr[D], xr[D][FM];
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (kb + d < ke) {
      wr[d] = load32(wsrc, kb + d);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) xr[d][fm] = load32(xsrc[fm], kb + d);
    }
  for (int kt0 = kb; kt0 < ke; kt0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int kt = kt0 + d;
      if (kt < ke) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) acc[fm] = mfma_32x32x64_fp8(wr[d], xr[d][fm], acc[fm]);
        if (kt + D < ke) {
          wr[d] = load32(wsrc, kt + D);
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) xr[d][fm] = load32(xsrc[fm], kt + D);
        }
      }
    }
  }

  // Partial sums of waves 1..3 -> LDS as 16-byte quarters (one ds_write_b128 /
  // ds_read_b128 per four accumulators); wave 0 adds them in wave order.
  v4f* red4 = reinterpret_cast<v4f*>(red);
  if (wave > 0) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        red4[(((wave - 1) * FM + fm) * 4 + q) * 64 + lane] =
            v4f{acc[fm][4 * q], acc[fm][4 * q + 1], acc[fm][4 * q + 2], acc[fm][4 * q + 3]};
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < WAVES; ++w)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f r = red4[(((w - 1) * FM + fm) * 4 + q) * 64 + lane];
        acc[fm][4 * q] += r.x;
        acc[fm][4 * q + 1] += r.y;
        acc[fm][4 * q + 2] += r.z;
        acc[fm][4 * q + 3] += r.w;
      }

  // Epilogue: MFMA row rho = 8*j + 4*h + tt of the block is column n0 + rho.
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int64_t m = t.row_base + 32 * fm + r32;
    const bool write = m < t.row_end;
    const bool zero = !write && m < t.zero_end;
    uint16_t* yrow = a.Y + m * N;
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      uint32_t e[2][2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * jp + jj;
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const float v0 = (acc[fm][4 * j + 2 * pr] * xsv[fm]) * wsv[j][2 * pr];
          const float v1 = (acc[fm][4 * j + 2 * pr + 1] * xsv[fm]) * wsv[j][2 * pr + 1];
          e[jj][pr] = pack_bf16x2(v0, v1);
        }
      }
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const auto sw = __builtin_amdgcn_permlane32_swap(e[0][pr], e[1][pr], false, false);
        e[0][pr] = sw[0];
        e[1][pr] = sw[1];
      }
      const int64_t c = n0 + 16 * jp + 8 * h;
      if (c < N) {
        if (write)
          *(v4i*)(yrow + c) = v4i{(int)e[0][0], (int)e[0][1], (int)e[1][0], (int)e[1][1]};
        else if (zero)
          *(v4i*)(yrow + c) = v4i{0, 0, 0, 0};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Zero fill (K == 0): a plain kernel rather than a memset, so the call can be
// captured into a graph without a memset node.
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(256) zero_fill_kernel(v4i* __restrict__ y, int64_t n_vec) {
  const v4i z = {0, 0, 0, 0};
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_vec; i += (int64_t)gridDim.x * 256) y[i] = z;
}

// ---------------------------------------------------------------------------
// Configuration table and launch dispatch
// ---------------------------------------------------------------------------

// kind: 0 = both operands through LDS (one tile per workgroup),
//       3 = small M: W and X straight to registers, K split across the 4 waves,
//       4 = kind 0 on a persistent grid whose last round may run as quarter tiles
//           (packed layouts: stacked, offsets, batched).
// pre: 1 = W pre-shuffled (the _preshuffle entry points), 0 = plain W.
//                      BM   BN   BK  WM WN stages kind wdepth twin pre
const KernelConfig kConfigs[] = {
    /* 0 */ {256, 256, 64, 2, 4, 4, 0, 0, 0},
    /* 1 */ {128, 256, 64, 2, 4, 4, 0, 0, 0},
    /* 2 */ {64, 256, 64, 1, 4, 2, 0, 0, 0},
    /* 3 */ {32, 128, 64, 1, 4, 2, 0, 0, 0},
    /* 4 */ {128, 256, 128, 2, 4, 3, 0, 0, 0, 1},
    /* 5 */ {64, 256, 128, 1, 4, 2, 0, 0, 0, 1},
    /* 6 */ {32, 128, 128, 1, 4, 3, 0, 0, 0, 1},
    /* 7 */ {256, 256, 128, 2, 4, 2, 0, 0, 0},
    /* 8 */ {256, 128, 128, 2, 4, 3, 0, 0, 0},
    /* 9 */ {128, 256, 128, 2, 4, 3, 0, 0, 0},
    /* 10 */ {128, 128, 128, 2, 2, 4, 0, 0, 0},
    /* 11 */ {256, 128, 128, 2, 2, 3, 0, 0, 0},
    /* 12 */ {128, 128, 64, 2, 2, 4, 0, 0, 0},
    /* 13 */ {32, 32, 64, 1, 4, 0, 3, 8, 0},
    /* 14 */ {64, 32, 64, 1, 4, 0, 3, 8, 0},
    /* 15 */ {32, 32, 64, 1, 4, 0, 3, 4, 0},
    /* 16 */ {256, 256, 128, 2, 4, 2, 4, 0, 7},
    /* 17 */ {128, 256, 128, 2, 4, 3, 4, 0, 9},
    /* 18 */ {32, 128, 128, 1, 4, 3, 0, 0, 0},
    /* 19 */ {32, 128, 64, 1, 4, 4, 0, 0, 0},
    /* 20 */ {32, 128, 128, 1, 4, 4, 0, 0, 0},
    /* 21 */ {32, 64, 128, 1, 2, 4, 0, 0, 0},
    /* 22 */ {32, 64, 128, 1, 2, 6, 0, 0, 0},
    /* 23 */ {32, 128, 128, 1, 4, 6, 0, 0, 0},
    /* 24 */ {32, 64, 128, 1, 2, 8, 0, 0, 0},
    /* 25 */ {256, 256, 128, 2, 4, 2, 0, 0, 0, 1},
    /* 26 */ {256, 256, 128, 2, 4, 2, 4, 0, 25, 1},
    /* 27 */ {32, 64, 128, 1, 2, 4, 0, 0, 0, 1},
    /* 28 */ {192, 256, 128, 2, 4, 2, 0, 0, 0},
};
const int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

template <int LAYOUT, int BM, int BN, int BK, int WM, int WN, int STAGES, bool PRE = false>
static hipError_t launch_lds(bool k_tail, const GemmArgs& a, int64_t grid, hipStream_t s) {
  const dim3 block(WM * WN * 64);
  if (k_tail)
    hipLaunchKernelGGL((gg_lds_kernel<LAYOUT, BM, BN, BK, WM, WN, STAGES, true, PRE>), dim3((uint32_t)grid), block,
                       0, s, a);
  else
    hipLaunchKernelGGL((gg_lds_kernel<LAYOUT, BM, BN, BK, WM, WN, STAGES, false, PRE>), dim3((uint32_t)grid), block,
                       0, s, a);
  return hipGetLastError();
}

template <int LAYOUT, int BM, int BN, int BK, int WM, int WN, int STAGES, bool PRE = false>
static hipError_t launch_persistent(bool k_tail, const GemmArgs& a, int grid, int tail_mode, hipStream_t s) {
  const dim3 block(WM * WN * 64);
  if (k_tail)
    hipLaunchKernelGGL((gg_persistent_kernel<LAYOUT, BM, BN, BK, WM, WN, STAGES, true, PRE>), dim3((uint32_t)grid),
                       block, 0, s, a, tail_mode);
  else
    hipLaunchKernelGGL((gg_persistent_kernel<LAYOUT, BM, BN, BK, WM, WN, STAGES, false, PRE>), dim3((uint32_t)grid),
                       block, 0, s, a, tail_mode);
  return hipGetLastError();
}

template <int LAYOUT, int BM, int D>
static hipError_t launch_skinny(bool k_tail, const GemmArgs& a, int64_t grid, hipStream_t s) {
  if (k_tail)
    hipLaunchKernelGGL((gg_skinny_kernel<LAYOUT, BM, D, true>), dim3((uint32_t)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gg_skinny_kernel<LAYOUT, BM, D, false>), dim3((uint32_t)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

// One case per row of kConfigs (same order).  Persistent rows (16, 17, 26) go
// through launch_gemm_persistent; the padded layout launches their twin here.
template <int LAYOUT>
static hipError_t launch_layout(int config_id, bool k_tail, const GemmArgs& a, int64_t grid, hipStream_t s) {
  switch (config_id) {
    case 0: return launch_lds<LAYOUT, 256, 256, 64, 2, 4, 4>(k_tail, a, grid, s);
    case 1: return launch_lds<LAYOUT, 128, 256, 64, 2, 4, 4>(k_tail, a, grid, s);
    case 2: return launch_lds<LAYOUT, 64, 256, 64, 1, 4, 2>(k_tail, a, grid, s);
    case 3: return launch_lds<LAYOUT, 32, 128, 64, 1, 4, 2>(k_tail, a, grid, s);
    case 4: return launch_lds<LAYOUT, 128, 256, 128, 2, 4, 3, true>(k_tail, a, grid, s);
    case 5: return launch_lds<LAYOUT, 64, 256, 128, 1, 4, 2, true>(k_tail, a, grid, s);
    case 6: return launch_lds<LAYOUT, 32, 128, 128, 1, 4, 3, true>(k_tail, a, grid, s);
    case 7: return launch_lds<LAYOUT, 256, 256, 128, 2, 4, 2>(k_tail, a, grid, s);
    case 8: return launch_lds<LAYOUT, 256, 128, 128, 2, 4, 3>(k_tail, a, grid, s);
    case 9: return launch_lds<LAYOUT, 128, 256, 128, 2, 4, 3>(k_tail, a, grid, s);
    case 10: return launch_lds<LAYOUT, 128, 128, 128, 2, 2, 4>(k_tail, a, grid, s);
    case 11: return launch_lds<LAYOUT, 256, 128, 128, 2, 2, 3>(k_tail, a, grid, s);
    case 12: return launch_lds<LAYOUT, 128, 128, 64, 2, 2, 4>(k_tail, a, grid, s);
    case 13: return launch_skinny<LAYOUT, 32, 8>(k_tail, a, grid, s);
    case 14: return launch_skinny<LAYOUT, 64, 8>(k_tail, a, grid, s);
    case 15: return launch_skinny<LAYOUT, 32, 4>(k_tail, a, grid, s);
    case 18: return launch_lds<LAYOUT, 32, 128, 128, 1, 4, 3>(k_tail, a, grid, s);
    case 19: return launch_lds<LAYOUT, 32, 128, 64, 1, 4, 4>(k_tail, a, grid, s);
    case 20: return launch_lds<LAYOUT, 32, 128, 128, 1, 4, 4>(k_tail, a, grid, s);
    case 21: return launch_lds<LAYOUT, 32, 64, 128, 1, 2, 4>(k_tail, a, grid, s);
    case 22: return launch_lds<LAYOUT, 32, 64, 128, 1, 2, 6>(k_tail, a, grid, s);
    case 23: return launch_lds<LAYOUT, 32, 128, 128, 1, 4, 6>(k_tail, a, grid, s);
    case 24: return launch_lds<LAYOUT, 32, 64, 128, 1, 2, 8>(k_tail, a, grid, s);
    case 25: return launch_lds<LAYOUT, 256, 256, 128, 2, 4, 2, true>(k_tail, a, grid, s);
    case 27: return launch_lds<LAYOUT, 32, 64, 128, 1, 2, 4, true>(k_tail, a, grid, s);
    case 28: return launch_lds<LAYOUT, 192, 256, 128, 2, 4, 2>(k_tail, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int LAYOUT>
static hipError_t launch_persistent_layout(int config_id, bool k_tail, const GemmArgs& a, int grid, int tail_mode,
                                           hipStream_t s) {
  switch (config_id) {
    case 16: return launch_persistent<LAYOUT, 256, 256, 128, 2, 4, 2>(k_tail, a, grid, tail_mode, s);
    case 17: return launch_persistent<LAYOUT, 128, 256, 128, 2, 4, 3>(k_tail, a, grid, tail_mode, s);
    case 26: return launch_persistent<LAYOUT, 256, 256, 128, 2, 4, 2, true>(k_tail, a, grid, tail_mode, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_persistent(int layout, int config_id, bool k_tail, const GemmArgs& a, int grid,
                                  int tail_mode, hipStream_t s) {
  switch (layout) {
    case kStacked: return launch_persistent_layout<kStacked>(config_id, k_tail, a, grid, tail_mode, s);
    case kOffsets: return launch_persistent_layout<kOffsets>(config_id, k_tail, a, grid, tail_mode, s);
    case kBatched: return launch_persistent_layout<kBatched>(config_id, k_tail, a, grid, tail_mode, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(int layout, int config_id, bool k_tail, const GemmArgs& a, int64_t grid,
                       hipStream_t s) {
  switch (layout) {
    case kStacked: return launch_layout<kStacked>(config_id, k_tail, a, grid, s);
    case kPadded: return launch_layout<kPadded>(config_id, k_tail, a, grid, s);
    case kOffsets: return launch_layout<kOffsets>(config_id, k_tail, a, grid, s);
    case kBatched: return launch_layout<kBatched>(config_id, k_tail, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int LAYOUT, int BM, int BN, int BK, int WM, int WN, int STAGES>
static hipError_t launch_ragged(bool k_tail, const GemmArgs& a, int64_t grid, hipStream_t s) {
  const dim3 block(WM * WN * 64);
  // k_offsets: the slices' lengths are device-side, so the tail mask is always in
  if (k_tail || LAYOUT == kKOffsets)
    hipLaunchKernelGGL((gg_ragged_kernel<LAYOUT, BM, BN, BK, WM, WN, STAGES, true>), dim3((uint32_t)grid), block, 0,
                       s, a);
  else
    hipLaunchKernelGGL((gg_ragged_kernel<LAYOUT, BM, BN, BK, WM, WN, STAGES, false>), dim3((uint32_t)grid), block,
                       0, s, a);
  return hipGetLastError();
}

// The configurations the ragged layouts are built for (a subset of kConfigs with
// plain W and one tile per workgroup).
template <int LAYOUT>
static hipError_t launch_ragged_layout(int config_id, bool k_tail, const GemmArgs& a, int64_t grid, hipStream_t s) {
  switch (config_id) {
    case 2: return launch_ragged<LAYOUT, 64, 256, 64, 1, 4, 2>(k_tail, a, grid, s);
    case 7: return launch_ragged<LAYOUT, 256, 256, 128, 2, 4, 2>(k_tail, a, grid, s);
    case 9: return launch_ragged<LAYOUT, 128, 256, 128, 2, 4, 3>(k_tail, a, grid, s);
    case 18: return launch_ragged<LAYOUT, 32, 128, 128, 1, 4, 3>(k_tail, a, grid, s);
    case 21: return launch_ragged<LAYOUT, 32, 64, 128, 1, 2, 4>(k_tail, a, grid, s);
    case 28: return launch_ragged<LAYOUT, 192, 256, 128, 2, 4, 2>(k_tail, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_ragged(int layout, int config_id, bool k_tail, const GemmArgs& a, int64_t grid,
                              hipStream_t s) {
  switch (layout) {
    case kNOffsets: return launch_ragged_layout<kNOffsets>(config_id, k_tail, a, grid, s);
    case kKOffsets: return launch_ragged_layout<kKOffsets>(config_id, k_tail, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

// Block-scaled configurations: 0 = 128 x 256 tiles (2 x 4 waves, 3 stages),
// 1 = 32 x 128 tiles (1 x 4 waves, 3 stages) for few rows per group, 2 = the
// 128 x 256 tiles on a persistent grid (grid = compute units).
template <int LAYOUT, bool PRE>
static hipError_t launch_blockscale(int config, const GemmArgs& a, int64_t grid, hipStream_t s) {
  switch (config) {
    case 0:
      hipLaunchKernelGGL((gg_blockscale_kernel<LAYOUT, 128, 256, 2, 4, 3, PRE>), dim3((uint32_t)grid), dim3(512), 0,
                         s, a);
      return hipGetLastError();
    case 1:
      hipLaunchKernelGGL((gg_blockscale_kernel<LAYOUT, 32, 128, 1, 4, 3, PRE>), dim3((uint32_t)grid), dim3(256), 0, s,
                         a);
      return hipGetLastError();
    case 2:
      if constexpr (LAYOUT == kPadded) {
        return hipErrorInvalidValue;   // the persistent grid walks packed rows only
      } else {
        hipLaunchKernelGGL((gg_blockscale_persistent_kernel<LAYOUT, 128, 256, 2, 4, 3, PRE>), dim3((uint32_t)grid),
                           dim3(512), 0, s, a);
        return hipGetLastError();
      }
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_blockscale(int layout, int config, bool preshuffled, const GemmArgs& a, int64_t grid,
                                  hipStream_t s) {
  switch (layout) {
#define FP8GG_BS_LAYOUT(L) \
  case L: return preshuffled ? launch_blockscale<L, true>(config, a, grid, s) : launch_blockscale<L, false>(config, a, grid, s);
    FP8GG_BS_LAYOUT(kStacked)
    FP8GG_BS_LAYOUT(kPadded)
    FP8GG_BS_LAYOUT(kOffsets)
    FP8GG_BS_LAYOUT(kBatched)
#undef FP8GG_BS_LAYOUT
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_zero_fill(uint16_t* Y, int64_t n_elems, hipStream_t s) {
  const int64_t n_vec = n_elems / 8;  // N % 8 == 0, so the output is whole 16-byte vectors
  if (n_vec == 0) return hipSuccess;
  int64_t blocks = (n_vec + 255) / 256;
  blocks = blocks > 4096 ? 4096 : blocks;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, (v4i*)Y, n_vec);
  return hipGetLastError();
}

hipError_t launch_shuffle_b(const uint8_t* W, uint8_t* Ws, int64_t G, int64_t N, int64_t K, hipStream_t s) {
  const int64_t chunks = G * N * K / 16;
  if (chunks == 0) return hipSuccess;
  int64_t blocks = (chunks + 255) / 256;
  blocks = blocks > 8192 ? 8192 : blocks;
  hipLaunchKernelGGL(shuffle_b_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, (const v4i*)W, (v4i*)Ws, G, N, K);
  return hipGetLastError();
}

}  // namespace fp8gg
