// Internal interface between the host API (validation, planning) and the
// device kernels of the fp8 rowwise-scaled grouped GEMM library.
#ifndef FP8GG_INTERNAL_H_
#define FP8GG_INTERNAL_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8gg {

enum Layout : int { kStacked = 0, kPadded = 1 };

// Operands of one grouped GEMM call, as the kernels see them.  Row-major, dense.
struct GemmArgs {
  const uint8_t* X;      // stacked: [M, K]; padded: [G * M, K] (M = expected_m)
  const uint8_t* W;      // [G, N, K] (plain) or the pre-shuffled blocks
  const float* xs;       // one scale per row of X
  const float* ws;       // [G, N]
  const int64_t* meta;   // stacked: M_sizes [G]; padded: zero_start_index_M [G]
  uint16_t* Y;           // bf16 bits, one row per row of X, N columns
  int64_t G, M, N, K;
  int64_t m_tiles;       // stacked: upper bound of M tiles over all groups; padded: per slab
  int64_t n_tiles;
  int32_t zeroing;       // padded: write zeros into padding rows
};

// A compiled kernel configuration (workgroup tile and pipeline).
struct KernelConfig {
  int BM;       // rows of X per workgroup
  int BN;       // columns of Y (rows of W) per workgroup
  int BK;       // K bytes per pipeline stage (64 or 128: one or two 32x32x64 MFMA steps)
  int WM, WN;   // waves along M and N (threads = 64 * WM * WN)
  int stages;   // LDS pipeline depth (X and W; X only when W is pre-shuffled)
  int kind;     // 0: X and W through LDS; 3: small M, W and X straight to registers with
                // K split across waves; 4: kind 0 on a persistent grid whose last wave
                // is split along K (stacked layout)
  int wdepth;   // kind 3: K steps of fragments held in flight in registers
  int twin;     // kind 4: the kind-0 configuration with the same tile (used without workspace)
  int pre;      // 1: W pre-shuffled by f8f8bf16_shuffle_b (the _preshuffle entry points)
};

enum { kKindLds = 0, kKindSkinny = 3, kKindSplitTail = 4 };

extern const KernelConfig kConfigs[];
extern const int kNumConfigs;

inline bool is_preshuffled(const KernelConfig& c) { return c.pre != 0; }

// Split-tail workspace for a grid of P workgroups: P uint32 counters first (at a
// fixed offset whatever the configuration, so a workspace shared by several
// configurations keeps them zero), then one fp32 partial tile per workgroup.
inline size_t tail_counters_bytes(int P) { return ((size_t)P * 4 + 255) / 256 * 256; }
inline size_t tail_workspace_bytes(const KernelConfig& c, int P) {
  return tail_counters_bytes(P) + (size_t)P * c.BM * c.BN * 4;
}

constexpr int kMaxTailSplit = 16;

// Number of K pieces for each tile of the last, partial wave of a persistent grid
// of P workgroups over T tiles of nk K stages (1: no split).  With rem = T % P
// tiles left over, s pieces per tile need rem * s <= P workgroups and at least one
// stage each.  Cost of the last wave, in tenths of a stage time (fitted on MI355X
// to device timestamps of the 128 x 256 tile and to gate_up's 256 x 256 tail timed
// at s = 1, 3, 4, 5):
//   unsplit:  10 * nk                (few busy compute units stream faster, but
//                                     the whole K loop is on the critical path)
//   split:    11 * ceil(nk / s)      (longest piece, all compute units busy)
//          + (26 + 16 * s) * r       (partial write and L2 write-back fence, then
//                                     the finisher's reload of s partials),
// r = partial bytes / stage bytes.  force > 0 requests a split factor instead,
// clamped to what the shape allows.
__host__ __device__ inline int tail_split(int64_t T, int64_t P, int64_t nk, int64_t stage_bytes,
                                          int64_t partial_bytes, int force) {
  const int64_t rem = P > 0 ? T % P : 0;
  if (rem == 0 || nk < 2) return 1;
  int64_t smax = P / rem;
  if (smax > nk) smax = nk;
  if (smax > kMaxTailSplit) smax = kMaxTailSplit;
  if (force > 0) return (int)(force < smax ? force : smax);
  int best = 1;
  int64_t best_cost = 10 * nk * stage_bytes;
  for (int s = 2; s <= smax; ++s) {
    const int64_t cost = 11 * ((nk + s - 1) / s) * stage_bytes + (26 + 16 * (int64_t)s) * partial_bytes;
    if (cost < best_cost) {
      best = s;
      best_cost = cost;
    }
  }
  return best;
}

inline int lds_bytes(const KernelConfig& c) {
  if (c.kind == kKindSkinny) return 3 * (c.BM / 32) * 16 * 64 * 4;
  const int stages = c.stages * (c.BM + c.BN) * c.BK;
  // split tail: two scale blocks, a dummy word per lane and the finisher flag
  return c.kind == kKindSplitTail ? stages + 2 * (c.BM + c.BN) * 4 + 256 + 4 : stages;
}

hipError_t launch_gemm(int layout, int config_id, bool k_tail, const GemmArgs& args,
                       int64_t grid, hipStream_t stream);
hipError_t launch_gemm_tail(int config_id, bool k_tail, const GemmArgs& args, int grid, float* partials,
                            uint32_t* counters, int force_split, hipStream_t stream);
hipError_t launch_zero_fill(uint16_t* Y, int64_t n_elems, hipStream_t stream);
hipError_t launch_shuffle_b(const uint8_t* W, uint8_t* Ws, int64_t G, int64_t N, int64_t K,
                            hipStream_t stream);

}  // namespace fp8gg

#endif  // FP8GG_INTERNAL_H_
