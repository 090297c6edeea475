// Internal interface between the host API (validation, planning) and the
// device kernels of the fp8 rowwise-scaled grouped GEMM library.
#ifndef FP8GG_INTERNAL_H_
#define FP8GG_INTERNAL_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8gg {

// Values match FP8GG_LAYOUT_* of the public header.
enum Layout : int { kStacked = 0, kPadded = 1, kOffsets = 2, kBatched = 3, kNOffsets = 4, kKOffsets = 5 };

// Layouts whose groups partition the output columns (n_offsets) or the
// contraction (k_offsets) instead of the rows.
inline bool is_ragged_layout(int layout) { return layout == kNOffsets || layout == kKOffsets; }

// Operands of one grouped GEMM call, as the kernels see them.  Row-major, dense.
struct GemmArgs {
  const uint8_t* X;      // stacked, offsets, k_offsets: [M, K]; padded, batched, n_offsets: [G * M, K]
  const uint8_t* W;      // [G, N, K] (plain) or the pre-shuffled blocks; n_offsets, k_offsets: [N, K]
  const float* xs;       // one scale per row of X; k_offsets: [G, M]; block scales: [rows, K / 128]
  const float* ws;       // [G, N]; n_offsets: [N]; block scales: [G, N / 128, K / 128]
  const int64_t* meta;   // stacked: M_sizes [G]; padded: zero_start_index_M [G]; else unused
  const int32_t* offs;   // inclusive int32 prefix [G]: rows (offsets), W rows (n_offsets), K (k_offsets)
  uint16_t* Y;           // bf16 bits, one row per row of X, N columns
  int64_t G, M, N, K;
  int64_t m_tiles;       // packed: upper bound of M tiles over all groups; padded: per slab
  int64_t n_tiles;
  int32_t zeroing;       // padded: write zeros into padding rows
  int32_t xcd_group;     // one-tile-per-workgroup grids: 1 = each XCD takes a contiguous share of the tiles (xcd_slot)
  int32_t skip_dead;     // 1: waves whose rows all lie past the tile's group issue no MFMAs
};

// A compiled kernel configuration (workgroup tile and pipeline).
struct KernelConfig {
  int BM;       // rows of X per workgroup
  int BN;       // columns of Y (rows of W) per workgroup
  int BK;       // K bytes per pipeline stage (64 or 128: one or two 32x32x64 MFMA steps)
  int WM, WN;   // waves along M and N (threads = 64 * WM * WN)
  int stages;   // LDS pipeline depth (X and W; X only when W is pre-shuffled)
  int kind;     // 0: X and W through LDS; 3: small M, W and X straight to registers with
                // K split across waves; 4: kind 0 on a persistent grid whose last round
                // may run as quarter tiles (packed layouts)
  int wdepth;   // kind 3: K steps of fragments held in flight in registers
  int twin;     // kind 4: the kind-0 configuration with the same tile (used for the padded layout)
  int pre;      // 1: W pre-shuffled by f8f8bf16_shuffle_b (the _preshuffle entry points)
};

enum { kKindLds = 0, kKindSkinny = 3, kKindPersistent = 4 };

extern const KernelConfig kConfigs[];
extern const int kNumConfigs;

inline bool is_preshuffled(const KernelConfig& c) { return c.pre != 0; }

// Whether the persistent grid of P workgroups computes the rem = T % P tiles of its
// last round as quarter tiles: mode 0 when they make at most two rounds of quarters
// (4 * rem <= 2 * P), mode 1 never, mode 2 whenever rem > 0.
__host__ __device__ inline bool tail_quarters(int64_t T, int64_t P, int mode) {
  const int64_t rem = P > 0 ? T % P : 0;
  if (rem == 0 || mode == 1) return false;
  return mode == 2 || 4 * rem <= 2 * P;
}

inline int lds_bytes(const KernelConfig& c) {
  if (c.kind == kKindSkinny) return 3 * (c.BM / 32) * 16 * 64 * 4;
  return c.stages * (c.BM + c.BN) * c.BK;
}

hipError_t launch_gemm(int layout, int config_id, bool k_tail, const GemmArgs& args,
                       int64_t grid, hipStream_t stream);
hipError_t launch_gemm_persistent(int layout, int config_id, bool k_tail, const GemmArgs& args, int grid,
                                  int tail_mode, hipStream_t stream);
hipError_t launch_gemm_ragged(int layout, int config_id, bool k_tail, const GemmArgs& args, int64_t grid,
                              hipStream_t stream);
// Block-scaled stacked GEMM: config 0 tiles 128 x 256, config 1 tiles 32 x 128,
// config 2 the 128 x 256 tiles on a persistent grid (one workgroup per CU).
constexpr int kBlockscaleTileM[3] = {128, 32, 128};
constexpr int kBlockscaleTileN[3] = {256, 128, 256};
constexpr int kBlockscalePersistent = 2;
hipError_t launch_gemm_blockscale(int layout, int config, bool preshuffled, const GemmArgs& args, int64_t grid,
                                  hipStream_t stream);
hipError_t launch_zero_fill(uint16_t* Y, int64_t n_elems, hipStream_t stream);
hipError_t launch_quantize_rowwise(const uint16_t* X, uint8_t* XQ, float* x_scale, int64_t rows, int64_t K,
                                   hipStream_t stream);
hipError_t launch_shuffle_b(const uint8_t* W, uint8_t* Ws, int64_t G, int64_t N, int64_t K,
                            hipStream_t stream);

}  // namespace fp8gg

#endif  // FP8GG_INTERNAL_H_
