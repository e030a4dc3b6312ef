// Host-side choice of the dense GEMM kernel for a shape.  The launch code in
// gemm.hip and the fp8gemm_run_path query of the C ABI both call choose_path(),
// so the path a call reports is the path it takes.
//
// Paths, from few output tiles to many:
//   * split-K: fewer than 128 tiles of 128 x 128 and K >= 1024.  64 x 64 tiles,
//     K cut into S slices so that tiles x S fills the GPU; the slices meet
//     through fp32 partial tiles in the workspace (the decode-like M = 128 shape
//     of "Hopper/Blackwell architecture features" §12.2.4);
//   * 128 x 128 tiles, one per workgroup, two workgroups per CU;
//   * 256 x 256 tiles, one per workgroup, once they give a tile per CU;
//   * persistent: 256 x 256 tiles walked by one workgroup per CU as a single copy
//     stream (§12.7.3 persistent kernels), from eight tiles per CU on, when every
//     tile is a full interior tile and the epilogue is the plain 16-bit one.
#pragma once

#include <stdint.h>

#include "launch.h"

namespace fp8gemm {

enum GemmPath : int {
  kPathNone = 0,        // nothing to launch (M or N is 0)
  kPathSplitK = 1,
  kPathTile128 = 2,
  kPathTile256 = 3,
  kPathPersistent = 4,
};

// Output tile edges of the configurations (gemm.hip checks its tile
// configurations against these).
constexpr int kBigTile = 256;
constexpr int kMidTile = 128;
constexpr int kSplitTile = 64;
// split-K: aim for one workgroup per CU of an MI355X
constexpr int kSplitTargetWgs = 256;
// the arrival counters (one int per split tile) fill the fixed counter head
constexpr int64_t kMaxSplitTiles = kSplitCounterBytes / 4;
// persistent streams pay off from about eight tiles per CU on (measured)
constexpr int64_t kPersistentTiles = 8 * 256;

struct SplitPlan {
  int splits = 1, tiles_m = 0, tiles_n = 0;
};

// K counts bytes of a code row (FP4: two elements per byte); blk_bytes is the
// byte length of one 32-element MX block (32, FP4 16).  Slices keep the interior
// path: whole 128-byte K tiles, and for MX whole 16-code groups (512 elements).
inline SplitPlan plan_split(int64_t M, int64_t N, int64_t K, int mode, int blk_bytes) {
  SplitPlan plan;
  const int64_t mid_tiles = ((M + kMidTile - 1) / kMidTile) * ((N + kMidTile - 1) / kMidTile);
  if (mid_tiles >= 128 || K < 1024) return plan;
  const int64_t tm = (M + kSplitTile - 1) / kSplitTile;
  const int64_t tn = (N + kSplitTile - 1) / kSplitTile;
  const int64_t gran = mode == kMx32 ? 16 * blk_bytes : 128;
  int best = 1;
  for (int s = 2; s <= 16; s *= 2) {
    if (K % (s * gran) != 0 || K / s < 512) break;
    best = s;
    if (tm * tn * s >= kSplitTargetWgs) break;
  }
  if (best == 1 || tm * tn > kMaxSplitTiles) return plan;
  // the partials are addressed with 32-bit buffer offsets
  if (tm * tn * best * kSplitTile * kSplitTile * 4 >= ((int64_t)1 << 31)) return plan;
  plan.splits = best;
  plan.tiles_m = (int)tm;
  plan.tiles_n = (int)tn;
  return plan;
}

// Workspace bytes of a plan: the counter head, then the fp32 partial tiles.
inline int64_t split_workspace_bytes(const SplitPlan& plan) {
  if (plan.splits <= 1) return 0;
  const int64_t tiles = (int64_t)plan.tiles_m * plan.tiles_n;
  return kSplitCounterBytes + tiles * plan.splits * kSplitTile * kSplitTile * 4;
}

// Workspace a dense GEMM needs (K in elements): the split-K plan of FP8
// operands; FP4 shapes split along K at most as often as FP8 ones of the same
// element count (their slices are whole 256-byte code groups), so this covers them.
inline int64_t gemm_workspace_need(int64_t M, int64_t N, int64_t K, int mode) {
  return split_workspace_bytes(plan_split(M, N, K, mode, 32));
}

// The byte span of a tile's rows fits the 32-bit offsets of a buffer descriptor.
inline bool spans_fit(int64_t rows, int64_t ld, int64_t K) {
  return rows * ld + K < ((int64_t)1 << 31);
}

// Path of a dense GEMM.  K counts bytes (FP4: K / 2 of the elements); fp4: both
// operands are e2m1; fused: a bias or activation, or the quantised output.
inline GemmPath choose_path(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int mode,
                            bool fp4, bool fused) {
  if (M <= 0 || N <= 0) return kPathNone;
  const int blk = fp4 ? 16 : 32;
  if (plan_split(M, N, K, mode, blk).splits > 1) return kPathSplitK;
  const int64_t big_tiles = ((M + kBigTile - 1) / kBigTile) * ((N + kBigTile - 1) / kBigTile);
  const bool big_interior = M % kBigTile == 0 && N % kBigTile == 0 &&
                            spans_fit(kBigTile, lda, K) && spans_fit(kBigTile, ldb, K);
  if (fp4) {
    // FP4: the large tile only when every tile runs the interior mainloop (K a whole
    // number of code groups, 32-bit spans; tiles cut by M or N included): its other
    // edge tiles would read their codes into registers and spill; no persistent stream
    if (big_tiles >= 256 && K % (16 * blk) == 0 && spans_fit(kBigTile, lda, K) &&
        spans_fit(kBigTile, ldb, K))
      return kPathTile256;
    return kPathTile128;
  }
  // MX with K % 128 != 0 reads its codes into registers: the large tile would spill
  const bool mx_ragged = mode == kMx32 && K % 128 != 0;
  if (big_tiles >= 256 && !mx_ragged) {
    if (!fused && big_tiles >= kPersistentTiles && big_interior && K % 512 == 0)
      return kPathPersistent;
    return kPathTile256;
  }
  return kPathTile128;
}

// Path of the GEMM with row-major B ([K][N], N contiguous) read by the kernels
// themselves (transposing LDS reads): the dense choice without the persistent
// stream.  kPathNone (with M, N > 0) where that form does not apply: K % 128 != 0
// (MX: K % 512 != 0, whole code groups) or spans past 32-bit buffer offsets; the
// caller then makes B K-contiguous first.
// K counts elements; fp4: MXFP4 operands (A rows of K / 2 bytes, B K-rows of
// packed pairs along N; MX only), planned like the K-contiguous FP4 GEMM.
inline GemmPath choose_path_kn(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                               int mode, bool fp4 = false) {
  if (M <= 0 || N <= 0) return kPathNone;
  if (fp4 && mode != kMx32) return kPathNone;
  if (K % (mode == kMx32 ? 512 : 128) != 0) return kPathNone;
  const int64_t ka = fp4 ? K / 2 : K;               // bytes of an A row
  if (!spans_fit(kBigTile, lda, ka) || !spans_fit(K, ldb, kBigTile)) return kPathNone;
  if (mode == kMx32 && !spans_fit(K / 32, N, kBigTile)) return kPathNone;
  if (plan_split(M, N, ka, mode, fp4 ? 16 : 32).splits > 1) return kPathSplitK;
  const int64_t big_tiles = ((M + kBigTile - 1) / kBigTile) * ((N + kBigTile - 1) / kBigTile);
  return big_tiles >= 256 ? kPathTile256 : kPathTile128;
}

// Path of the MXFP6 GEMM (K in elements, K % 128 == 0; lda, ldb in bytes): the
// 256 x 256 tile once it gives a tile per CU and its 256-row spans fit 32-bit
// offsets, else 128 x 128 tiles.
inline GemmPath choose_path_fp6(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
  if (M <= 0 || N <= 0) return kPathNone;
  const int64_t kb = K / 4 * 3;
  const int64_t big_tiles = ((M + kBigTile - 1) / kBigTile) * ((N + kBigTile - 1) / kBigTile);
  if (big_tiles >= 256 && spans_fit(kBigTile, lda, kb) && spans_fit(kBigTile, ldb, kb))
    return kPathTile256;
  return kPathTile128;
}

}  // namespace fp8gemm
