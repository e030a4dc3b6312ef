// Dense scaled FP8 GEMM kernels for gfx950: one C tile per workgroup.
//
// Tile order.  "Hopper/Blackwell architecture features" §12.7.1 reorders program
// ids in groups of GROUP_M tile rows so that concurrently running tiles share A
// rows and B columns in L2.  MI355X has one L2 per XCD (8 XCDs of 32 CUs) and the
// hardware deals workgroup ids round-robin over the XCDs, so the id is first
// remapped to make each XCD own a contiguous range of the grouped order: the
// tiles running together on one XCD then form a compact GROUP_M x k block.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_tile.h"
#include "launch.h"
#include "tile_order.h"

namespace fp8gemm {
namespace {

template <class Cfg, int MODE, typename OutT, bool KALIGNED>
__global__ __launch_bounds__(Cfg::kThreads, Cfg::kWavesPerEu) void gemm_kernel(GemmProblem p,
                                                                              int tiles_m,
                                                              int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Cfg::kLdsBytes];
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, kGroupM, &tm, &tn);
  const int m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;

  TileOperands op;
  op.A = p.A + (int64_t)m0 * p.lda;
  op.lda = p.lda;
  op.a_rows = p.M - m0;
  op.B = p.B + (int64_t)n0 * p.ldb;
  op.ldb = p.ldb;
  op.b_rows = p.N - n0;
  op.K = p.K;
  const float* fsa = static_cast<const float*>(p.scale_a);
  const float* fsb = static_cast<const float*>(p.scale_b);
  op.sa = op.sb = nullptr;
  op.ra = op.rb = nullptr;
  if (MODE == kMx32) {
    op.sa = static_cast<const uint8_t*>(p.scale_a) + (int64_t)m0 * (p.K / 32);
    op.sb = static_cast<const uint8_t*>(p.scale_b) + (int64_t)n0 * (p.K / 32);
  }
  if (MODE == kRowwise) {
    op.ra = fsa + m0;
    op.rb = fsb + n0;
  }

  const float ts = (MODE == kTensor) ? fsa[0] * fsb[0] : 1.0f;
  gemm_tile<Cfg, MODE, OutT, KALIGNED>(op, lds, static_cast<OutT*>(p.C), p.ldc, m0, p.M, n0, p.N,
                                       ts);
}

template <class Cfg, int MODE, typename OutT>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t stream) {
  const int tiles_m = (p.M + Cfg::BM - 1) / Cfg::BM;
  const int tiles_n = (p.N + Cfg::BN - 1) / Cfg::BN;
  const int grid = tiles_m * tiles_n;
  if (p.K % 128 == 0)
    hipLaunchKernelGGL((gemm_kernel<Cfg, MODE, OutT, true>), dim3(grid), dim3(Cfg::kThreads), 0,
                       stream, p, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((gemm_kernel<Cfg, MODE, OutT, false>), dim3(grid), dim3(Cfg::kThreads), 0,
                       stream, p, tiles_m, tiles_n);
  return hipGetLastError();
}

// Large-problem tile.  FP8GEMM_BIG_CFG selects it (tuning switch):
//   0: 256 x 256, 4 wavefronts of 128 x 128, one workgroup per CU, 4-slot ring
//   1: 256 x 128, 4 wavefronts of 128 x 64, two workgroups per CU, 3-slot ring
#ifndef FP8GEMM_BIG_CFG
#define FP8GEMM_BIG_CFG 0
#endif
#if FP8GEMM_BIG_CFG == 0
using Big = TileCfg<256, 256, 128, 128, 4, 1>;
#else
using Big = TileCfg<256, 128, 128, 64, 3, 2>;
#endif
using Mid = TileCfg<128, 128, 64, 64, 4, 2>;

template <int MODE, typename OutT>
hipError_t launch_mode(const GemmProblem& p, hipStream_t stream) {
  // Large tiles when they still give at least one tile per CU; otherwise smaller
  // tiles for more parallelism.
  const int64_t big_tiles = (int64_t)((p.M + Big::BM - 1) / Big::BM) * ((p.N + Big::BN - 1) / Big::BN);
  // MX with K % 128 != 0 reads its codes into registers: the large tile would spill
  const bool mx_ragged = MODE == kMx32 && p.K % 128 != 0;
  if (big_tiles >= 256 * Big::kWgPerCu && !mx_ragged) return launch_cfg<Big, MODE, OutT>(p, stream);
  return launch_cfg<Mid, MODE, OutT>(p, stream);
}

}  // namespace

hipError_t launch_gemm(const GemmProblem& p, int mode, int out, hipStream_t stream) {
  if (out == kF16) {
    if (mode == kTensor) return launch_mode<kTensor, _Float16>(p, stream);
    if (mode == kRowwise) return launch_mode<kRowwise, _Float16>(p, stream);
    return launch_mode<kMx32, _Float16>(p, stream);
  }
  if (mode == kTensor) return launch_mode<kTensor, __bf16>(p, stream);
  if (mode == kRowwise) return launch_mode<kRowwise, __bf16>(p, stream);
  return launch_mode<kMx32, __bf16>(p, stream);
}

}  // namespace fp8gemm
