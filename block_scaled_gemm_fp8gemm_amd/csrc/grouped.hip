// Grouped (mixture-of-experts) scaled FP8 GEMM for gfx950: a persistent kernel
// that walks the output tiles of all experts.
//
// The JAX/Triton Blackwell FP8 GEMM post extends the GEMM to MoE as a grouped GEMM
// in which expert weights are shared between the programs that use them (TMA
// multicast on that hardware); "Hopper/Blackwell architecture features" §12.7.3
// recommends persistent kernels (grid = number of SMs, each program loops over
// tiles) for launch cost and L2 reuse.  Here:
//   * the grid is one workgroup per CU; expert row offsets stay on the device and
//     every workgroup derives the per-expert tile counts ceil(m_g/BM)*ceil(N/BN)
//     and their prefix sums in LDS, so the host never synchronizes;
//   * tiles are numbered expert by expert, tile rows fastest, so the tiles
//     running at the same time share the same expert weight columns; the slot of
//     a workgroup inside each round of the persistent loop is remapped so one XCD
//     runs a contiguous run of tiles and reads each weight tile into its own L2
//     once (the MI355X counterpart of sharing expert weights by multicast);
//   * each tile uses the dense mainloop and epilogue, with rows past the expert's
//     end clamped on load and masked on store (ragged experts, empty experts).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_tile.h"
#include "launch.h"
#include "tile_order.h"

namespace fp8gemm {
namespace {

constexpr int kMaxGroups = 1024;

template <class Cfg, int MODE, typename OutT, bool KALIGNED>
__global__ __launch_bounds__(Cfg::kThreads, Cfg::kWavesPerEu) void grouped_kernel(GroupedProblem p,
                                                                                 int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Cfg::kLdsBytes];
  __shared__ int tile_start[kMaxGroups + 1];
  __shared__ int row_begin[kMaxGroups];
  __shared__ int row_end[kMaxGroups];

  if (threadIdx.x == 0) {
    // Offsets are clamped into [0, total_m] so no row outside A or C is touched
    // even when they break the documented rules.
    int acc = 0;
    tile_start[0] = 0;
    for (int g = 0; g < p.groups; ++g) {
      int a = p.offsets[g], b = p.offsets[g + 1];
      a = a < 0 ? 0 : (a > p.total_m ? p.total_m : a);
      b = b < a ? a : (b > p.total_m ? p.total_m : b);
      row_begin[g] = a;
      row_end[g] = b;
      acc += ((b - a + Cfg::BM - 1) / Cfg::BM) * tiles_n;
      tile_start[g + 1] = acc;
    }
  }
  __syncthreads();
  const int total = tile_start[p.groups];
  const int slot = xcd_linear(blockIdx.x, gridDim.x);
  const float* fsa = static_cast<const float*>(p.scale_a);
  const float* fsb = static_cast<const float*>(p.scale_b);

  for (int t = slot; t < total; t += gridDim.x) {
    // expert of tile t: last g with tile_start[g] <= t
    int lo = 0, hi = p.groups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_start[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    const int g = lo;
    const int local = t - tile_start[g];
    const int rows_g = row_end[g] - row_begin[g];
    const int tiles_m_g = (rows_g + Cfg::BM - 1) / Cfg::BM;
    const int tm = local % tiles_m_g, tn = local / tiles_m_g;
    const int m0 = row_begin[g] + tm * Cfg::BM;
    const int m_end = row_end[g];
    const int n0 = tn * Cfg::BN;

    TileOperands op;
    op.A = p.A + (int64_t)m0 * p.lda;
    op.lda = p.lda;
    op.a_rows = m_end - m0;
    const uint8_t* Bg = p.B + (int64_t)g * p.stride_b;
    op.B = Bg + (int64_t)n0 * p.ldb;
    op.ldb = p.ldb;
    op.b_rows = p.N - n0;
    op.K = p.K;
    op.sld = p.K / 32;
    op.sa = op.sb = nullptr;
    op.ra = op.rb = nullptr;
    if (MODE == kMx32) {
      const int nblk = p.K / 32;
      op.sa = static_cast<const uint8_t*>(p.scale_a) + (int64_t)m0 * nblk;
      op.sb = static_cast<const uint8_t*>(p.scale_b) + ((int64_t)g * p.N + n0) * nblk;
    }
    if (MODE == kRowwise) {
      op.ra = fsa + m0;
      op.rb = fsb + (int64_t)g * p.N + n0;
    }

    __syncthreads();  // the previous tile's epilogue is done with LDS
    const float ts = (MODE == kTensor) ? fsa[0] * fsb[g] : 1.0f;
    gemm_tile<Cfg, MODE, OutT, KALIGNED>(op, lds, static_cast<OutT*>(p.C), p.ldc, m0, m_end, n0,
                                         p.N, ts);
  }
}

#ifndef FP8GEMM_BIG_CFG
#define FP8GEMM_BIG_CFG 0
#endif
#if FP8GEMM_BIG_CFG == 0
using Big = TileCfg<256, 256, 128, 128, 4, 1>;
#else
using Big = TileCfg<256, 128, 128, 64, 3, 2>;
#endif
// MX with K % 128 != 0 reads its codes into registers: the large tile would spill
using Mid = TileCfg<128, 128, 64, 64, 4, 2>;

template <class Cfg, int MODE, typename OutT>
hipError_t launch_cfg(const GroupedProblem& p, hipStream_t stream) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
  }
  const int tiles_n = (p.N + Cfg::BN - 1) / Cfg::BN;
  // never more workgroups than the largest possible tile count
  const int64_t max_tiles = (int64_t)((p.total_m + Cfg::BM - 1) / Cfg::BM + p.groups) * tiles_n;
  const int64_t slots = (int64_t)cus * Cfg::kWgPerCu;
  const int grid = (int)(max_tiles < slots ? max_tiles : slots);
  if (grid <= 0) return hipSuccess;
  if (p.K % 128 == 0)
    hipLaunchKernelGGL((grouped_kernel<Cfg, MODE, OutT, true>), dim3(grid), dim3(Cfg::kThreads), 0,
                       stream, p, tiles_n);
  else
    hipLaunchKernelGGL((grouped_kernel<Cfg, MODE, OutT, false>), dim3(grid), dim3(Cfg::kThreads),
                       0, stream, p, tiles_n);
  return hipGetLastError();
}

}  // namespace

int grouped_max_groups() { return kMaxGroups; }

hipError_t launch_grouped_gemm(const GroupedProblem& p, int mode, int out, hipStream_t stream) {
  if (out == kF16) {
    if (mode == kTensor) return launch_cfg<Big, kTensor, _Float16>(p, stream);
    if (mode == kRowwise) return launch_cfg<Big, kRowwise, _Float16>(p, stream);
    if (p.K % 128 != 0) return launch_cfg<Mid, kMx32, _Float16>(p, stream);
    return launch_cfg<Big, kMx32, _Float16>(p, stream);
  }
  if (mode == kTensor) return launch_cfg<Big, kTensor, __bf16>(p, stream);
  if (mode == kRowwise) return launch_cfg<Big, kRowwise, __bf16>(p, stream);
  if (p.K % 128 != 0) return launch_cfg<Mid, kMx32, __bf16>(p, stream);
  return launch_cfg<Big, kMx32, __bf16>(p, stream);
}

}  // namespace fp8gemm
