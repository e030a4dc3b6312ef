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
//   * tiles are numbered expert by expert and, inside an expert, in the same
//     grouped order as the dense GEMM (groups of a few tile rows, column-major
//     inside a group); the slot of a workgroup inside each round of the
//     persistent loop is remapped so one XCD runs a contiguous run of tiles, and
//     the ~32 tiles resident on an XCD cover a few tile rows by several tile
//     columns of one expert: both the activation rows and the expert weight
//     columns they read are shared in that XCD's L2 (the MI355X counterpart of
//     sharing expert weights by multicast).  Walking all tile rows of one column
//     first instead shares the weights but makes each XCD stream ~1 MB of
//     distinct activations per 128-deep K step, which measured 2.3x slower;
//   * each tile uses the dense mainloop and epilogue, with rows past the expert's
//     end masked on store (ragged experts, empty experts); with K % 512 == 0 the
//     tiles cut by an expert's last row stay in the copy stream unless they
//     reach past the end of A.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_tile.h"
#include "launch.h"
#include "tile_order.h"

namespace fp8gemm {
namespace {

constexpr int kMaxGroups = 1024;

// The tiles of one persistent workgroup: list entry i is tile slot + i * stride
// of the expert-major order (expert by expert, grouped order inside an expert).
template <class Cfg, int MODE>
struct GroupedTiles {
  GroupedProblem p;
  const int* tile_start;   // LDS: first tile of each expert, prefix sums
  const int* row_begin;    // LDS: clamped expert row ranges
  const int* row_end;
  int tiles_n, slot, stride;

  struct Where {
    int g, m0, m_end, n0;
  };
  __device__ Where where(int i) const {
    const int t = slot + i * stride;
    int lo = 0, hi = p.groups - 1;          // expert of tile t: last g with tile_start[g] <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tile_start[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    // the values come from LDS, so the compiler cannot see that they are the same
    // in every lane; they are, and keeping them in scalar registers keeps every
    // address derived from them (buffer descriptors included) scalar
    Where w;
    w.g = __builtin_amdgcn_readfirstlane(lo);
    const int local = t - __builtin_amdgcn_readfirstlane(tile_start[w.g]);
    const int rb = __builtin_amdgcn_readfirstlane(row_begin[w.g]);
    w.m_end = __builtin_amdgcn_readfirstlane(row_end[w.g]);
    const int tiles_m_g = (w.m_end - rb + Cfg::BM - 1) / Cfg::BM;
    int tm, tn;
    grouped_tile(local, tiles_m_g, tiles_n, kGroupM, &tm, &tn);
    w.m0 = rb + tm * Cfg::BM;
    w.n0 = tn * Cfg::BN;
    return w;
  }
  __device__ TileOperands op_at(const Where& w) const {
    TileOperands op;
    op.A = p.A + (int64_t)w.m0 * p.lda;
    op.lda = p.lda;
    op.a_rows = w.m_end - w.m0;
    op.B = p.B + (int64_t)w.g * p.stride_b + (int64_t)w.n0 * p.ldb;
    op.ldb = p.ldb;
    op.b_rows = p.N - w.n0;
    op.K = p.K;
    op.sld = p.K / kBlkBytes;
    op.sa = op.sb = nullptr;
    op.ra = op.rb = nullptr;
    if (MODE == kMx32) {
      op.sa = static_cast<const uint8_t*>(p.scale_a) + (int64_t)w.m0 * op.sld;
      op.sb = static_cast<const uint8_t*>(p.scale_b) + ((int64_t)w.g * p.N + w.n0) * op.sld;
    }
    if (MODE == kRowwise) {
      op.ra = static_cast<const float*>(p.scale_a) + w.m0;
      op.rb = static_cast<const float*>(p.scale_b) + (int64_t)w.g * p.N + w.n0;
    }
    return op;
  }
  __device__ TileOperands op(int i) const { return op_at(where(i)); }
};

// ALL_INTERIOR: every tile runs the interior mainloop (MXFP4 experts with K a
// multiple of 512 and 32-bit spans; the launch checks), so the kernel carries no
// edge path.
template <class Cfg, int MODE, typename OutT, bool KALIGNED, bool ALL_INTERIOR = false>
__global__ __launch_bounds__(Cfg::kThreads, Cfg::kWavesPerEu) void grouped_kernel(GroupedProblem p,
                                                                                 int tiles_n) {
  // One LDS object holds the tile ring and the expert tables: with several LDS
  // variables the compiler no longer proves that fragment reads and the ring's
  // DMA writes are independent and waits for every copy before every read.
  constexpr int kTableOff = (Cfg::kLdsBytes + 15) / 16 * 16;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kTableOff + (3 * kMaxGroups + 1) * 4];
  int* tile_start = reinterpret_cast<int*>(lds + kTableOff);
  int* row_begin = tile_start + kMaxGroups + 1;
  int* row_end = row_begin + kMaxGroups;

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
  const int total = __builtin_amdgcn_readfirstlane(tile_start[p.groups]);
  const GroupedTiles<Cfg, MODE> src{p, tile_start, row_begin, row_end, tiles_n,
                                    xcd_linear(blockIdx.x, gridDim.x), (int)gridDim.x};
  const int count = total > src.slot ? (total - src.slot + src.stride - 1) / src.stride : 0;
  const float* fsa = static_cast<const float*>(p.scale_a);
  const float* fsb = static_cast<const float*>(p.scale_b);
  OutT* C = static_cast<OutT*>(p.C);
  // with K % 512 == 0, tiles whole in N run as copy streams (one per run of such
  // tiles); so do tiles cut by an expert's last row whose BM rows still lie
  // inside A: they read the next expert's rows (and their row scales or codes)
  // as a whole tile would and store only their own rows.  Tiles cut by N or by
  // the end of A take the general path (FP4: every tile).
  constexpr bool kStream = KALIGNED && Cfg::kSlots == 4 && !kF4;
  // (their stores address a tile's rows with 32-bit offsets)
  const bool ranged = (int64_t)Cfg::BM * p.ldc * (int64_t)sizeof(OutT) < ((int64_t)1 << 31);
  auto streamable = [&](int i) __attribute__((always_inline)) {
    if (!kStream || p.K % 512 != 0 || !ranged) return false;
    const auto w = src.where(i);
    const TileOperands op = src.op_at(w);
    return op.b_rows >= Cfg::BN && w.m0 + Cfg::BM <= p.total_m && interior_k<Cfg, MODE>(op);
  };
  auto epi = [&](const v16f (&acc)[Cfg::kFragM][Cfg::kFragN], int i, int rbuf)
                 __attribute__((always_inline)) {
    const auto w = src.where(i);
    const float ts = (MODE == kTensor) ? fsa[0] * fsb[w.g] : 1.0f;
    epilogue_direct_rows<Cfg, MODE, OutT>(acc, lds, C, p.ldc, w.m0, w.n0, ts, rbuf,
                                          w.m_end - w.m0);
  };

  int i = 0;
  while (i < count) {
    __syncthreads();  // the previous tile's epilogue is done with LDS
    bool streamed = false;
    if constexpr (kStream) {
      if (streamable(i)) {
        int j = i + 1;
        while (j < count && streamable(j)) ++j;
        stream_interior<Cfg, MODE, 2 * Cfg::kFragM * Cfg::kFragN>(src, i, j, lds, epi);
        i = j;
        streamed = true;
      }
    }
    if (!streamed) {
      const auto w = src.where(i);
      const float ts = (MODE == kTensor) ? fsa[0] * fsb[w.g] : 1.0f;
      // tiles cut by an expert's last row (or by N): with ALL_INTERIOR on the
      // interior loop too, their copies ending at the last valid row or column;
      // otherwise on the edge path (FP8: tiles that did not stream above; an
      // interior instance here would inflate the stream's loop)
      if constexpr (ALL_INTERIOR)
        gemm_tile_interior<Cfg, MODE, OutT>(src.op_at(w), lds, C, p.ldc, w.m0, w.m_end, w.n0,
                                            p.N, ts);
      else
        gemm_tile<Cfg, MODE, OutT, KALIGNED, false, false>(src.op_at(w), lds, C, p.ldc, w.m0,
                                                           w.m_end, w.n0, p.N, ts);
      ++i;
    }
  }
}

// the dense GEMM's large tile: 256 x 256, 4 wavefronts of 128 x 128, one per CU
using Big = TileCfg<256, 256, 128, 128, 4, 1>;
// MX with K % 128 != 0 reads its codes into registers: the large tile would spill
using Mid = TileCfg<128, 128, 64, 64, 4, 2>;

template <class Cfg, int MODE, typename OutT>
hipError_t launch_cfg(const GroupedProblem& p, hipStream_t stream) {
  const int cus = device_cu_count();
  const int tiles_n = (p.N + Cfg::BN - 1) / Cfg::BN;
  // never more workgroups than the largest possible tile count
  const int64_t max_tiles = (int64_t)((p.total_m + Cfg::BM - 1) / Cfg::BM + p.groups) * tiles_n;
  const int64_t slots = (int64_t)cus * Cfg::kWgPerCu;
  const int grid = (int)(max_tiles < slots ? max_tiles : slots);
  if (grid <= 0) return hipSuccess;
  // MXFP4 with whole 512-element code groups (K counts bytes) and 32-bit spans:
  // every tile interior
  constexpr bool kAllInterior = kF4 && Cfg::BM == 256;
  const bool all_interior = kAllInterior && MODE == kMx32 && p.K % 256 == 0 &&
                            (int64_t)Cfg::BM * p.lda + p.K < ((int64_t)1 << 31) &&
                            (int64_t)Cfg::BN * p.ldb + p.K < ((int64_t)1 << 31);
  if (all_interior)
    hipLaunchKernelGGL((grouped_kernel<Cfg, MODE, OutT, true, kAllInterior>),
                       dim3(grid), dim3(Cfg::kThreads), 0, stream, p, tiles_n);
  else if (p.K % 128 == 0)
    hipLaunchKernelGGL((grouped_kernel<Cfg, MODE, OutT, true>), dim3(grid), dim3(Cfg::kThreads), 0,
                       stream, p, tiles_n);
  else
    hipLaunchKernelGGL((grouped_kernel<Cfg, MODE, OutT, false>), dim3(grid), dim3(Cfg::kThreads),
                       0, stream, p, tiles_n);
  return hipGetLastError();
}

}  // namespace

#if FP8GEMM_FMT_A == 4 && FP8GEMM_FMT_B == 4
// MXFP4 experts (K, lda, ldb and stride_b in bytes): the large tile, one tile at
// a time; with K % 512 == 0 every tile on the interior mainloop (tiles cut by an
// expert's last row or by N included), else full tiles only; a K tail takes
// 128 x 128 tiles.
hipError_t launch_grouped_gemm_e2m1_e2m1(const GroupedProblem& p, int mode, int out,
                                         hipStream_t stream) {
  if (mode != kMx32) return hipErrorInvalidValue;
  if (out == kF16) {
    if (p.K % 128 != 0) return launch_cfg<Mid, kMx32, _Float16>(p, stream);
    return launch_cfg<Big, kMx32, _Float16>(p, stream);
  }
  if (p.K % 128 != 0) return launch_cfg<Mid, kMx32, __bf16>(p, stream);
  return launch_cfg<Big, kMx32, __bf16>(p, stream);
}
#else
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
#endif

}  // namespace fp8gemm
