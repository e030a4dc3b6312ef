// Dense scaled FP8 GEMM kernels for gfx950: one C tile per workgroup, and a
// split-K kernel for shapes with too few output tiles to fill the GPU.
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
#include "plan.h"
#include "tile_order.h"

// FP8GEMM_KN=1 builds the kernels for row-major B ([K][N]): every tile runs the
// interior mainloop in its transposing-read form (no persistent kernel).
#ifndef FP8GEMM_KN
#define FP8GEMM_KN 0
#endif

namespace fp8gemm {
namespace {

constexpr bool kKn = FP8GEMM_KN;

template <class Cfg, int MODE, typename OutT, bool KALIGNED, bool FUSED>
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
  op.B = kKn ? p.B + (kF4 ? n0 / 2 : n0) : p.B + (int64_t)n0 * p.ldb;
  op.ldb = p.ldb;
  op.b_rows = p.N - n0;
  op.K = p.K;
  op.sld = p.K / kBlkBytes;
  op.sldb = p.N;                         // row-major B: its codes are [K/32][N]
  const float* fsa = static_cast<const float*>(p.scale_a);
  const float* fsb = static_cast<const float*>(p.scale_b);
  op.sa = op.sb = nullptr;
  op.ra = op.rb = nullptr;
  if (MODE == kMx32) {
    op.sa = static_cast<const uint8_t*>(p.scale_a) + (int64_t)m0 * op.sld;
    op.sb = static_cast<const uint8_t*>(p.scale_b) + (kKn ? (int64_t)n0 : (int64_t)n0 * op.sld);
  }
  if (MODE == kRowwise) {
    op.ra = fsa + m0;
    op.rb = fsb + n0;
  }

  const float ts = (MODE == kTensor) ? fsa[0] * fsb[0] : 1.0f;
  if constexpr (kKn)
    gemm_tile_kn<Cfg, MODE, OutT, FUSED>(op, lds, static_cast<OutT*>(p.C), p.ldc, m0, p.M, n0,
                                         p.N, ts, p.bias, p.act, p.cs, p.ldcs);
  else
    gemm_tile<Cfg, MODE, OutT, KALIGNED, FUSED>(op, lds, static_cast<OutT*>(p.C), p.ldc, m0, p.M,
                                                n0, p.N, ts, p.bias, p.act, p.cs, p.ldcs);
}

// Operands of the tiles of one persistent workgroup: tile i of the list is the
// tile at position slot + i * stride of the grouped order, where the slot of a
// workgroup is XCD-aware (the workgroups of one XCD hold consecutive slots), so
// in every round each XCD works on a contiguous stretch of the grouped order.
template <class Cfg, int MODE>
struct DenseTiles {
  GemmProblem p;
  int tiles_m, tiles_n, slot, stride;
  __device__ void coords(int i, int& m0, int& n0) const {
    int tm, tn;
    grouped_tile(slot + i * stride, tiles_m, tiles_n, kGroupM, &tm, &tn);
    m0 = tm * Cfg::BM;
    n0 = tn * Cfg::BN;
  }
  __device__ TileOperands op(int i) const {
    int m0, n0;
    coords(i, m0, n0);
    TileOperands op;
    op.A = p.A + (int64_t)m0 * p.lda;
    op.lda = p.lda;
    op.a_rows = p.M - m0;
    op.B = p.B + (int64_t)n0 * p.ldb;
    op.ldb = p.ldb;
    op.b_rows = p.N - n0;
    op.K = p.K;
    op.sld = p.K / kBlkBytes;
    op.sa = op.sb = nullptr;
    op.ra = op.rb = nullptr;
    if (MODE == kMx32) {
      op.sa = static_cast<const uint8_t*>(p.scale_a) + (int64_t)m0 * op.sld;
      op.sb = static_cast<const uint8_t*>(p.scale_b) + (int64_t)n0 * op.sld;
    }
    if (MODE == kRowwise) {
      op.ra = static_cast<const float*>(p.scale_a) + m0;
      op.rb = static_cast<const float*>(p.scale_b) + n0;
    }
    return op;
  }
};

// Persistent form for shapes whose tiles are all interior: one workgroup per CU
// walks its tiles as one copy stream (the next tile's first K tiles are fetched
// while the current one finishes, its epilogue runs while they land).
template <class Cfg, int MODE, typename OutT>
__global__ __launch_bounds__(Cfg::kThreads, 1) void gemm_persistent_kernel(GemmProblem p,
                                                                           int tiles_m,
                                                                           int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Cfg::kLdsBytes];
  const int total = tiles_m * tiles_n;
  DenseTiles<Cfg, MODE> src{p, tiles_m, tiles_n, xcd_linear(blockIdx.x, gridDim.x),
                            (int)gridDim.x};
  const int count = (total - src.slot + src.stride - 1) / src.stride;
  const float* fsa = static_cast<const float*>(p.scale_a);
  const float* fsb = static_cast<const float*>(p.scale_b);
  const float ts = (MODE == kTensor) ? fsa[0] * fsb[0] : 1.0f;
  OutT* C = static_cast<OutT*>(p.C);
  auto epi = [&](const v16f (&acc)[Cfg::kFragM][Cfg::kFragN], int i, int rbuf)
                 __attribute__((always_inline)) {
    int m0, n0;
    src.coords(i, m0, n0);
    epilogue_direct<Cfg, MODE, OutT>(acc, lds, C, p.ldc, m0, n0, ts, rbuf, nullptr, kActNone, p.cs,
                                     p.ldcs);
  };
  // epilogue_direct issues two 16-byte stores per 32 x 32 block and lane
  if (count > 0)
    stream_interior<Cfg, MODE, 2 * Cfg::kFragM * Cfg::kFragN>(src, 0, count, lds, epi);
}

template <class Cfg, int MODE, typename OutT, bool FUSED>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t stream) {
  const int tiles_m = (p.M + Cfg::BM - 1) / Cfg::BM;
  const int tiles_n = (p.N + Cfg::BN - 1) / Cfg::BN;
  const int grid = tiles_m * tiles_n;
  if constexpr (kKn)   // K % 128 == 0 on this path
    hipLaunchKernelGGL((gemm_kernel<Cfg, MODE, OutT, true, FUSED>), dim3(grid),
                       dim3(Cfg::kThreads), 0, stream, p, tiles_m, tiles_n);
  else if (p.K % 128 == 0)
    hipLaunchKernelGGL((gemm_kernel<Cfg, MODE, OutT, true, FUSED>), dim3(grid),
                       dim3(Cfg::kThreads), 0, stream, p, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((gemm_kernel<Cfg, MODE, OutT, false, FUSED>), dim3(grid),
                       dim3(Cfg::kThreads), 0, stream, p, tiles_m, tiles_n);
  return hipGetLastError();
}

// Large-problem tile: 256 x 256, 4 wavefronts of 128 x 128, one workgroup per CU
// (the interior path's two 128-K ring slots plus code buffers need its 144 KiB of
// LDS); mid-size tile: 128 x 128, 4 wavefronts of 64 x 64, two workgroups per CU.
using Big = TileCfg<256, 256, 128, 128, 4, 1>;
using Mid = TileCfg<128, 128, 64, 64, 4, 2>;
static_assert(Big::BM == kBigTile && Big::BN == kBigTile && Big::kWgPerCu == 1, "plan.h tiles");
static_assert(Mid::BM == kMidTile && Mid::BN == kMidTile, "plan.h tiles");

template <class Cfg, int MODE, typename OutT>
hipError_t launch_persistent(const GemmProblem& p, hipStream_t stream) {
  const int tiles_m = p.M / Cfg::BM, tiles_n = p.N / Cfg::BN;
  const int total = tiles_m * tiles_n;
  const int cus = device_cu_count();
  const int grid = total < cus ? total : cus;
  hipLaunchKernelGGL((gemm_persistent_kernel<Cfg, MODE, OutT>), dim3(grid), dim3(Cfg::kThreads), 0,
                     stream, p, tiles_m, tiles_n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-K.  The decode-like shape M = 128, N = K = 4096 of "Hopper/Blackwell
// architecture features" §12.2.4 is bound by streaming B (16 MiB) from HBM, yet
// it has only 32 output tiles of 128 x 128.  Here the output is cut into
// 64 x 64 tiles and K into `splits` slices, so that tiles x splits >= 256
// workgroups each stream an equal share of B.  Each workgroup runs the mainloop
// over its slice (4-deep ring of 128-K tiles: a slice has few K tiles and its
// copies come from HBM), stores its fp32 partial tile in the workspace and
// counts its arrival on the tile's counter.  The last to arrive sums the
// partials of slices 0, 1, ..., splits-1 in that order (so the result does not
// depend on arrival order), resets the counter to zero for the next call and
// runs the epilogue.
// ---------------------------------------------------------------------------
// 64 x 64 split tiles, 4 wavefronts of 32 x 32, one workgroup per CU.  For M =
// 128, N = K = 4096 the 64 x 64 tiles split K in two instead of four and halve
// the fp32 partials exchanged against 128 x 64 tiles (8 -> 4 MiB written):
// 14.9 -> 13.5 us (measured; two workgroups per CU 14.3 us, an eight-deep ring
// 4 % slower, so the copy stream of a slice is not bound by the bytes in flight).
using SplitCfg = TileCfg<64, 64, 32, 32, 8, 1>;
static_assert(SplitCfg::BM == kSplitTile && SplitCfg::BN == kSplitTile, "plan.h tiles");
static_assert(128 * 128 * 128 / (SplitCfg::BM * SplitCfg::BN) <= kMaxSplitTiles,
              "counters for every split plan");

// ring depth of the split-K mainloop in 128-K tiles
constexpr int kSplitRing = 4;

template <class Cfg, int MODE, typename OutT, bool FUSED>
__global__ __launch_bounds__(Cfg::kThreads, Cfg::kWavesPerEu) void splitk_kernel(GemmProblem p, int tiles_m,
                                                                    int splits) {
  // the arrival flag lives in the same LDS object as the ring: a second LDS
  // variable makes the compiler wait for every ring copy before every LDS read
  constexpr int kFlagOff = (Cfg::kLdsBytes + 15) / 16 * 16;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kFlagOff + 16];
  int& s_last = *reinterpret_cast<int*>(lds + kFlagOff);
  constexpr int FM = Cfg::kFragM, FN = Cfg::kFragN;
  // XCD-aware: the workgroups of one XCD hold a contiguous run of (tile, slice)
  // pairs, so the tile rows that share B columns (and, for row-major B, the
  // neighbouring column tiles that share its 128-byte lines) meet in one L2
  const int lin = xcd_linear(blockIdx.x, gridDim.x);
  const int tile = lin / splits, ks = lin % splits;
  const int tm = tile % tiles_m, tn = tile / tiles_m;
  const int m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;
  const int kslice = p.K / splits, k0 = ks * kslice;

  TileOperands op;
  op.A = p.A + (int64_t)m0 * p.lda + k0;
  op.lda = p.lda;
  op.a_rows = p.M - m0;
  // (row-major FP4 B: K-rows 2 k0 on, columns n0 on in bytes n0 / 2)
  op.B = kKn ? p.B + (int64_t)(kF4 ? 2 * k0 : k0) * p.ldb + (kF4 ? n0 / 2 : n0)
             : p.B + (int64_t)n0 * p.ldb + k0;
  op.ldb = p.ldb;
  op.b_rows = p.N - n0;
  op.K = kslice;
  op.sld = p.K / kBlkBytes;
  op.sldb = p.N;
  const float* fsa = static_cast<const float*>(p.scale_a);
  const float* fsb = static_cast<const float*>(p.scale_b);
  op.sa = op.sb = nullptr;
  op.ra = op.rb = nullptr;
  if (MODE == kMx32) {
    op.sa = static_cast<const uint8_t*>(p.scale_a) + (int64_t)m0 * op.sld + k0 / kBlkBytes;
    op.sb = static_cast<const uint8_t*>(p.scale_b) +
            (kKn ? (int64_t)(k0 / kBlkBytes) * p.N + n0 : (int64_t)n0 * op.sld + k0 / kBlkBytes);
  }
  if (MODE == kRowwise) {
    op.ra = fsa + m0;
    op.rb = fsb + n0;
  }

  v16f acc[FM][FN];
  if constexpr (kKn) mainloop_interior<Cfg, MODE, kSplitRing, true>(op, lds, acc);
  else if (interior_k<Cfg, MODE>(op)) mainloop_interior<Cfg, MODE, kSplitRing>(op, lds, acc);
  else mainloop<Cfg, MODE, !kF4>(op, lds, acc);

  // partial tile: float4 r of thread x at [tile][slice][r][x] (coalesced per r)
  const int tiles = tiles_m * (int)((p.N + Cfg::BN - 1) / Cfg::BN);
  int* counters = static_cast<int*>(p.workspace);
  constexpr int kVec = FM * FN * 4;
  const __amdgpu_buffer_rsrc_t rp =
      buffer_rsrc(static_cast<uint8_t*>(p.workspace) + kSplitCounterBytes,
                  (uint32_t)((int64_t)tiles * splits * kVec * Cfg::kThreads * 16));
  auto poff = [&](int slice, int r) {
    return ((((tile * splits + slice) * kVec) + r) * Cfg::kThreads + (int)threadIdx.x) * 16;
  };
  // Partials travel as 16-byte buffer accesses with the SC1 cache policy, the
  // policy of relaxed agent-scope atomics on gfx950: stores are written through
  // to, and loads read from, the memory level shared by all XCDs, so ordering
  // only needs the stores to have completed before the arrival is counted.  (An
  // agent-scope release/acquire fence pair would write back and invalidate the
  // whole L2 of the XCD instead, which cost more than the GEMM.)
  constexpr int kSc1 = 16;
  {
#pragma unroll
    for (int r = 0; r < kVec; ++r) {
      const v16f& a = acc[(r >> 2) / FN][(r >> 2) % FN];
      const int g = r & 3;
      const v4f v{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), rp, poff(ks, r), 0, kSc1);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);                       // this thread's partial stored
  __syncthreads();                                     // ... and every thread's
  if (threadIdx.x == 0) {
    const int prev =
        __hip_atomic_fetch_add(&counters[tile], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == splits - 1;
  }
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x == 0)                                // ready for the next call
    __hip_atomic_store(&counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // sum the slices in order 0, 1, ..., splits - 1 (own slice from registers);
  // the loads of up to four slices are issued together
  constexpr int kBatch = 4;
  v16f sum[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) sum[i][j] = v16f{};
  for (int s0 = 0; s0 < splits; s0 += kBatch) {
    v4f v[kBatch][kVec];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int slice = s0 + b;
      if (slice < splits && slice != ks) {
#pragma unroll
        for (int r = 0; r < kVec; ++r)
          v[b][r] = __builtin_bit_cast(
              v4f, __builtin_amdgcn_raw_buffer_load_b128(rp, poff(slice, r), 0, kSc1));
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int slice = s0 + b;
      if (slice >= splits) break;
      if (slice == ks) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) sum[i][j] += acc[i][j];
      } else {
#pragma unroll
        for (int r = 0; r < kVec; ++r) {
          v16f& d = sum[(r >> 2) / FN][(r >> 2) % FN];
          const int g = r & 3;
#pragma unroll
          for (int e = 0; e < 4; ++e) d[4 * g + e] += v[b][r][e];
        }
      }
    }
  }
  const float ts = (MODE == kTensor) ? fsa[0] * fsb[0] : 1.0f;
  if constexpr (FUSED || std::is_same<OutT, uint8_t>::value)
    epilogue_fused<Cfg, MODE, OutT>(sum, lds, static_cast<OutT*>(p.C), p.ldc, m0, p.M, n0, p.N, ts,
                                    p.bias, p.act, p.cs, p.ldcs);
  else
    epilogue<Cfg, MODE, OutT>(sum, lds, static_cast<OutT*>(p.C), p.ldc, m0, p.M, n0, p.N, ts, p.cs,
                              p.ldcs);
}

template <int MODE, typename OutT, bool FUSED>
hipError_t launch_split(const GemmProblem& p, const SplitPlan& plan, hipStream_t stream) {
  const int grid = plan.tiles_m * plan.tiles_n * plan.splits;
  hipLaunchKernelGGL((splitk_kernel<SplitCfg, MODE, OutT, FUSED>), dim3(grid),
                     dim3(SplitCfg::kThreads), 0, stream, p, plan.tiles_m, plan.splits);
  return hipGetLastError();
}

template <int MODE, typename OutT, bool FUSED>
hipError_t launch_plan(const GemmProblem& p, hipStream_t stream) {
  constexpr bool kNoStream = FUSED || std::is_same<OutT, uint8_t>::value;
  // (K of the problem counts bytes for FP4, elements for the row-major form's plan)
  const GemmPath path = kKn ? choose_path_kn(p.M, p.N, kF4 ? 2 * (int64_t)p.K : p.K, p.lda,
                                             p.ldb, MODE, kF4)
                            : choose_path(p.M, p.N, p.K, p.lda, p.ldb, MODE, kF4, kNoStream);
  // row-major B outside the in-kernel form: the caller transposes B first
  if (kKn && path == kPathNone && p.M > 0 && p.N > 0) return hipErrorInvalidValue;
  switch (path) {
    case kPathSplitK:
      return launch_split<MODE, OutT, FUSED>(p, plan_split(p.M, p.N, p.K, MODE, kBlkBytes),
                                             stream);
    case kPathPersistent:
      // (the fused epilogue stages through the ring, so it never runs in a stream)
      if constexpr (!kNoStream && !kF4 && !kKn) return launch_persistent<Big, MODE, OutT>(p, stream);
      return hipErrorInvalidValue;
    case kPathTile256:
      return launch_cfg<Big, MODE, OutT, FUSED>(p, stream);
    case kPathTile128:
      return launch_cfg<Mid, MODE, OutT, FUSED>(p, stream);
    default:
      return hipSuccess;
  }
}

// kernels with the fused bias / activation epilogue only when it is asked for
// (the e4m3 + MX-scale output, OutT = uint8_t, quantises interior tiles without
// one straight from registers and the other tiles in the fused epilogue's loop)
template <int MODE, typename OutT>
hipError_t launch_any(const GemmProblem& p, hipStream_t stream) {
  if (p.bias != nullptr || p.act != kActNone) return launch_plan<MODE, OutT, true>(p, stream);
  return launch_plan<MODE, OutT, false>(p, stream);
}

}  // namespace

// This file is compiled once per pair of operand formats (FP8GEMM_FMT_A/B); the
// e4m3 x e4m3 build also defines the workspace query (the plan does not depend
// on the formats).
#if FP8GEMM_KN && FP8GEMM_FMT_A == 0 && FP8GEMM_FMT_B == 0
#define FP8GEMM_LAUNCH_NAME launch_gemm_kn
#elif FP8GEMM_KN && FP8GEMM_FMT_A == 1 && FP8GEMM_FMT_B == 1
#define FP8GEMM_LAUNCH_NAME launch_gemm_kn_e5m2_e5m2
#elif FP8GEMM_KN && FP8GEMM_FMT_A == 0 && FP8GEMM_FMT_B == 1
#define FP8GEMM_LAUNCH_NAME launch_gemm_kn_e4m3_e5m2
#elif FP8GEMM_KN && FP8GEMM_FMT_A == 1 && FP8GEMM_FMT_B == 0
#define FP8GEMM_LAUNCH_NAME launch_gemm_kn_e5m2_e4m3
#elif FP8GEMM_KN && FP8GEMM_FMT_A == 4 && FP8GEMM_FMT_B == 4
#define FP8GEMM_LAUNCH_NAME launch_gemm_kn_e2m1_e2m1
#elif FP8GEMM_FMT_A == 0 && FP8GEMM_FMT_B == 0
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int mode) {
  return (size_t)gemm_workspace_need(M, N, K, mode);
}
#define FP8GEMM_LAUNCH_NAME launch_gemm
#elif FP8GEMM_FMT_A == 1 && FP8GEMM_FMT_B == 1
#define FP8GEMM_LAUNCH_NAME launch_gemm_e5m2_e5m2
#elif FP8GEMM_FMT_A == 0 && FP8GEMM_FMT_B == 1
#define FP8GEMM_LAUNCH_NAME launch_gemm_e4m3_e5m2
#elif FP8GEMM_FMT_A == 1 && FP8GEMM_FMT_B == 0
#define FP8GEMM_LAUNCH_NAME launch_gemm_e5m2_e4m3
#elif FP8GEMM_FMT_A == 4 && FP8GEMM_FMT_B == 4
#define FP8GEMM_LAUNCH_NAME launch_gemm_e2m1_e2m1
#endif

hipError_t FP8GEMM_LAUNCH_NAME(const GemmProblem& p, int mode, int out, hipStream_t stream) {
#if FP8GEMM_FMT_A == 4
  // MXFP4: E8M0 block scales only; K, lda and ldb count bytes (two codes each)
  if (mode != kMx32) return hipErrorInvalidValue;
  if (out == kF16) return launch_any<kMx32, _Float16>(p, stream);
#if !FP8GEMM_KN
  if (out == kE4M3Mx) return launch_any<kMx32, uint8_t>(p, stream);
  if (out == kBF16Max) return launch_any<kMx32, bf16_max>(p, stream);
#endif
  return launch_any<kMx32, __bf16>(p, stream);
#else
#if !FP8GEMM_KN
  // the bf16 output with its maxima: the same kernels and epilogue arithmetic as
  // the plain bf16 output (so its values are those of fp8gemm_run_ex)
  if (out == kBF16Max) {
    if (mode == kTensor) return launch_any<kTensor, bf16_max>(p, stream);
    if (mode == kRowwise) return launch_any<kRowwise, bf16_max>(p, stream);
    return launch_any<kMx32, bf16_max>(p, stream);
  }
#endif
  if (out == kE4M3Mx) {
    if (mode == kTensor) return launch_any<kTensor, uint8_t>(p, stream);
    if (mode == kRowwise) return launch_any<kRowwise, uint8_t>(p, stream);
    return launch_any<kMx32, uint8_t>(p, stream);
  }
  if (out == kF16) {
    if (mode == kTensor) return launch_any<kTensor, _Float16>(p, stream);
    if (mode == kRowwise) return launch_any<kRowwise, _Float16>(p, stream);
    return launch_any<kMx32, _Float16>(p, stream);
  }
  if (mode == kTensor) return launch_any<kTensor, __bf16>(p, stream);
  if (mode == kRowwise) return launch_any<kRowwise, __bf16>(p, stream);
  return launch_any<kMx32, __bf16>(p, stream);
#endif
}

}  // namespace fp8gemm
