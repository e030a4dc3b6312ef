// One output tile of the scaled FP8 GEMM on gfx950 MFMA: the K mainloop and the
// scale/cast epilogue.  Used by the dense kernel (one tile per workgroup) and the
// grouped kernel (a persistent loop over expert tiles).
//
// Prior art and what is kept.  "Hopper/Blackwell architecture features" §12.7
// tiles C into BLOCK_M x BLOCK_N tiles, walks K in BLOCK_K steps accumulating
// fp32 and casts on store; §12.4 overlaps the load of the next K tile with the
// math on the current one through a multi-stage shared-memory ring whose size
// per stage is (BLOCK_M + BLOCK_N) * BLOCK_K * element size (§12.4.3).  The
// TMA/mbarrier/warp-specialised machinery of §12.2/§12.3 has no CDNA
// counterpart; instead every wavefront both loads and computes:
//   * K tiles of 128 bytes are copied global -> LDS with gfx950's direct
//     `global_load_lds_dwordx4` (16 bytes per lane, no VGPR staging) into a
//     two-stage ring: (BM + BN) * 128 bytes per stage (64 KiB for 256 x 256).
//   * LDS rows are 128 bytes; the sixteen-byte chunk c of row r is stored at
//     chunk position c ^ (r & 7), so the eight rows a group of lanes reads
//     together fall on distinct banks.  The XOR is applied on the load side by
//     choosing which global chunk each lane fetches.
//   * Each wavefront owns a WM x WN sub-tile made of 32 x 32 MFMA blocks and
//     runs V_MFMA_SCALE_F32_32X32X64_F8F6F4 on e4m3 operands.  Per lane an
//     operand fragment is two 16-byte K chunks, k = 32*(byte/16) + 16*(lane/32)
//     + byte%16, for row lane%32; the E8M0 scale of (row r, 32-K block b) is
//     byte 0 of the scale register of lane r + 32*b.  Per-tensor and row-wise
//     operands pass constant zero scales (the plain MFMA); MX operands pass the
//     E8M0 codes so the block scales are applied inside the instruction.
//   * The instruction is issued with B as its first operand, so the fp32 result
//     is C transposed: a lane holds four consecutive output columns of one row,
//     which are scaled, rounded to fp16/bf16 and stored as 8 bytes.
//   * Rows past the matrix edge are read from the last valid row (and never
//     stored); K chunks past K are read from column 0 and zeroed in registers
//     before use, together with their scales (set to 2^0).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_utils.h"
#include "launch.h"

namespace fp8gemm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

template <int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int kBK = 128;
  static constexpr int kWavesM = BM / WM, kWavesN = BN / WN;
  static constexpr int kWaves = kWavesM * kWavesN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kFragM = WM / 32, kFragN = WN / 32;
  static constexpr int kStageBytes = (BM + BN) * kBK;
  static constexpr int kStages = 2;
  static constexpr int kLdsBytes = kStages * kStageBytes;
  static constexpr int kLoadsA = BM / 8 / kWaves;  // 1 KiB (8 rows) per load instruction
  static constexpr int kLoadsB = BN / 8 / kWaves;
  static_assert(BM % (8 * kWaves) == 0 && BN % (8 * kWaves) == 0, "whole load instructions");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "32x32 MFMA blocks");
  static_assert(kLdsBytes <= 160 * 1024, "LDS per workgroup");
};

// Where a tile's operands live and how many of its rows are valid.
struct TileOperands {
  const uint8_t* A;     // first row of this tile's A rows
  int64_t lda;
  int a_rows;           // valid A rows from A (>= 1)
  const uint8_t* B;     // first row (output column) of this tile's B
  int64_t ldb;
  int b_rows;           // valid B rows (output columns) from B (>= 1)
  const uint8_t* sa;    // MX: E8M0 codes of A's first tile row, K/32 per row
  const uint8_t* sb;    // MX: E8M0 codes of B's first tile row
  int K;
};

__device__ __forceinline__ void lds_dma16(const uint8_t* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

template <class Cfg, bool KTAIL>
__device__ __forceinline__ void load_stage(const TileOperands& op, uint8_t* stage, int k0, int wave,
                                           int lane) {
  const int sub = lane >> 3;                  // row within the 8-row group
  const int chunk = (lane & 7) ^ sub;         // logical K chunk fetched (XOR layout)
  int kc = k0 + 16 * chunk;
  if (KTAIL && kc >= op.K) kc = 0;            // in-bounds dummy, zeroed later
#pragma unroll
  for (int t = 0; t < Cfg::kLoadsA; ++t) {
    const int grp = wave * Cfg::kLoadsA + t;
    int row = grp * 8 + sub;
    row = row < op.a_rows ? row : op.a_rows - 1;
    lds_dma16(op.A + (int64_t)row * op.lda + kc, stage + grp * 1024);
  }
  uint8_t* stageB = stage + Cfg::BM * Cfg::kBK;
#pragma unroll
  for (int t = 0; t < Cfg::kLoadsB; ++t) {
    const int grp = wave * Cfg::kLoadsB + t;
    int row = grp * 8 + sub;
    row = row < op.b_rows ? row : op.b_rows - 1;
    lds_dma16(op.B + (int64_t)row * op.ldb + kc, stageB + grp * 1024);
  }
}

// Raw scale bytes of one fragment row for K tile kt, as loaded.  Nothing is done
// with them until the next K step (after its wait), so the loads stay in flight
// together with the LDS prefetch; mx_scale_word() then arranges them.
struct MxRaw {
  uint32_t lo, hi;
};

template <bool KALIGNED>
__device__ __forceinline__ MxRaw load_mx_scales(const uint8_t* s, int row, int kt, int nblk,
                                                int h) {
  const uint8_t* p = s + (int64_t)row * nblk;
  MxRaw r;
  if (KALIGNED) {
    r.lo = *reinterpret_cast<const uint32_t*>(p + 4 * kt);  // blocks 4kt .. 4kt+3
    r.hi = 0;
  } else {
    const int b0 = 4 * kt + h, b1 = b0 + 2;
    r.lo = b0 < nblk ? p[b0] : 127u;
    r.hi = b1 < nblk ? p[b1] : 127u;
  }
  return r;
}

// Scale register for both MFMA K halves of a K tile: byte0 = block 4kt + h (first
// half), byte2 = block 4kt + 2 + h (second half), h = lane/32.
template <bool KALIGNED>
__device__ __forceinline__ uint32_t mx_scale_word(MxRaw r, int h) {
  if (KALIGNED) return r.lo >> (8 * h);
  return r.lo | (r.hi << 16);
}

template <class Cfg, int MODE, bool KALIGNED>
__device__ __forceinline__ void mainloop(const TileOperands& op, uint8_t* lds,
                                         v16f (&acc)[Cfg::kFragM][Cfg::kFragN]) {
  constexpr int FM = Cfg::kFragM, FN = Cfg::kFragN;
  constexpr bool KTAIL = !KALIGNED;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const int h = lane >> 5;
  const int nk = (op.K + Cfg::kBK - 1) / Cfg::kBK;
  const int nblk = op.K / 32;

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

  // fragment rows (tile-local) of this lane
  int arow[FM], brow[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) arow[i] = wm * Cfg::WM + i * 32 + (lane & 31);
#pragma unroll
  for (int j = 0; j < FN; ++j) brow[j] = wn * Cfg::WN + j * 32 + (lane & 31);

  MxRaw sa_nxt[FM], sb_nxt[FN];
  uint32_t sa_cur[FM], sb_cur[FN];
  auto load_scales = [&](int kt) {
    if (MODE == kMx32) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = arow[i] < op.a_rows ? arow[i] : op.a_rows - 1;
        sa_nxt[i] = load_mx_scales<KALIGNED>(op.sa, r, kt, nblk, h);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = brow[j] < op.b_rows ? brow[j] : op.b_rows - 1;
        sb_nxt[j] = load_mx_scales<KALIGNED>(op.sb, r, kt, nblk, h);
      }
    }
  };

  load_stage<Cfg, KTAIL>(op, lds, 0, wave, lane);
  load_scales(0);

  for (int kt = 0; kt < nk; ++kt) {
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of stage kt have landed
    __syncthreads();                 // ... and everyone's; stage kt+1's slot is free
    if (MODE == kMx32) {
#pragma unroll
      for (int i = 0; i < FM; ++i) sa_cur[i] = mx_scale_word<KALIGNED>(sa_nxt[i], h);
#pragma unroll
      for (int j = 0; j < FN; ++j) sb_cur[j] = mx_scale_word<KALIGNED>(sb_nxt[j], h);
    }
    if (kt + 1 < nk) {
      load_stage<Cfg, KTAIL>(op, lds + ((kt + 1) & 1) * Cfg::kStageBytes, (kt + 1) * Cfg::kBK,
                             wave, lane);
      load_scales(kt + 1);
    }
    const uint8_t* sA = lds + (kt & 1) * Cfg::kStageBytes;
    const uint8_t* sB = sA + Cfg::BM * Cfg::kBK;
    const int k0 = kt * Cfg::kBK;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c0 = 4 * kk + h, c1 = c0 + 2;
      bool z0 = false, z1 = false;
      if (KTAIL) {
        z0 = k0 + 16 * c0 >= op.K;
        z1 = k0 + 16 * c1 >= op.K;
      }
      v8i af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint8_t* rowp = sA + arow[i] * Cfg::kBK;
        const int sw = arow[i] & 7;
        v4i lo = *reinterpret_cast<const v4i*>(rowp + 16 * (c0 ^ sw));
        v4i hi = *reinterpret_cast<const v4i*>(rowp + 16 * (c1 ^ sw));
        if (KTAIL) {
          if (z0) lo = v4i{};
          if (z1) hi = v4i{};
        }
        af[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint8_t* rowp = sB + brow[j] * Cfg::kBK;
        const int sw = brow[j] & 7;
        v4i lo = *reinterpret_cast<const v4i*>(rowp + 16 * (c0 ^ sw));
        v4i hi = *reinterpret_cast<const v4i*>(rowp + 16 * (c1 ^ sw));
        if (KTAIL) {
          if (z0) lo = v4i{};
          if (z1) hi = v4i{};
        }
        bf[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if (MODE == kMx32) {
            const int scb = (int)(sb_cur[j] >> (16 * kk));
            const int sca = (int)(sa_cur[i] >> (16 * kk));
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bf[j], af[i], acc[i][j], 0, 0, 0, scb, 0, sca);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bf[j], af[i], acc[i][j], 0, 0, 0, 0, 0, 0);
          }
        }
    }
  }
}

// Scale, round and store a tile.  m0/n0: global coordinates of the tile origin;
// rows at or past m_end / columns at or past N are not stored.  Output row m
// lives at C + m * ldc.
template <class Cfg, int MODE, typename OutT>
__device__ __forceinline__ void epilogue(const v16f (&acc)[Cfg::kFragM][Cfg::kFragN], OutT* C,
                                         int64_t ldc, int m0, int m_end, int n0, int N,
                                         float tensor_scale, const float* row_sa,
                                         const float* col_sb) {
  constexpr int FM = Cfg::kFragM, FN = Cfg::kFragN;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const int h = lane >> 5;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * Cfg::WM + i * 32 + (lane & 31);
    if (m >= m_end) continue;
    float fa = 1.0f;
    if (MODE == kTensor) fa = tensor_scale;
    if (MODE == kRowwise) fa = row_sa[m];
    OutT* crow = C + (int64_t)m * ldc;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * Cfg::WN + j * 32 + 8 * g + 4 * h;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e] * fa;
        if (MODE == kRowwise) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= (n + e < N) ? col_sb[n + e] : 0.0f;
        }
        if (n + 3 < N) {
          *reinterpret_cast<uint2*>(crow + n) = pack4<OutT>(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) crow[n + e] = to_out<OutT>(v[e]);
        }
      }
    }
  }
}

}  // namespace fp8gemm
