// One output tile of the scaled FP8 GEMM on gfx950 MFMA: the K mainloop and the
// scale/cast epilogue.  Used by the dense kernel (one tile per workgroup) and the
// grouped kernel (a persistent loop over expert tiles).
//
// Prior art and what is kept.  "Hopper/Blackwell architecture features" §12.7
// tiles C into BLOCK_M x BLOCK_N tiles, walks K in BLOCK_K steps accumulating
// fp32 and casts on store; §12.4 overlaps the load of later K tiles with the math
// on the current one through a multi-stage shared-memory ring whose size per
// stage is (BLOCK_M + BLOCK_N) * BLOCK_K * element size (§12.4.3).  The
// TMA/mbarrier/warp-specialised machinery of §12.2/§12.3 has no CDNA
// counterpart; here every wavefront both copies and computes:
//   * K is walked in 64-byte sub-tiles (one V_MFMA_SCALE_F32_32X32X64_F8F6F4 K
//     step).  A ring of four LDS slots of (BM + BN) * 64 bytes (32 KiB for
//     256 x 256) is filled by gfx950's direct `global_load_lds_dwordx4` copies
//     (16 bytes per lane, no VGPR staging) issued four sub-tiles ahead.  Each
//     sub-tile waits only for the copies of the next one (an s_waitcnt vmcnt
//     count that leaves the two newer sub-tiles in flight) and one workgroup
//     barrier, so 64-96 KiB stay in flight per CU; with a single 64 KiB stage the
//     copy stream stalls on latency at about half the rate it sustains here.
//   * LDS rows are 64 bytes; 16-byte chunk c of tile row r is stored at chunk
//     c ^ ((r >> 2) & 3).  A fragment read touches 16 consecutive rows at one
//     logical chunk per 16-lane group, and the XOR spreads them over all 64
//     banks.  The XOR is applied on the copy side by choosing which global chunk
//     each lane fetches.
//   * Each wavefront owns a WM x WN sub-tile of 32 x 32 MFMA blocks.  Per lane an
//     operand fragment is two 16-byte K chunks, k = 32*(byte/16) + 16*(lane/32)
//     + byte%16, of row lane%32; the E8M0 scale of (row r, 32-K block b) is byte
//     0 of the scale register of lane r + 32*b.  Per-tensor and row-wise operands
//     use the unscaled MFMA; MX operands pass the E8M0 codes, so block scales are
//     applied inside the instruction.  MX codes travel through LDS next to their
//     tile (one dword = four blocks per row per 128 K).
//   * Fragments are double-buffered in registers: the LDS reads of sub-tile t+1
//     are interleaved with the MFMAs of sub-tile t.
//   * The instruction takes B as its first operand, so the accumulator holds C^T
//     blocks: a lane has four consecutive output columns of one row.  The
//     epilogue scales them (row-wise scales come from LDS, copied at tile start),
//     rounds to fp16/bf16, transposes the tile through LDS and writes C with
//     fully coalesced 16-byte stores.
//   * Rows past the matrix edge are read from the last valid row and never
//     stored; K chunks past K are read from column 0 and zeroed in registers,
//     their MX scales set to 2^0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_utils.h"
#include "launch.h"

// Element formats of the A and B codes, fixed per translation unit: the library
// compiles the GEMM once per format pair, and the inline namespace keeps the
// instances of these header templates apart.
#ifndef FP8GEMM_FMT_A
#define FP8GEMM_FMT_A 0
#endif
#ifndef FP8GEMM_FMT_B
#define FP8GEMM_FMT_B 0
#endif
#define FP8GEMM_FMT_NS_(a, b) fmt_##a##b
#define FP8GEMM_FMT_NS(a, b) FP8GEMM_FMT_NS_(a, b)

#ifndef FP8GEMM_DIRECT_EPILOGUE
#define FP8GEMM_DIRECT_EPILOGUE 1
#endif
#ifndef FP8GEMM_SCHED
#define FP8GEMM_SCHED 1
#endif
#ifndef FP8GEMM_F4_UNROLL
#define FP8GEMM_F4_UNROLL 1    // FP4 interior loop: code groups per unrolled body (1 or 2)
#endif

namespace fp8gemm {
inline namespace FP8GEMM_FMT_NS(FP8GEMM_FMT_A, FP8GEMM_FMT_B) {

// operand-format fields of the F8F6F4 MFMA (B is its first operand)
constexpr int kFmtA = FP8GEMM_FMT_A, kFmtB = FP8GEMM_FMT_B;
// FP4 (e2m1, format field 4) operands: two codes per byte, so one 64-byte K
// sub-tile holds 128 K elements and feeds two MFMAs of 64 K.  The instruction
// takes 16 bytes per lane for FP4 (32 elements of row lane % 32 from 32-K block
// lane / 32, low nibble first; probed on gfx950), so the two 16-byte chunks a
// lane reads for an FP8 fragment are exactly the operands of those two MFMAs,
// and an E8M0 block covers 16 bytes instead of 32.  A lane takes chunks 2h and
// 2h + 1 of a 64-byte step (h = lane / 32): the first MFMA then covers blocks
// 4s and 4s + 2, the second 4s + 1 and 4s + 3 (the order of K inside an MFMA
// does not matter), and the two code bytes a lane needs, 4s + 2h and 4s + 2h + 1,
// are adjacent: one 16-bit read, byte 0 for the first MFMA and byte 1 (op_sel 1,
// probed) for the second.  Only FP4 x FP4 is built.
constexpr bool kF4 = kFmtA == 4;
static_assert((kFmtA == 4) == (kFmtB == 4), "FP4 operands pair with FP4 operands only");
constexpr int kBlkBytes = kF4 ? 16 : 32;     // bytes of one 32-element MX block

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// The 16-byte halves of an FP8 fragment as FP4 operands (the instruction reads
// the first four registers of an FP4 operand, so no copies are made).
__device__ __forceinline__ v8i lo16(const v8i& v) {
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, 0, 1, 2, 3);
}
__device__ __forceinline__ v8i hi16(const v8i& v) {
  return __builtin_shufflevector(v, v, 4, 5, 6, 7, 4, 5, 6, 7);
}

// BM x BN output tile, WM x WN per wavefront, SLOTS-deep LDS ring, and the number
// of workgroups meant to share a CU (their waves then share each SIMD, so one
// workgroup's barrier waits are covered by the other's MFMAs).
template <int BM_, int BN_, int WM_, int WN_, int SLOTS_ = 4, int WG_PER_CU_ = 1>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int kBK = 64;                              // K bytes per sub-tile
  static constexpr int kSlots = SLOTS_;                       // LDS ring depth
  static constexpr int kWgPerCu = WG_PER_CU_;
  static constexpr int kWavesM = BM / WM, kWavesN = BN / WN;
  static constexpr int kWaves = kWavesM * kWavesN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kFragM = WM / 32, kFragN = WN / 32;
  static constexpr int kSlotBytes = (BM + BN) * kBK;
  static constexpr int kScaleSlotBytes = (BM + BN) * 4;       // MX: 4 codes per row per 128 K
  // MX codes of a 128-K tile are copied with its first sub-tile, kSlots sub-tiles
  // ahead, and read until its last one: kSlots / 2 K tiles are live at once
  static constexpr int kScaleSlots = kSlots / 2 > 2 ? kSlots / 2 : 2;
  // row-wise: fp32 per row / column, two buffers (persistent kernels alternate)
  static constexpr int kRowScaleBytes = 2 * (BM + BN) * 4;
  static constexpr int kScaleOff = kSlots * kSlotBytes;
  static constexpr int kRowScaleOff = kScaleOff + kScaleSlots * kScaleSlotBytes;
  // interior path, MX: two buffers of 16 code bytes (512 K) per row after the ring
  static constexpr int kCodeBytes = 2 * (BM + BN) * 16;
  static constexpr int kLdsBytes = kRowScaleOff + kRowScaleBytes > kScaleOff + kCodeBytes
                                       ? kRowScaleOff + kRowScaleBytes
                                       : kScaleOff + kCodeBytes;
  // copies per sub-tile and wavefront: 1 KiB (16 rows of 64 bytes) per instruction
  static constexpr int kTileLoads = (BM + BN) * kBK / 1024 / kWaves;
  // dword copies (MX codes per 128 K, row-wise scales) per wavefront: one dword per
  // row, 64 rows per instruction; waves without a full share repeat the last one
  static constexpr int kScaleInsts = (BM + BN) / 64;
  static constexpr int kScaleLoads = (kScaleInsts + kWaves - 1) / kWaves;
  // epilogue staging: 32 rows of one wavefront's columns (+16 bytes against conflicts)
  static constexpr int kStagePitch = WN * 2 + 16;
  static_assert((BM + BN) * kBK % (1024 * kWaves) == 0, "equal copy share per wavefront");
  static_assert(BM % 64 == 0 && BN % 64 == 0, "whole copy instructions per operand");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "32x32 MFMA blocks");
  static_assert(kWaves * 32 * kStagePitch <= kSlots * kSlotBytes, "epilogue staging fits");
  static_assert(kLdsBytes * kWgPerCu <= 160 * 1024, "LDS per CU");
  static_assert(kSlots >= 3, "ring keeps one sub-tile being read and one in flight");
  // waves per SIMD, for __launch_bounds__ (caps registers at 512 / this)
  static constexpr int kWavesPerEu = kWgPerCu * kWaves / 4 > 0 ? kWgPerCu * kWaves / 4 : 1;
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
  const float* ra;      // row-wise: fp32 scale of A's first tile row
  const float* rb;      // row-wise: fp32 scale of B's first tile row
  int K;                // K extent of this tile's product (a split's slice under split-K)
  int sld;              // MX: bytes between the codes of consecutive rows
  // Row-major B ([K][N], N contiguous; the kn kernels): B is this tile's first
  // column of K-row 0, ldb the bytes between K-rows, b_rows the valid columns;
  // sb the tile's first column of the codes [K/32][N], sldb the bytes between
  // their rows.
  int sldb = 0;
};

// A copy of a tile's operand description with every field read from the first
// lane.  The values are wave-uniform by construction; where they come through a
// data-dependent search (grouped tiles) or a struct the compiler keeps in memory,
// its divergence analysis may no longer see that, and it would then compute the
// copy offsets in vector registers and wrap every copy in a loop over the lanes'
// distinct descriptors.  For values already in scalar registers this is free.
template <class T>
__device__ __forceinline__ T first_lane_ptr(T p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<T>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int64_t first_lane_i64(int64_t v) {
  const uint64_t a = (uint64_t)v;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ TileOperands first_lane(const TileOperands& o) {
  TileOperands u;
  u.A = first_lane_ptr(o.A);
  u.lda = first_lane_i64(o.lda);
  u.a_rows = __builtin_amdgcn_readfirstlane(o.a_rows);
  u.B = first_lane_ptr(o.B);
  u.ldb = first_lane_i64(o.ldb);
  u.b_rows = __builtin_amdgcn_readfirstlane(o.b_rows);
  u.sa = first_lane_ptr(o.sa);
  u.sb = first_lane_ptr(o.sb);
  u.ra = first_lane_ptr(o.ra);
  u.rb = first_lane_ptr(o.rb);
  u.K = __builtin_amdgcn_readfirstlane(o.K);
  u.sld = __builtin_amdgcn_readfirstlane(o.sld);
  u.sldb = __builtin_amdgcn_readfirstlane(o.sldb);
  return u;
}

// Row-major B in LDS: a 128-K tile is 128 K-rows of BN bytes; 16-byte chunk c of
// K-row k sits at chunk c ^ kn_swz(k).  A transposing read takes 8 K-rows at one
// 32-column fragment (two chunks, both halves): with this XOR the 32 lanes of a
// half-wave hit 32 distinct bank pairs for BN = 64, 128 and 256 (rows of 64 B
// share a 256-byte bank line four ways, rows of 128 B two ways).
template <int BN>
__device__ __forceinline__ int kn_swz(int k) {
  return 2 * ((k / (256 / BN)) & (BN / 32 - 1));
}

// The same for packed FP4 B: a K-row holds BN / 2 bytes (two codes per byte),
// a 32-column fragment is one 16-byte chunk, and a transposing read
// (ds_read_b64_tr_b4; probed on gfx950: in each 16-lane group, 4-bit element j
// of lane i is element i of the 16 addressed by lane j) takes 16 K-rows at one
// fragment (both 8-byte halves).  Chunk c of K-row k sits at c ^ kn4_swz(k): the
// 16 rows of a half-wave's read land on 16 distinct 16-byte bank groups for BN =
// 64, 128 and 256 (period 16 in k).
template <int BN>
__device__ __forceinline__ int kn4_swz(int k) {
  return (k / (512 / BN)) & (BN / 32 - 1);
}

__device__ __forceinline__ void lds_dma16(const uint8_t* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

__device__ __forceinline__ void lds_dma4(const void* g, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

// Chunk swizzle of a 64-byte LDS row.
__device__ __forceinline__ int lds_swz(int r) { return (r >> 2) & 3; }

// s_waitcnt with vmcnt(n) (n < 64), lgkmcnt(0), no expcnt wait (gfx9 encoding).
#define FP8GEMM_WAIT_VM_LGKM0(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | ((((n) >> 4) & 3) << 14))

// Copies of sub-tile s (K bytes [64 s, 64 s + 64)) into an LDS slot: A rows, then
// B rows; instruction g covers tile rows 16 g .. 16 g + 15 of [A; B].
template <class Cfg, bool KTAIL>
__device__ __forceinline__ void copy_subtile(const TileOperands& op, uint8_t* slot, int s,
                                             int wave, int lane) {
  constexpr int nA = Cfg::BM / 16;
  const int sub = lane >> 2;                    // row within the 16-row group
#pragma unroll
  for (int j = 0; j < Cfg::kTileLoads; ++j) {
    const int g = wave * Cfg::kTileLoads + j;   // wave-uniform instruction index
    const bool isA = g < nA;
    const int row_t = (isA ? g : g - nA) * 16 + sub;
    const int chunk = (lane & 3) ^ lds_swz(row_t);
    int kc = s * Cfg::kBK + 16 * chunk;
    if (KTAIL && kc >= op.K) kc = 0;            // in-bounds dummy, zeroed before use
    const uint8_t* base = isA ? op.A : op.B;
    const int64_t ld = isA ? op.lda : op.ldb;
    const int rows = isA ? op.a_rows : op.b_rows;
    const int row = row_t < rows ? row_t : rows - 1;
    lds_dma16(base + (int64_t)row * ld + kc, slot + g * 1024);
  }
}

// Dword copies (one lane per row, 64 rows per instruction) of every A row and then
// every B row of a tile, spread over the wavefronts without branches: every wave
// issues kScaleLoads instructions (so copy counts stay uniform for the vmcnt
// waits); indices past the last instruction repeat it, rewriting the same bytes.
// Row r of A lands at dst[4 r], row r of B at dst[4 (BM + r)].
template <class Cfg>
__device__ __forceinline__ void dword_rows_ab(const uint8_t* pa, int64_t lda, int a_rows,
                                              const uint8_t* pb, int64_t ldb, int b_rows,
                                              int byte_off, uint8_t* dst, int wave, int lane) {
  constexpr int nA = Cfg::BM / 64;
#pragma unroll
  for (int j = 0; j < Cfg::kScaleLoads; ++j) {
    int i = wave * Cfg::kScaleLoads + j;         // wave-uniform
    i = i < Cfg::kScaleInsts ? i : Cfg::kScaleInsts - 1;
    const bool isA = i < nA;
    const uint8_t* base = isA ? pa : pb;
    const int64_t ld = isA ? lda : ldb;
    const int rows = isA ? a_rows : b_rows;
    const int row_t = (isA ? i : i - nA) * 64 + lane;
    const int row = row_t < rows ? row_t : rows - 1;
    lds_dma4(base + (int64_t)row * ld + byte_off, dst + i * 256);
  }
}

// The j-th of this wave's tile copy instructions for sub-tile s (see copy_subtile).
template <class Cfg, bool KTAIL>
__device__ __forceinline__ void copy_one(const TileOperands& op, uint8_t* slot, int s, int j,
                                         int wave, int lane) {
  constexpr int nA = Cfg::BM / 16;
  const int g = wave * Cfg::kTileLoads + j;     // wave-uniform instruction index
  const bool isA = g < nA;
  const int row_t = (isA ? g : g - nA) * 16 + (lane >> 2);
  const int chunk = (lane & 3) ^ lds_swz(row_t);
  int kc = s * Cfg::kBK + 16 * chunk;
  if (KTAIL && kc >= op.K) kc = 0;
  const uint8_t* base = isA ? op.A : op.B;
  const int64_t ld = isA ? op.lda : op.ldb;
  const int rows = isA ? op.a_rows : op.b_rows;
  const int row = row_t < rows ? row_t : rows - 1;
  lds_dma16(base + (int64_t)row * ld + kc, slot + g * 1024);
}

// The j-th of this wave's dword copy instructions (see dword_rows_ab).
template <class Cfg>
__device__ __forceinline__ void dword_one(const uint8_t* pa, int64_t lda, int a_rows,
                                          const uint8_t* pb, int64_t ldb, int b_rows, int byte_off,
                                          uint8_t* dst, int j, int wave, int lane) {
  constexpr int nA = Cfg::BM / 64;
  int i = wave * Cfg::kScaleLoads + j;
  i = i < Cfg::kScaleInsts ? i : Cfg::kScaleInsts - 1;
  const bool isA = i < nA;
  const uint8_t* base = isA ? pa : pb;
  const int64_t ld = isA ? lda : ldb;
  const int rows = isA ? a_rows : b_rows;
  const int row_t = (isA ? i : i - nA) * 64 + lane;
  const int row = row_t < rows ? row_t : rows - 1;
  lds_dma4(base + (int64_t)row * ld + byte_off, dst + i * 256);
}

// One 16-byte fragment read: r < 2*FM -> A fragment r/2, else B fragment; r odd ->
// the second K chunk.  Zeroed when it lies past K (KTAIL).
template <class Cfg, bool KTAIL>
__device__ __forceinline__ v4i read_one(const uint8_t* slot, int r, int k0, int K,
                                        const int (&arow)[Cfg::kFragM],
                                        const int (&brow)[Cfg::kFragN], int h) {
  const bool isA = r < 2 * Cfg::kFragM;
  const int idx = isA ? r >> 1 : (r - 2 * Cfg::kFragM) >> 1;
  const int row = isA ? arow[idx] : Cfg::BM + brow[idx];
  const int c = kF4 ? 2 * h + (r & 1) : h + 2 * (r & 1);
  v4i v = *reinterpret_cast<const v4i*>(slot + row * Cfg::kBK + 16 * (c ^ lds_swz(row)));
  if (KTAIL && k0 + 16 * c >= K) v = v4i{};
  return v;
}

// Operand fragments of one sub-tile for all of a wave's MFMA blocks.
template <class Cfg, bool KTAIL>
__device__ __forceinline__ void read_frags(const uint8_t* slot, int k0, int K,
                                           const int (&arow)[Cfg::kFragM],
                                           const int (&brow)[Cfg::kFragN], int h,
                                           v8i (&af)[Cfg::kFragM], v8i (&bf)[Cfg::kFragN]) {
  const int c0 = kF4 ? 2 * h : h, c1 = kF4 ? 2 * h + 1 : h + 2;
  bool z0 = false, z1 = false;
  if (KTAIL) {
    z0 = k0 + 16 * c0 >= K;
    z1 = k0 + 16 * c1 >= K;
  }
  const uint8_t* sB = slot + Cfg::BM * Cfg::kBK;
#pragma unroll
  for (int i = 0; i < Cfg::kFragM; ++i) {
    const uint8_t* rowp = slot + arow[i] * Cfg::kBK;
    const int sw = lds_swz(arow[i]);
    v4i lo = *reinterpret_cast<const v4i*>(rowp + 16 * (c0 ^ sw));
    v4i hi = *reinterpret_cast<const v4i*>(rowp + 16 * (c1 ^ sw));
    if (KTAIL) {
      if (z0) lo = v4i{};
      if (z1) hi = v4i{};
    }
    af[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
#pragma unroll
  for (int j = 0; j < Cfg::kFragN; ++j) {
    const uint8_t* rowp = sB + brow[j] * Cfg::kBK;
    const int sw = lds_swz(brow[j]);
    v4i lo = *reinterpret_cast<const v4i*>(rowp + 16 * (c0 ^ sw));
    v4i hi = *reinterpret_cast<const v4i*>(rowp + 16 * (c1 ^ sw));
    if (KTAIL) {
      if (z0) lo = v4i{};
      if (z1) hi = v4i{};
    }
    bf[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// All MFMA blocks of a wave for one sub-tile.  B is the instruction's first
// operand (rows n), A the second (columns m): the accumulators hold C^T blocks.
template <class Cfg, int MODE>
__device__ __forceinline__ void mfma_subtile(v16f (&acc)[Cfg::kFragM][Cfg::kFragN],
                                             const v8i (&af)[Cfg::kFragM],
                                             const v8i (&bf)[Cfg::kFragN],
                                             const uint32_t (&sa)[Cfg::kFragM],
                                             const uint32_t (&sb)[Cfg::kFragN]) {
#pragma unroll
  for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::kFragN; ++j) {
      if (MODE == kMx32) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            bf[j], af[i], acc[i][j], kFmtB, kFmtA, 0, (int)sb[j], 0, (int)sa[i]);
      } else {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[j], af[i], acc[i][j], kFmtB,
                                                                    kFmtA, 0, 0, 0, 0);
      }
    }
}

// Interleaving hint for one sub-tile region (AMDGPU scheduler group masks: 0x008
// MFMA, 0x020 VMEM read, 0x100 DS read): LDS reads early, copies spread out.
template <class Cfg, int NVMEM, int NDS>
__device__ __forceinline__ void sched_subtile() {
#if FP8GEMM_SCHED
  constexpr int kMfma = Cfg::kFragM * Cfg::kFragN;
  constexpr int kD = (NDS + kMfma / 2 - 1) / (kMfma / 2);   // reads in the first half
  constexpr int kV = (NVMEM + kMfma - 1) / kMfma;
#pragma unroll
  for (int i = 0; i < kMfma; ++i) {
    if (i < kMfma / 2) __builtin_amdgcn_sched_group_barrier(0x100, kD, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, kV, 0);
  }
#endif
}

// The K loop of one tile.  Per sub-tile t (64 K):
//   wait: own copies of sub-tile t+1 landed (the S-2 newer sub-tiles may stay
//         in flight) and own LDS reads done; workgroup barrier
//   copy sub-tile t+S into slot t%S (free: its fragments are in registers) and,
//         every 128 K, the MX codes of that K tile
//   LDS reads of sub-tile t+1 (and MX codes)     || MFMAs of sub-tile t
// The loop runs an even number of sub-tiles (K tails are zero-filled) and copies
// past the end re-fetch the last sub-tile, so counts per sub-tile are constant.
// With K % 128 != 0 the MX codes are read with byte loads and every wait drains
// all copies (a rarely used, simpler path).  FP4 operands always take that path
// here (KALIGNED = false): their interior tiles run mainloop_interior.
template <class Cfg, int MODE, bool KALIGNED>
__device__ __forceinline__ void mainloop(const TileOperands& op, uint8_t* lds,
                                         v16f (&acc)[Cfg::kFragM][Cfg::kFragN]) {
  constexpr int FM = Cfg::kFragM, FN = Cfg::kFragN;
  static_assert(!(kF4 && KALIGNED), "FP4 edge tiles read their codes into registers");
  constexpr bool KTAIL = !KALIGNED;
  constexpr bool kMxLds = (MODE == kMx32) && KALIGNED;
  constexpr bool kMxReg = (MODE == kMx32) && !KALIGNED;
  // copies issued per sub-tile by this wave: even sub-tiles also carry MX codes
  constexpr int S = Cfg::kSlots;
  constexpr int kLoadsOdd = Cfg::kTileLoads;
  constexpr int kLoadsEven = Cfg::kTileLoads + (kMxLds ? Cfg::kScaleLoads : 0);
  // copies allowed in flight at the barrier of an even / odd sub-tile t: those of
  // sub-tiles t+2 .. t+S-1; in the prologue: sub-tiles 1 .. S-1
  constexpr int kWaitEven = ((S - 2) / 2) * (kLoadsOdd + kLoadsEven) + ((S - 2) % 2) * kLoadsEven;
  constexpr int kWaitOdd = ((S - 2) / 2) * (kLoadsOdd + kLoadsEven) + ((S - 2) % 2) * kLoadsOdd;
  constexpr int kWaitPrologue = ((S - 1) / 2) * (kLoadsOdd + kLoadsEven) + ((S - 1) % 2) * kLoadsOdd;
  static_assert(kWaitPrologue < 64, "vmcnt range");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const int h = lane >> 5;
  const int nsub = ((op.K + 127) / 128) * 2;     // even number of 64-K sub-tiles
  const int nvalid = (op.K + Cfg::kBK - 1) / Cfg::kBK;
  const int nblk = op.K / kBlkBytes;

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

  int arow[FM], brow[FN];        // tile-local fragment rows of this lane
#pragma unroll
  for (int i = 0; i < FM; ++i) arow[i] = wm * Cfg::WM + i * 32 + (lane & 31);
#pragma unroll
  for (int j = 0; j < FN; ++j) brow[j] = wn * Cfg::WN + j * 32 + (lane & 31);

  auto slot_ptr = [&](int s) { return lds + (s % S) * Cfg::kSlotBytes; };
  auto copy = [&](int s) {
    const int sc = s < nvalid ? s : nvalid - 1;  // past the end: harmless re-fetch
    copy_subtile<Cfg, KTAIL>(op, slot_ptr(s), sc, wave, lane);
    if (kMxLds && (s & 1) == 0) {
      uint8_t* sslot = lds + Cfg::kScaleOff + ((s >> 1) % Cfg::kScaleSlots) * Cfg::kScaleSlotBytes;
      dword_rows_ab<Cfg>(op.sa, op.sld, op.a_rows, op.sb, op.sld, op.b_rows, 4 * (sc >> 1), sslot,
                         wave, lane);
    }
  };

  // MX scale registers.  K % 128 == 0: one word per fragment row and K tile,
  // pre-shifted so byte 0 / byte 2 are the codes of its even / odd sub-tile
  // (cur = this K tile, nxt = the next).  Otherwise: the code of the current /
  // next sub-tile in byte 0.
  uint32_t sa_cur[FM], sb_cur[FN], sa_nxt[FM], sb_nxt[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) sa_cur[i] = sa_nxt[i] = 0;
#pragma unroll
  for (int j = 0; j < FN; ++j) sb_cur[j] = sb_nxt[j] = 0;
  // words of K tile kt (resident in scale slot kt & 1)
  auto read_lds_codes = [&](int kt, uint32_t (&a)[FM], uint32_t (&b)[FN]) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(lds + Cfg::kScaleOff +
                                                          (kt % Cfg::kScaleSlots) * Cfg::kScaleSlotBytes);
#pragma unroll
    for (int i = 0; i < FM; ++i) a[i] = w[arow[i]] >> (8 * h);
#pragma unroll
    for (int j = 0; j < FN; ++j) b[j] = w[Cfg::BM + brow[j]] >> (8 * h);
  };
  // codes of sub-tile s straight from global memory (K % 128 != 0): block 2s + h.
  // FP4: blocks 4s + 2h (first MFMA, bits 0-7) and 4s + 2h + 1 (second MFMA, bits
  // 8-15, which it reads through op_sel 1)
  auto load_reg_codes = [&](int s, uint32_t (&a)[FM], uint32_t (&b)[FN]) {
    const int blk = kF4 ? 4 * s + 2 * h : 2 * s + h;
    auto code = [&](const uint8_t* base, int b) { return b < nblk ? (uint32_t)base[b] : 127u; };
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = arow[i] < op.a_rows ? arow[i] : op.a_rows - 1;
      const uint8_t* row = op.sa + (int64_t)r * op.sld;
      a[i] = kF4 ? code(row, blk) | (code(row, blk + 1) << 8) : code(row, blk);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = brow[j] < op.b_rows ? brow[j] : op.b_rows - 1;
      const uint8_t* row = op.sb + (int64_t)r * op.sld;
      b[j] = kF4 ? code(row, blk) | (code(row, blk + 1) << 8) : code(row, blk);
    }
  };

  v8i af0[FM], bf0[FN], af1[FM], bf1[FN];

  // prologue: sub-tiles 0..3 in flight; wait for sub-tile 0; its fragments in registers
  if (MODE == kRowwise) {
    dword_rows_ab<Cfg>(reinterpret_cast<const uint8_t*>(op.ra), 4, op.a_rows,
                       reinterpret_cast<const uint8_t*>(op.rb), 4, op.b_rows, 0,
                       lds + Cfg::kRowScaleOff, wave, lane);
  }
#pragma unroll
  for (int s = 0; s < S; ++s) copy(s);
  if (KALIGNED) FP8GEMM_WAIT_VM_LGKM0(kWaitPrologue);
  else __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  read_frags<Cfg, KTAIL>(slot_ptr(0), 0, op.K, arow, brow, h, af0, bf0);
  if (kMxLds) read_lds_codes(0, sa_cur, sb_cur);
  if (kMxReg) load_reg_codes(0, sa_cur, sb_cur);

  // One sub-tile, issued in a fixed order (sched_barrier fences): for each MFMA q,
  // the MFMA, then its share of the copy instructions of sub-tile t+S and of the
  // LDS reads of sub-tile t+1.  The matrix pipe never waits behind a burst of
  // memory instructions, and the copies / reads trickle out between MFMAs.
  constexpr int kMfma = FM * FN;
  constexpr int kReads = 2 * (FM + FN);
  auto step = [&](int t, v8i (&fa)[FM], v8i (&fb)[FN], v8i (&na)[FM], v8i (&nb)[FN],
                  auto odd_c) {
    constexpr bool odd = decltype(odd_c)::value;
    constexpr int kVmem = Cfg::kTileLoads + ((kMxLds && !odd) ? Cfg::kScaleLoads : 0);
    constexpr int kDs = kReads + ((kMxLds && odd) ? FM + FN : 0);
    __builtin_amdgcn_sched_barrier(0);
    if (!KALIGNED) __builtin_amdgcn_s_waitcnt(0);     // copies of sub-tile t+1 landed
    else if (odd) FP8GEMM_WAIT_VM_LGKM0(kWaitOdd);
    else FP8GEMM_WAIT_VM_LGKM0(kWaitEven);
    __builtin_amdgcn_s_barrier();                      // ... for every wave; slot t%S free
    __builtin_amdgcn_sched_barrier(0);
    if (kMxReg) load_reg_codes(t + 1, sa_nxt, sb_nxt);
    const int sn = t + S;                              // sub-tile to copy
    const int sc = sn < nvalid ? sn : nvalid - 1;      // past the end: harmless re-fetch
    uint8_t* cslot = slot_ptr(sn);
    uint8_t* sslot = lds + Cfg::kScaleOff + ((sn >> 1) % Cfg::kScaleSlots) * Cfg::kScaleSlotBytes;
    const uint8_t* rslot = slot_ptr(t + 1);
    const int rk0 = (t + 1) * Cfg::kBK;
    const uint32_t* wsc = reinterpret_cast<const uint32_t*>(
        lds + Cfg::kScaleOff + (((t + 1) >> 1) % Cfg::kScaleSlots) * Cfg::kScaleSlotBytes);
    v4i rd[kReads];
#pragma unroll
    for (int q = 0; q < kMfma; ++q) {
      const int i = q / FN, j = q % FN;
      if (kF4) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            lo16(fb[j]), lo16(fa[i]), acc[i][j], kFmtB, kFmtA, 0, (int)sb_cur[j], 0,
            (int)sa_cur[i]);
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            hi16(fb[j]), hi16(fa[i]), acc[i][j], kFmtB, kFmtA, 1, (int)sb_cur[j], 1,
            (int)sa_cur[i]);
      } else if (MODE == kMx32) {
        const uint32_t sa = (kMxLds && odd) ? sa_cur[i] >> 16 : sa_cur[i];
        const uint32_t sb = (kMxLds && odd) ? sb_cur[j] >> 16 : sb_cur[j];
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fb[j], fa[i], acc[i][j], kFmtB, kFmtA, 0, (int)sb, 0, (int)sa);
      } else {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], kFmtB,
                                                                    kFmtA, 0, 0, 0, 0);
      }
#pragma unroll
      for (int v = q * kVmem / kMfma; v < (q + 1) * kVmem / kMfma; ++v) {
        if (v < Cfg::kTileLoads) {
          copy_one<Cfg, KTAIL>(op, cslot, sc, v, wave, lane);
        } else if (kMxLds) {
          dword_one<Cfg>(op.sa, op.sld, op.a_rows, op.sb, op.sld, op.b_rows, 4 * (sc >> 1), sslot,
                         v - Cfg::kTileLoads, wave, lane);
        }
      }
#pragma unroll
      for (int d = q * kDs / kMfma; d < (q + 1) * kDs / kMfma; ++d) {
        if (d < kReads) {
          rd[d] = read_one<Cfg, KTAIL>(rslot, d, rk0, op.K, arow, brow, h);
        } else if (kMxLds) {
          const int e = d - kReads;
          if (e < FM) sa_nxt[e] = wsc[arow[e]] >> (8 * h);
          else sb_nxt[e - FM] = wsc[Cfg::BM + brow[e - FM]] >> (8 * h);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) na[i] = __builtin_shufflevector(rd[2 * i], rd[2 * i + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      nb[j] = __builtin_shufflevector(rd[2 * FM + 2 * j], rd[2 * FM + 2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
    if (kMxReg || (kMxLds && odd)) {
#pragma unroll
      for (int i = 0; i < FM; ++i) sa_cur[i] = sa_nxt[i];
#pragma unroll
      for (int j = 0; j < FN; ++j) sb_cur[j] = sb_nxt[j];
    }
  };

  for (int t = 0; t < nsub; t += 2) {
    step(t, af0, bf0, af1, bf1, std::false_type{});
    step(t + 1, af1, bf1, af0, bf0, std::true_type{});
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0);     // no copy may still target LDS
  __builtin_amdgcn_s_barrier();      // every wave is done with the ring
}

// ---------------------------------------------------------------------------
// Interior tiles.  Two changes against mainloop(), both about the copy stream,
// which bounds this kernel on gfx950:
//   * Whole cache lines.  A copy instruction that reads 64 bytes from each of 16
//     rows costs as many memory requests as one reading 128 bytes from each of
//     them; measured on MI355X, 64-byte row pieces stream at about 14 TB/s and
//     128-byte pieces at about 25 TB/s into LDS.  The ring therefore holds two
//     128-K tiles of (BM + BN) rows x 128 bytes (the same 2 x 64 KiB for
//     256 x 256), each tile is consumed as two 64-K MFMA steps, and the copies
//     of K tile u + 2 go out while K tile u + 1 is consumed.
//     LDS rows are 128 bytes; 16-byte chunk c of row r sits at chunk
//     c ^ ((r >> 1) & 7), which spreads the 16 rows of a fragment read over all
//     64 banks.
//   * MX codes are fetched 16 bytes (512 K) per row at a time instead of 4 bytes
//     per 128 K: each code copy touches one cache line per row, so this cuts its
//     requests by four.
// No vector-ALU work is left inside the K loop (each VALU instruction between
// the MFMAs of the single wavefront of a SIMD delays the next MFMA): copies go
// through buffer descriptors of the tile's rows with a loop-invariant lane
// offset and a scalar offset; LDS reads use per-lane base registers with the
// slot, K half and fragment folded into the instruction offset (the loop is
// unrolled over the ring); MX codes are read as single bytes, the form the MFMA
// takes.
// Conditions: every row of the tile valid; K % 128 == 0 (MX: a whole 16-byte code
// group per row, K % 512 == 0, FP4 K % 256 == 0 bytes); the byte span of a tile's
// rows fits a 32-bit buffer offset.
// FP4: a 64-K step of the description below is a 64-byte step of 128 K elements,
// two MFMAs per fragment pair, each with its own code byte; a code group then
// covers two K tiles instead of four.
// ---------------------------------------------------------------------------

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  // gfx9 raw buffer descriptor: no stride, no swizzle, 32-bit data format word
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ void buffer_dma16(__amdgpu_buffer_rsrc_t rs, uint8_t* lds, int voff,
                                             int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, soff, 0, 0);
}

// The same copy issued from inline assembly, so that the compiler does not track
// it.  The compiler makes every LDS read that it cannot tell apart from a pending
// direct-to-LDS copy wait for all of them (s_waitcnt vmcnt(0)); it does so for
// the transposing reads (ds_read_b64_tr_b8), which would serialise the copy ring.
// Loops that issue their copies here keep their own explicit waits, which count
// these copies like any other (they are ordinary vector-memory operations); the
// instruction writes no VGPR.  rs: the four descriptor words (buffer_rsrc_words).
typedef unsigned v4u_rs __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4u_rs buffer_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return v4u_rs{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}
// lds_base: LDS byte address of the destination area (wave-uniform), lds_off its
// offset; soff the scalar byte offset into the buffer.  The sums are formed at
// the copy from values passed through an empty volatile asm (scalar_fresh), so
// the compiler cannot hoist one SGPR per copy out of an unrolled loop.
__device__ __forceinline__ uint32_t lds_address(const uint8_t* lds) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)lds);
}
template <class T>
__device__ __forceinline__ T scalar_fresh(T v) {
  asm volatile("" : "+s"(v));
  return v;
}
__device__ __forceinline__ void buffer_dma16_untracked(v4u_rs rs, uint32_t lds_base,
                                                       uint32_t lds_off, int voff, int soff) {
  const uint32_t m0 = scalar_fresh(lds_base) + lds_off;
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(rs), "s"(soff)
               : "memory", "m0");
}

// An opaque copy of v: the compiler cannot fold constants through it, so an LDS
// base stays in one register and the constant parts stay in the offset field.
__device__ __forceinline__ int opaque(int v) {
  asm("" : "+v"(v));
  return v;
}

// Compile-time loop: f(integral_constant<int, I>) for I = B .. E - 1.
template <int B, int E>
struct Unroll {
  template <class F>
  static __device__ __forceinline__ void run(F&& f) {
    if constexpr (B < E) {
      f(std::integral_constant<int, B>{});
      Unroll<B + 1, E>::run(f);
    }
  }
};

// Whether a tile's K extent and spans suit the interior mainloop (whole 128-K
// tiles, MX whole code groups, 32-bit buffer offsets); uniform over the
// workgroup.  Rows past M or N are read as zero there, so tiles cut by the edges
// qualify too (their epilogue masks the stores).
template <class Cfg, int MODE>
__device__ __forceinline__ bool interior_k(const TileOperands& op) {
  return op.K % (MODE == kMx32 ? 16 * kBlkBytes : 128) == 0 &&
         (int64_t)Cfg::BM * op.lda + op.K < ((int64_t)1 << 31) &&
         (int64_t)Cfg::BN * op.ldb + op.K < ((int64_t)1 << 31);
}
// ... and the tile is whole (every row and column valid): the copy-stream and
// register-direct epilogue paths.
template <class Cfg, int MODE>
__device__ __forceinline__ bool interior_tile(const TileOperands& op) {
  return op.a_rows >= Cfg::BM && op.b_rows >= Cfg::BN && interior_k<Cfg, MODE>(op);
}

#ifndef FP8GEMM_READ_SPAN
#define FP8GEMM_READ_SPAN 4    // eighths of a step's MFMAs over which its LDS reads are spread
#endif
#ifndef FP8GEMM_COPY_SPAN
#define FP8GEMM_COPY_SPAN 8    // eighths of a step's MFMAs over which its copies are spread
#endif

// NS: ring depth in 128-K tiles (2 for the 256 x 256 tile; 4 or 8 for the split-K
// tiles, whose K slices are short and whose copies come from HBM: a slice streams
// at about the ring's bytes per HBM latency).
//
// KN: B is row-major [K][N] (the layout of the pages' Triton listings, e.g.
// "Hopper/Blackwell architecture features" §12.7.1, where the B pointer advances
// by BLOCK_K * stride_bk).  Its K tile is copied as 128 K-rows of BN bytes (whole
// lines, chunks XOR-swizzled by kn_swz) and each B fragment is assembled from
// four transposing LDS reads (ds_read_b64_tr_b8; probed on gfx950: in each
// 16-lane group, byte j of lane i comes from byte i % 8 of the 8 bytes addressed
// by lane 2 j + i / 8).  Lanes 2 m and 2 m + 1 of a group address K-row kb + m at
// the group's 16 columns, so lane i receives column i at K-rows kb .. kb + 7: the
// eight K bytes of operand bytes 8 q .. 8 q + 7 (kb = 32 (q / 2) + 16 h + 8 (q % 2)
// within the 64-K step).  Packed FP4 B (two codes per byte along N): a K tile is
// 256 K-rows of BN / 2 bytes, a fragment step four ds_read_b64_tr_b4 of 16
// K-rows each (lane w of a 16-lane group addresses K-row kb + w at the 8-byte
// half G of the fragment's chunk; see kn4_swz), and its two codes per step are
// two bytes in two registers.  MX codes of B come as [K/32][N] and sit in LDS as
// [16 blocks][BN] per group.  Tiles cut by M or N run here too: A rows past the edge
// read as zero (the copy range ends at the last valid row) and B columns past N
// hold whatever the copy finds there; neither is ever stored.
template <class Cfg, int MODE, int NS = 2, bool KN = false>
__device__ __forceinline__ void mainloop_interior(const TileOperands& op_in, uint8_t* lds,
                                                  v16f (&acc)[Cfg::kFragM][Cfg::kFragN]) {
  const TileOperands op = first_lane(op_in);
  constexpr int FM = Cfg::kFragM, FN = Cfg::kFragN;
  constexpr bool kMx = MODE == kMx32;
  constexpr int kRowB = 128;                          // bytes per LDS row (one K tile)
  constexpr int kTile = (Cfg::BM + Cfg::BN) * kRowB;  // one ring slot
  constexpr int nA = Cfg::BM / 8;                     // 8-row copy blocks of A
  constexpr int kLoads = kTile / 1024 / Cfg::kWaves;  // tile copies per wave and K tile
  constexpr int kCodeInsts = (Cfg::BM + Cfg::BN) / 64;
  constexpr int kCodeLoads = (kCodeInsts + Cfg::kWaves - 1) / Cfg::kWaves;
  constexpr int kCodeBuf = (Cfg::BM + Cfg::BN) * 16;  // 16 code bytes per row
  constexpr int kCodeOff = NS * kTile;
  constexpr bool kUniformOperand = nA % kLoads == 0;  // a wave copies rows of one operand
  static_assert(NS == 2 || NS == 4 || NS == 8, "ring of 2, 4 or 8 K tiles");
  static_assert(NS * kTile <= Cfg::kScaleOff, "ring fits");
  static_assert(kCodeOff + 2 * kCodeBuf <= Cfg::kLdsBytes, "code buffers fit");
  static_assert(kTile % (1024 * Cfg::kWaves) == 0, "equal copy share per wave");
  static_assert(kLoads % 2 == 0, "copy blocks of both swizzle phases per wave");
  static_assert((NS - 1) * kLoads + kCodeLoads < 64, "vmcnt range");
  // KN: bytes per B K-row in LDS (FP4: two codes per byte), K-rows of B per K
  // tile, K-rows per B copy instruction, 16-byte chunks per K-row; the MX code
  // rows of B hold one byte per column whatever the format
  constexpr int kBRowB = kF4 ? Cfg::BN / 2 : Cfg::BN;
  constexpr int kKTileRows = kF4 ? 2 * kRowB : kRowB;
  constexpr int kKRows = 1024 / kBRowB, kChunks = kBRowB / 16;
  constexpr int kCRows = 1024 / Cfg::BN, kCChunks = Cfg::BN / 16;
  constexpr int kSwzPeriod = kF4 ? 16 : 8;
  auto swz_b = [](int k) { return kF4 ? kn4_swz<Cfg::BN>(k) : kn_swz<Cfg::BN>(k); };
  // ring slots reachable from one base register through the 16-bit offset field
  // (KN: the B reads add up to 104 K-rows of BN bytes)
  constexpr int kMaxFrag0 = ((FM > FN ? FM : FN) - 1) * 32 * kRowB;
  constexpr int kMaxFrag = KN && 104 * Cfg::BN > kMaxFrag0 ? 104 * Cfg::BN : kMaxFrag0;
  constexpr int kPerBase = (NS >= 4 && 3 * kTile + kMaxFrag < 65536) ? 4
                           : (NS >= 2 && kTile + kMaxFrag < 65536) ? 2 : 1;
  constexpr int kBases = NS / kPerBase;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const int h = lane >> 5;
  const int nk = op.K / kRowB;                     // K tiles
  const int nblk = op.K / kBlkBytes;
  const int ncode = nblk / 16;                     // 16-byte code groups per row
  constexpr int kGroupTiles = 16 * kBlkBytes / kRowB;   // K tiles per code group (4, FP4 2)
  constexpr int kCodes = 1;                        // code reads per fragment and step
  // B code registers per fragment and step: row-major FP4 B keeps its two codes
  // (rows BN bytes apart) in two registers, each the MFMA's byte 0, rather than
  // joining them into one with a VALU op that would wait on both reads
  constexpr bool kCodePair = KN && kF4;
  constexpr int kCodesB = kCodePair ? 2 : 1;

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

  // ---- copy side ----
  // copy instruction g of a K tile covers rows 8g .. 8g+7 of [A; B]: lane -> row
  // (lane >> 3) of the block, LDS chunk lane & 7, global chunk (lane & 7) ^
  // ((row >> 1) & 7); the swizzle of even and odd blocks differs
  const int g0 = wave * kLoads;                   // first block of this wave
  // valid rows (KN: B columns) of the tile: copies of rows past the edge of A
  // (and of a K-contiguous B) read zero, so tiles cut by M or N run here too
  const int a_tile = op.a_rows < Cfg::BM ? op.a_rows : Cfg::BM;
  const int b_tile = op.b_rows < Cfg::BN ? op.b_rows : Cfg::BN;
  const uint32_t nrA = (uint32_t)((a_tile - 1) * op.lda + op.K);
  const uint32_t nrB = KN ? (uint32_t)((op.K / kRowB * kKTileRows - 1) * op.ldb +
                                       (kF4 ? (b_tile + 1) / 2 : b_tile))
                          : (uint32_t)((b_tile - 1) * op.ldb + op.K);
  const __amdgpu_buffer_rsrc_t rsA = buffer_rsrc(op.A, nrA);
  const __amdgpu_buffer_rsrc_t rsB = buffer_rsrc(op.B, nrB);
  // KN: the copies go out untracked (see buffer_dma16_untracked)
  const v4u_rs wsA = buffer_rsrc_words(op.A, nrA), wsB = buffer_rsrc_words(op.B, nrB);
  const int lda = (int)op.lda, ldb = (int)op.ldb;
  const int crow = lane >> 3;
  const int sw0 = 16 * ((lane & 7) ^ ((crow >> 1) & 7));
  const int sw1 = 16 * ((lane & 7) ^ (((crow + 8) >> 1) & 7));
  // per-instruction lane offsets (loop invariant); KN: B instruction g covers
  // K-rows kKRows (g - nA) .. + kKRows - 1 (that first K-row goes in the scalar
  // offset), lane -> K-row lane / kChunks, LDS chunk lane % kChunks, global chunk
  // (lane % kChunks) ^ kn_swz(K-row); kn_swz has period 8 in the K-row and every
  // wave's first B instruction starts at a multiple of 8 K-rows, so at most two
  // distinct lane offsets remain
  static_assert(!KN || ((kLoads * kKRows) % kSwzPeriod == 0 && (nA * kKRows) % kSwzPeriod == 0),
                "B copy blocks start on the swizzle period");
  int voff[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const bool isA = g0 + j < nA;
    if (KN && !isA) {
      const int kr = lane / kChunks;
      voff[j] = kr * ldb + 16 * ((lane % kChunks) ^ swz_b(((j * kKRows) & (kSwzPeriod - 1)) + kr));
    } else {
      voff[j] = crow * (isA ? lda : ldb) + ((j & 1) ? sw1 : sw0);
    }
  }
  uint8_t* const cdst = lds + g0 * 1024;
  const uint32_t lds_base = KN ? lds_address(lds) : 0u;
  const uint32_t ncA = (uint32_t)((a_tile - 1) * op.sld + nblk);
  const uint32_t ncB = KN ? (uint32_t)((nblk - 1) * op.sldb + b_tile)
                          : (uint32_t)((b_tile - 1) * op.sld + nblk);
  const __amdgpu_buffer_rsrc_t rcA = buffer_rsrc(op.sa, ncA);
  const __amdgpu_buffer_rsrc_t rcB = buffer_rsrc(op.sb, ncB);
  const v4u_rs wcA = buffer_rsrc_words(op.sa, ncA), wcB = buffer_rsrc_words(op.sb, ncB);
  const int cvoff = lane * op.sld;
  // KN: each wave copies rows of one operand (kUniformOperand), so its
  // descriptor, lane offsets and the linear scalar offset of a copy, soff =
  // g * t_row + kt * t_kt + t_base for copy block g of K tile kt, are set once.
  static_assert(!KN || kUniformOperand, "KN: a wave copies rows of one operand");
  const bool wave_a = g0 < nA;
  const v4u_rs ws_t = wave_a ? wsA : wsB;
  const int t_row = wave_a ? 8 * lda : kKRows * ldb;
  const int t_kt = wave_a ? kRowB : kKTileRows * ldb;
  const int t_base = wave_a ? 0 : -nA * kKRows * ldb;
  // KN, MX: B code copy jj covers code rows (32-K blocks) kCRows li .. + kCRows - 1
  // of the group, lane -> block lane / kCChunks, 16 columns at 16 (lane % kCChunks);
  // A code copies as in the K-contiguous layout.  soff = grp * c_grp + c_base.
  int cv[kCodeLoads], c_grp[kCodeLoads], c_base[kCodeLoads];
  v4u_rs wc[kCodeLoads];
#pragma unroll
  for (int jj = 0; jj < kCodeLoads; ++jj) {
    int ci = wave * kCodeLoads + jj;
    ci = ci < kCodeInsts ? ci : kCodeInsts - 1;
    const bool code_a = ci < Cfg::BM / 64;
    const int li = code_a ? ci : ci - Cfg::BM / 64;
    cv[jj] = code_a ? lane * op.sld
                    : (li * kCRows + lane / kCChunks) * op.sldb + 16 * (lane % kCChunks);
    c_grp[jj] = code_a ? 16 : 16 * op.sldb;
    c_base[jj] = code_a ? li * 64 * op.sld : 0;
    wc[jj] = code_a ? wcA : wcB;
  }

  auto tile_copy = [&](int j, int slot, int kt) {       // j-th copy of K tile kt
    const int g = g0 + j;                               // wave-uniform
    const bool isA = kUniformOperand ? g0 < nA : g < nA;
    if constexpr (KN) {
      const int soff = g * scalar_fresh(t_row) + kt * scalar_fresh(t_kt) + t_base;
      buffer_dma16_untracked(ws_t, lds_base, (uint32_t)(g * 1024 + slot * kTile), voff[j], soff);
    } else {
      const int soff = isA ? g * 8 * lda + kt * kRowB : (g - nA) * 8 * ldb + kt * kRowB;
      buffer_dma16(isA ? rsA : rsB, cdst + slot * kTile + j * 1024, voff[j], soff);
    }
  };
  auto code_copy = [&](int jj, int buf, int grp) {      // jj-th code copy of group grp
    int ci = wave * kCodeLoads + jj;
    ci = ci < kCodeInsts ? ci : kCodeInsts - 1;
    const bool isA = ci < Cfg::BM / 64;
    const int li = isA ? ci : ci - Cfg::BM / 64;
    if constexpr (KN) {
      buffer_dma16_untracked(wc[jj], lds_base, (uint32_t)(kCodeOff + buf * kCodeBuf + ci * 1024),
                             cv[jj], grp * scalar_fresh(c_grp[jj]) + c_base[jj]);
    } else {
      buffer_dma16(isA ? rcA : rcB, lds + kCodeOff + buf * kCodeBuf + ci * 1024, cvoff,
                   li * 64 * op.sld + 16 * grp);
    }
  };

  // ---- read side: per-lane LDS bases, constant offsets ----
  // fragment row r = wave base + 32 i + lane % 32; logical chunk 4p + 2c + h
  // (K half p, chunk pair c; FP4 4p + 2h + c) sits at (chunk) ^ ((r >> 1) & 7)
  const int rsw = ((lane & 31) >> 1) & 7;
  const int ra = (wm * Cfg::WM + (lane & 31)) * kRowB;
  const int rb = (Cfg::BM + wn * Cfg::WN + (lane & 31)) * kRowB;
  int ba[kBases][2][2], bb[kBases][2][2];              // [base][half][chunk pair]
#pragma unroll
  for (int s = 0; s < kBases; ++s)
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int ch = 16 * ((kF4 ? 4 * p + 2 * h + c : 4 * p + 2 * c + h) ^ rsw);
        ba[s][p][c] = opaque(s * kPerBase * kTile + ra + ch);
        if (!KN) bb[s][p][c] = opaque(s * kPerBase * kTile + rb + ch);
      }
  // KN: lane (16-lane group G, position w) addresses K-row kb + w / 2 at columns
  // 32 j + 16 G + 8 (w % 2) of fragment j: chunk 2 j' + G, j' = this wave's
  // fragment column / 32, at (2 j' + G) ^ kn_swz(w / 2) (kb % 8 == 0 leaves the
  // swizzle to the lane); base per fragment, K offsets in the offset field
  // (FP4: lane (G, w) addresses K-row 64 h + w of the step's 128 at 8-byte half G
  // of the fragment's chunk j' = this wave's fragment column / 32, which sits at
  // j' ^ kn4_swz(w); the four reads of a fragment start 16 K-rows apart)
  int bk[kBases][KN ? FN : 1];
  if constexpr (KN && kF4) {
    const int w = lane & 15, G = (lane >> 4) & 1;
    const int swz = kn4_swz<Cfg::BN>(w);
#pragma unroll
    for (int s = 0; s < kBases; ++s)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int c1 = (wn * Cfg::WN + 32 * j) / 32;
        bk[s][j] = opaque(s * kPerBase * kTile + Cfg::BM * kRowB + (64 * h + w) * kBRowB +
                          16 * (c1 ^ swz) + 8 * G);
      }
  } else if constexpr (KN) {
    const int w = lane & 15, G = (lane >> 4) & 1;
    const int swz = kn_swz<Cfg::BN>(w >> 1);
#pragma unroll
    for (int s = 0; s < kBases; ++s)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int c2 = (wn * Cfg::WN + 32 * j) / 16;      // even
        bk[s][j] = opaque(s * kPerBase * kTile + Cfg::BM * kRowB + (16 * h + (w >> 1)) * Cfg::BN +
                          16 * ((c2 ^ swz) + G) + 8 * (w & 1));
      }
  }
  // MX codes: byte 4 (u % 4) + 2 p + h of the row's 16-byte group u / 4 (FP4:
  // bytes 8 (u % 2) + 4 p + 2 h + c of group u / 2, c = the step's MFMA); the
  // group of the current K tile is in buffer `cur`, the next one in `nxt`
  int cur_a = 0, cur_b = 0, nxt_a = 0, nxt_b = 0;
  int cbuf = 0;                                        // buffer index of the current group
  if (kMx) {
    cur_a = opaque(kCodeOff + (wm * Cfg::WM + (lane & 31)) * 16 + (kF4 ? 2 * h : h));
    cur_b = KN ? opaque(kCodeOff + Cfg::BM * 16 + (kF4 ? 2 * h : h) * Cfg::BN + wn * Cfg::WN +
                        (lane & 31))
               : opaque(kCodeOff + (Cfg::BM + wn * Cfg::WN + (lane & 31)) * 16 + (kF4 ? 2 * h : h));
    nxt_a = opaque(cur_a + kCodeBuf);
    nxt_b = opaque(cur_b + kCodeBuf);
  }

  auto rd16 = [&](int addr) { return *reinterpret_cast<const v4i*>(lds + addr); };
  auto rdtr = [&](int addr) {
    auto* a = reinterpret_cast<__attribute__((address_space(3))) v2i*>(
        (__attribute__((address_space(3))) uint8_t*)(lds + addr));
    if constexpr (kF4) return __builtin_amdgcn_ds_read_tr4_b64_v2i32(a);
    else return __builtin_amdgcn_ds_read_tr8_b64_v2i32(a);
  };
  // a step's LDS reads: 16-byte reads of A (and of B), KN: four 8-byte
  // transposing reads per B fragment
  constexpr int kReadsA = 2 * FM, kReadsB = (KN ? 4 : 2) * FN;
  struct Reads {
    v4i rd[kReadsA + (KN ? 0 : kReadsB)];
    v2i rt[KN ? kReadsB : 1];
  };
  // the d-th read of a step's fragments (ring slot s, half p)
  auto read_frag = [&](auto s_c, auto p_c, int d, Reads& r) {
    constexpr int s = decltype(s_c)::value, p = decltype(p_c)::value;
    constexpr int b = s / kPerBase, o = (s % kPerBase) * kTile;
    const int c = d & 1;
    if (d < kReadsA) {
      r.rd[d] = rd16(ba[b][p][c] + o + (d >> 1) * 32 * kRowB);
    } else if constexpr (KN && kF4) {
      const int e = d - kReadsA, q = e & 3;
      r.rt[e] = rdtr(bk[b][e >> 2] + o + (128 * p + 16 * q) * kBRowB);
    } else if constexpr (KN) {
      const int e = d - kReadsA, q = e & 3;
      r.rt[e] = rdtr(bk[b][e >> 2] + o + (64 * p + 32 * (q >> 1) + 8 * (q & 1)) * Cfg::BN);
    } else {
      r.rd[d] = rd16(bb[b][p][c] + o + ((d - kReadsA) >> 1) * 32 * kRowB);
    }
  };
  // fragments from a step's reads
  auto frags = [&](const Reads& r, v8i (&fa)[FM], v8i (&fb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[i] = __builtin_shufflevector(r.rd[2 * i], r.rd[2 * i + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if constexpr (KN) {
        const v4i lo = __builtin_shufflevector(r.rt[4 * j], r.rt[4 * j + 1], 0, 1, 2, 3);
        const v4i hi = __builtin_shufflevector(r.rt[4 * j + 2], r.rt[4 * j + 3], 0, 1, 2, 3);
        fb[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      } else {
        fb[j] = __builtin_shufflevector(r.rd[kReadsA + 2 * j], r.rd[kReadsA + 2 * j + 1], 0, 1, 2,
                                        3, 4, 5, 6, 7);
      }
    }
  };
  uint32_t ca[2][kCodes][FM], cb[2][kCodesB][FN];     // codes: [register set][MFMA][fragment]
#pragma unroll
  for (int z = 0; z < 2; ++z)
#pragma unroll
    for (int c = 0; c < kCodesB; ++c) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        if (c < kCodes) ca[z][c][i] = 0;
#pragma unroll
      for (int j = 0; j < FN; ++j) cb[z][c][j] = 0;
    }
  // the e-th code byte read of a step: K tile u with u % kGroupTiles == q, half p
  auto read_code = [&](int base_a, int base_b, int q, int p, int e,
                       uint32_t (&a)[kCodes][FM], uint32_t (&b)[kCodesB][FN]) {
    const int c = e / (FM + FN), f = e % (FM + FN);
    if constexpr (kF4) {           // the two adjacent code bytes of the step's MFMAs
      const int off = 8 * q + 4 * p;
      if (f < FM) a[c][f] = *reinterpret_cast<const uint16_t*>(lds + base_a + off + f * 32 * 16);
      else if (KN) {               // code rows of B: blocks off + 2 h and + 1 at one column
        b[0][f - FM] = lds[base_b + off * Cfg::BN + (f - FM) * 32];
        b[kCodesB - 1][f - FM] = lds[base_b + (off + 1) * Cfg::BN + (f - FM) * 32];
      }
      else b[c][f - FM] = *reinterpret_cast<const uint16_t*>(lds + base_b + off + (f - FM) * 32 * 16);
    } else {
      const int off = 4 * q + 2 * p;
      if (f < FM) a[c][f] = lds[base_a + off + f * 32 * 16];
      else if (KN) b[c][f - FM] = lds[base_b + off * Cfg::BN + (f - FM) * 32];
      else b[c][f - FM] = lds[base_b + off + (f - FM) * 32 * 16];
    }
  };

  v8i af0[FM], bf0[FN], af1[FM], bf1[FN];

  // ---- prologue: K tiles 0 .. NS-1 (and code group 0) in flight; wait for tile 0 ----
  if (MODE == kRowwise) {
    dword_rows_ab<Cfg>(reinterpret_cast<const uint8_t*>(op.ra), 4, op.a_rows,
                       reinterpret_cast<const uint8_t*>(op.rb), 4, op.b_rows, 0,
                       lds + Cfg::kRowScaleOff, wave, lane);
  }
#pragma unroll
  for (int j = 0; j < kLoads; ++j) tile_copy(j, 0, 0);
  if (kMx) {
#pragma unroll
    for (int jj = 0; jj < kCodeLoads; ++jj) code_copy(jj, 0, 0);
  }
#pragma unroll
  for (int s = 1; s < NS; ++s) {
    const int ks = s < nk ? s : nk - 1;               // short K: harmless re-fetch
#pragma unroll
    for (int j = 0; j < kLoads; ++j) tile_copy(j, s, ks);
  }
  FP8GEMM_WAIT_VM_LGKM0((NS - 1) * kLoads);
  __builtin_amdgcn_s_barrier();
  {
    Reads r0;
#pragma unroll
    for (int d = 0; d < kReadsA + kReadsB; ++d)
      read_frag(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, d, r0);
    frags(r0, af0, bf0);
    if (kMx) {
#pragma unroll
      for (int e = 0; e < kCodes * (FM + FN); ++e) read_code(cur_a, cur_b, 0, 0, e, ca[0], cb[0]);
    }
  }

  // ---- one 64-K step t: K tile u = t / 2, half p; T = t mod (unrolled steps) ----
  constexpr int kMfma = FM * FN;
  constexpr int kReads = kReadsA + kReadsB;
  constexpr int kReadSpan = (kMfma * FP8GEMM_READ_SPAN + 7) / 8 > 0 ? (kMfma * FP8GEMM_READ_SPAN + 7) / 8 : 1;
  constexpr int kCopySpan = (kMfma * FP8GEMM_COPY_SPAN + 7) / 8 > 0 ? (kMfma * FP8GEMM_COPY_SPAN + 7) / 8 : 1;
  auto step = [&](int t, auto T_c, v8i (&fa)[FM], v8i (&fb)[FN], v8i (&na)[FM], v8i (&nb)[FN]) {
    constexpr int T = decltype(T_c)::value;
    constexpr int p = T & 1, ku = T >> 1;        // half, K tile within the unrolled body
    constexpr int q = ku % kGroupTiles, slot = ku % NS;
    constexpr int Z = T & 1;                     // code register set used by this step
    // what step t + 1 reads: same K tile, other half; or the next K tile
    constexpr int np = p ^ 1, nslot = p ? (ku + 1) % NS : slot;
    constexpr int nq = p ? (q + 1) % kGroupTiles : q;
    constexpr bool kCodeStep = kMx && p == 1 && q == 0;   // code group copy rides along
    constexpr int kVmem = p ? kLoads + (kCodeStep ? kCodeLoads : 0) : 0;
    constexpr int kDs = kReads + (kMx ? kCodes * (FM + FN) : 0);
    // code bytes of step t + 1 live in the group of K tile (t + 1) / 2
    constexpr bool kNextGroup = p && q == kGroupTiles - 1;
    // copies allowed in flight once K tile u + 1 has landed: those of K tiles
    // u + 2 .. u + NS - 1 and a code group issued after K tile u + 1's copies.
    // On the last K tile of a group this step also reads the next group, whose
    // copy went out in K tile u - q right after that tile's copies of K tile
    // u - q + NS: then only the tile copies of the q - 1 K tiles since may remain.
    constexpr int kAfterTile = (NS - 2) * kLoads + ((kMx && q >= 1 && q + 1 <= NS) ? kCodeLoads : 0);
    constexpr int kAfterCode = (q - 1) * kLoads;
    constexpr int kWaitOdd =
        (kNextGroup && kAfterCode < kAfterTile) ? kAfterCode : kAfterTile;
    const int u = t >> 1;
    __builtin_amdgcn_sched_barrier(0);
    if (p) {
      // copies of K tile u + 1 landed for every wave; slot of K tile u free (its
      // last fragments were read in the previous step)
      FP8GEMM_WAIT_VM_LGKM0(kWaitOdd);
      __builtin_amdgcn_s_barrier();
    } else {
      __builtin_amdgcn_s_waitcnt(0xc07f);        // lgkmcnt(0): fragments in registers
    }
    __builtin_amdgcn_sched_barrier(0);
    const int kc = (u + NS) < nk ? u + NS : nk - 1;  // past the end: harmless re-fetch
    const int grp = u / kGroupTiles + 1 < ncode ? u / kGroupTiles + 1 : ncode - 1;
    Reads rd;
#pragma unroll
    for (int m = 0; m < kMfma; ++m) {
      const int i = m / FN, j = m % FN;
      if (kF4) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            lo16(fb[j]), lo16(fa[i]), acc[i][j], kFmtB, kFmtA, 0, (int)cb[Z][0][j], 0,
            (int)ca[Z][0][i]);
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            hi16(fb[j]), hi16(fa[i]), acc[i][j], kFmtB, kFmtA, kCodePair ? 0 : 1,
            (int)cb[Z][kCodesB - 1][j], 1,
            (int)ca[Z][0][i]);
      } else if (kMx) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fb[j], fa[i], acc[i][j], kFmtB, kFmtA, 0, (int)cb[Z][0][j], 0, (int)ca[Z][0][i]);
      } else {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], kFmtB,
                                                                    kFmtA, 0, 0, 0, 0);
      }
      if (m < kCopySpan) {
#pragma unroll
        for (int v = m * kVmem / kCopySpan; v < (m + 1) * kVmem / kCopySpan; ++v) {
          if (v < kLoads) tile_copy(v, slot, kc);
          else if (kCodeStep) code_copy(v - kLoads, cbuf ^ 1, grp);
        }
      }
      if (m < kReadSpan) {
#pragma unroll
        for (int d = m * kDs / kReadSpan; d < (m + 1) * kDs / kReadSpan; ++d) {
          if (d < kReads) {
            read_frag(std::integral_constant<int, nslot>{}, std::integral_constant<int, np>{}, d,
                      rd);
          } else if (kMx) {
            read_code(kNextGroup ? nxt_a : cur_a, kNextGroup ? nxt_b : cur_b, nq, np, d - kReads,
                      ca[Z ^ 1], cb[Z ^ 1]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    frags(rd, na, nb);
    if (kMx && kNextGroup) {                      // the next group is current from step t + 1
      cbuf ^= 1;
      const int ta = cur_a, tb = cur_b;
      cur_a = nxt_a;
      cur_b = nxt_b;
      nxt_a = ta;
      nxt_b = tb;
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  using I6 = std::integral_constant<int, 6>;
  using I7 = std::integral_constant<int, 7>;

  // unrolled over 4 K tiles (4-deep ring), an MX code group (4 K tiles, FP4 2)
  // or the 2-deep ring
  constexpr int kUnrollK = NS >= 4 ? NS : kMx ? kGroupTiles * (kF4 ? FP8GEMM_F4_UNROLL : 1) : 2;
  static_assert(!kMx || kUnrollK % kGroupTiles == 0, "whole code groups per unrolled body");
  static_assert(kUnrollK == 2 || kUnrollK == 4 || kUnrollK == 8, "2, 4 or 8 K tiles per body");
  int u = 0;
  if constexpr (kUnrollK == 8) {
    // the eight-deep ring: sixteen steps per body, then whole K tiles (MX: whole
    // code groups) one by one
    for (; u + kUnrollK <= nk; u += kUnrollK) {
      const int t = 2 * u;
      Unroll<0, kUnrollK>::run([&](auto k_c) __attribute__((always_inline)) {
        constexpr int k = decltype(k_c)::value;
        step(t + 2 * k, std::integral_constant<int, 2 * k>{}, af0, bf0, af1, bf1);
        step(t + 2 * k + 1, std::integral_constant<int, 2 * k + 1>{}, af1, bf1, af0, bf0);
      });
    }
    const int t = 2 * u;
    constexpr int kG = kMx ? kGroupTiles : 1;
    Unroll<0, kUnrollK / kG - 1>::run([&](auto g_c) __attribute__((always_inline)) {
      constexpr int g = decltype(g_c)::value;
      if (u + g * kG < nk) {
        Unroll<g * kG, (g + 1) * kG>::run([&](auto k_c) __attribute__((always_inline)) {
          constexpr int k = decltype(k_c)::value;
          step(t + 2 * k, std::integral_constant<int, 2 * k>{}, af0, bf0, af1, bf1);
          step(t + 2 * k + 1, std::integral_constant<int, 2 * k + 1>{}, af1, bf1, af0, bf0);
        });
      }
    });
  } else {
  for (; u + kUnrollK <= nk; u += kUnrollK) {
    const int t = 2 * u;
    step(t, I0{}, af0, bf0, af1, bf1);
    step(t + 1, I1{}, af1, bf1, af0, bf0);
    step(t + 2, I2{}, af0, bf0, af1, bf1);
    step(t + 3, I3{}, af1, bf1, af0, bf0);
    if constexpr (kUnrollK == 4) {
      step(t + 4, I4{}, af0, bf0, af1, bf1);
      step(t + 5, I5{}, af1, bf1, af0, bf0);
      step(t + 6, I6{}, af0, bf0, af1, bf1);
      step(t + 7, I7{}, af1, bf1, af0, bf0);
    }
  }
  // remaining K tiles: for MX one code group (FP4 with two groups per body);
  // otherwise any K tiles left
  if constexpr (kMx && kUnrollK > kGroupTiles) {
    static_assert(2 * kGroupTiles == kUnrollK, "one group left at most");
    const int t = 2 * u;
    if (u < nk) {
      step(t, I0{}, af0, bf0, af1, bf1);
      step(t + 1, I1{}, af1, bf1, af0, bf0);
      step(t + 2, I2{}, af0, bf0, af1, bf1);
      step(t + 3, I3{}, af1, bf1, af0, bf0);
    }
  }
  if constexpr (!kMx) {
    const int t = 2 * u;
    if (u < nk) {
      step(t, I0{}, af0, bf0, af1, bf1);
      step(t + 1, I1{}, af1, bf1, af0, bf0);
    }
    if constexpr (kUnrollK == 4) {
      if (u + 1 < nk) {
        step(t + 2, I2{}, af0, bf0, af1, bf1);
        step(t + 3, I3{}, af1, bf1, af0, bf0);
      }
      if (u + 2 < nk) {
        step(t + 4, I4{}, af0, bf0, af1, bf1);
        step(t + 5, I5{}, af1, bf1, af0, bf0);
      }
    }
  }
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0);     // no copy may still target LDS
  __builtin_amdgcn_s_barrier();      // every wave is done with the ring
}

// ---------------------------------------------------------------------------
// A run of interior tiles as one copy stream (persistent kernels).  Tiles
// first .. last-1 of a workgroup's list (src.op(i)) share lda, ldb and K; their
// 128-K tiles are consumed back to back, so the copies of the next tile's first
// K tiles (and its first MX code group) go out while the current tile's last K
// tiles are consumed, and the register fragments of its first step are read
// during the current tile's last step.  Each tile's epilogue (epi(acc, i, buf),
// buf = row-scale buffer) then runs while those copies are in flight, instead of
// a new workgroup starting cold.  Row-wise scales of tile i are copied into LDS
// buffer i % 2 during its K loop.
// Conditions: every tile interior (interior_tile), K % 512 == 0.
// ---------------------------------------------------------------------------
template <class Cfg, int MODE, int kEpiStores, class Src, class Epi>
__device__ __forceinline__ void stream_interior(const Src& src, int first, int last,
                                                uint8_t* lds, Epi&& epi) {
  static constexpr int NS = 2;
  static_assert(!kF4, "FP4 GEMMs run one tile per workgroup");
  static constexpr int FM = Cfg::kFragM, FN = Cfg::kFragN;
  static constexpr bool kMx = MODE == kMx32;
  static constexpr bool kRow = MODE == kRowwise;
  static constexpr int kRowB = 128;
  static constexpr int kTile = (Cfg::BM + Cfg::BN) * kRowB;
  static constexpr int nA = Cfg::BM / 8;
  static constexpr int kLoads = kTile / 1024 / Cfg::kWaves;
  static constexpr int kCodeInsts = (Cfg::BM + Cfg::BN) / 64;           // also row-scale copies
  static constexpr int kCodeLoads = (kCodeInsts + Cfg::kWaves - 1) / Cfg::kWaves;
  static constexpr int kCodeBuf = (Cfg::BM + Cfg::BN) * 16;
  static constexpr int kCodeOff = NS * kTile;
  static constexpr int kRowScaleBuf = (Cfg::BM + Cfg::BN) * 4;
  static constexpr bool kUniformOperand = nA % kLoads == 0;
  static constexpr bool kSide = kMx || kRow;                              // side copies every 512 K
  static constexpr int kSideLoads = kSide ? kCodeLoads : 0;
  static_assert(NS * kTile <= Cfg::kScaleOff, "ring fits");
  static_assert(kCodeOff + 2 * kCodeBuf <= Cfg::kLdsBytes, "code buffers fit");
  static_assert(Cfg::kRowScaleOff + 2 * kRowScaleBuf <= Cfg::kLdsBytes, "row-scale buffers fit");
  static_assert(kTile % (1024 * Cfg::kWaves) == 0, "equal copy share per wave");
  static_assert(kLoads % 2 == 0, "copy blocks of both swizzle phases per wave");
  static constexpr int kMaxFrag = ((FM > FN ? FM : FN) - 1) * 32 * kRowB;
  static constexpr int kPerBase = (kTile + kMaxFrag < 65536) ? 2 : 1;
  static constexpr int kBases = NS / kPerBase;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const int h = lane >> 5;
  const TileOperands op0 = src.op(first);
  const int nk = op0.K / kRowB;                    // K tiles per output tile (% 4 == 0)
  const int nblk = op0.K / 32;
  const int ncode = nblk / 16;
  const int lda = (int)op0.lda, ldb = (int)op0.ldb, sld = op0.sld;

  // base addresses of a tile's A rows, B rows, A codes / row scales and B codes /
  // column scales (scalar values; buffer descriptors are formed where used).
  // Everything below passes them as separate scalars: a struct argument to the
  // helper lambdas kept whole frames in scratch memory.
  auto side_a = [](const TileOperands& op) __attribute__((always_inline)) {
    return kMx ? static_cast<const void*>(op.sa) : static_cast<const void*>(op.ra);
  };
  auto side_b = [](const TileOperands& op) __attribute__((always_inline)) {
    return kMx ? static_cast<const void*>(op.sb) : static_cast<const void*>(op.rb);
  };
  const uint32_t bytes_a = (uint32_t)((Cfg::BM - 1) * op0.lda + op0.K);
  const uint32_t bytes_b = (uint32_t)((Cfg::BN - 1) * op0.ldb + op0.K);
  const uint32_t bytes_sa = kMx ? (uint32_t)((Cfg::BM - 1) * op0.sld + nblk) : Cfg::BM * 4;
  const uint32_t bytes_sb = kMx ? (uint32_t)((Cfg::BN - 1) * op0.sld + nblk) : Cfg::BN * 4;

  // ---- copy side ----
  const int g0 = wave * kLoads;
  const int crow = lane >> 3;
  const int sw0 = 16 * ((lane & 7) ^ ((crow >> 1) & 7));
  const int sw1 = 16 * ((lane & 7) ^ (((crow + 8) >> 1) & 7));
  int voff[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const bool isA = g0 + j < nA;
    voff[j] = crow * (isA ? lda : ldb) + ((j & 1) ? sw1 : sw0);
  }
  uint8_t* const cdst = lds + g0 * 1024;
  const int cvoff = kMx ? lane * sld : lane * 4;

  // (selects below are on values: a select between two members of one object
  // would select addresses and force the object into scratch memory)
  auto tile_copy = [&](const void* pa, const void* pb, int j, int slot, int kt)
                       __attribute__((always_inline)) {
    const int g = g0 + j;
    const bool isA = kUniformOperand ? (g0 < nA) : (g < nA);
    buffer_dma16(buffer_rsrc(isA ? pa : pb, isA ? bytes_a : bytes_b),
                 cdst + slot * kTile + j * 1024, voff[j],
                 (isA ? g : g - nA) * 8 * (isA ? lda : ldb) + kt * kRowB);
  };
  // jj-th side copy: MX code group grp into code buffer buf, or row scales into
  // row-scale buffer buf
  auto side_copy = [&](const void* psa, const void* psb, int jj, int buf, int grp)
                       __attribute__((always_inline)) {
    int ci = wave * kCodeLoads + jj;
    ci = ci < kCodeInsts ? ci : kCodeInsts - 1;
    const bool isA = ci < Cfg::BM / 64;
    const int li = isA ? ci : ci - Cfg::BM / 64;
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(isA ? psa : psb, isA ? bytes_sa : bytes_sb);
    if (kMx) {
      buffer_dma16(rs, lds + kCodeOff + buf * kCodeBuf + ci * 1024, cvoff,
                   li * 64 * sld + 16 * grp);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs,
          (__attribute__((address_space(3))) void*)(lds + Cfg::kRowScaleOff + buf * kRowScaleBuf +
                                                    ci * 256),
          4, cvoff, li * 64 * 4, 0, 0);
    }
  };

  // ---- read side ----
  const int rsw = ((lane & 31) >> 1) & 7;
  const int ra = (wm * Cfg::WM + (lane & 31)) * kRowB;
  const int rb = (Cfg::BM + wn * Cfg::WN + (lane & 31)) * kRowB;
  int ba[kBases][2][2], bb[kBases][2][2];
#pragma unroll
  for (int s = 0; s < kBases; ++s)
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int ch = 16 * ((4 * p + 2 * c + h) ^ rsw);
        ba[s][p][c] = opaque(s * kPerBase * kTile + ra + ch);
        bb[s][p][c] = opaque(s * kPerBase * kTile + rb + ch);
      }
  int cur_a = 0, cur_b = 0, nxt_a = 0, nxt_b = 0;
  int cbuf = 0;
  if (kMx) {
    cur_a = opaque(kCodeOff + (wm * Cfg::WM + (lane & 31)) * 16 + h);
    cur_b = opaque(kCodeOff + (Cfg::BM + wn * Cfg::WN + (lane & 31)) * 16 + h);
    nxt_a = opaque(cur_a + kCodeBuf);
    nxt_b = opaque(cur_b + kCodeBuf);
  }
  auto rd16 = [&](int addr) __attribute__((always_inline)) { return *reinterpret_cast<const v4i*>(lds + addr); };
  auto read_frag = [&](auto s_c, auto p_c, int d, v4i (&rd)[2 * (FM + FN)]) __attribute__((always_inline)) {
    constexpr int s = decltype(s_c)::value, p = decltype(p_c)::value;
    constexpr int b = s / kPerBase, o = (s % kPerBase) * kTile;
    const int c = d & 1;
    if (d < 2 * FM) rd[d] = rd16(ba[b][p][c] + o + (d >> 1) * 32 * kRowB);
    else rd[d] = rd16(bb[b][p][c] + o + ((d - 2 * FM) >> 1) * 32 * kRowB);
  };
  uint32_t ca[2][FM], cb[2][FN];
#pragma unroll
  for (int z = 0; z < 2; ++z) {
#pragma unroll
    for (int i = 0; i < FM; ++i) ca[z][i] = 0;
#pragma unroll
    for (int j = 0; j < FN; ++j) cb[z][j] = 0;
  }
  auto read_code = [&](int base_a, int base_b, int q, int p, int e, uint32_t (&a)[FM],
                       uint32_t (&b)[FN]) __attribute__((always_inline)) {
    const int off = 4 * q + 2 * p;
    if (e < FM) a[e] = lds[base_a + off + e * 32 * 16];
    else b[e - FM] = lds[base_b + off + (e - FM) * 32 * 16];
  };

  v8i af0[FM], bf0[FN], af1[FM], bf1[FN];
  v16f acc[FM][FN];

  // ---- stream prologue: K tiles 0, 1 of the first tile (and its code group 0) ----
  // current (c) and next (n) tile of the stream
  const void *ca_ = op0.A, *cb_ = op0.B, *csa = side_a(op0), *csb = side_b(op0);
  const void *na_ = ca_, *nb_ = cb_, *nsa = csa, *nsb = csb;
  if (first + 1 < last) {
    const TileOperands o1 = src.op(first + 1);
    na_ = o1.A;
    nb_ = o1.B;
    nsa = side_a(o1);
    nsb = side_b(o1);
  }
#pragma unroll
  for (int j = 0; j < kLoads; ++j) tile_copy(ca_, cb_, j, 0, 0);
  if (kMx) {
#pragma unroll
    for (int jj = 0; jj < kCodeLoads; ++jj) side_copy(csa, csb, jj, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < kLoads; ++j) tile_copy(ca_, cb_, j, 1, 1);
  FP8GEMM_WAIT_VM_LGKM0(kLoads);
  __builtin_amdgcn_s_barrier();
  {
    v4i rd[2 * (FM + FN)];
#pragma unroll
    for (int d = 0; d < 2 * (FM + FN); ++d)
      read_frag(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, d, rd);
#pragma unroll
    for (int i = 0; i < FM; ++i) af0[i] = __builtin_shufflevector(rd[2 * i], rd[2 * i + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      bf0[j] = __builtin_shufflevector(rd[2 * FM + 2 * j], rd[2 * FM + 2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
    if (kMx) {
#pragma unroll
      for (int e = 0; e < FM + FN; ++e) read_code(cur_a, cur_b, 0, 0, e, ca[0], cb[0]);
    }
  }

  static constexpr int kMfma = FM * FN;
  static constexpr int kReads = 2 * (FM + FN);
  static constexpr int kReadSpan = (kMfma * FP8GEMM_READ_SPAN + 7) / 8 > 0 ? (kMfma * FP8GEMM_READ_SPAN + 7) / 8 : 1;
  static constexpr int kCopySpan = (kMfma * FP8GEMM_COPY_SPAN + 7) / 8 > 0 ? (kMfma * FP8GEMM_COPY_SPAN + 7) / 8 : 1;
  int rbuf = 0;                                    // row-scale buffer of the current tile
  bool has_next = first + 1 < last;
  bool fresh = true;                               // no epilogue stores in flight yet
  // one 64-K step of the current tile: K tile u = t / 2, T = t % 8
  auto step = [&](int t, auto T_c, v8i (&fa)[FM], v8i (&fb)[FN], v8i (&na)[FM], v8i (&nb)[FN]) __attribute__((always_inline)) {
    constexpr int T = decltype(T_c)::value;
    constexpr int p = T & 1, ku = T >> 1;
    constexpr int q = ku & 3, slot = ku % NS;
    constexpr int Z = T & 1;
    constexpr int np = p ^ 1, nslot = p ? (ku + 1) % NS : slot, nq = p ? (q + 1) & 3 : q;
    constexpr bool kSideStep = kSide && p == 1 && q == 0;
    constexpr int kVmem = p ? kLoads + (kSideStep ? kSideLoads : 0) : 0;
    constexpr int kDs = kReads + (kMx ? FM + FN : 0);
    // in flight once K tile u + 1 has landed: a side copy issued after it (q == 1)
    constexpr int kWaitOdd = (kSide && q == 1) ? kSideLoads : 0;
    const int u = t >> 1;
    __builtin_amdgcn_sched_barrier(0);
    if (p) {
      // first odd step after an epilogue: its C stores were issued after the
      // copies of this K tile and may stay in flight (vmcnt retires in order)
      if (T == 1 && u == 0 && !fresh) FP8GEMM_WAIT_VM_LGKM0(kWaitOdd + kEpiStores);
      else FP8GEMM_WAIT_VM_LGKM0(kWaitOdd);
      __builtin_amdgcn_s_barrier();
    } else {
      __builtin_amdgcn_s_waitcnt(0xc07f);
    }
    __builtin_amdgcn_sched_barrier(0);
    // copy target: K tile u + 2 of this tile, else of the next tile, else a
    // harmless re-fetch of this tile's last K tile
    const int k2 = u + NS;
    const bool to_next = k2 >= nk;
    const bool tn = to_next && has_next;
    const void* ta = tn ? na_ : ca_;
    const void* tb = tn ? nb_ : cb_;
    const int kt = to_next ? (has_next ? k2 - nk : nk - 1) : k2;
    const int g1 = (u >> 2) + 1;                   // MX code group of K tile u + 4
    const bool g_next = g1 >= ncode;
    const bool gn = g_next && has_next;
    const void* gsa = gn ? nsa : csa;
    const void* gsb = gn ? nsb : csb;
    const int grp = g_next ? (has_next ? 0 : ncode - 1) : g1;
    constexpr bool kNextGroup = p && q == 3;
    v4i rd[kReads];
#pragma unroll
    for (int m = 0; m < kMfma; ++m) {
      const int i = m / FN, j = m % FN;
      if (kMx) {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            fb[j], fa[i], acc[i][j], kFmtB, kFmtA, 0, (int)cb[Z][j], 0, (int)ca[Z][i]);
      } else {
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], kFmtB,
                                                                    kFmtA, 0, 0, 0, 0);
      }
      if (m < kCopySpan) {
#pragma unroll
        for (int v = m * kVmem / kCopySpan; v < (m + 1) * kVmem / kCopySpan; ++v) {
          if (v < kLoads) tile_copy(ta, tb, v, slot, kt);
          else if (kMx && kSideStep) side_copy(gsa, gsb, v - kLoads, cbuf ^ 1, grp);
          else if (kRow && kSideStep) side_copy(csa, csb, v - kLoads, rbuf, 0);
        }
      }
      if (m < kReadSpan) {
#pragma unroll
        for (int d = m * kDs / kReadSpan; d < (m + 1) * kDs / kReadSpan; ++d) {
          if (d < kReads) {
            read_frag(std::integral_constant<int, nslot>{}, std::integral_constant<int, np>{}, d,
                      rd);
          } else if (kMx) {
            read_code(kNextGroup ? nxt_a : cur_a, kNextGroup ? nxt_b : cur_b, nq, np, d - kReads,
                      ca[Z ^ 1], cb[Z ^ 1]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) na[i] = __builtin_shufflevector(rd[2 * i], rd[2 * i + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      nb[j] = __builtin_shufflevector(rd[2 * FM + 2 * j], rd[2 * FM + 2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
    if (kMx && kNextGroup) {
      cbuf ^= 1;
      const int ta = cur_a, tb = cur_b;
      cur_a = nxt_a;
      cur_b = nxt_b;
      nxt_a = ta;
      nxt_b = tb;
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  using I6 = std::integral_constant<int, 6>;
  using I7 = std::integral_constant<int, 7>;

  for (int tile = first; tile < last; ++tile) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};
    for (int u = 0; u < nk; u += 4) {
      const int t = 2 * u;
      step(t, I0{}, af0, bf0, af1, bf1);
      step(t + 1, I1{}, af1, bf1, af0, bf0);
      step(t + 2, I2{}, af0, bf0, af1, bf1);
      step(t + 3, I3{}, af1, bf1, af0, bf0);
      step(t + 4, I4{}, af0, bf0, af1, bf1);
      step(t + 5, I5{}, af1, bf1, af0, bf0);
      step(t + 6, I6{}, af0, bf0, af1, bf1);
      step(t + 7, I7{}, af1, bf1, af0, bf0);
    }
    __builtin_amdgcn_sched_barrier(0);
    epi(acc, tile, rbuf);
    __builtin_amdgcn_sched_barrier(0);
    fresh = false;
    // advance: the next tile becomes current
    rbuf ^= 1;
    if (has_next) {
      ca_ = na_;
      cb_ = nb_;
      csa = nsa;
      csb = nsb;
      has_next = tile + 2 < last;
      if (has_next) {
        const TileOperands o2 = src.op(tile + 2);
        na_ = o2.A;
        nb_ = o2.B;
        nsa = side_a(o2);
        nsb = side_b(o2);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0);     // no copy may still target LDS
  __builtin_amdgcn_s_barrier();      // every wave is done with the ring
}

// Scale, round and store a tile through LDS.  m0/n0: global coordinates of the
// tile origin; rows at or past m_end and columns at or past N are not stored.
// Output row m lives at C + m * ldc (ldc * sizeof(OutT) a multiple of 16 and C
// 16-byte aligned).  The LDS ring must be idle (mainloop() ends with a barrier);
// row-wise scales are read from the LDS copy mainloop() made.
// Fused epilogue operations after the scales: bias[n] added, then an activation
// (the Cutlass-named Triton FP8 post fuses a bias_add_relu epilogue to save the
// round trip of C; GELU, erf form, and SiLU are the other common choices).
// Activations of the fused epilogue in fp32, from the hardware reciprocal and
// exp2 (v_rcp_f32, v_exp_f32; about an ulp each):
//   GELU(v) = v Phi(v) = v (1 + erf(v / sqrt 2)) / 2, with erf(z), z >= 0, from
//     the rational approximation 7.1.26 of Abramowitz and Stegun's Handbook of
//     Mathematical Functions: erf(z) = 1 - t (a1 + t (a2 + ... + t a5)) e^(-z^2),
//     t = 1 / (1 + p z), |error| <= 1.5e-7.  With q = (1 - erf(|v| / sqrt 2)) / 2,
//     Phi(v) = 1 - q for v >= 0 and q for v < 0.
//   SiLU(v) = v / (1 + e^-v).
// About 16 and 5 vector instructions per value.
__device__ __forceinline__ float gelu_f32(float v) {
  // z = |v| / sqrt 2 folded into p (t = 1 / (1 + p |v| / sqrt 2)), the 1/2 of q
  // into a1 .. a5, and e^(-z^2) = 2^(-v^2 log2(e) / 2)
  constexpr double kP = 0.3275911, kA1 = 0.254829592, kA2 = -0.284496736;
  constexpr double kA3 = 1.421413741, kA4 = -1.453152027, kA5 = 1.061405429;
  constexpr float kPs = (float)(kP * 0.70710678118654752);
  constexpr float kB1 = (float)(kA1 / 2), kB2 = (float)(kA2 / 2), kB3 = (float)(kA3 / 2);
  constexpr float kB4 = (float)(kA4 / 2), kB5 = (float)(kA5 / 2);
  constexpr float kE = (float)(-0.5 * 1.4426950408889634);
  const float t = __builtin_amdgcn_rcpf(fmaf(kPs, fabsf(v), 1.0f));
  const float hpoly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, kB5, kB4), kB3), kB2), kB1);
  const float q = hpoly * __builtin_amdgcn_exp2f((v * v) * kE);
  return v * (v >= 0.0f ? 1.0f - q : q);
}
__device__ __forceinline__ float silu_f32(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * 1.4426950408889634f));
}
__device__ __forceinline__ float activate(float v, int act) {
  if (act == kActRelu) return fmaxf(v, 0.0f);
  if (act == kActGelu) return gelu_f32(v);
  if (act == kActSilu) return silu_f32(v);
  return v;
}

// Maxima of the requantised output (OutT = bf16_max): cs holds them as uint32_t
// (the bits of a non-negative float order like the float); ldcs != 0: one per
// row of C, else one for the whole output.  fold_row_max reduces a value over the
// `width` consecutive lanes that hold pieces of row m and lets the group's first
// lane fold it into that row (valid rows only); with one maximum it returns the
// running maximum instead, which fold_tensor_max folds once per wave.  Every lane
// of the wave takes part in both (shuffles).
__device__ __forceinline__ float fold_row_max(uint8_t* cs, int64_t ldcs, int m, bool valid, float a,
                                              int width, int lane, float run) {
  if (ldcs != 0) {
    a = group_max(a, width);
    if (lane % width == 0 && valid && a > 0.0f)
      atomicMax(reinterpret_cast<uint32_t*>(cs) + m, __float_as_uint(a));
    return run;
  }
  return fmaxf(run, a);
}

__device__ __forceinline__ void fold_tensor_max(uint8_t* cs, int64_t ldcs, float run, int lane) {
  if (ldcs == 0) {
    run = wave_max(run);
    if (lane == 0 && run > 0.0f) atomicMax(reinterpret_cast<uint32_t*>(cs), __float_as_uint(run));
  }
}

// The same for the register epilogues, where row r's values sit in lanes r and
// r + 32 (h = lane / 32): the pair's maximum, folded by the low lane.
__device__ __forceinline__ float fold_pair_max(uint8_t* cs, int64_t ldcs, int m, float a, int h,
                                               float run) {
  if (ldcs != 0) {
    a = fmaxf(a, __shfl_xor(a, 32, 64));
    if (h == 0 && a > 0.0f) atomicMax(reinterpret_cast<uint32_t*>(cs) + m, __float_as_uint(a));
    return run;
  }
  return fmaxf(run, a);
}

template <class Cfg, int MODE, typename OutT>
__device__ __forceinline__ void epilogue(const v16f (&acc)[Cfg::kFragM][Cfg::kFragN], uint8_t* lds,
                                         OutT* C, int64_t ldc, int m0, int m_end, int n0, int N,
                                         float tensor_scale, uint8_t* cs = nullptr,
                                         int64_t ldcs = 0) {
  constexpr int FM = Cfg::kFragM, FN = Cfg::kFragN;
  constexpr int kChunksPerRow = Cfg::WN * 2 / 16;        // 16-byte chunks of a staged row
  constexpr int kRowsPerInst = 64 / kChunksPerRow;
  static_assert(sizeof(OutT) == 2, "16-bit outputs");
  static_assert(64 % kChunksPerRow == 0, "whole rows per store instruction");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const int h = lane >> 5;
  uint8_t* stage = lds + wave * 32 * Cfg::kStagePitch;
  const float* rsc = reinterpret_cast<const float*>(lds + Cfg::kRowScaleOff);
  float run = 0.0f;                                      // bf16_max, one maximum: this wave's
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = lane & 31;                             // staged row of this lane
    float fa = 1.0f;
    if (MODE == kTensor) fa = tensor_scale;
    if (MODE == kRowwise) fa = rsc[wm * Cfg::WM + i * 32 + r];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = j * 32 + 8 * g + 4 * h;             // staged column of value 0
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e] * fa;
        if (MODE == kRowwise) {
          const v4f fb = *reinterpret_cast<const v4f*>(rsc + Cfg::BM + wn * Cfg::WN + c);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= fb[e];
        }
        *reinterpret_cast<uint2*>(stage + r * Cfg::kStagePitch + c * 2) =
            pack4<OutT>(v[0], v[1], v[2], v[3]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);                  // lgkmcnt(0): staged rows written
#pragma unroll
    for (int q = 0; q < 32 / kRowsPerInst; ++q) {
      const int rr = q * kRowsPerInst + lane / kChunksPerRow;
      const int ch = lane % kChunksPerRow;
      const v4i val = *reinterpret_cast<const v4i*>(stage + rr * Cfg::kStagePitch + ch * 16);
      const int m = m0 + wm * Cfg::WM + i * 32 + rr;
      const int n = n0 + wn * Cfg::WN + ch * 8;
      float a = 0.0f;
      if (m < m_end) {
        OutT* dst = C + (int64_t)m * ldc + n;
        if (n + 8 <= N) {
          *reinterpret_cast<v4i*>(dst) = val;
          if constexpr (kTrackMax<OutT>)
            a = absmax_bf16(reinterpret_cast<const uint32_t*>(&val), 4);
        } else {
          OutT o[8];
          __builtin_memcpy(o, &val, 16);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (n + e < N) {
              dst[e] = o[e];
              if constexpr (kTrackMax<OutT>) {
                const uint32_t b = (uint32_t)__builtin_bit_cast(uint16_t, o[e]);
                a = fmaxf(a, absmax_bf16(&b, 1));
              }
            }
        }
      }
      if constexpr (kTrackMax<OutT>)
        run = fold_row_max(cs, ldcs, m, m < m_end, a, kChunksPerRow, lane, run);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);                  // reads done before the next block
  }
  if constexpr (kTrackMax<OutT>) fold_tensor_max(cs, ldcs, run, lane);
}

// Bias (and ReLU) epilogue of a full tile from registers, the layout of
// epilogue_direct below.  Each wave first copies the bias of its WN columns into
// a wave-private stretch of the (free) ring, then reads four columns at a time
// like the row-wise column scales (bias == nullptr: zeros).
template <class Cfg, int MODE, typename OutT, int ACT>
__device__ __forceinline__ void epilogue_direct_bias(const v16f (&acc)[Cfg::kFragM][Cfg::kFragN],
                                                     uint8_t* lds, OutT* C, int64_t ldc,
                                                     int m0, int n0, float tensor_scale,
                                                     const float* bias, uint8_t* cs,
                                                     int64_t ldcs) {
  constexpr int FM = Cfg::kFragM, FN = Cfg::kFragN;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const int h = lane >> 5;
  const float* rsc = reinterpret_cast<const float*>(lds + Cfg::kRowScaleOff);
  const int nw = n0 + wn * Cfg::WN;                      // first column of this wave
  static_assert(Cfg::kWaves * Cfg::WN * 4 <= Cfg::kSlots * Cfg::kSlotBytes, "bias fits the ring");
  float* bl = reinterpret_cast<float*>(lds) + wave * Cfg::WN;
#pragma unroll
  for (int c = lane; c < Cfg::WN; c += 64) bl[c] = bias != nullptr ? bias[nw + c] : 0.0f;
  float am[FM];                                          // bf16_max: row maxima of the lane
#pragma unroll
  for (int i = 0; i < FM; ++i) am[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * Cfg::WM + i * 32 + (lane & 31);
      float fa = 1.0f;
      if (MODE == kTensor) fa = tensor_scale;
      if (MODE == kRowwise) fa = rsc[r];
      OutT* crow = C + (int64_t)(m0 + r) * ldc + nw;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        uint2 w[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int g = 2 * k + q;
          const int c = j * 32 + 8 * g + 4 * h;
          v4f fb{1.0f, 1.0f, 1.0f, 1.0f};
          if (MODE == kRowwise) fb = *reinterpret_cast<const v4f*>(rsc + Cfg::BM + wn * Cfg::WN + c);
          const v4f bv = *reinterpret_cast<const v4f*>(bl + c);
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = acc[i][j][4 * g + e] * fa;
            if (MODE == kRowwise) v[e] *= fb[e];
            v[e] = activate(v[e] + bv[e], ACT);
          }
          w[q] = pack4<OutT>(v[0], v[1], v[2], v[3]);
          if constexpr (kTrackMax<OutT>) am[i] = fmaxf(am[i], absmax_bf16(&w[q].x, 2));
        }
        const auto sx = __builtin_amdgcn_permlane32_swap(w[0].x, w[1].x, false, false);
        const auto sy = __builtin_amdgcn_permlane32_swap(w[0].y, w[1].y, false, false);
        const v4i out{(int)sx[0], (int)sy[0], (int)sx[1], (int)sy[1]};
        *reinterpret_cast<v4i*>(crow + j * 32 + 16 * k + 8 * h) = out;
      }
    }
  }
  if constexpr (kTrackMax<OutT>) {
    float run = 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      run = fold_pair_max(cs, ldcs, m0 + wm * Cfg::WM + i * 32 + (lane & 31), am[i], h, run);
    fold_tensor_max(cs, ldcs, run, lane);
  }
}

// Epilogue of a full tile straight from registers.  After the MFMAs a lane holds,
// for each 32 x 32 block and group g of four accumulators, four consecutive
// output columns 8g + 4h .. 8g + 4h + 3 (h = lane / 32) of row lane % 32.  One
// V_PERMLANE32_SWAP per packed dword exchanges group 2k + 1 of the low half-wave
// with group 2k of the high half, after which every lane owns eight consecutive
// columns (16 bytes) of its row: C is written with 16-byte stores and no LDS
// staging, so the epilogue costs a few hundred instructions and no waits.
// BIAS (fused kernels, interior tiles): the bias of the lane's 16 columns of
// block j is loaded once per j and added after the scales, then the activation
// `act` (one instance of the loop per activation, chosen once).
template <class Cfg, int MODE, typename OutT, bool BIAS = false>
__device__ __forceinline__ void epilogue_direct(const v16f (&acc)[Cfg::kFragM][Cfg::kFragN],
                                                uint8_t* lds, OutT* C, int64_t ldc, int m0,
                                                int n0, float tensor_scale, int rbuf = 0,
                                                const float* bias = nullptr, int act = kActNone,
                                                uint8_t* cs = nullptr, int64_t ldcs = 0) {
  constexpr int FM = Cfg::kFragM, FN = Cfg::kFragN;
  static_assert(sizeof(OutT) == 2, "16-bit outputs");
  if constexpr (BIAS) {
    if (act == kActGelu)
      epilogue_direct_bias<Cfg, MODE, OutT, kActGelu>(acc, lds, C, ldc, m0, n0, tensor_scale, bias,
                                                      cs, ldcs);
    else if (act == kActSilu)
      epilogue_direct_bias<Cfg, MODE, OutT, kActSilu>(acc, lds, C, ldc, m0, n0, tensor_scale, bias,
                                                      cs, ldcs);
    else if (act == kActRelu)
      epilogue_direct_bias<Cfg, MODE, OutT, kActRelu>(acc, lds, C, ldc, m0, n0, tensor_scale, bias,
                                                      cs, ldcs);
    else
      epilogue_direct_bias<Cfg, MODE, OutT, kActNone>(acc, lds, C, ldc, m0, n0, tensor_scale, bias,
                                                      cs, ldcs);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const int h = lane >> 5;
  const float* rsc =
      reinterpret_cast<const float*>(lds + Cfg::kRowScaleOff + rbuf * (Cfg::BM + Cfg::BN) * 4);
  float run = 0.0f;                                      // bf16_max, one maximum: this wave's
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = wm * Cfg::WM + i * 32 + (lane & 31);   // tile row of this lane
    float fa = 1.0f;
    if (MODE == kTensor) fa = tensor_scale;
    if (MODE == kRowwise) fa = rsc[r];
    OutT* crow = C + (int64_t)(m0 + r) * ldc + n0 + wn * Cfg::WN;
    float am = 0.0f;                                     // bf16_max: this lane's row maximum
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        uint2 w[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int g = 2 * k + q;
          const int c = j * 32 + 8 * g + 4 * h;           // wave-local column of value 0
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e] * fa;
          if (MODE == kRowwise) {
            const v4f fb = *reinterpret_cast<const v4f*>(rsc + Cfg::BM + wn * Cfg::WN + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] *= fb[e];
          }
          w[q] = pack4<OutT>(v[0], v[1], v[2], v[3]);
          if constexpr (kTrackMax<OutT>) am = fmaxf(am, absmax_bf16(&w[q].x, 2));
        }
        // low half keeps group 2k and takes the high half's; high half keeps 2k + 1
        const auto sx = __builtin_amdgcn_permlane32_swap(w[0].x, w[1].x, false, false);
        const auto sy = __builtin_amdgcn_permlane32_swap(w[0].y, w[1].y, false, false);
        const v4i out{(int)sx[0], (int)sy[0], (int)sx[1], (int)sy[1]};
        *reinterpret_cast<v4i*>(crow + j * 32 + 16 * k + 8 * h) = out;
      }
    }
    if constexpr (kTrackMax<OutT>) run = fold_pair_max(cs, ldcs, m0 + r, am, h, run);
  }
  if constexpr (kTrackMax<OutT>) fold_tensor_max(cs, ldcs, run, lane);
}

// The register epilogue for tiles of which only the first `rows` rows are stored
// (tiles cut by M inside a copy stream; no bias, 16-bit outputs): the stores go
// through a buffer descriptor whose range ends at the last valid row, so the
// hardware drops the others and every wave still issues all its stores (the
// stream's waits count them).  Rows 0 .. BM-1 of the tile must be addressable
// with 32-bit offsets: BM * ldc * sizeof(OutT) < 2^31.
template <class Cfg, int MODE, typename OutT>
__device__ __forceinline__ void epilogue_direct_rows(const v16f (&acc)[Cfg::kFragM][Cfg::kFragN],
                                                     const uint8_t* lds, OutT* C, int64_t ldc,
                                                     int m0, int n0, float tensor_scale, int rbuf,
                                                     int rows) {
  constexpr int FM = Cfg::kFragM, FN = Cfg::kFragN;
  static_assert(sizeof(OutT) == 2 && !kTrackMax<OutT>, "16-bit outputs");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const int h = lane >> 5;
  const float* rsc =
      reinterpret_cast<const float*>(lds + Cfg::kRowScaleOff + rbuf * (Cfg::BM + Cfg::BN) * 4);
  const int vr = rows < Cfg::BM ? rows : Cfg::BM;
  const __amdgpu_buffer_rsrc_t rs =
      buffer_rsrc(C + (int64_t)m0 * ldc, (uint32_t)(vr * (int)ldc * (int)sizeof(OutT)));
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = wm * Cfg::WM + i * 32 + (lane & 31);   // tile row of this lane
    float fa = 1.0f;
    if (MODE == kTensor) fa = tensor_scale;
    if (MODE == kRowwise) fa = rsc[r];
    const int vrow = (r * (int)ldc + n0 + wn * Cfg::WN + 8 * h) * (int)sizeof(OutT);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        uint2 w[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int g = 2 * k + q;
          const int c = j * 32 + 8 * g + 4 * h;           // wave-local column of value 0
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e] * fa;
          if (MODE == kRowwise) {
            const v4f fb = *reinterpret_cast<const v4f*>(rsc + Cfg::BM + wn * Cfg::WN + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] *= fb[e];
          }
          w[q] = pack4<OutT>(v[0], v[1], v[2], v[3]);
        }
        // low half keeps group 2k and takes the high half's; high half keeps 2k + 1
        const auto sx = __builtin_amdgcn_permlane32_swap(w[0].x, w[1].x, false, false);
        const auto sy = __builtin_amdgcn_permlane32_swap(w[0].y, w[1].y, false, false);
        typedef unsigned v4u_st __attribute__((ext_vector_type(4)));
        const v4u_st out{sx[0], sy[0], sx[1], sy[1]};
        __builtin_amdgcn_raw_buffer_store_b128(out, rs,
                                               vrow + (j * 32 + 16 * k) * (int)sizeof(OutT), 0, 0);
      }
    }
  }
}

// The output quantised for the next layer, straight from registers (interior
// tiles without bias or activation): e4m3 codes with one E8M0 code per 32
// consecutive columns of a row, by the quantisers' MX rule.  A 32 x 32 block j
// of row r is one MX block, held by lanes r (columns 8g .. 8g + 3) and r + 32
// (8g + 4 .. 8g + 7): the block maximum is the lane's 16 values and one swap
// with its partner (v_permlane32_swap); after encoding, a second swap of the
// 4-byte groups leaves each lane two 8-byte runs of its row (columns 16k + 8h ..
// 16k + 8h + 7).  Needs N % 32 == 0 (every interior tile is whole).
template <class Cfg, int MODE>
__device__ __forceinline__ void epilogue_direct_q(const v16f (&acc)[Cfg::kFragM][Cfg::kFragN],
                                                  const uint8_t* lds, uint8_t* C, int64_t ldc,
                                                  int m0, int n0, float tensor_scale,
                                                  uint8_t* cs, int64_t ldcs) {
  constexpr int FM = Cfg::kFragM, FN = Cfg::kFragN;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const int h = lane >> 5;
  const float* rsc = reinterpret_cast<const float*>(lds + Cfg::kRowScaleOff);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = wm * Cfg::WM + i * 32 + (lane & 31);   // tile row of this lane
    float fa = 1.0f;
    if (MODE == kTensor) fa = tensor_scale;
    if (MODE == kRowwise) fa = rsc[r];
    uint8_t* crow = C + (int64_t)(m0 + r) * ldc + n0 + wn * Cfg::WN;
    uint8_t* srow = cs + (int64_t)(m0 + r) * ldcs + ((n0 + wn * Cfg::WN) >> 5);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      float v[16];
      float a = 0.0f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = j * 32 + 8 * g + 4 * h;             // wave-local column of value 0
        v4f fb{1.0f, 1.0f, 1.0f, 1.0f};
        if (MODE == kRowwise) fb = *reinterpret_cast<const v4f*>(rsc + Cfg::BM + wn * Cfg::WN + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[4 * g + e] = acc[i][j][4 * g + e] * fa;
          if (MODE == kRowwise) v[4 * g + e] *= fb[e];
          a = fmaxf(a, fabsf(v[4 * g + e]));
        }
      }
      const auto am = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a),
                                                       false, false);
      // one of the pair is this lane's own maximum, the other its partner's
      a = fmaxf(__uint_as_float(am[0]), __uint_as_float(am[1]));
      const uint32_t code = mx_code_from_amax<kE4M3>(a);
      const int e = 127 - (int)code;
      uint32_t w[4];
#pragma unroll
      for (int g = 0; g < 4; ++g)
        w[g] = encode4_e4m3(ldexpf(v[4 * g], e), ldexpf(v[4 * g + 1], e), ldexpf(v[4 * g + 2], e),
                            ldexpf(v[4 * g + 3], e));
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        // low half keeps group 2k and takes the high half's; high half keeps 2k + 1
        const auto sw = __builtin_amdgcn_permlane32_swap(w[2 * k], w[2 * k + 1], false, false);
        uint2 out;
        out.x = sw[0];
        out.y = sw[1];
        *reinterpret_cast<uint2*>(crow + j * 32 + 16 * k + 8 * h) = out;
      }
      if (h == 0) srow[j] = (uint8_t)code;
    }
  }
}

// Fused epilogue (bias, activation).  The scaled fp32 tile goes through LDS, one
// block of 32 rows per wavefront at a time, and the bias, the activation, the
// cast and the stores run in a loop over 16-byte pieces: four copies of the
// activation's math instead of one per accumulator register.  (Inlining
// it into the register epilogues made those kernels many times larger and the
// fused GEMM slower than a separate pass over C; kernels without a fused
// epilogue are separate instances and carry none of this code.)  Needs the ring
// free: it runs after the mainloop's final barrier, never inside a copy stream.
// With OutT = uint8_t the output is quantised again for the next layer: e4m3
// codes with one E8M0 code per 32 consecutive columns of a row (the MX rule of
// the quantisers), written to cs[m * ldcs + n / 32]; N % 32 == 0.  The 32
// columns of a block are the four-column pieces of 8 consecutive lanes, so the
// block maximum takes three xor-shuffles.
// With OutT = bf16_max the stored bf16 values' magnitudes are also folded into
// the maxima at cs (see fold_row_max).
template <class Cfg, int MODE, typename OutT>
__device__ __forceinline__ void epilogue_fused(const v16f (&acc)[Cfg::kFragM][Cfg::kFragN],
                                               uint8_t* lds, OutT* C, int64_t ldc, int m0,
                                               int m_end, int n0, int N, float tensor_scale,
                                               const float* bias, int act,
                                               uint8_t* cs = nullptr, int64_t ldcs = 0) {
  constexpr bool kQ = std::is_same<OutT, uint8_t>::value;
  constexpr int FM = Cfg::kFragM, FN = Cfg::kFragN;
  constexpr int kPitch = Cfg::WN + 4;                    // staged fp32 row (+16 bytes)
  constexpr int kPiecesPerRow = Cfg::WN / 4;
  constexpr int kIters = 32 * kPiecesPerRow / 64;
  static_assert(Cfg::kWaves * 32 * kPitch * 4 <= Cfg::kSlots * Cfg::kSlotBytes,
                "fp32 staging fits in the ring");
  static_assert((32 * kPiecesPerRow) % 64 == 0, "whole store instructions");
  static_assert(64 % kPiecesPerRow == 0, "a lane keeps its columns over the store loop");
  static_assert(sizeof(OutT) == 2 || kQ, "16-bit outputs or e4m3 codes");
  static_assert(!kQ || kPiecesPerRow % 8 == 0, "32-column blocks inside one lane group");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const int h = lane >> 5;
  float* stage = reinterpret_cast<float*>(lds) + wave * 32 * kPitch;
  // the store loop hands each lane the same four columns every time: their bias
  // is loaded once, before any wait on the staged rows
  const int cc = (lane % kPiecesPerRow) * 4;            // wave-local column of the lane
  const int n = n0 + wn * Cfg::WN + cc;
  float bv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (bias != nullptr) {
#pragma unroll
    for (int e = 0; e < 4; ++e) bv[e] = n + e < N ? bias[n + e] : 0.0f;
  }
  const float* rsc = reinterpret_cast<const float*>(lds + Cfg::kRowScaleOff);
  float run = 0.0f;                                      // bf16_max, one maximum: this wave's
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = lane & 31;
    float fa = 1.0f;
    if (MODE == kTensor) fa = tensor_scale;
    if (MODE == kRowwise) fa = rsc[wm * Cfg::WM + i * 32 + r];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = j * 32 + 8 * g + 4 * h;
        v4f v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e] * fa;
        if (MODE == kRowwise) {
          const v4f fb = *reinterpret_cast<const v4f*>(rsc + Cfg::BM + wn * Cfg::WN + c);
          v *= fb;
        }
        *reinterpret_cast<v4f*>(stage + r * kPitch + c) = v;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);                  // lgkmcnt(0): staged rows written
    // unrolled by 4: the LDS reads of four pieces are in flight together
#pragma unroll 4
    for (int it = 0; it < kIters; ++it) {
      const int rr = (it * 64 + lane) / kPiecesPerRow;
      const v4f val = *reinterpret_cast<const v4f*>(stage + rr * kPitch + cc);
      const int m = m0 + wm * Cfg::WM + i * 32 + rr;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = activate(val[e] + bv[e], act);
      if constexpr (kQ) {
        float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
        a = fmaxf(a, __shfl_xor(a, 1, 64));
        a = fmaxf(a, __shfl_xor(a, 2, 64));
        a = fmaxf(a, __shfl_xor(a, 4, 64));
        const uint32_t code = mx_code_from_amax<kE4M3>(a);
        const int e = 127 - (int)code;
        const uint32_t w = encode4_e4m3(ldexpf(v[0], e), ldexpf(v[1], e), ldexpf(v[2], e),
                                        ldexpf(v[3], e));
        if (m < m_end && n < N) {           // N % 32 == 0: a block is all in or all out
          *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(C) + (int64_t)m * ldc + n) = w;
          if ((lane & 7) == 0) cs[(int64_t)m * ldcs + (n >> 5)] = (uint8_t)code;
        }
      } else {
        const uint2 w = pack4<OutT>(v[0], v[1], v[2], v[3]);
        float a = 0.0f;
        if (m < m_end) {
          OutT* dst = C + (int64_t)m * ldc + n;
          if (n + 4 <= N) {
            *reinterpret_cast<uint2*>(dst) = w;
            if constexpr (kTrackMax<OutT>) a = absmax_bf16(&w.x, 2);
          } else {
            for (int e = 0; e < 4; ++e)
              if (n + e < N) {
                const OutT o = to_out<OutT>(v[e]);
                dst[e] = o;
                if constexpr (kTrackMax<OutT>) {
                  const uint32_t b = (uint32_t)__builtin_bit_cast(uint16_t, o);
                  a = fmaxf(a, absmax_bf16(&b, 1));
                }
              }
          }
        }
        if constexpr (kTrackMax<OutT>)
          run = fold_row_max(cs, ldcs, m, m < m_end, a, kPiecesPerRow, lane, run);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);                  // reads done before the next block
  }
  if constexpr (kTrackMax<OutT>) fold_tensor_max(cs, ldcs, run, lane);
}

// Epilogue of a full interior tile (every row and column valid): straight from
// the accumulators where the output allows it.
template <class Cfg, int MODE, typename OutT, bool FUSED>
__device__ __forceinline__ void epilogue_full_tile(const v16f (&acc)[Cfg::kFragM][Cfg::kFragN],
                                                   uint8_t* lds, OutT* C, int64_t ldc, int m0,
                                                   int m_end, int n0, int N, float tensor_scale,
                                                   const float* bias, int act, uint8_t* cs,
                                                   int64_t ldcs) {
  if constexpr (FUSED && !std::is_same<OutT, uint8_t>::value) {
    epilogue_direct<Cfg, MODE, OutT, true>(acc, lds, C, ldc, m0, n0, tensor_scale, 0, bias, act,
                                           cs, ldcs);
  } else if constexpr (FUSED) {
    epilogue_fused<Cfg, MODE, OutT>(acc, lds, C, ldc, m0, m_end, n0, N, tensor_scale, bias, act,
                                    cs, ldcs);
  } else if constexpr (std::is_same<OutT, uint8_t>::value) {
    epilogue_direct_q<Cfg, MODE>(acc, lds, C, ldc, m0, n0, tensor_scale, cs, ldcs);
  } else {
#if FP8GEMM_DIRECT_EPILOGUE
    epilogue_direct<Cfg, MODE, OutT>(acc, lds, C, ldc, m0, n0, tensor_scale, 0, nullptr, kActNone,
                                     cs, ldcs);
#else
    epilogue<Cfg, MODE, OutT>(acc, lds, C, ldc, m0, m_end, n0, N, tensor_scale, cs, ldcs);
#endif
  }
}

// Epilogue of any tile (rows and columns past the edges are not stored).
template <class Cfg, int MODE, typename OutT, bool FUSED>
__device__ __forceinline__ void epilogue_any_tile(const v16f (&acc)[Cfg::kFragM][Cfg::kFragN],
                                                  uint8_t* lds, OutT* C, int64_t ldc, int m0,
                                                  int m_end, int n0, int N, float tensor_scale,
                                                  const float* bias, int act, uint8_t* cs,
                                                  int64_t ldcs) {
  if constexpr (FUSED || sizeof(OutT) != 2)
    epilogue_fused<Cfg, MODE, OutT>(acc, lds, C, ldc, m0, m_end, n0, N, tensor_scale, bias, act,
                                    cs, ldcs);
  else
    epilogue<Cfg, MODE, OutT>(acc, lds, C, ldc, m0, m_end, n0, N, tensor_scale, cs, ldcs);
}

// One output tile: the interior mainloop when the tile qualifies, else the
// general (clamped) one, then the epilogue.  Each branch has its own accumulators
// and epilogue so no accumulator copies join the two paths.  EDGE_INTERIOR: tiles
// cut by M or N take the interior mainloop too (the grouped kernel keeps them on
// the general one: its copy-stream path spills once the extra branch is there).
template <class Cfg, int MODE, typename OutT, bool KALIGNED, bool FUSED = false,
          bool EDGE_INTERIOR = true>
__device__ __forceinline__ void gemm_tile(const TileOperands& op, uint8_t* lds, OutT* C,
                                          int64_t ldc, int m0, int m_end, int n0, int N,
                                          float tensor_scale, const float* bias = nullptr,
                                          int act = kActNone, uint8_t* cs = nullptr,
                                          int64_t ldcs = 0) {
  if constexpr (KALIGNED && Cfg::kSlots == 4) {
    if (EDGE_INTERIOR ? interior_k<Cfg, MODE>(op) : interior_tile<Cfg, MODE>(op)) {
      v16f acc[Cfg::kFragM][Cfg::kFragN];
      mainloop_interior<Cfg, MODE>(op, lds, acc);
      if (!EDGE_INTERIOR || (op.a_rows >= Cfg::BM && op.b_rows >= Cfg::BN))
        epilogue_full_tile<Cfg, MODE, OutT, FUSED>(acc, lds, C, ldc, m0, m_end, n0, N,
                                                   tensor_scale, bias, act, cs, ldcs);
      else                                        // a tile cut by M or N
        epilogue_any_tile<Cfg, MODE, OutT, FUSED>(acc, lds, C, ldc, m0, m_end, n0, N,
                                                  tensor_scale, bias, act, cs, ldcs);
      return;
    }
  }
  v16f acc[Cfg::kFragM][Cfg::kFragN];
  mainloop<Cfg, MODE, KALIGNED && !kF4>(op, lds, acc);
  epilogue_any_tile<Cfg, MODE, OutT, FUSED>(acc, lds, C, ldc, m0, m_end, n0, N, tensor_scale,
                                            bias, act, cs, ldcs);
}

// One output tile on the interior mainloop, whole or cut by M or N (the caller
// guarantees interior_k(op)); plain 16-bit epilogue.
template <class Cfg, int MODE, typename OutT>
__device__ __forceinline__ void gemm_tile_interior(const TileOperands& op, uint8_t* lds, OutT* C,
                                                   int64_t ldc, int m0, int m_end, int n0, int N,
                                                   float tensor_scale) {
  v16f acc[Cfg::kFragM][Cfg::kFragN];
  mainloop_interior<Cfg, MODE>(op, lds, acc);
  if (op.a_rows >= Cfg::BM && op.b_rows >= Cfg::BN)
    epilogue_full_tile<Cfg, MODE, OutT, false>(acc, lds, C, ldc, m0, m_end, n0, N, tensor_scale,
                                               nullptr, kActNone, nullptr, 0);
  else
    epilogue_any_tile<Cfg, MODE, OutT, false>(acc, lds, C, ldc, m0, m_end, n0, N, tensor_scale,
                                              nullptr, kActNone, nullptr, 0);
}

// One output tile with row-major B ([K][N]): the interior mainloop in its KN
// form for every tile (the caller guarantees K % 128 == 0, MX K % 512 == 0, and
// 32-bit spans); tiles cut by M or N end in the general epilogue.
template <class Cfg, int MODE, typename OutT, bool FUSED = false>
__device__ __forceinline__ void gemm_tile_kn(const TileOperands& op, uint8_t* lds, OutT* C,
                                             int64_t ldc, int m0, int m_end, int n0, int N,
                                             float tensor_scale, const float* bias = nullptr,
                                             int act = kActNone, uint8_t* cs = nullptr,
                                             int64_t ldcs = 0) {
  v16f acc[Cfg::kFragM][Cfg::kFragN];
  mainloop_interior<Cfg, MODE, 2, true>(op, lds, acc);
  if (op.a_rows >= Cfg::BM && op.b_rows >= Cfg::BN)
    epilogue_full_tile<Cfg, MODE, OutT, FUSED>(acc, lds, C, ldc, m0, m_end, n0, N, tensor_scale,
                                               bias, act, cs, ldcs);
  else
    epilogue_any_tile<Cfg, MODE, OutT, FUSED>(acc, lds, C, ldc, m0, m_end, n0, N, tensor_scale,
                                              bias, act, cs, ldcs);
}

}  // inline namespace
}  // namespace fp8gemm
