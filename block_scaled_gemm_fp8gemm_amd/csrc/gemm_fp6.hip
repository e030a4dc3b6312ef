// MXFP6 GEMM for gfx950: e2m3 / e3m2 operands with E8M0 block scales, through
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 at an FP6 format field (2 = e2m3, 3 = e3m2).
//
// "Hopper/Blackwell architecture features" §12.6.1 lists FP6 with micro-scaling
// among the new tensor-core formats.  The element formats and the packed layout
// follow OCP MX v1.0: a row of codes is a little-endian 6-bit stream, so a
// 32-element block is 24 contiguous bytes.  For an FP6 operand the instruction
// takes 24 bytes per lane, the 32 elements of block lane / 32 of row lane % 32,
// low bits first (probed on gfx950), and the block scale from byte 0 of the scale
// operand of lane row + 32 * block: a lane's operand is exactly the 24 packed
// bytes of its block.
//
// Tile 128 x 128, 4 wavefronts of 64 x 64, two workgroups per CU.  K is walked in
// 64-element steps (one MFMA K step, 48 bytes per row).  A four-slot LDS ring of
// (128 + 128) rows x 48 bytes is filled by direct-to-LDS copies: a slot is 12
// KiB, copied as 12 instructions of 1 KiB over the flat [row][48] layout (lane l
// of instruction j carries bytes 1024 j + 16 l).  A fragment is three 8-byte LDS
// reads per lane (row stride 48 bytes: 16 consecutive rows hit distinct bank
// pairs).  The E8M0 codes travel through LDS in groups of 16 per row (8 steps),
// double-buffered, as dword copies.  Per step: one wait for the next step's
// copies and one workgroup barrier.  Rows past M / N read the last valid row and
// are never stored.  Conditions: K % 128 == 0 (whole 2-step tiles; code rows are
// dword multiples).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_tile.h"
#include "launch.h"
#include "plan.h"
#include "tile_order.h"

namespace fp8gemm {
namespace fp6 {
namespace {

using Cfg = TileCfg<128, 128, 64, 64, 4, 2>;     // the epilogue's view of the tile
constexpr int BM = 128, BN = 128, kRows = BM + BN;
constexpr int kStepBytes = 48;                   // 64 FP6 codes of a row
constexpr int NS = 4;                            // ring slots (steps in flight)
constexpr int kSlot = kRows * kStepBytes;        // 12 KiB
constexpr int kLoads = kSlot / 1024 / 4;         // copy instructions per wave and step
constexpr int kCodeOff = NS * kSlot;             // two groups of 16 codes x 256 rows
constexpr int kCodeBuf = kRows * 16;
constexpr int kLdsBytes = kCodeOff + 2 * kCodeBuf;
constexpr int kGroupSteps = 8;                   // steps per 16-code group
static_assert(kSlot % 4096 == 0 && kLoads == 3, "equal copy share per wave");
static_assert(kLoads * 2 * 1024 == BM * kStepBytes, "waves 0-1 copy A rows, 2-3 B rows");
static_assert(Cfg::kWaves * 32 * (Cfg::WN + 4) * 4 <= kCodeOff, "epilogue staging fits the ring");
static_assert(2 * kLdsBytes <= 160 * 1024, "two workgroups per CU");

template <int FA, int FB, int MODE, typename OutT, bool FUSED>
__global__ __launch_bounds__(256, 2) void fp6_kernel(GemmProblem p, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];
  constexpr int FM = Cfg::kFragM, FN = Cfg::kFragN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, kGroupM, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const int h = lane >> 5;
  const int a_rows = p.M - m0 < BM ? p.M - m0 : BM;
  const int b_rows = p.N - n0 < BN ? p.N - n0 : BN;
  const int kbytes = p.K / 4 * 3;
  const int nsteps = p.K / 64;
  const int nblk = p.K / 32, sld = nblk;         // E8M0 codes per row

  // ---- copy side ----
  const bool a_wave = wave < 2;                  // waves 0-1: A rows, 2-3: B rows
  const __amdgpu_buffer_rsrc_t rs = a_wave
      ? buffer_rsrc(p.A + (int64_t)m0 * p.lda, (uint32_t)((a_rows - 1) * p.lda + kbytes))
      : buffer_rsrc(p.B + (int64_t)n0 * p.ldb, (uint32_t)((b_rows - 1) * p.ldb + kbytes));
  const int ld = (int)(a_wave ? p.lda : p.ldb), rows = a_wave ? a_rows : b_rows;
  int voff[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int f = (wave * kLoads + j) * 1024 + 16 * lane;     // flat byte of the slot
    int r = f / kStepBytes - (a_wave ? 0 : BM);
    r = r < rows ? r : rows - 1;
    voff[j] = r * ld + f % kStepBytes;
  }
  auto copy_step = [&](int slot, int s) __attribute__((always_inline)) {
    s = s < nsteps ? s : nsteps - 1;             // past the end: harmless re-fetch
#pragma unroll
    for (int j = 0; j < kLoads; ++j)
      buffer_dma16(rs, lds + slot * kSlot + (wave * kLoads + j) * 1024, voff[j], s * kStepBytes);
  };
  // codes: wave w copies rows 64w .. 64w + 63 (lane = row), dword i of group g
  // lands at kCodeOff + buf * kCodeBuf + (4w + i) * 256 + 4 lane
  const __amdgpu_buffer_rsrc_t rc = a_wave
      ? buffer_rsrc(static_cast<const uint8_t*>(p.scale_a) + (int64_t)m0 * sld,
                    (uint32_t)((a_rows - 1) * sld + nblk))
      : buffer_rsrc(static_cast<const uint8_t*>(p.scale_b) + (int64_t)n0 * sld,
                    (uint32_t)((b_rows - 1) * sld + nblk));
  int crow = (wave & 1) * 64 + lane;
  crow = crow < rows ? crow : rows - 1;
  const int cvoff = crow * sld;
  const int ngroups = (nsteps + kGroupSteps - 1) / kGroupSteps;
  auto copy_codes = [&](int buf, int g) __attribute__((always_inline)) {
    g = g < ngroups ? g : ngroups - 1;           // past the end: harmless re-fetch
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rc,
          (__attribute__((address_space(3))) void*)(lds + kCodeOff + buf * kCodeBuf +
                                                    (4 * wave + i) * 256),
          4, cvoff, 16 * g + 4 * i, 0, 0);
  };

  // ---- read side: lane (row lane % 32, block h of the step) ----
  int arow[FM], brow[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) arow[i] = wm * Cfg::WM + i * 32 + (lane & 31);
#pragma unroll
  for (int j = 0; j < FN; ++j) brow[j] = BM + wn * Cfg::WN + j * 32 + (lane & 31);
  auto frag = [&](int slot, int row) __attribute__((always_inline)) {
    const uint8_t* base = lds + slot * kSlot + row * kStepBytes + 24 * h;
    const uint2 d0 = *reinterpret_cast<const uint2*>(base);
    const uint2 d1 = *reinterpret_cast<const uint2*>(base + 8);
    const uint2 d2 = *reinterpret_cast<const uint2*>(base + 16);
    return v8i{(int)d0.x, (int)d0.y, (int)d1.x, (int)d1.y, (int)d2.x, (int)d2.y, 0, 0};
  };
  // code of block 2s + h of a row: group s / 8, byte 2 (s % 8) + h of the group
  auto code = [&](int buf, int row, int pos) __attribute__((always_inline)) {
    const int b = 2 * pos + h;                   // block within the group
    return (uint32_t)lds[kCodeOff + buf * kCodeBuf + (4 * (row >> 6) + (b >> 2)) * 256 +
                         4 * (row & 63) + (b & 3)];
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};
  v8i af[2][FM], bf[2][FN];
  uint32_t sa[2][FM], sb[2][FN];

  // ---- prologue: code group 0, steps 0 .. NS-1; wait for step 0 ----
  copy_codes(0, 0);
#pragma unroll
  for (int s = 0; s < NS; ++s) copy_step(s, s);
  FP8GEMM_WAIT_VM_LGKM0((NS - 1) * kLoads);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    af[0][i] = frag(0, arow[i]);
    sa[0][i] = code(0, arow[i], 0);
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    bf[0][j] = frag(0, brow[j]);
    sb[0][j] = code(0, brow[j], 0);
  }

  // ---- step t (position P = t % 8 in its code group): wait for step t + 1's
  // copies; at P = 0 copy the next code group; copy step t + NS into the slot of
  // step t; read step t + 1's fragments and codes; the MFMAs of step t ----
  auto step = [&](int t, auto P_c) __attribute__((always_inline)) {
    constexpr int P = decltype(P_c)::value;
    constexpr int cur = P & 1, nxt = cur ^ 1;
    // copies issued after step t + 1's: the two steps before t, with a code group
    // copy where one of them started a group
    constexpr int kAfter = (NS - 2) * kLoads + ((P == 1 || P == 2) ? 4 : 0);
    __builtin_amdgcn_sched_barrier(0);
    FP8GEMM_WAIT_VM_LGKM0(kAfter);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int g = t / kGroupSteps;
    if (P == 0) copy_codes((g + 1) & 1, g + 1);
    copy_step(t % NS, t + NS);
    if (t + 1 < nsteps) {
      const int ns = (t + 1) % NS;
      const int cbuf = ((t + 1) / kGroupSteps) & 1;
      constexpr int np = (P + 1) % kGroupSteps;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        af[nxt][i] = frag(ns, arow[i]);
        sa[nxt][i] = code(cbuf, arow[i], np);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        bf[nxt][j] = frag(ns, brow[j]);
        sb[nxt][j] = code(cbuf, brow[j], np);
      }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            bf[cur][j], af[cur][i], acc[i][j], FB, FA, 0, (int)sb[cur][j], 0, (int)sa[cur][i]);
  };
  for (int t0 = 0; t0 < nsteps; t0 += kGroupSteps) {
    Unroll<0, kGroupSteps>::run([&](auto P_c) __attribute__((always_inline)) {
      constexpr int P = decltype(P_c)::value;
      if (t0 + P < nsteps) step(t0 + P, P_c);
    });
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0);                 // no copy may still target LDS
  __builtin_amdgcn_s_barrier();

  OutT* C = static_cast<OutT*>(p.C);
  if constexpr (FUSED || std::is_same<OutT, uint8_t>::value)
    epilogue_fused<Cfg, MODE, OutT>(acc, lds, C, p.ldc, m0, p.M, n0, p.N, 1.0f, p.bias, p.act,
                                    p.cs, p.ldcs);
  else
    epilogue<Cfg, MODE, OutT>(acc, lds, C, p.ldc, m0, p.M, n0, p.N, 1.0f, p.cs, p.ldcs);
}

// ---------------------------------------------------------------------------
// 256 x 256 tiles for shapes with a tile per CU: 4 wavefronts of 128 x 128, one
// workgroup per CU.  A 64-K step of a 128 x 128 wavefront tile reads 8 fragments
// for 16 MFMAs; the 128 x 128 tile above reads 4 for 4, and at two workgroups per
// CU asks for more LDS bandwidth than there is.
//   * K tiles of 96 bytes per row (128 codes, two MFMA steps), so no step
//     straddles two tiles, in a three-slot ring: A plane (3 x 256 rows x 96 B),
//     then B plane, then two buffers of 16 E8M0 codes per row: 160 KiB.  With the
//     planes apart every slot is in reach of one base register per piece.
//   * A K tile holds four 32-element blocks of 24 bytes.  Step 0 feeds lane h
//     block 2 h, step 1 block 2 h + 1 (any order of K inside an MFMA sums the
//     same, and a lane still holds one whole MX block with its own code).  A
//     lane reads the two whole 16-byte chunks its block lies in (chunks 3 h,
//     3 h + 1 for the even block, 3 h + 1, 3 h + 2 for the odd one) into eight
//     registers like an FP8 fragment, and the MFMA takes registers 0-5 or 2-7:
//     a third more LDS reads than the 24 bytes, but operands the register
//     allocator places without copies.
//   * Row stride 96 bytes puts rows r and r + 8 on the same banks; chunk c of
//     row r is stored at (c + ((r >> 3) & 1)) mod 6, which makes the 16-byte
//     reads of 16 rows conflict-free.
//   * Copy instruction j of a wave covers flat chunks 64 j .. 64 j + 63 of its
//     operand's 128 rows (row F / 6, position F % 6); instructions j and j + 3 are
//     32 rows apart with the same pattern, so a lane has three offsets and the
//     row offset goes in the scalar offset.
//   * K tile u: step 0 reads step 1's fragments (same slot) during its MFMAs;
//     step 1 waits for K tile u + 1, meets the other waves at the one barrier
//     of the K tile, copies K tile u + 3 into the slot of K tile u (and, at the
//     first K tile of a code group, the next group) and reads K tile u + 1.
//   * Rows past M or N read as zero (the copy range ends at the last valid row).
namespace big {

using Cfg = TileCfg<256, 256, 128, 128, 4, 1>;
constexpr int BM = 256, BN = 256;
constexpr int kTileB = 96;                         // bytes per row and K tile
constexpr int NS = 3;                              // ring slots
constexpr int kSlot = BM * kTileB;                 // one operand's slot, 24 KiB
constexpr int kPlane = NS * kSlot;                 // 72 KiB per operand
constexpr int kCodeOff = 2 * kPlane;
constexpr int kCodeBuf = (BM + BN) * 16;           // 16 codes (512 K) per row
constexpr int kLdsBytes = kCodeOff + 2 * kCodeBuf;
constexpr int kLoads = kSlot / 1024 / 2;           // copies per wave and K tile (2 waves per operand)
constexpr int kCodeLoads = 2;                      // 16-byte code copies per wave and group
constexpr int kGroupTiles = 4;                     // K tiles per code group
constexpr int kBody = 12;                          // K tiles per unrolled body (3 slots x 4)
static_assert(kLoads == 12 && kLoads % 3 == 0, "copy pattern repeats every 3 instructions");
static_assert(kLdsBytes <= 160 * 1024, "one workgroup per CU");
static_assert(Cfg::kWaves * 32 * Cfg::kStagePitch <= kCodeOff, "epilogue staging fits the ring");
static_assert(Cfg::kSlots * Cfg::kSlotBytes <= kCodeOff, "fused epilogue staging fits the ring");
static_assert((NS - 1) * kLoads + kCodeLoads < 64, "vmcnt range");

template <int FA, int FB, int MODE, typename OutT, bool FUSED>
__global__ __launch_bounds__(256, 1) void fp6_big_kernel(GemmProblem p, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];
  constexpr int FM = Cfg::kFragM, FN = Cfg::kFragN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, kGroupM, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
  const int h = lane >> 5;
  const int a_rows = p.M - m0 < BM ? p.M - m0 : BM;
  const int b_rows = p.N - n0 < BN ? p.N - n0 : BN;
  const int kbytes = p.K / 4 * 3;
  const int nk = p.K / 128;                        // K tiles
  const int nblk = p.K / 32, sld = nblk;
  const int ngroups = (nk + kGroupTiles - 1) / kGroupTiles;

  // ---- copy side: waves 0-1 copy A rows, 2-3 B rows (128 rows each) ----
  const bool a_wave = wave < 2;
  const int ld = (int)(a_wave ? p.lda : p.ldb);
  const __amdgpu_buffer_rsrc_t rs = a_wave
      ? buffer_rsrc(p.A + (int64_t)m0 * p.lda, (uint32_t)((a_rows - 1) * p.lda + kbytes))
      : buffer_rsrc(p.B + (int64_t)n0 * p.ldb, (uint32_t)((b_rows - 1) * p.ldb + kbytes));
  int voff[3];
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const int f = ((wave & 1) * kLoads + q) * 64 + lane;     // flat chunk of the operand's slot
    const int r = f / 6, cp = f % 6;
    const int c = (cp + 6 - ((r >> 3) & 1)) % 6;              // global chunk held at position cp
    voff[q] = r * ld + 16 * c;
  }
  uint8_t* const cdst = lds + (a_wave ? 0 : kPlane) + (wave & 1) * kLoads * 1024;
  auto copy_tile = [&](int slot, int kt) __attribute__((always_inline)) {
    kt = kt < nk ? kt : nk - 1;                    // past the end: harmless re-fetch
#pragma unroll
    for (int j = 0; j < kLoads; ++j)
      buffer_dma16(rs, cdst + slot * kSlot + j * 1024, voff[j % 3], (j / 3) * 32 * ld + kt * kTileB);
  };
  // codes: copy instruction ci = 2 wave + jj covers rows 64 ci .. 64 ci + 63 of
  // [A; B] (16 bytes per row: lane = row)
  const __amdgpu_buffer_rsrc_t rc = a_wave
      ? buffer_rsrc(static_cast<const uint8_t*>(p.scale_a) + (int64_t)m0 * sld,
                    (uint32_t)((a_rows - 1) * sld + nblk))
      : buffer_rsrc(static_cast<const uint8_t*>(p.scale_b) + (int64_t)n0 * sld,
                    (uint32_t)((b_rows - 1) * sld + nblk));
  auto copy_codes = [&](int buf, int g) __attribute__((always_inline)) {
    g = g < ngroups ? g : ngroups - 1;             // past the end: harmless re-fetch
#pragma unroll
    for (int jj = 0; jj < kCodeLoads; ++jj)
      buffer_dma16(rc, lds + kCodeOff + buf * kCodeBuf + (2 * wave + jj) * 1024,
                   (64 * (2 * (wave & 1) + jj) + lane) * sld, 16 * g);
  };

  // ---- read side: lane (row lane % 32, h = lane / 32); chunk c of the row at
  // position (c + rot) mod 6, rot = (row >> 3) & 1 = (lane >> 3) & 1; step pp
  // reads chunks 3 h + pp and 3 h + pp + 1 ----
  const int rot = (lane >> 3) & 1;
  auto pos = [&](int c) { return 16 * ((c + rot) % 6); };
  int ba0[2], ba1[2], bb0[2], bb1[2];
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
    const int ra = (wm * Cfg::WM + (lane & 31)) * kTileB;
    const int rb = kPlane + (wn * Cfg::WN + (lane & 31)) * kTileB;
    ba0[pp] = opaque(ra + pos(3 * h + pp));
    ba1[pp] = opaque(ra + pos(3 * h + pp + 1));
    bb0[pp] = opaque(rb + pos(3 * h + pp));
    bb1[pp] = opaque(rb + pos(3 * h + pp + 1));
  }
  auto rd16 = [&](int addr) __attribute__((always_inline)) {
    return *reinterpret_cast<const v4i*>(lds + addr);
  };
  // a fragment: the two chunks in eight registers; the block is registers 0-5
  // (step 0, even block) or 2-7 (step 1, odd block)
  auto frag = [&](int a0, int a1, auto pp_c) __attribute__((always_inline)) {
    const v8i v = __builtin_shufflevector(rd16(a0), rd16(a1), 0, 1, 2, 3, 4, 5, 6, 7);
    if constexpr (decltype(pp_c)::value == 0)
      return __builtin_shufflevector(v, v, 0, 1, 2, 3, 4, 5, -1, -1);
    else
      return __builtin_shufflevector(v, v, 2, 3, 4, 5, 6, 7, -1, -1);
  };
  // codes of (row, block b of the group): kCodeOff + buf * kCodeBuf + row * 16 + b;
  // the lane's block of step pp in K tile q4 of the group is 4 q4 + 2 h + pp
  int cur_a = opaque(kCodeOff + (wm * Cfg::WM + (lane & 31)) * 16 + 2 * h);
  int cur_b = opaque(kCodeOff + (BM + wn * Cfg::WN + (lane & 31)) * 16 + 2 * h);
  int nxt_a = opaque(cur_a + kCodeBuf), nxt_b = opaque(cur_b + kCodeBuf);

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};
  v8i af[2][FM], bf[2][FN];
  uint32_t sa[2][FM], sb[2][FN];

  // fragments and codes of step pp of the K tile in ring slot s, K tile q4 of its
  // code group, into register set z
  // fragment f (A fragments, then B) of step pp of the K tile in ring slot s,
  // K tile q4 of its code group, and its code
  auto read_one = [&](int s, auto pp_c, int q4, int ca, int cb, int f, v8i (&fa)[FM],
                      v8i (&fb)[FN], uint32_t (&xa)[FM], uint32_t (&xb)[FN])
                      __attribute__((always_inline)) {
    constexpr int pp = decltype(pp_c)::value;
    if (f < FM) {
      const int o = s * kSlot + f * 32 * kTileB;
      fa[f] = frag(ba0[pp] + o, ba1[pp] + o, pp_c);
      xa[f] = lds[ca + f * 32 * 16 + 4 * q4 + pp];
    } else {
      const int j = f - FM, o = s * kSlot + j * 32 * kTileB;
      fb[j] = frag(bb0[pp] + o, bb1[pp] + o, pp_c);
      xb[j] = lds[cb + j * 32 * 16 + 4 * q4 + pp];
    }
  };
  auto read_step = [&](int s, auto pp_c, int q4, int ca, int cb, v8i (&fa)[FM], v8i (&fb)[FN],
                       uint32_t (&xa)[FM], uint32_t (&xb)[FN]) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < FM + FN; ++f) read_one(s, pp_c, q4, ca, cb, f, fa, fb, xa, xb);
  };
  // the MFMAs of register set z, the reads of the next step (`next(f)`, one
  // fragment before each of the first FM + FN MFMAs) interleaved in a fixed order
  auto mfmas = [&](int z, auto&& next) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < FM * FN; ++m) {
      const int i = m / FN, j = m % FN;
      if (m < FM + FN) next(m);
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          bf[z][j], af[z][i], acc[i][j], FB, FA, 0, (int)sb[z][j], 0, (int)sa[z][i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- prologue: code group 0 and K tiles 0 .. 2 in flight; wait for K tile 0 ----
  copy_codes(0, 0);
#pragma unroll
  for (int s = 0; s < NS; ++s) copy_tile(s, s);
  FP8GEMM_WAIT_VM_LGKM0((NS - 1) * kLoads);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  read_step(0, std::integral_constant<int, 0>{}, 0, cur_a, cur_b, af[0], bf[0], sa[0], sb[0]);

  // ---- K tile u (k = u mod 12 of the body: slot k mod 3, K tile k mod 4 of
  // its code group) ----
  auto ktile = [&](int u, auto k_c) __attribute__((always_inline)) {
    constexpr int k = decltype(k_c)::value;
    constexpr int slot = k % NS, q4 = k % kGroupTiles, nslot = (k + 1) % NS;
    constexpr bool kNextGroup = q4 == kGroupTiles - 1;   // K tile u + 1 starts a group
    // step 0: fragments of step 1 during the MFMAs of step 0
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xc07f);            // lgkmcnt(0): step 0's fragments in registers
    __builtin_amdgcn_sched_barrier(0);
    mfmas(0, [&](int f) __attribute__((always_inline)) {
      read_one(slot, std::integral_constant<int, 1>{}, q4, cur_a, cur_b, f, af[1], bf[1], sa[1],
               sb[1]);
    });
    // step 1: K tile u + 1 landed for every wave; the slot of K tile u is free
    // (copies issued after K tile u + 1's: K tile u + 2, and a code group when
    // K tile u - 1 started one)
    constexpr int kAfter = kLoads + (((k + kBody - 1) % kGroupTiles == 0) ? kCodeLoads : 0);
    __builtin_amdgcn_sched_barrier(0);
    FP8GEMM_WAIT_VM_LGKM0(kAfter);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (q4 == 0) copy_codes((u / kGroupTiles + 1) & 1, u / kGroupTiles + 1);
    copy_tile(slot, u + NS);
    // (after the last K tile these reads find a stale slot and are never used;
    // a condition here would keep both register sets live across it)
    mfmas(1, [&](int f) __attribute__((always_inline)) {
      if constexpr (kNextGroup)
        read_one(nslot, std::integral_constant<int, 0>{}, 0, nxt_a, nxt_b, f, af[0], bf[0],
                 sa[0], sb[0]);
      else
        read_one(nslot, std::integral_constant<int, 0>{}, q4 + 1, cur_a, cur_b, f, af[0], bf[0],
                 sa[0], sb[0]);
    });
    if constexpr (kNextGroup) {                    // the next group is current from K tile u + 1
      const int ta = cur_a, tb = cur_b;
      cur_a = nxt_a;
      cur_b = nxt_b;
      nxt_a = ta;
      nxt_b = tb;
    }
  };
  // whole bodies without branches (a branch between K tiles makes the compiler
  // shuffle the fragment registers), then the K tiles left one by one
  int u0 = 0;
  for (; u0 + kBody <= nk; u0 += kBody) {
    Unroll<0, kBody>::run([&](auto k_c) __attribute__((always_inline)) {
      ktile(u0 + decltype(k_c)::value, k_c);
    });
  }
  Unroll<0, kBody - 1>::run([&](auto k_c) __attribute__((always_inline)) {
    constexpr int k = decltype(k_c)::value;
    if (u0 + k < nk) ktile(u0 + k, k_c);
  });
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0);                   // no copy may still target LDS
  __builtin_amdgcn_s_barrier();

  OutT* C = static_cast<OutT*>(p.C);
  if (a_rows == BM && b_rows == BN)
    epilogue_full_tile<Cfg, MODE, OutT, FUSED>(acc, lds, C, p.ldc, m0, p.M, n0, p.N, 1.0f, p.bias,
                                               p.act, p.cs, p.ldcs);
  else
    epilogue_any_tile<Cfg, MODE, OutT, FUSED>(acc, lds, C, p.ldc, m0, p.M, n0, p.N, 1.0f, p.bias,
                                              p.act, p.cs, p.ldcs);
}

}  // namespace big

template <int FA, int FB, typename OutT, bool FUSED>
hipError_t launch_typed(const GemmProblem& p, hipStream_t stream) {
  if (choose_path_fp6(p.M, p.N, p.K, p.lda, p.ldb) == kPathTile256) {
    const int tiles_m = (p.M + big::BM - 1) / big::BM, tiles_n = (p.N + big::BN - 1) / big::BN;
    hipLaunchKernelGGL((big::fp6_big_kernel<FA, FB, kMx32, OutT, FUSED>),
                       dim3(tiles_m * tiles_n), dim3(256), 0, stream, p, tiles_m, tiles_n);
    return hipGetLastError();
  }
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  hipLaunchKernelGGL((fp6_kernel<FA, FB, kMx32, OutT, FUSED>), dim3(tiles_m * tiles_n),
                     dim3(256), 0, stream, p, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int FA, int FB>
hipError_t launch_formats(const GemmProblem& p, int out, hipStream_t stream) {
  const bool fused = p.bias != nullptr || p.act != kActNone;
  if (out == kE4M3Mx) return launch_typed<FA, FB, uint8_t, true>(p, stream);
  if (out == kBF16Max)
    return fused ? launch_typed<FA, FB, bf16_max, true>(p, stream)
                 : launch_typed<FA, FB, bf16_max, false>(p, stream);
  if (out == kF16)
    return fused ? launch_typed<FA, FB, _Float16, true>(p, stream)
                 : launch_typed<FA, FB, _Float16, false>(p, stream);
  return fused ? launch_typed<FA, FB, __bf16, true>(p, stream)
               : launch_typed<FA, FB, __bf16, false>(p, stream);
}

}  // namespace
}  // namespace fp6

hipError_t launch_gemm_fp6(const GemmProblem& p, int fmt_a, int fmt_b, int out,
                           hipStream_t stream) {
  using namespace fp6;
  if (p.K % 128 != 0) return hipErrorInvalidValue;
  if (fmt_a == kE2M3 && fmt_b == kE2M3) return launch_formats<kE2M3, kE2M3>(p, out, stream);
  if (fmt_a == kE3M2 && fmt_b == kE3M2) return launch_formats<kE3M2, kE3M2>(p, out, stream);
  if (fmt_a == kE2M3 && fmt_b == kE3M2) return launch_formats<kE2M3, kE3M2>(p, out, stream);
  if (fmt_a == kE3M2 && fmt_b == kE2M3) return launch_formats<kE3M2, kE2M3>(p, out, stream);
  return hipErrorInvalidValue;
}

}  // namespace fp8gemm
