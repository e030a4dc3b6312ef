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
    epilogue<Cfg, MODE, OutT>(acc, lds, C, p.ldc, m0, p.M, n0, p.N, 1.0f);
}

template <int FA, int FB, typename OutT, bool FUSED>
hipError_t launch_typed(const GemmProblem& p, hipStream_t stream) {
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  hipLaunchKernelGGL((fp6_kernel<FA, FB, kMx32, OutT, FUSED>), dim3(tiles_m * tiles_n),
                     dim3(256), 0, stream, p, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int FA, int FB>
hipError_t launch_formats(const GemmProblem& p, int out, hipStream_t stream) {
  const bool fused = p.bias != nullptr || p.act != kActNone;
  if (out == kE4M3Mx) return launch_typed<FA, FB, uint8_t, true>(p, stream);
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
