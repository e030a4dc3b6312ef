// Byte-matrix transpose for gfx950: the row-major [K, N] B operand (N contiguous,
// the layout of the pages' Triton listings, e.g. "Hopper/Blackwell architecture
// features" §12.7.1, where b_ptr advances by BLOCK_K * stride_bk) turned into the
// K-contiguous [N][K] rows the GEMM's copies read, and its MX codes [K/32][N] into
// [N][K/32].  HBM-bound: each byte is read once and written once.
//
// A workgroup transposes a 64 x 64 byte tile through LDS: 256 threads read it as
// 64 rows of four 16-byte pieces, and write the transposed tile the same way
// (each thread gathers its 16 output bytes from one LDS column).  Tiles cut by the
// matrix edge move byte by byte, guarded.  Packed FP4 codes (two per byte) take a
// nibble transpose with the same tile shape in elements.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace fp8gemm {
namespace {

constexpr int kT = 64;              // tile edge (bytes)
constexpr int kPitch = kT + 4;      // LDS row pitch (bytes), off the bank period

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void transpose_u8_kernel(const uint8_t* __restrict__ in,
                                                           int64_t ldi, uint8_t* __restrict__ out,
                                                           int64_t ldo, int rows, int cols,
                                                           int tiles_c) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kT * kPitch];
  const int tr = blockIdx.x / tiles_c, tc = blockIdx.x % tiles_c;
  const int r0 = tr * kT, c0 = tc * kT;
  const int t = threadIdx.x;
  const int lr = t >> 2, lc = (t & 3) * 16;         // this thread's row and 16-byte piece
  const bool full = r0 + kT <= rows && c0 + kT <= cols;
  // in: rows r0 .. r0+63, columns c0 .. c0+63
  if (full && (((uintptr_t)in | (uintptr_t)ldi) & 15) == 0) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(in + (int64_t)(r0 + lr) * ldi + c0 + lc);
    uint32_t* dst = reinterpret_cast<uint32_t*>(tile + lr * kPitch + lc);   // 4-byte aligned
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = v[e];
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = r0 + lr, c = c0 + lc + e;
      tile[lr * kPitch + lc + e] = (r < rows && c < cols) ? in[(int64_t)r * ldi + c] : 0;
    }
  }
  __syncthreads();
  // out: rows c0 .. c0+63 (input columns), columns r0 .. r0+63 (input rows)
  uint8_t b[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) b[e] = tile[(lc + e) * kPitch + lr];
  const int orow = c0 + lr, ocol = r0 + lc;
  if (full && (((uintptr_t)out | (uintptr_t)ldo) & 15) == 0) {
    u32x4 v;
    __builtin_memcpy(&v, b, 16);
    *reinterpret_cast<u32x4*>(out + (int64_t)orow * ldo + ocol) = v;
  } else if (orow < cols) {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (ocol + e < rows) out[(int64_t)orow * ldo + ocol + e] = b[e];
  }
}

// Nibble transpose of a packed FP4 matrix: in holds rows x cols 4-bit codes, two
// per byte along a row (element (r, c) in byte in[r * ldi + c / 2], low nibble for
// even c); out receives the cols x rows transpose packed the same way (element
// (c, r) in byte out[c * ldo + r / 2]).  rows % 2 == 0, so every output byte takes
// two whole input rows.  A workgroup moves a 64 x 64 element tile: 256 threads
// read it as 64 rows of four 8-byte pieces into LDS, then each thread assembles 8
// output bytes (16 consecutive input rows of one column) from one LDS column.
__global__ __launch_bounds__(256) void transpose_u4_kernel(const uint8_t* __restrict__ in,
                                                           int64_t ldi, uint8_t* __restrict__ out,
                                                           int64_t ldo, int rows, int cols,
                                                           int tiles_c) {
  constexpr int kB = kT / 2;                        // bytes per tile row
  __shared__ __attribute__((aligned(16))) uint8_t tile[kT * (kB + 4)];
  const int tr = blockIdx.x / tiles_c, tc = blockIdx.x % tiles_c;
  const int r0 = tr * kT, c0 = tc * kT;             // elements
  const int t = threadIdx.x;
  const int lr = t >> 2, lb = (t & 3) * 8;          // tile row, first byte of the piece
  const int cb = (cols + 1) / 2;                    // bytes of an input row
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = r0 + lr, b = c0 / 2 + lb + e;
    tile[lr * (kB + 4) + lb + e] = (r < rows && b < cb) ? in[(int64_t)r * ldi + b] : 0;
  }
  __syncthreads();
  // output row c0 + oc (an input column), bytes for input rows r0 + 16 q .. + 15
  const int oc = t >> 2, q = t & 3;
  const int c = c0 + oc;
  const int shift = (oc & 1) * 4;
  uint8_t ob[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int lr0 = 16 * q + 2 * e;
    const uint8_t lo = (tile[lr0 * (kB + 4) + oc / 2] >> shift) & 0xF;
    const uint8_t hi = (tile[(lr0 + 1) * (kB + 4) + oc / 2] >> shift) & 0xF;
    ob[e] = (uint8_t)(lo | (hi << 4));
  }
  if (c < cols) {
    const int ob0 = (r0 + 16 * q) / 2;               // first output byte of the run
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (2 * (ob0 + e) < rows) out[(int64_t)c * ldo + ob0 + e] = ob[e];
  }
}

}  // namespace

hipError_t launch_transpose_u4(const uint8_t* in, int64_t ldi, uint8_t* out, int64_t ldo,
                               int64_t rows, int64_t cols, hipStream_t stream) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int64_t tiles_r = (rows + kT - 1) / kT, tiles_c = (cols + kT - 1) / kT;
  hipLaunchKernelGGL(transpose_u4_kernel, dim3((unsigned)(tiles_r * tiles_c)), dim3(256), 0,
                     stream, in, ldi, out, ldo, (int)rows, (int)cols, (int)tiles_c);
  return hipGetLastError();
}

hipError_t launch_transpose_u8(const uint8_t* in, int64_t ldi, uint8_t* out, int64_t ldo,
                               int64_t rows, int64_t cols, hipStream_t stream) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int64_t tiles_r = (rows + kT - 1) / kT, tiles_c = (cols + kT - 1) / kT;
  hipLaunchKernelGGL(transpose_u8_kernel, dim3((unsigned)(tiles_r * tiles_c)), dim3(256), 0,
                     stream, in, ldi, out, ldo, (int)rows, (int)cols, (int)tiles_c);
  return hipGetLastError();
}

}  // namespace fp8gemm
