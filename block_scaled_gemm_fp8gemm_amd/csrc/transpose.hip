// Byte-matrix transpose for gfx950: the row-major [K, N] B operand (N contiguous,
// the layout of the pages' Triton listings, e.g. "Hopper/Blackwell architecture
// features" §12.7.1, where b_ptr advances by BLOCK_K * stride_bk) turned into the
// K-contiguous [N][K] rows the GEMM's copies read, and its MX codes [K/32][N] into
// [N][K/32].  HBM-bound: each byte is read once and written once.
//
// A workgroup transposes a 64 x 64 byte tile through LDS: 256 threads read it as
// 64 rows of four 16-byte pieces, and write the transposed tile the same way
// (each thread gathers its 16 output bytes from one LDS column).  Tiles cut by the
// matrix edge move byte by byte, guarded.
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

}  // namespace

hipError_t launch_transpose_u8(const uint8_t* in, int64_t ldi, uint8_t* out, int64_t ldo,
                               int64_t rows, int64_t cols, hipStream_t stream) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int64_t tiles_r = (rows + kT - 1) / kT, tiles_c = (cols + kT - 1) / kT;
  hipLaunchKernelGGL(transpose_u8_kernel, dim3((unsigned)(tiles_r * tiles_c)), dim3(256), 0,
                     stream, in, ldi, out, ldo, (int)rows, (int)cols, (int)tiles_c);
  return hipGetLastError();
}

}  // namespace fp8gemm
