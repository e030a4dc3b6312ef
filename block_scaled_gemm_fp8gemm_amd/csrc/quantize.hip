// fp32 -> e4m3fn quantisation kernels for gfx950 (scale computation and encoding).
//
// What is computed (the E4M3 operands with per-block scale factors of the
// JAX/Triton Blackwell FP8 GEMM post, the row-wise FP8 GEMM of "Hopper/Blackwell
// architecture features" §12.3.4 and the MXFP8 format of its §12.6.1):
//   per-tensor : s = fl32(amax / 448) over the whole tensor (1 if amax = 0),
//                q = RNE_sat(fl32(x / s))
//   row-wise   : the same with one amax per row (reduction along K)
//   MX (32)    : per 32-element K block, E8M0 code = clamp(floor(log2 amax) - 8 + 127,
//                0, 254) (127 if amax = 0), q = RNE_sat(x * 2^(127 - code))
//
// All kernels are HBM-streaming: 16 consecutive fp32 (four 16-byte loads) per
// thread and unit of work, one 16-byte store of codes, reductions by wavefront
// shuffles and LDS.  The division is IEEE binary32 (correctly rounded), as the
// codes must be bit-exact.  Per-tensor scaling takes two passes (partial maxima,
// then quantise) because the scale depends on the whole tensor; the other modes
// read each element once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_utils.h"
#include "launch.h"

namespace fp8gemm {
namespace {

constexpr int kThreads = 256;

typedef float f4 __attribute__((ext_vector_type(4)));

struct Vec16 {
  f4 v[4];
};

__device__ __forceinline__ Vec16 load16(const float* p) {
  const f4* p4 = reinterpret_cast<const f4*>(p);
  Vec16 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.v[i] = __builtin_nontemporal_load(p4 + i);
  return r;
}

__device__ __forceinline__ float absmax16(const Vec16& x) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = fmaxf(m, fmaxf(fmaxf(fabsf(x.v[i].x), fabsf(x.v[i].y)),
                       fmaxf(fabsf(x.v[i].z), fabsf(x.v[i].w))));
  }
  return m;
}

// Quotient by s (binary32 division), then encode: 16 codes in a uint4.
__device__ __forceinline__ uint4 encode16_div(const Vec16& x, float s) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = encode4_e4m3(x.v[i].x / s, x.v[i].y / s, x.v[i].z / s, x.v[i].w / s);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Exact power-of-two scaling by 2^e, then encode.
__device__ __forceinline__ uint4 encode16_ldexp(const Vec16& x, int e) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = encode4_e4m3(ldexpf(x.v[i].x, e), ldexpf(x.v[i].y, e), ldexpf(x.v[i].z, e),
                        ldexpf(x.v[i].w, e));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Block-wide max of one value per thread (kThreads threads).
__device__ __forceinline__ float block_max(float v, float* lds) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[wave] = v;
  __syncthreads();
  float r = lds[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, lds[i]);
  __syncthreads();
  return r;
}

// ---- per-tensor: pass 1, one partial maximum per workgroup -------------------
__global__ __launch_bounds__(kThreads) void amax_partial_kernel(const float* __restrict__ x,
                                                                uint32_t units_per_row,
                                                                uint32_t units, int64_t ldx,
                                                                float* __restrict__ partials) {
  __shared__ float red[kThreads / 64];
  float m = 0.0f;
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < units; u += stride) {
    const uint32_t r = u / units_per_row;
    const uint32_t c = u - r * units_per_row;
    m = fmaxf(m, absmax16(load16(x + (int64_t)r * ldx + 16 * c)));
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// ---- per-tensor: pass 2, scale from the partial maxima, then encode ----------
__global__ __launch_bounds__(kThreads) void quant_tensor_kernel(
    const float* __restrict__ x, uint32_t units_per_row, uint32_t units, int64_t ldx,
    uint8_t* __restrict__ q, int64_t ldq, const float* __restrict__ partials, int nparts,
    float* __restrict__ scale_out) {
  __shared__ float red[kThreads / 64];
  float m = 0.0f;
  for (int i = threadIdx.x; i < nparts; i += kThreads) m = fmaxf(m, partials[i]);
  const float amax = block_max(m, red);
  const float s = (amax == 0.0f) ? 1.0f : amax / kE4M3Max;
  if (blockIdx.x == 0 && threadIdx.x == 0) scale_out[0] = s;
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < units; u += stride) {
    const uint32_t r = u / units_per_row;
    const uint32_t c = u - r * units_per_row;
    const Vec16 v = load16(x + (int64_t)r * ldx + 16 * c);
    *reinterpret_cast<uint4*>(q + (int64_t)r * ldq + 16 * c) = encode16_div(v, s);
  }
}

// ---- row-wise: one lane group of T threads per row, U units cached per thread --
template <int T, int U>
__global__ __launch_bounds__(kThreads) void quant_row_kernel(const float* __restrict__ x, int rows,
                                                             int units_per_row, int64_t ldx,
                                                             uint8_t* __restrict__ q, int64_t ldq,
                                                             float* __restrict__ scales) {
  static_assert(T == 64 || T == 128 || T == 256, "row group is 1, 2 or 4 wavefronts");
  constexpr int kRowsPerBlock = kThreads / T;
  constexpr int kWavesPerRow = T / 64;
  __shared__ float red[kThreads / 64];
  const int g = threadIdx.x / T;  // row slot in this block
  const int t = threadIdx.x % T;
  for (int row0 = blockIdx.x * kRowsPerBlock; row0 < rows; row0 += gridDim.x * kRowsPerBlock) {
    const int r = row0 + g;
    const bool live = r < rows;
    const float* xr = x + (int64_t)(live ? r : 0) * ldx;
    Vec16 v[U];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int c = t + j * T;
      if (live && c < units_per_row) {
        v[j] = load16(xr + 16 * c);
        m = fmaxf(m, absmax16(v[j]));
      }
    }
    m = wave_max(m);
    if (kWavesPerRow > 1) {
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
      __syncthreads();
      m = red[g * kWavesPerRow];
#pragma unroll
      for (int i = 1; i < kWavesPerRow; ++i) m = fmaxf(m, red[g * kWavesPerRow + i]);
      __syncthreads();
    }
    const float s = (m == 0.0f) ? 1.0f : m / kE4M3Max;
    if (live && t == 0) scales[r] = s;
    uint8_t* qr = q + (int64_t)(live ? r : 0) * ldq;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int c = t + j * T;
      if (live && c < units_per_row)
        *reinterpret_cast<uint4*>(qr + 16 * c) = encode16_div(v[j], s);
    }
  }
}

// ---- row-wise, long rows: two passes over the row (the second mostly from cache)
__global__ __launch_bounds__(kThreads) void quant_row_long_kernel(
    const float* __restrict__ x, int rows, int units_per_row, int64_t ldx,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ scales) {
  __shared__ float red[kThreads / 64];
  for (int r = blockIdx.x; r < rows; r += gridDim.x) {
    const float* xr = x + (int64_t)r * ldx;
    float m = 0.0f;
    for (int c = threadIdx.x; c < units_per_row; c += kThreads) m = fmaxf(m, absmax16(load16(xr + 16 * c)));
    m = block_max(m, red);
    const float s = (m == 0.0f) ? 1.0f : m / kE4M3Max;
    if (threadIdx.x == 0) scales[r] = s;
    uint8_t* qr = q + (int64_t)r * ldq;
    for (int c = threadIdx.x; c < units_per_row; c += kThreads)
      *reinterpret_cast<uint4*>(qr + 16 * c) = encode16_div(load16(xr + 16 * c), s);
  }
}

// ---- MX: two lanes per 32-element block, 16 elements each ----------------------
__global__ __launch_bounds__(kThreads) void quant_mx_kernel(const float* __restrict__ x,
                                                            uint32_t blocks_per_row,
                                                            uint32_t blocks, int64_t ldx,
                                                            uint8_t* __restrict__ q, int64_t ldq,
                                                            uint8_t* __restrict__ codes) {
  const uint32_t stride = gridDim.x * (kThreads / 2);
  const int half = threadIdx.x & 1;
  // every lane runs the same number of iterations so the pair shuffle is always matched
  for (uint32_t b0 = blockIdx.x * (kThreads / 2); b0 < blocks; b0 += stride) {
    const uint32_t bi = b0 + (threadIdx.x >> 1);
    const bool live = bi < blocks;
    const uint32_t r = live ? bi / blocks_per_row : 0;
    const uint32_t c = live ? bi - r * blocks_per_row : 0;
    Vec16 v;
    float m = 0.0f;
    if (live) {
      v = load16(x + (int64_t)r * ldx + 32 * c + 16 * half);
      m = absmax16(v);
    }
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    const uint32_t code = mx_code_from_amax(m);
    if (live) {
      *reinterpret_cast<uint4*>(q + (int64_t)r * ldq + 32 * c + 16 * half) =
          encode16_ldexp(v, 127 - (int)code);
      if (half == 0) codes[(int64_t)r * blocks_per_row + c] = (uint8_t)code;
    }
  }
}

int grid_for(uint64_t work_items, int per_block, int cap) {
  uint64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > (uint64_t)cap) g = cap;
  return (int)g;
}

}  // namespace

hipError_t launch_quantize_tensor(const float* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* q,
                                  int64_t ldq, float* scale, float* partials, hipStream_t stream) {
  const uint32_t upr = (uint32_t)(k / 16);
  const uint32_t units = (uint32_t)(rows * upr);
  const int grid = grid_for(units, kThreads, kQuantPartials);
  hipLaunchKernelGGL(amax_partial_kernel, dim3(grid), dim3(kThreads), 0, stream, x, upr, units,
                     ldx, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grid2 = grid_for(units, kThreads, 4096);
  hipLaunchKernelGGL(quant_tensor_kernel, dim3(grid2), dim3(kThreads), 0, stream, x, upr, units,
                     ldx, q, ldq, partials, grid, scale);
  return hipGetLastError();
}

template <int T, int U>
static void launch_row(const float* x, int rows, int upr, int64_t ldx, uint8_t* q, int64_t ldq,
                       float* scales, hipStream_t stream) {
  const int rows_per_block = kThreads / T;
  const int grid = grid_for((uint64_t)rows, rows_per_block, 65535);
  hipLaunchKernelGGL((quant_row_kernel<T, U>), dim3(grid), dim3(kThreads), 0, stream, x, rows, upr,
                     ldx, q, ldq, scales);
}

hipError_t launch_quantize_rowwise(const float* x, int64_t rows, int64_t k, int64_t ldx,
                                   uint8_t* q, int64_t ldq, float* scales, hipStream_t stream) {
  const int upr = (int)(k / 16);
  const int r = (int)rows;
  if (upr <= 64) launch_row<64, 1>(x, r, upr, ldx, q, ldq, scales, stream);
  else if (upr <= 128) launch_row<128, 1>(x, r, upr, ldx, q, ldq, scales, stream);
  else if (upr <= 256) launch_row<256, 1>(x, r, upr, ldx, q, ldq, scales, stream);
  else if (upr <= 512) launch_row<256, 2>(x, r, upr, ldx, q, ldq, scales, stream);
  else if (upr <= 1024) launch_row<256, 4>(x, r, upr, ldx, q, ldq, scales, stream);
  else {
    const int grid = grid_for((uint64_t)rows, 1, 65535);
    hipLaunchKernelGGL(quant_row_long_kernel, dim3(grid), dim3(kThreads), 0, stream, x, r, upr,
                       ldx, q, ldq, scales);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_mx(const float* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* q,
                              int64_t ldq, uint8_t* codes, hipStream_t stream) {
  const uint32_t bpr = (uint32_t)(k / 32);
  const uint32_t blocks = (uint32_t)(rows * bpr);
  const int grid = grid_for(blocks, kThreads / 2, 8192);
  hipLaunchKernelGGL(quant_mx_kernel, dim3(grid), dim3(kThreads), 0, stream, x, bpr, blocks, ldx,
                     q, ldq, codes);
  return hipGetLastError();
}

}  // namespace fp8gemm
