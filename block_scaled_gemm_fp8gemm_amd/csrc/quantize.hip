// fp32 -> e4m3fn / e5m2 / e2m3 / e3m2 / e2m1 quantisation kernels for gfx950
// (scale computation and encoding).
//
// What is computed (the E4M3 operands with per-block scale factors of the
// JAX/Triton Blackwell FP8 GEMM post, the row-wise FP8 GEMM of "Hopper/Blackwell
// architecture features" §12.3.4 and the MXFP8 format of its §12.6.1):
//   per-tensor : s = fl32(amax / 448) over the whole tensor (1 if amax = 0),
//                q = RNE_sat(fl32(x / s))
//   row-wise   : the same with one amax per row (reduction along K)
//   MX (32)    : per 32-element K block, E8M0 code = clamp(floor(log2 amax) - 8 + 127,
//                0, 254) (127 if amax = 0), q = RNE_sat(x * 2^(127 - code))
// and the same with 57344 and 15 in place of 448 and 8 for e5m2 codes (the post's
// second FP8 format); MX only, 6 and 2 for e2m1 (FP4, two codes per byte, the
// first in the low nibble: the MXFP4 format of the architecture page's §12.6.1),
// 7.5 and 2 for e2m3 and 28 and 4 for e3m2 (FP6, the MXFP6 elements of the same
// table; four codes in three bytes, a little-endian 6-bit stream).
//
// All kernels are HBM-streaming.  The unit of work is 1024 consecutive values of
// a row, taken by one wavefront so that every load and store instruction covers
// one contiguous KiB (see load_unit); maxima are reduced with wavefront shuffles
// and LDS.  The division is IEEE binary32 (correctly rounded), as the codes must
// be bit-exact.  Per-tensor scaling takes two passes (partial maxima, then
// quantise) because the scale depends on the whole tensor; the other modes read
// each element once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_utils.h"
#include "launch.h"

namespace fp8gemm {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

typedef float f4 __attribute__((ext_vector_type(4)));

// A unit is 1024 consecutive values of one row, handled by one wavefront: lane l
// holds the float4s at columns 256 j + 4 l (j = 0..3), so each of the four loads
// (and each of the four code stores) covers one contiguous KiB across the
// wavefront and every cache line is fetched by a single instruction.  Columns at
// or past k are neither read nor written (and count as zero for the maxima).
struct Unit {
  f4 v[4];
};

__device__ __forceinline__ Unit load_unit(const float* row, int col0, int k, int lane) {
  Unit u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = col0 + 256 * j + 4 * lane;
    u.v[j] = c < k ? __builtin_nontemporal_load(reinterpret_cast<const f4*>(row + c)) : f4{};
  }
  return u;
}

__device__ __forceinline__ void store_codes(uint8_t* qrow, int col0, int k, int lane,
                                            const uint32_t (&w)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = col0 + 256 * j + 4 * lane;
    if (c < k) *reinterpret_cast<uint32_t*>(qrow + c) = w[j];
  }
}

__device__ __forceinline__ float absmax4(f4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

__device__ __forceinline__ float absmax_unit(const Unit& u) {
  return fmaxf(fmaxf(absmax4(u.v[0]), absmax4(u.v[1])), fmaxf(absmax4(u.v[2]), absmax4(u.v[3])));
}

// Quotient by s (binary32 division), then encode.
template <int FMT>
__device__ __forceinline__ void encode_unit_div(const Unit& u, float s, uint32_t (&w)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = encode4<FMT>(u.v[j].x / s, u.v[j].y / s, u.v[j].z / s, u.v[j].w / s);
}

// Block-wide max of one value per thread.
__device__ __forceinline__ float block_max(float v, float* lds) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[wave] = v;
  __syncthreads();
  float r = lds[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = fmaxf(r, lds[i]);
  __syncthreads();
  return r;
}

// ---- per-tensor: pass 1, one partial maximum per workgroup -------------------
// Units are dealt to wavefronts in turn, two per wavefront and iteration.
__global__ __launch_bounds__(kThreads) void amax_partial_kernel(const float* __restrict__ x, int k,
                                                                int upr, int units,
                                                                int64_t ldx,
                                                                float* __restrict__ partials) {
  __shared__ float red[kWaves];
  const int lane = threadIdx.x & 63;
  const int w0 = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int nw = gridDim.x * kWaves;
  float m = 0.0f;
  for (int u = w0; u < units; u += 2 * nw) {
    const int u2 = u + nw;
    const int r = u / upr, r2 = u2 / upr;
    const Unit a = load_unit(x + (int64_t)r * ldx, (u - r * upr) * 1024, k, lane);
    Unit b{};
    if (u2 < units) b = load_unit(x + (int64_t)r2 * ldx, (u2 - r2 * upr) * 1024, k, lane);
    m = fmaxf(m, fmaxf(absmax_unit(a), absmax_unit(b)));
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// ---- per-tensor: pass 2, scale from the partial maxima, then encode ----------
template <int FMT>
__global__ __launch_bounds__(kThreads) void quant_tensor_kernel(
    const float* __restrict__ x, int k, int upr, int units, int64_t ldx,
    uint8_t* __restrict__ q, int64_t ldq, const float* __restrict__ partials, int nparts,
    float* __restrict__ scale_out) {
  __shared__ float red[kWaves];
  float m = 0.0f;
  for (int i = threadIdx.x; i < nparts; i += kThreads) m = fmaxf(m, partials[i]);
  const float amax = block_max(m, red);
  const float s = (amax == 0.0f) ? 1.0f : amax / elem_max<FMT>();
  if (blockIdx.x == 0 && threadIdx.x == 0) scale_out[0] = s;
  const int lane = threadIdx.x & 63;
  const int w0 = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int nw = gridDim.x * kWaves;
  for (int u = w0; u < units; u += 2 * nw) {
    const int u2 = u + nw;
    const int r = u / upr, r2 = u2 / upr;
    const int c0 = (u - r * upr) * 1024, c2 = (u2 - r2 * upr) * 1024;
    const Unit a = load_unit(x + (int64_t)r * ldx, c0, k, lane);
    Unit b{};
    if (u2 < units) b = load_unit(x + (int64_t)r2 * ldx, c2, k, lane);
    uint32_t w[4];
    encode_unit_div<FMT>(a, s, w);
    store_codes(q + (int64_t)r * ldq, c0, k, lane, w);
    if (u2 < units) {
      encode_unit_div<FMT>(b, s, w);
      store_codes(q + (int64_t)r2 * ldq, c2, k, lane, w);
    }
  }
}

// ---- row-wise: one workgroup per row, the row cached in registers -------------
// Wave w holds units w, w + 4, ... (up to U of them); rows longer than 4 U units
// take the two-pass kernel below.
template <int U, int FMT>
__global__ __launch_bounds__(kThreads) void quant_row_kernel(const float* __restrict__ x, int rows,
                                                             int k, int upr, int64_t ldx,
                                                             uint8_t* __restrict__ q, int64_t ldq,
                                                             float* __restrict__ scales) {
  __shared__ float red[kWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int r = blockIdx.x; r < rows; r += gridDim.x) {
    const float* xr = x + (int64_t)r * ldx;
    Unit v[U];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = wave + j * kWaves;
      v[j] = u < upr ? load_unit(xr, u * 1024, k, lane) : Unit{};
      m = fmaxf(m, absmax_unit(v[j]));
    }
    m = block_max(m, red);
    const float s = (m == 0.0f) ? 1.0f : m / elem_max<FMT>();
    if (threadIdx.x == 0) scales[r] = s;
    uint8_t* qr = q + (int64_t)r * ldq;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = wave + j * kWaves;
      if (u < upr) {
        uint32_t w[4];
        encode_unit_div<FMT>(v[j], s, w);
        store_codes(qr, u * 1024, k, lane, w);
      }
    }
  }
}

// ---- row-wise, long rows: two passes over the row (the second mostly from cache)
template <int FMT>
__global__ __launch_bounds__(kThreads) void quant_row_long_kernel(
    const float* __restrict__ x, int rows, int k, int upr, int64_t ldx, uint8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scales) {
  __shared__ float red[kWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int r = blockIdx.x; r < rows; r += gridDim.x) {
    const float* xr = x + (int64_t)r * ldx;
    float m = 0.0f;
    for (int u = wave; u < upr; u += kWaves) m = fmaxf(m, absmax_unit(load_unit(xr, u * 1024, k, lane)));
    m = block_max(m, red);
    const float s = (m == 0.0f) ? 1.0f : m / elem_max<FMT>();
    if (threadIdx.x == 0) scales[r] = s;
    uint8_t* qr = q + (int64_t)r * ldq;
    for (int u = wave; u < upr; u += kWaves) {
      uint32_t w[4];
      encode_unit_div<FMT>(load_unit(xr, u * 1024, k, lane), s, w);
      store_codes(qr, u * 1024, k, lane, w);
    }
  }
}

// ---- MX: a 32-element block is one float4 of 8 consecutive lanes ---------------
// Block maxima by xor-shuffles inside each group of 8 lanes; the first lane of a
// group writes the block's E8M0 code.
template <int FMT>
__device__ __forceinline__ void mx_unit(const Unit& u, uint8_t* qrow, uint8_t* crow, int col0,
                                        int k, int lane) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float m = absmax4(u.v[j]);
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    m = fmaxf(m, __shfl_xor(m, 4, 64));
    const uint32_t code = mx_code_from_amax<FMT>(m);
    const int e = 127 - (int)code;
    const float x0 = ldexpf(u.v[j].x, e), x1 = ldexpf(u.v[j].y, e);
    const float x2 = ldexpf(u.v[j].z, e), x3 = ldexpf(u.v[j].w, e);
    if constexpr (FMT == kE2M1) w[j] = encode4_e2m1(x0, x1, x2, x3);
    else if constexpr (FMT == kE2M3 || FMT == kE3M2) w[j] = encode4_fp6<FMT>(x0, x1, x2, x3);
    else w[j] = encode4<FMT>(x0, x1, x2, x3);
    const int c = col0 + 256 * j + 4 * lane;
    if ((lane & 7) == 0 && c < k) crow[c >> 5] = (uint8_t)code;
  }
  if constexpr (FMT == kE2M3 || FMT == kE3M2) {
    // Four codes in three bytes: the lane's float4 is 24 bits; lanes 4i .. 4i + 3
    // (16 columns) make the 96-bit run at byte 192 j + 12 i, stored as three
    // dwords by lanes 4i, 4i + 1, 4i + 2 (dword t = bits 32t .. 32t + 31: the
    // lane's own 24 bits shifted down by 8t and the next lane's shifted up).
    const int t = lane & 3;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t nxt = (uint32_t)__shfl_down((int)w[j], 1, 64);
      const uint32_t word = (w[j] >> (8 * t)) | (t < 3 ? nxt << (24 - 8 * t) : 0u);
      const int cg = col0 + 256 * j + 16 * (lane >> 2);   // first column of the run
      if (t < 3 && cg < k) *reinterpret_cast<uint32_t*>(qrow + cg / 4 * 3 + 4 * t) = word;
    }
  } else if constexpr (FMT == kE2M1) {
    // Two codes per byte: lane l holds the 16 bits of bytes 128 j + 2 l and + 1.
    // Lanes 2i and 2i + 1 swap halves so that the even lane stores the word at
    // 128 j + 4 i for j = 0, 2 and the odd lane the one for j = 1, 3: two 4-byte
    // stores per lane, each instruction covering two 128-byte runs.
    const bool odd = lane & 1;
    const int pair = lane >> 1;
#pragma unroll
    for (int jp = 0; jp < 4; jp += 2) {
      const uint32_t keep = odd ? w[jp + 1] : w[jp];
      const uint32_t give = odd ? w[jp] : w[jp + 1];
      const uint32_t got = (uint32_t)__shfl_xor((int)give, 1, 64);
      const uint32_t word = odd ? (got | (keep << 16)) : (keep | (got << 16));
      const int j = jp + (odd ? 1 : 0);
      const int c = col0 + 256 * j + 8 * pair;          // first of the word's 8 columns
      if (c < k) *reinterpret_cast<uint32_t*>(qrow + (c >> 1)) = word;
    }
  } else {
    store_codes(qrow, col0, k, lane, w);
  }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void quant_mx_kernel(const float* __restrict__ x, int k,
                                                            int upr, int units, int64_t ldx,
                                                            uint8_t* __restrict__ q, int64_t ldq,
                                                            uint8_t* __restrict__ codes) {
  const int lane = threadIdx.x & 63;
  const int w0 = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int nw = gridDim.x * kWaves;
  const int bpr = k / 32;
  for (int u = w0; u < units; u += 2 * nw) {
    const int u2 = u + nw;
    const int r = u / upr, r2 = u2 / upr;
    const int c0 = (u - r * upr) * 1024, c2 = (u2 - r2 * upr) * 1024;
    const Unit a = load_unit(x + (int64_t)r * ldx, c0, k, lane);
    Unit b{};
    if (u2 < units) b = load_unit(x + (int64_t)r2 * ldx, c2, k, lane);
    mx_unit<FMT>(a, q + (int64_t)r * ldq, codes + (int64_t)r * bpr, c0, k, lane);
    if (u2 < units) mx_unit<FMT>(b, q + (int64_t)r2 * ldq, codes + (int64_t)r2 * bpr, c2, k, lane);
  }
}

// ---- the requantised GEMM output: maxima from the GEMM epilogue, then encode ---
// The GEMM kernels stored y in bf16 and folded the stored values' magnitudes into
// amax (per row or one for the output; zeroed by zero_words_kernel before the
// GEMM); this pass derives the scales by the per-tensor / row-wise rule above and
// encodes y's values (exact in fp32) with it, as quantising the bf16 output
// would.  One wavefront per row (rows dealt to wavefronts in turn), 2048 columns
// per step: lane l takes the 8 values at columns 512 j + 8 l (j = 0 .. 3), so
// each 16-byte load and 8-byte code store instruction covers one contiguous run.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int FMT, bool PER_ROW>
__global__ __launch_bounds__(kThreads) void requant_kernel(const uint16_t* __restrict__ y,
                                                           int rows, int n, int64_t ldy,
                                                           const uint32_t* __restrict__ amax,
                                                           uint8_t* __restrict__ q, int64_t ldq,
                                                           float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int w0 = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int nw = gridDim.x * kWaves;
  float s = 1.0f;
  if constexpr (!PER_ROW) {
    const float m = __uint_as_float(amax[0]);
    s = (m == 0.0f) ? 1.0f : m / elem_max<FMT>();
    if (blockIdx.x == 0 && threadIdx.x == 0) scales[0] = s;
  }
  for (int r = w0; r < rows; r += nw) {
    if constexpr (PER_ROW) {
      const float m = __uint_as_float(amax[r]);
      s = (m == 0.0f) ? 1.0f : m / elem_max<FMT>();
      if (lane == 0) scales[r] = s;
    }
    const uint16_t* yr = y + (int64_t)r * ldy;
    uint8_t* qr = q + (int64_t)r * ldq;
    // 2048 columns per step: the four loads go out before any is used
    for (int c0 = 0; c0 < n; c0 += 2048) {
      u32x4 w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = c0 + 512 * j + 8 * lane;
        w[j] = c < n ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(yr + c)) : u32x4{};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = c0 + 512 * j + 8 * lane;
        if (c < n) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(w[j][e] << 16);
            x[2 * e + 1] = __uint_as_float(w[j][e] & 0xffff0000u);
          }
          uint2 o;
          o.x = encode4<FMT>(x[0] / s, x[1] / s, x[2] / s, x[3] / s);
          o.y = encode4<FMT>(x[4] / s, x[5] / s, x[6] / s, x[7] / s);
          *reinterpret_cast<uint2*>(qr + c) = o;
        }
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void zero_words_kernel(uint32_t* __restrict__ p,
                                                              int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * kThreads)
    p[i] = 0u;
}

int grid_for(uint64_t work_items, int per_block, int cap) {
  uint64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > (uint64_t)cap) g = cap;
  return (int)g;
}

template <int FMT>
hipError_t quantize_tensor_fmt(const float* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* q,
                               int64_t ldq, float* scale, float* partials, hipStream_t stream) {
  const int upr = (int)((k + 1023) / 1024);
  const int units = (int)(rows * upr);
  // two units per wavefront and iteration
  const int grid = grid_for((uint64_t)units, 2 * kWaves, kQuantPartials);
  hipLaunchKernelGGL(amax_partial_kernel, dim3(grid), dim3(kThreads), 0, stream, x, (int)k, upr,
                     units, ldx, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grid2 = grid_for((uint64_t)units, 2 * kWaves, 8192);
  hipLaunchKernelGGL((quant_tensor_kernel<FMT>), dim3(grid2), dim3(kThreads), 0, stream, x,
                     (int)k, upr, units, ldx, q, ldq, partials, grid, scale);
  return hipGetLastError();
}

template <int FMT>
hipError_t quantize_rowwise_fmt(const float* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* q,
                                int64_t ldq, float* scales, hipStream_t stream) {
  const int upr = (int)((k + 1023) / 1024);
  const int r = (int)rows;
  const int grid = grid_for((uint64_t)rows, 1, 65535);
  if (upr <= kWaves)
    hipLaunchKernelGGL((quant_row_kernel<1, FMT>), dim3(grid), dim3(kThreads), 0, stream, x, r,
                       (int)k, upr, ldx, q, ldq, scales);
  else if (upr <= 2 * kWaves)
    hipLaunchKernelGGL((quant_row_kernel<2, FMT>), dim3(grid), dim3(kThreads), 0, stream, x, r,
                       (int)k, upr, ldx, q, ldq, scales);
  else if (upr <= 4 * kWaves)
    hipLaunchKernelGGL((quant_row_kernel<4, FMT>), dim3(grid), dim3(kThreads), 0, stream, x, r,
                       (int)k, upr, ldx, q, ldq, scales);
  else
    hipLaunchKernelGGL((quant_row_long_kernel<FMT>), dim3(grid), dim3(kThreads), 0, stream, x, r,
                       (int)k, upr, ldx, q, ldq, scales);
  return hipGetLastError();
}

template <int FMT>
hipError_t quantize_mx_fmt(const float* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* q,
                           int64_t ldq, uint8_t* codes, hipStream_t stream) {
  const int upr = (int)((k + 1023) / 1024);
  const int units = (int)(rows * upr);
  const int grid = grid_for((uint64_t)units, 2 * kWaves, 8192);
  hipLaunchKernelGGL((quant_mx_kernel<FMT>), dim3(grid), dim3(kThreads), 0, stream, x, (int)k,
                     upr, units, ldx, q, ldq, codes);
  return hipGetLastError();
}

template <int FMT>
hipError_t requant_fmt(const uint16_t* y, int64_t rows, int64_t n, int64_t ldy,
                       const uint32_t* amax, bool per_row, uint8_t* q, int64_t ldq, float* scales,
                       hipStream_t stream) {
  const int grid = grid_for((uint64_t)rows, kWaves, 16384);
  if (per_row)
    hipLaunchKernelGGL((requant_kernel<FMT, true>), dim3(grid), dim3(kThreads), 0, stream, y,
                       (int)rows, (int)n, ldy, amax, q, ldq, scales);
  else
    hipLaunchKernelGGL((requant_kernel<FMT, false>), dim3(grid), dim3(kThreads), 0, stream, y,
                       (int)rows, (int)n, ldy, amax, q, ldq, scales);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_tensor(const float* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* q,
                                  int64_t ldq, float* scale, float* partials, int fmt,
                                  hipStream_t stream) {
  if (fmt == kE5M2)
    return quantize_tensor_fmt<kE5M2>(x, rows, k, ldx, q, ldq, scale, partials, stream);
  return quantize_tensor_fmt<kE4M3>(x, rows, k, ldx, q, ldq, scale, partials, stream);
}

hipError_t launch_quantize_rowwise(const float* x, int64_t rows, int64_t k, int64_t ldx,
                                   uint8_t* q, int64_t ldq, float* scales, int fmt,
                                   hipStream_t stream) {
  if (fmt == kE5M2) return quantize_rowwise_fmt<kE5M2>(x, rows, k, ldx, q, ldq, scales, stream);
  return quantize_rowwise_fmt<kE4M3>(x, rows, k, ldx, q, ldq, scales, stream);
}

hipError_t launch_quantize_mx(const float* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* q,
                              int64_t ldq, uint8_t* codes, int fmt, hipStream_t stream) {
  if (fmt == kE5M2) return quantize_mx_fmt<kE5M2>(x, rows, k, ldx, q, ldq, codes, stream);
  if (fmt == kE2M1) return quantize_mx_fmt<kE2M1>(x, rows, k, ldx, q, ldq, codes, stream);
  if (fmt == kE2M3) return quantize_mx_fmt<kE2M3>(x, rows, k, ldx, q, ldq, codes, stream);
  if (fmt == kE3M2) return quantize_mx_fmt<kE3M2>(x, rows, k, ldx, q, ldq, codes, stream);
  return quantize_mx_fmt<kE4M3>(x, rows, k, ldx, q, ldq, codes, stream);
}

hipError_t launch_zero_words(uint32_t* p, int64_t count, hipStream_t stream) {
  const int grid = grid_for((uint64_t)count, kThreads, 1024);
  hipLaunchKernelGGL(zero_words_kernel, dim3(grid), dim3(kThreads), 0, stream, p, count);
  return hipGetLastError();
}

hipError_t launch_requant(const uint16_t* y, int64_t rows, int64_t n, int64_t ldy,
                          const uint32_t* amax, bool per_row, uint8_t* q, int64_t ldq,
                          float* scales, int fmt, hipStream_t stream) {
  if (fmt == kE5M2)
    return requant_fmt<kE5M2>(y, rows, n, ldy, amax, per_row, q, ldq, scales, stream);
  return requant_fmt<kE4M3>(y, rows, n, ldy, amax, per_row, q, ldq, scales, stream);
}

}  // namespace fp8gemm
