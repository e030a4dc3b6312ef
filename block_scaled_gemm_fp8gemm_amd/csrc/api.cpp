// C ABI of the scaled FP8 GEMM library: argument validation and kernel dispatch.
//
// Every check runs on the host before the first HIP call, so an invalid call
// returns its status without touching the device (this is also what lets the
// error paths be tested on machines without a GPU).  The rules follow the
// descriptor constraints of "Hopper/Blackwell architecture features" §12.2.3
// (16-byte aligned base, unit stride in the last dimension, other strides a
// multiple of 16 bytes): here they are requirements of the 16-byte vector and
// direct-to-LDS loads, and a violation is an error rather than a slow path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/fp8gemm.h"
#include "launch.h"
#include "plan.h"

namespace fp8gemm {

// One cached CU count per device (0 = not queried yet).  Concurrent first calls
// may both query; they store the same value.
int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace fp8gemm

namespace {

using fp8gemm::kMx32;
using fp8gemm::kRowwise;
using fp8gemm::kTensor;

constexpr int64_t kMaxDim = INT32_MAX;
constexpr int kMaxGroups = 1024;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_mode(int mode) { return mode == kTensor || mode == kRowwise || mode == kMx32; }
bool valid_out(int out) { return out == FP8GEMM_OUT_F16 || out == FP8GEMM_OUT_BF16; }
bool valid_format(int f) {
  return f == FP8GEMM_FORMAT_E4M3 || f == FP8GEMM_FORMAT_E5M2 || f == FP8GEMM_FORMAT_E2M3 ||
         f == FP8GEMM_FORMAT_E3M2 || f == FP8GEMM_FORMAT_E2M1;
}
bool is_fp6(int f) { return f == FP8GEMM_FORMAT_E2M3 || f == FP8GEMM_FORMAT_E3M2; }
// bits of one code of format f (packed formats share bytes)
int code_bits(int f) { return f == FP8GEMM_FORMAT_E2M1 ? 4 : is_fp6(f) ? 6 : 8; }
bool valid_act(int a) {
  return a == FP8GEMM_ACT_NONE || a == FP8GEMM_ACT_RELU || a == FP8GEMM_ACT_GELU ||
         a == FP8GEMM_ACT_SILU;
}

fp8gemm_status from_hip(hipError_t e) {
  return e == hipSuccess ? FP8GEMM_SUCCESS : FP8GEMM_ERROR_LAUNCH;
}

// Checks shared by the dense and grouped GEMM (M is the number of A rows; bits is
// the size of one operand code: 8, 6 for FP6 or 4 for FP4, so a row of K codes
// takes K * bits / 8 bytes and K must keep rows of whole 16-byte chunks).
fp8gemm_status check_gemm_common(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                                 const uint8_t* B, int64_t ldb, int mode, const void* scale_a,
                                 const void* scale_b, const void* C, int64_t ldc, int out,
                                 int bits = 8) {
  if (!A || !B || !C || !scale_a || !scale_b) return FP8GEMM_ERROR_INVALID_VALUE;
  if (lda * 8 < K * bits || ldb * 8 < K * bits || ldc < N) return FP8GEMM_ERROR_INVALID_VALUE;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim || lda > kMaxDim || ldb > kMaxDim ||
      ldc > kMaxDim)
    return FP8GEMM_ERROR_NOT_SUPPORTED;
  if ((K * bits) % 128 != 0) return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (mode == kMx32 && K % 32 != 0) return FP8GEMM_ERROR_NOT_SUPPORTED;
  // the grid is one workgroup per 128 x 128 tile at most: keep it below 2^31
  if (((M + 127) / 128) * ((N + 127) / 128) > kMaxDim) return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16)) return FP8GEMM_ERROR_MISALIGNED;
  if (lda % 16 != 0 || ldb % 16 != 0 || (ldc * 2) % 16 != 0) return FP8GEMM_ERROR_MISALIGNED;
  if (!aligned(scale_a, 4) || !aligned(scale_b, 4)) return FP8GEMM_ERROR_MISALIGNED;
  (void)out;
  return FP8GEMM_SUCCESS;
}

}  // namespace

extern "C" {

size_t fp8gemm_quantize_workspace_size(int64_t rows, int64_t k, int mode) {
  (void)rows;
  (void)k;
  return mode == kTensor ? sizeof(float) * fp8gemm::kQuantPartials : 0;
}

fp8gemm_status fp8gemm_quantize(const float* x, int64_t rows, int64_t k, int64_t ldx, int mode,
                                uint8_t* q, int64_t ldq, void* scales, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return fp8gemm_quantize_ex(x, rows, k, ldx, mode, FP8GEMM_FORMAT_E4M3, q, ldq, scales, workspace,
                             workspace_bytes, stream);
}

fp8gemm_status fp8gemm_quantize_ex(const float* x, int64_t rows, int64_t k, int64_t ldx, int mode,
                                   int format, uint8_t* q, int64_t ldq, void* scales,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_mode(mode) || !valid_format(format) || rows < 0 || k <= 0)
    return FP8GEMM_ERROR_INVALID_VALUE;
  const int bits = code_bits(format);
  if (bits < 8 && mode != kMx32) return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (rows == 0) return FP8GEMM_SUCCESS;
  if (!x || !q || !scales) return FP8GEMM_ERROR_INVALID_VALUE;
  if (ldx < k || ldq * 8 < k * bits) return FP8GEMM_ERROR_INVALID_VALUE;
  if (k % 16 != 0) return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (mode == kMx32 && k % 32 != 0) return FP8GEMM_ERROR_NOT_SUPPORTED;
  // 32-bit unit indexing inside the kernels: at most 2^32 - 1 elements per call
  if (rows > kMaxDim || ldx > kMaxDim || ldq > kMaxDim || rows * k >= (int64_t(1) << 32))
    return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (!aligned(x, 16) || !aligned(q, 16)) return FP8GEMM_ERROR_MISALIGNED;
  if ((ldx * 4) % 16 != 0 || ldq % 16 != 0) return FP8GEMM_ERROR_MISALIGNED;
  if (mode != kMx32 && !aligned(scales, 4)) return FP8GEMM_ERROR_MISALIGNED;
  const size_t need = fp8gemm_quantize_workspace_size(rows, k, mode);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 4)))
    return FP8GEMM_ERROR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == kTensor)
    return from_hip(fp8gemm::launch_quantize_tensor(x, rows, k, ldx, q, ldq,
                                                    static_cast<float*>(scales),
                                                    static_cast<float*>(workspace), format, s));
  if (mode == kRowwise)
    return from_hip(fp8gemm::launch_quantize_rowwise(x, rows, k, ldx, q, ldq,
                                                     static_cast<float*>(scales), format, s));
  return from_hip(fp8gemm::launch_quantize_mx(x, rows, k, ldx, q, ldq,
                                              static_cast<uint8_t*>(scales), format, s));
}

size_t fp8gemm_workspace_size(int64_t M, int64_t N, int64_t K, int mode) {
  if (!valid_mode(mode) || M <= 0 || N <= 0 || K <= 0) return 0;
  return fp8gemm::gemm_workspace_bytes(M, N, K, mode);
}

fp8gemm_status fp8gemm_run(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                           const uint8_t* B, int64_t ldb, int mode, const void* scale_a,
                           const void* scale_b, void* C, int64_t ldc, int out_dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return fp8gemm_run_ex(M, N, K, A, lda, FP8GEMM_FORMAT_E4M3, B, ldb, FP8GEMM_FORMAT_E4M3, mode,
                        scale_a, scale_b, nullptr, FP8GEMM_ACT_NONE, C, ldc, out_dtype, workspace,
                        workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The dense GEMM behind fp8gemm_run_ex (16-bit outputs), fp8gemm_run_mxout
// (out_dtype kE4M3Mx: e4m3 codes to C, E8M0 codes to cs) and fp8gemm_run_qout
// (kBF16Max: the bf16 output to C and its maxima to cs).
fp8gemm_status run_dense(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                         int a_format, const uint8_t* B, int64_t ldb, int b_format, int mode,
                         const void* scale_a, const void* scale_b, const float* bias,
                         int activation, void* C, int64_t ldc, int out_dtype, uint8_t* cs,
                         int64_t ldcs, void* workspace, size_t workspace_bytes, void* stream,
                         bool dry_run = false) {
  const bool qout = out_dtype == fp8gemm::kE4M3Mx;
  const bool bfmax = out_dtype == fp8gemm::kBF16Max;     // bf16 y + maxima (requantised output)
  if (!valid_mode(mode) || !(valid_out(out_dtype) || qout || bfmax) || !valid_format(a_format) ||
      !valid_format(b_format) || !valid_act(activation) || M < 0 || N < 0 || K <= 0)
    return FP8GEMM_ERROR_INVALID_VALUE;
  // FP4 pairs with FP4 only, FP6 with FP6 (e2m3 / e3m2 in any pairing), both
  // with MX block scales only; FP6 needs K % 128 == 0
  const bool fp4 = a_format == FP8GEMM_FORMAT_E2M1 || b_format == FP8GEMM_FORMAT_E2M1;
  const bool fp6 = is_fp6(a_format) || is_fp6(b_format);
  if (fp4 && (a_format != b_format || mode != kMx32)) return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (fp6 && (!is_fp6(a_format) || !is_fp6(b_format) || mode != kMx32))
    return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (fp6 && K % 128 != 0) return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (M == 0 || N == 0) return FP8GEMM_SUCCESS;
  if (qout) {
    if (!cs || ldcs < N / 32) return FP8GEMM_ERROR_INVALID_VALUE;
    if (N % 32 != 0) return FP8GEMM_ERROR_NOT_SUPPORTED;
    if (ldcs > kMaxDim) return FP8GEMM_ERROR_NOT_SUPPORTED;
    if (ldc % 16 != 0) return FP8GEMM_ERROR_MISALIGNED;      // byte rows of codes
  }
  fp8gemm_status st = check_gemm_common(M, N, K, A, lda, B, ldb, mode, scale_a, scale_b, C, ldc,
                                        out_dtype, fp4 ? 4 : fp6 ? 6 : 8);
  if (st != FP8GEMM_SUCCESS) return st;
  if (bias && !aligned(bias, 4)) return FP8GEMM_ERROR_MISALIGNED;
  // FP6 tiles: 128 rows of A (and of B) addressed with 32-bit buffer offsets
  if (fp6 && (127 * lda + K / 4 * 3 >= ((int64_t)1 << 31) ||
              127 * ldb + K / 4 * 3 >= ((int64_t)1 << 31)))
    return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (dry_run) return FP8GEMM_SUCCESS;              // every check but the workspace's passed
  // FP4 shapes split along K at most as often as FP8 ones of the same element
  // count, so the query (K in elements) covers them too
  const size_t need = fp8gemm_workspace_size(M, N, K, mode);
  if (need > 0 && (!workspace || workspace_bytes < need)) return FP8GEMM_ERROR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 16)) return FP8GEMM_ERROR_MISALIGNED;

  fp8gemm::GemmProblem p;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)(fp4 ? K / 2 : K);        // FP4: the kernels walk K in bytes
  p.A = A;
  p.lda = lda;
  p.B = B;
  p.ldb = ldb;
  p.scale_a = scale_a;
  p.scale_b = scale_b;
  p.C = C;
  p.ldc = ldc;
  p.workspace = need > 0 ? workspace : nullptr;
  p.bias = bias;
  p.act = activation;
  p.cs = cs;
  p.ldcs = ldcs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fp6) {
    p.K = (int)K;                        // the FP6 kernel walks K in elements
    p.workspace = nullptr;
    return from_hip(fp8gemm::launch_gemm_fp6(p, a_format, b_format, out_dtype, s));
  }
  if (fp4) return from_hip(fp8gemm::launch_gemm_e2m1_e2m1(p, mode, out_dtype, s));
  if (a_format == FP8GEMM_FORMAT_E5M2 && b_format == FP8GEMM_FORMAT_E5M2)
    return from_hip(fp8gemm::launch_gemm_e5m2_e5m2(p, mode, out_dtype, s));
  if (a_format == FP8GEMM_FORMAT_E5M2)
    return from_hip(fp8gemm::launch_gemm_e5m2_e4m3(p, mode, out_dtype, s));
  if (b_format == FP8GEMM_FORMAT_E5M2)
    return from_hip(fp8gemm::launch_gemm_e4m3_e5m2(p, mode, out_dtype, s));
  return from_hip(fp8gemm::launch_gemm(p, mode, out_dtype, s));
}

}  // namespace

extern "C" {

fp8gemm_status fp8gemm_run_ex(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                              int a_format, const uint8_t* B, int64_t ldb, int b_format, int mode,
                              const void* scale_a, const void* scale_b, const float* bias,
                              int activation, void* C, int64_t ldc, int out_dtype,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_out(out_dtype)) return FP8GEMM_ERROR_INVALID_VALUE;
  return run_dense(M, N, K, A, lda, a_format, B, ldb, b_format, mode, scale_a, scale_b, bias,
                   activation, C, ldc, out_dtype, nullptr, 0, workspace, workspace_bytes, stream);
}

fp8gemm_status fp8gemm_run_mxout(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                                 int a_format, const uint8_t* B, int64_t ldb, int b_format,
                                 int mode, const void* scale_a, const void* scale_b,
                                 const float* bias, int activation, uint8_t* C, int64_t ldc,
                                 uint8_t* c_scales, int64_t ldcs, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return run_dense(M, N, K, A, lda, a_format, B, ldb, b_format, mode, scale_a, scale_b, bias,
                   activation, C, ldc, fp8gemm::kE4M3Mx, c_scales, ldcs, workspace,
                   workspace_bytes, stream);
}

namespace {

// Workspace of the requantised output: the dense GEMM's own first (never less
// than its 4 KiB of split-K counters, so that no call of another shape finds y
// there), then the maxima (M words, zeroed by each call), then y in bf16 with
// rows of 128-byte multiples.
struct QoutLayout {
  size_t maxima, y, total;
  int64_t ldy;
};

QoutLayout qout_layout(int64_t M, int64_t N, int64_t K, int mode) {
  auto up = [](size_t v, size_t a) { return (v + a - 1) / a * a; };
  QoutLayout l;
  size_t g = fp8gemm::gemm_workspace_bytes(M, N, K, mode);
  if (g < (size_t)fp8gemm::kSplitCounterBytes) g = fp8gemm::kSplitCounterBytes;
  l.maxima = up(g, 256);
  l.y = l.maxima + up((size_t)M * 4, 256);
  l.ldy = (int64_t)up((size_t)N, 64);
  l.total = l.y + (size_t)M * (size_t)l.ldy * 2;
  return l;
}

}  // namespace

size_t fp8gemm_qout_workspace_size(int64_t M, int64_t N, int64_t K, int mode) {
  if (!valid_mode(mode) || M <= 0 || N <= 0 || K <= 0) return 0;
  return qout_layout(M, N, K, mode).total;
}

fp8gemm_status fp8gemm_run_qout(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                                int a_format, const uint8_t* B, int64_t ldb, int b_format,
                                int mode, const void* scale_a, const void* scale_b,
                                const float* bias, int activation, int out_mode, int c_format,
                                uint8_t* C, int64_t ldc, float* c_scales, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if ((out_mode != kTensor && out_mode != kRowwise) || !valid_format(c_format))
    return FP8GEMM_ERROR_INVALID_VALUE;
  // every check of the GEMM itself, with the codes standing in for its output
  fp8gemm_status st =
      run_dense(M, N, K, A, lda, a_format, B, ldb, b_format, mode, scale_a, scale_b, bias,
                activation, C, ldc, fp8gemm::kBF16Max, nullptr, 0, nullptr, 0, stream, true);
  if (st != FP8GEMM_SUCCESS || M == 0 || N == 0) return st;
  if (c_format != FP8GEMM_FORMAT_E4M3 && c_format != FP8GEMM_FORMAT_E5M2)
    return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (!c_scales) return FP8GEMM_ERROR_INVALID_VALUE;
  if (N % 16 != 0) return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (ldc % 16 != 0 || !aligned(c_scales, 4)) return FP8GEMM_ERROR_MISALIGNED;
  const QoutLayout l = qout_layout(M, N, K, mode);
  if (!workspace || workspace_bytes < l.total) return FP8GEMM_ERROR_WORKSPACE;
  if (!aligned(workspace, 16)) return FP8GEMM_ERROR_MISALIGNED;

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint32_t* maxima = reinterpret_cast<uint32_t*>(ws + l.maxima);
  uint16_t* y = reinterpret_cast<uint16_t*>(ws + l.y);
  const bool per_row = out_mode == kRowwise;
  hipError_t e = fp8gemm::launch_zero_words(maxima, per_row ? M : 1, s);
  if (e != hipSuccess) return FP8GEMM_ERROR_LAUNCH;
  st = run_dense(M, N, K, A, lda, a_format, B, ldb, b_format, mode, scale_a, scale_b, bias,
                 activation, y, l.ldy, fp8gemm::kBF16Max, reinterpret_cast<uint8_t*>(maxima),
                 per_row ? 1 : 0, workspace, l.maxima, stream);
  if (st != FP8GEMM_SUCCESS) return st;
  return from_hip(fp8gemm::launch_requant(
      y, M, N, l.ldy, maxima, per_row, C, ldc, c_scales,
      c_format == FP8GEMM_FORMAT_E5M2 ? fp8gemm::kE5M2 : fp8gemm::kE4M3, s));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// fp8gemm_run_noalloc: fp8gemm_run_ex for callers that cannot allocate (code
// under graph capture, serving loops that forbid allocation).  The split-K
// counters and partial tiles live in `scratch`, a static device array of
// FP8GEMM_NOALLOC_SCRATCH_BYTES that each device holds from the library's load
// until the process ends.  Host code never uses the array's name as an address
// (on the host it only names the symbol): the first call on a device, with that
// device current, looks its device address up with hipGetSymbolAddress, keeps
// it for the device and zeroes the counter head with a fill kernel on the
// caller's stream; from then on every call leaves the counters at zero.  The
// kernels get that address as their workspace, as fp8gemm_run_ex's kernels get
// the caller's workspace.
// ---------------------------------------------------------------------------
namespace {

static __device__ __align__(256) uint8_t scratch[FP8GEMM_NOALLOC_SCRATCH_BYTES];

__global__ void zero_words(int* p, int n) {
  for (int i = (int)threadIdx.x; i < n; i += (int)blockDim.x) p[i] = 0;
}

// Device address of `scratch` on the current device (nullptr on a HIP error).
void* scratch_address(hipStream_t stream) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    hipLaunchKernelGGL(zero_words, dim3(1), dim3(256), 0, stream, static_cast<int*>(p),
                       (int)(fp8gemm::kSplitCounterBytes / 4));
    if (hipGetLastError() != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

extern "C" {

fp8gemm_status fp8gemm_run_noalloc(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                                   int a_format, const uint8_t* B, int64_t ldb, int b_format,
                                   int mode, const void* scale_a, const void* scale_b,
                                   const float* bias, int activation, void* C, int64_t ldc,
                                   int out_dtype, void* stream) {
  if (!valid_out(out_dtype)) return FP8GEMM_ERROR_INVALID_VALUE;
  // every argument check first, without a workspace and without any HIP call
  fp8gemm_status st = run_dense(M, N, K, A, lda, a_format, B, ldb, b_format, mode, scale_a,
                                scale_b, bias, activation, C, ldc, out_dtype, nullptr, 0, nullptr,
                                0, stream, /*dry_run=*/true);
  if (st != FP8GEMM_SUCCESS || M == 0 || N == 0) return st;
  const size_t need = fp8gemm_workspace_size(M, N, K, mode);
  if (need > (size_t)FP8GEMM_NOALLOC_SCRATCH_BYTES) return FP8GEMM_ERROR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_address(s);
    if (ws == nullptr) return FP8GEMM_ERROR_LAUNCH;
  }
  return run_dense(M, N, K, A, lda, a_format, B, ldb, b_format, mode, scale_a, scale_b, bias,
                   activation, C, ldc, out_dtype, nullptr, 0, ws,
                   need > 0 ? (size_t)FP8GEMM_NOALLOC_SCRATCH_BYTES : 0, stream);
}

// Row-major B: the workspace starts with the GEMM's own workspace (at least the
// split-K counter head, so the counters keep their fixed place and a workspace
// shared with fp8gemm_run calls never has them overwritten), then the
// K-contiguous copy of B ([N][K] bytes) and, for MX, its codes ([N][K/32]), each
// rounded up to 256 bytes.
namespace {
constexpr int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }
int64_t kn_head_bytes(int64_t M, int64_t N, int64_t K, int mode) {
  const int64_t g = (int64_t)fp8gemm_workspace_size(M, N, K, mode);
  return round256(g > fp8gemm::kSplitCounterBytes ? g : fp8gemm::kSplitCounterBytes);
}
int64_t kn_b_bytes(int64_t N, int64_t K) { return round256(N * K); }
int64_t kn_code_bytes(int64_t N, int64_t K, int mode) {
  return mode == kMx32 ? round256(N * (K / 32)) : 0;
}
// Whether fp8gemm_run_kn reads the row-major B inside the GEMM kernels
// (transposing LDS reads) instead of making it K-contiguous in the workspace
// first: FP8 codes or MXFP4 (even N: whole bytes per K-row), MX code rows of
// whole 16-byte chunks, and a shape the in-kernel form takes (K % 128 == 0, MX
// K % 512 == 0, 32-bit spans).
bool kn_in_kernel(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int a_format,
                  int b_format, int mode) {
  const bool fp8 = code_bits(a_format) == 8 && code_bits(b_format) == 8;
  const bool fp4 = a_format == FP8GEMM_FORMAT_E2M1 && b_format == FP8GEMM_FORMAT_E2M1 &&
                   N % 2 == 0;
  return (fp8 || fp4) && (mode != kMx32 || N % 16 == 0) &&
         fp8gemm::choose_path_kn(M, N, K, lda, ldb, mode, fp4) != fp8gemm::kPathNone;
}
}  // namespace

size_t fp8gemm_workspace_size_kn(int64_t M, int64_t N, int64_t K, int mode) {
  if (!valid_mode(mode) || M <= 0 || N <= 0 || K <= 0) return 0;
  return (size_t)(kn_head_bytes(M, N, K, mode) + kn_b_bytes(N, K) + kn_code_bytes(N, K, mode));
}

fp8gemm_status fp8gemm_run_kn(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                              int a_format, const uint8_t* B, int64_t ldb, int b_format, int mode,
                              const void* scale_a, const void* scale_b, const float* bias,
                              int activation, void* C, int64_t ldc, int out_dtype,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_mode(mode) || !valid_out(out_dtype) || !valid_format(a_format) ||
      !valid_format(b_format) || !valid_act(activation) || M < 0 || N < 0 || K <= 0)
    return FP8GEMM_ERROR_INVALID_VALUE;
  // FP8 pairs, or FP4 with FP4 (MX only; row-major FP4 B packs two codes per byte
  // along N); no FP6 here
  const bool fp4 = a_format == FP8GEMM_FORMAT_E2M1 || b_format == FP8GEMM_FORMAT_E2M1;
  if (fp4 && (a_format != b_format || mode != kMx32)) return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (is_fp6(a_format) || is_fp6(b_format)) return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (M == 0 || N == 0) return FP8GEMM_SUCCESS;
  if (!B || !scale_b) return FP8GEMM_ERROR_INVALID_VALUE;
  if (fp4 ? ldb * 2 < N : ldb < N) return FP8GEMM_ERROR_INVALID_VALUE;
  if (N > kMaxDim || K > kMaxDim || ldb > kMaxDim) return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (K % 16 != 0 || (mode == kMx32 && K % 32 != 0)) return FP8GEMM_ERROR_NOT_SUPPORTED;
  // one transpose workgroup per 64 x 64 tile: keep the grid below 2^31
  if (((K + 63) / 64) * ((N + 63) / 64) > kMaxDim) return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (!aligned(B, 16) || ldb % 16 != 0) return FP8GEMM_ERROR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kn_in_kernel(M, N, K, lda, ldb, a_format, b_format, mode)) {
    // B's own checks passed above; the row of a K-contiguous B stands in for its pitch
    fp8gemm_status st = check_gemm_common(M, N, K, A, lda, B, fp4 ? K / 2 : K, mode, scale_a,
                                          scale_b, C, ldc, out_dtype, fp4 ? 4 : 8);
    if (st != FP8GEMM_SUCCESS) return st;
    if (bias && !aligned(bias, 4)) return FP8GEMM_ERROR_MISALIGNED;
    const size_t need = fp8gemm_workspace_size(M, N, K, mode);
    if (need > 0 && (!workspace || workspace_bytes < need)) return FP8GEMM_ERROR_WORKSPACE;
    if (need > 0 && !aligned(workspace, 16)) return FP8GEMM_ERROR_MISALIGNED;
    fp8gemm::GemmProblem p;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)(fp4 ? K / 2 : K);        // FP4: the kernels walk K in bytes of A
    p.A = A;
    p.lda = lda;
    p.B = B;
    p.ldb = ldb;
    p.scale_a = scale_a;
    p.scale_b = scale_b;
    p.C = C;
    p.ldc = ldc;
    p.workspace = need > 0 ? workspace : nullptr;
    p.bias = bias;
    p.act = activation;
    if (fp4) return from_hip(fp8gemm::launch_gemm_kn_e2m1_e2m1(p, mode, out_dtype, s));
    if (a_format == FP8GEMM_FORMAT_E5M2 && b_format == FP8GEMM_FORMAT_E5M2)
      return from_hip(fp8gemm::launch_gemm_kn_e5m2_e5m2(p, mode, out_dtype, s));
    if (a_format == FP8GEMM_FORMAT_E5M2)
      return from_hip(fp8gemm::launch_gemm_kn_e5m2_e4m3(p, mode, out_dtype, s));
    if (b_format == FP8GEMM_FORMAT_E5M2)
      return from_hip(fp8gemm::launch_gemm_kn_e4m3_e5m2(p, mode, out_dtype, s));
    return from_hip(fp8gemm::launch_gemm_kn(p, mode, out_dtype, s));
  }
  const size_t need = fp8gemm_workspace_size_kn(M, N, K, mode);
  if (!workspace || workspace_bytes < need) return FP8GEMM_ERROR_WORKSPACE;
  if (!aligned(workspace, 16)) return FP8GEMM_ERROR_MISALIGNED;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* ws_gemm = ws;
  uint8_t* bt = ws + kn_head_bytes(M, N, K, mode);
  uint8_t* codes_t = bt + kn_b_bytes(N, K);
  const size_t gemm_bytes = fp8gemm_workspace_size(M, N, K, mode);
  // the GEMM's checks run first, on the transposed operands, so a call they
  // reject enqueues nothing
  const int64_t ldbt = fp4 ? K / 2 : K;       // K % 16 == 0 (FP4: K % 32): 16-byte rows
  fp8gemm_status st = check_gemm_common(M, N, K, A, lda, bt, ldbt, mode, scale_a,
                                        mode == kMx32 ? codes_t : scale_b, C, ldc, out_dtype,
                                        fp4 ? 4 : 8);
  if (st != FP8GEMM_SUCCESS) return st;
  if (bias && !aligned(bias, 4)) return FP8GEMM_ERROR_MISALIGNED;
  hipError_t e = fp4 ? fp8gemm::launch_transpose_u4(B, ldb, bt, ldbt, K, N, s)
                     : fp8gemm::launch_transpose_u8(B, ldb, bt, ldbt, K, N, s);
  if (e != hipSuccess) return FP8GEMM_ERROR_LAUNCH;
  const void* sb = scale_b;
  if (mode == kMx32) {
    e = fp8gemm::launch_transpose_u8(static_cast<const uint8_t*>(scale_b), N, codes_t, K / 32,
                                     K / 32, N, s);
    if (e != hipSuccess) return FP8GEMM_ERROR_LAUNCH;
    sb = codes_t;
  }
  return fp8gemm_run_ex(M, N, K, A, lda, a_format, bt, ldbt, b_format, mode, scale_a, sb, bias,
                        activation, C, ldc, out_dtype, gemm_bytes ? ws_gemm : nullptr, gemm_bytes,
                        stream);
}

size_t fp8gemm_grouped_workspace_size(int32_t num_groups, int64_t total_m, int64_t N, int64_t K,
                                      int mode) {
  (void)num_groups;
  (void)total_m;
  (void)N;
  (void)K;
  (void)mode;
  return 0;
}

fp8gemm_status fp8gemm_grouped_run(int32_t num_groups, int64_t total_m, int64_t N, int64_t K,
                                   const uint8_t* A, int64_t lda, const int32_t* offsets,
                                   const uint8_t* B, int64_t ldb, int64_t stride_b, int mode,
                                   const void* scale_a, const void* scale_b, void* C,
                                   int64_t ldc, int out_dtype, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return fp8gemm_grouped_run_ex(num_groups, total_m, N, K, A, lda, FP8GEMM_FORMAT_E4M3, offsets,
                                B, ldb, FP8GEMM_FORMAT_E4M3, stride_b, mode, scale_a, scale_b, C,
                                ldc, out_dtype, workspace, workspace_bytes, stream);
}

fp8gemm_status fp8gemm_grouped_run_ex(int32_t num_groups, int64_t total_m, int64_t N, int64_t K,
                                      const uint8_t* A, int64_t lda, int a_format,
                                      const int32_t* offsets, const uint8_t* B, int64_t ldb,
                                      int b_format, int64_t stride_b, int mode,
                                      const void* scale_a, const void* scale_b, void* C,
                                      int64_t ldc, int out_dtype, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (!valid_mode(mode) || !valid_out(out_dtype) || !valid_format(a_format) ||
      !valid_format(b_format) || num_groups < 1 || total_m < 0 || N < 0 || K <= 0)
    return FP8GEMM_ERROR_INVALID_VALUE;
  // e4m3 experts, or MXFP4 activations and experts
  const bool fp4 = a_format == FP8GEMM_FORMAT_E2M1 && b_format == FP8GEMM_FORMAT_E2M1;
  if (!fp4 && (a_format != FP8GEMM_FORMAT_E4M3 || b_format != FP8GEMM_FORMAT_E4M3))
    return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (fp4 && mode != kMx32) return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (num_groups > kMaxGroups) return FP8GEMM_ERROR_NOT_SUPPORTED;
  if (total_m == 0 || N == 0) return FP8GEMM_SUCCESS;
  if (!offsets) return FP8GEMM_ERROR_INVALID_VALUE;
  fp8gemm_status st = check_gemm_common(total_m, N, K, A, lda, B, ldb, mode, scale_a, scale_b, C,
                                        ldc, out_dtype, fp4 ? 4 : 8);
  if (st != FP8GEMM_SUCCESS) return st;
  if (stride_b < N * ldb) return FP8GEMM_ERROR_INVALID_VALUE;
  if (stride_b % 16 != 0) return FP8GEMM_ERROR_MISALIGNED;
  if (!aligned(offsets, 4)) return FP8GEMM_ERROR_MISALIGNED;
  const size_t need = fp8gemm_grouped_workspace_size(num_groups, total_m, N, K, mode);
  if (need > 0 && (!workspace || workspace_bytes < need)) return FP8GEMM_ERROR_WORKSPACE;

  fp8gemm::GroupedProblem p;
  p.groups = num_groups;
  p.total_m = (int)total_m;
  p.N = (int)N;
  p.K = (int)(fp4 ? K / 2 : K);        // FP4: the kernels walk K in bytes
  p.A = A;
  p.lda = lda;
  p.offsets = offsets;
  p.B = B;
  p.ldb = ldb;
  p.stride_b = stride_b;
  p.scale_a = scale_a;
  p.scale_b = scale_b;
  p.C = C;
  p.ldc = ldc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fp4) return from_hip(fp8gemm::launch_grouped_gemm_e2m1_e2m1(p, mode, out_dtype, s));
  return from_hip(fp8gemm::launch_grouped_gemm(p, mode, out_dtype, s));
}

int fp8gemm_run_path(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int a_format,
                     int b_format, int mode, int fused) {
  if (!valid_mode(mode) || !valid_format(a_format) || !valid_format(b_format) || M < 0 || N < 0 ||
      K <= 0 || lda < 0 || ldb < 0)
    return FP8GEMM_PATH_NONE;
  const bool fp4 = a_format == FP8GEMM_FORMAT_E2M1 || b_format == FP8GEMM_FORMAT_E2M1;
  if (fp4 && (a_format != b_format || mode != kMx32)) return FP8GEMM_PATH_NONE;
  const bool fp6 = is_fp6(a_format) || is_fp6(b_format);
  if (fp6) {
    if (!is_fp6(a_format) || !is_fp6(b_format) || mode != kMx32) return FP8GEMM_PATH_NONE;
    return fp8gemm::choose_path_fp6(M, N, K, lda, ldb);
  }
  return fp8gemm::choose_path(M, N, fp4 ? K / 2 : K, lda, ldb, mode, fp4, fused != 0);
}

int fp8gemm_run_kn_path(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                        int a_format, int b_format, int mode) {
  if (!valid_mode(mode) || !valid_format(a_format) || !valid_format(b_format) || M <= 0 ||
      N <= 0 || K <= 0 || lda < 0 || ldb < 0)
    return FP8GEMM_PATH_NONE;
  if (!kn_in_kernel(M, N, K, lda, ldb, a_format, b_format, mode)) return FP8GEMM_PATH_NONE;
  return fp8gemm::choose_path_kn(M, N, K, lda, ldb, mode, a_format == FP8GEMM_FORMAT_E2M1);
}

const char* fp8gemm_status_string(int status) {
  switch (status) {
    case FP8GEMM_SUCCESS: return "FP8GEMM_SUCCESS";
    case FP8GEMM_ERROR_INVALID_VALUE: return "FP8GEMM_ERROR_INVALID_VALUE";
    case FP8GEMM_ERROR_MISALIGNED: return "FP8GEMM_ERROR_MISALIGNED";
    case FP8GEMM_ERROR_NOT_SUPPORTED: return "FP8GEMM_ERROR_NOT_SUPPORTED";
    case FP8GEMM_ERROR_WORKSPACE: return "FP8GEMM_ERROR_WORKSPACE";
    case FP8GEMM_ERROR_LAUNCH: return "FP8GEMM_ERROR_LAUNCH";
    default: return "FP8GEMM_ERROR_UNKNOWN";
  }
}

int fp8gemm_version(void) { return FP8GEMM_VERSION; }

}  // extern "C"
