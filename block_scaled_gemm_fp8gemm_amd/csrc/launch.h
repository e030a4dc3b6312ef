// Internal launch entry points of the gfx950 kernels (host side).  Arguments are
// validated by the C ABI layer (api.cpp) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8gemm {

// Compute units of the current device, queried once per device and cached (256
// on an MI355X; the persistent kernels launch one workgroup per CU).
int device_cu_count();

// Per-tensor quantisation keeps one partial maximum per workgroup of its first pass.
constexpr int kQuantPartials = 1024;

// fmt: element format of the codes (kE4M3 or kE5M2, device_utils.h).
hipError_t launch_quantize_tensor(const float* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* q,
                                  int64_t ldq, float* scale, float* partials, int fmt,
                                  hipStream_t stream);
hipError_t launch_quantize_rowwise(const float* x, int64_t rows, int64_t k, int64_t ldx,
                                   uint8_t* q, int64_t ldq, float* scales, int fmt,
                                   hipStream_t stream);
hipError_t launch_quantize_mx(const float* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* q,
                              int64_t ldq, uint8_t* codes, int fmt, hipStream_t stream);

enum ScaleMode : int { kTensor = 0, kRowwise = 1, kMx32 = 2 };
// kE4M3Mx: e4m3 codes with an E8M0 scale per 32 columns of each row (the fused
// epilogue quantises the output for the next layer; codes to C, scales to cs).
// kBF16Max: the bf16 result to C exactly as kBF16 writes it, and the maxima of
// the stored values' magnitudes folded into cs, read as uint32_t (atomic max on
// the bits of non-negative floats): one per row when ldcs != 0, one for the whole
// output when ldcs == 0; the first half of the requantised output
// (launch_requant encodes).
enum OutType : int { kF16 = 0, kBF16 = 1, kE4M3Mx = 2, kBF16Max = 3 };
// Element formats of the codes; the values are the operand-format fields of the
// F8F6F4 MFMA (e2m3 / e3m2 = FP6, four codes in three bytes; e2m1 = FP4, two
// codes per byte; the narrow formats take MX scales only).
enum ElemFormat : int { kE4M3 = 0, kE5M2 = 1, kE2M3 = 2, kE3M2 = 3, kE2M1 = 4 };
// Activation of the fused epilogue (applied after the scales and the bias).
enum Activation : int { kActNone = 0, kActRelu = 1, kActGelu = 2, kActSilu = 3 };

struct GemmProblem {
  int M, N, K;
  const uint8_t* A;
  int64_t lda;
  const uint8_t* B;
  int64_t ldb;
  const void* scale_a;
  const void* scale_b;
  void* C;
  int64_t ldc;
  void* workspace;      // split-K partials and tile counters (gemm_workspace_bytes)
  const float* bias;    // fused epilogue: fp32 [N] added after the scales, or null
  int act;              // fused epilogue: Activation applied last
  uint8_t* cs = nullptr;  // kE4M3Mx: E8M0 codes of C, cs[m * ldcs + n / 32]; kBF16Max: maxima
  int64_t ldcs = 0;
};

// The split-K arrival counters: the first kSplitCounterBytes of a GEMM workspace,
// whatever the shape (every call leaves the counters it used at zero).
constexpr int64_t kSplitCounterBytes = 4096;

// Device workspace a dense GEMM of this shape needs (0: none).  Shapes with too
// few output tiles to fill the GPU are split along K; the workspace then holds
// the fp32 partial tiles and one arrival counter per output tile.  The counters
// must be zero before the first call and every call leaves them zero.
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int mode);

hipError_t launch_gemm(const GemmProblem& p, int mode, int out, hipStream_t stream);
// The same GEMM for e5m2 operands (A format first, then B).
hipError_t launch_gemm_e5m2_e5m2(const GemmProblem& p, int mode, int out, hipStream_t stream);
hipError_t launch_gemm_e4m3_e5m2(const GemmProblem& p, int mode, int out, hipStream_t stream);
hipError_t launch_gemm_e5m2_e4m3(const GemmProblem& p, int mode, int out, hipStream_t stream);
// The same GEMMs with B row-major [K][N] (ldb: bytes between K-rows; MX codes of
// B [K/32][N]) read by the kernels through transposing LDS reads; only for
// shapes where choose_path_kn() finds a path (else hipErrorInvalidValue).
hipError_t launch_gemm_kn(const GemmProblem& p, int mode, int out, hipStream_t stream);
hipError_t launch_gemm_kn_e5m2_e5m2(const GemmProblem& p, int mode, int out, hipStream_t stream);
hipError_t launch_gemm_kn_e4m3_e5m2(const GemmProblem& p, int mode, int out, hipStream_t stream);
hipError_t launch_gemm_kn_e5m2_e4m3(const GemmProblem& p, int mode, int out, hipStream_t stream);
// MXFP4 with row-major B: K and lda as launch_gemm_e2m1_e2m1 (bytes), B K-rows of
// ldb bytes holding two codes per byte along N (mode kMx32, 16-bit outputs).
hipError_t launch_gemm_kn_e2m1_e2m1(const GemmProblem& p, int mode, int out, hipStream_t stream);
// MXFP4 x MXFP4 (mode kMx32 only): K, lda and ldb of the problem count bytes
// (two e2m1 codes each), the E8M0 codes stay one per 32 elements.
hipError_t launch_gemm_e2m1_e2m1(const GemmProblem& p, int mode, int out, hipStream_t stream);
// MXFP6 (e2m3 / e3m2 operands, MX scales): K counts elements (K % 128 == 0),
// lda and ldb bytes (four codes in three bytes).
hipError_t launch_gemm_fp6(const GemmProblem& p, int fmt_a, int fmt_b, int out,
                           hipStream_t stream);

struct GroupedProblem {
  int groups;
  int total_m, N, K;
  const uint8_t* A;
  int64_t lda;
  const int32_t* offsets;
  const uint8_t* B;
  int64_t ldb, stride_b;
  const void* scale_a;
  const void* scale_b;
  void* C;
  int64_t ldc;
};

// Second half of the requantised output: y bf16 [rows][n] (pitch ldy elements,
// a multiple of 8) to codes q (fmt kE4M3 or kE5M2, pitch ldq bytes) with s =
// fl32(amax / max of the format) (1 if amax = 0) and q = RNE_sat(fl32(y / s)),
// the quantisers' rule on y's values.  per_row: amax[r] (uint32_t bits of a
// non-negative float) for row r and scales[r] = s; else amax[0] and scales[0] for
// every row.  n % 8 == 0 (whole 8-byte code groups).
hipError_t launch_requant(const uint16_t* y, int64_t rows, int64_t n, int64_t ldy,
                          const uint32_t* amax, bool per_row, uint8_t* q, int64_t ldq,
                          float* scales, int fmt, hipStream_t stream);
// p[0 .. count) = 0 with a kernel (no memset node, so the call can be captured).
hipError_t launch_zero_words(uint32_t* p, int64_t count, hipStream_t stream);

// out[c][r] = in[r][c] for a rows x cols byte matrix (row pitches ldi >= cols and
// ldo >= rows bytes): the row-major B operand and its MX codes made K-contiguous.
hipError_t launch_transpose_u8(const uint8_t* in, int64_t ldi, uint8_t* out, int64_t ldo,
                               int64_t rows, int64_t cols, hipStream_t stream);
// The same for packed FP4 codes (two per byte along a row, low nibble first):
// element (r, c) at in[r * ldi + c / 2] goes to out[c * ldo + r / 2]; rows even.
hipError_t launch_transpose_u4(const uint8_t* in, int64_t ldi, uint8_t* out, int64_t ldo,
                               int64_t rows, int64_t cols, hipStream_t stream);

hipError_t launch_grouped_gemm(const GroupedProblem& p, int mode, int out, hipStream_t stream);
// MXFP4 experts (mode kMx32 only; K, lda, ldb and stride_b count bytes).
hipError_t launch_grouped_gemm_e2m1_e2m1(const GroupedProblem& p, int mode, int out,
                                         hipStream_t stream);

}  // namespace fp8gemm
