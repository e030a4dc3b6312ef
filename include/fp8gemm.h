/*
 * fp8gemm.h - C ABI of the MI355X (gfx950) scaled FP8 GEMM library.
 *
 * The library computes C = (sA . A_e4m3)(sB . B_e4m3) with fp32 accumulation and
 * an fp16 / bf16 epilogue, for per-tensor, row-wise and 32-element microscaled
 * (MX, E8M0 block-scale) operands, and the grouped (mixture-of-experts) form.
 *
 * Sources: the kernels in "Hopper/Blackwell architecture features" §12.7.1 and
 * §12.7.2 take raw pointers, sizes and strides, accumulate into an fp32 tile and
 * cast it on store; the JAX/Triton Blackwell FP8 GEMM post's kernel pseudocode
 * does the same with E4M3 operands and an fp16 result, and its MoE paragraph
 * extends the GEMM to grouped experts.  §12.2.3 of the first page requires 16-byte
 * aligned bases and row strides (16-byte multiples, unit stride in the last
 * dimension); §12.4.3 treats a resource overflow as an error; the Cutlass-named
 * Triton FP8 post's monitoring list asks for launch errors to be checked.
 *
 * Conventions for every entry point
 *   - All data pointers are DEVICE pointers (HIP device memory of the current
 *     device).  Sizes and strides are host integers.  `stream` is a hipStream_t
 *     (NULL = the default stream).
 *   - Calls are asynchronous on `stream`: they validate their arguments on the
 *     host, enqueue kernels and return.  The library never allocates, frees or
 *     synchronizes, and keeps no state between calls.  The caller owns every
 *     buffer and must keep it alive until the enqueued work completes.
 *   - Validation runs before any HIP call; a non-SUCCESS status means nothing
 *     was enqueued (except FP8GEMM_ERROR_LAUNCH, which reports a failed launch).
 *   - A is row-major [M,K] (element (m,k) at A[m*lda+k]).  B is column-major
 *     [K,N], i.e. stored as N rows of K contiguous bytes (element (k,n) at
 *     B[n*ldb+k]).  C is row-major [M,N] (element (m,n) at C[m*ldc+n]).
 *   - Operand codes are OCP e4m3fn bytes (bias 7, no infinity, NaN = S.1111.111,
 *     max 448).  E8M0 scale codes encode 2^(code-127); 0xFF (NaN) is never
 *     produced by fp8gemm_quantize.
 *   - Inputs are expected finite; NaN/Inf inputs give unspecified results.
 *   - Thread safety: calls from several host threads are safe; calls whose
 *     buffers overlap must be ordered by the caller.
 */
#ifndef FP8GEMM_H_
#define FP8GEMM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8GEMM_VERSION 190 /* 1.9.0: e5m2, fused epilogues, row-major B read in-kernel, MXFP4 (dense, grouped), MXFP6 (dense), MX output, requantised output with fresh per-tensor / per-row scales, path queries, no-allocation GEMM */

typedef enum fp8gemm_status {
  FP8GEMM_SUCCESS = 0,
  FP8GEMM_ERROR_INVALID_VALUE = 1, /* null pointer, negative size, ld too small, bad enum */
  FP8GEMM_ERROR_MISALIGNED = 2,    /* pointer or row pitch (bytes) not a multiple of 16   */
  FP8GEMM_ERROR_NOT_SUPPORTED = 3, /* K not a multiple of 16 (32 for MX), or mode not offered */
  FP8GEMM_ERROR_WORKSPACE = 4,     /* workspace missing or smaller than the size query    */
  FP8GEMM_ERROR_LAUNCH = 5         /* a kernel launch failed (hipGetLastError)            */
} fp8gemm_status;

typedef enum fp8gemm_scale_mode {
  FP8GEMM_SCALE_TENSOR = 0,  /* one fp32 scale per operand                         */
  FP8GEMM_SCALE_ROWWISE = 1, /* fp32 scale per row of A / per column of B           */
  FP8GEMM_SCALE_MX32 = 2     /* E8M0 scale per 32 contiguous K elements (MXFP8)     */
} fp8gemm_scale_mode;

typedef enum fp8gemm_out_dtype {
  FP8GEMM_OUT_F16 = 0, /* IEEE binary16, round to nearest even */
  FP8GEMM_OUT_BF16 = 1 /* bfloat16, round to nearest even      */
} fp8gemm_out_dtype;

/* Element format of operand codes (the JAX/Triton Blackwell FP8 GEMM post names
   both FP8 formats, E4M3 and E5M2, in its second paragraph). */
typedef enum fp8gemm_format {
  FP8GEMM_FORMAT_E4M3 = 0, /* OCP e4m3fn: bias 7, no infinity, max 448 (the default)      */
  FP8GEMM_FORMAT_E5M2 = 1, /* OCP e5m2: bias 15, infinities and NaNs, max 57344           */
  /* FP6, the MXFP6 elements (§12.6.1 of the same page lists FP6 with micro-scaling):
     OCP MX e2m3 (bias 1, 3 mantissa bits, max 7.5) and e3m2 (bias 3, 2 mantissa bits,
     max 28), no infinity or NaN, sign = bit 5 of a code.  Four codes in three bytes:
     a row is a little-endian 6-bit stream, element i in bits 6i .. 6i+5 (element
     (r,i) starts at bit 6i of the row's bytes).  MX32 scales only. */
  FP8GEMM_FORMAT_E2M3 = 2,
  FP8GEMM_FORMAT_E3M2 = 3,
  /* FP4, the MXFP4 element ("Hopper/Blackwell architecture features" §12.6.1 lists FP4
     next to FP8 with micro-scaling): OCP MX e2m1, bias 1, magnitudes 0, .5, 1, 1.5, 2,
     3, 4, 6, no infinity or NaN.  Two codes per byte, element 2i in bits 0-3 and
     element 2i+1 in bits 4-7 (sign = bit 3 of a code).  MX32 scales only. */
  FP8GEMM_FORMAT_E2M1 = 4
} fp8gemm_format;

/* Activation of the fused epilogue (the Cutlass-named Triton FP8 post fuses a
   bias_add_relu epilogue to save a round trip of C through memory). */
typedef enum fp8gemm_activation {
  FP8GEMM_ACT_NONE = 0,
  FP8GEMM_ACT_RELU = 1, /* max(y, 0)                              */
  FP8GEMM_ACT_GELU = 2, /* y * (1 + erf(y / sqrt(2))) / 2          */
  FP8GEMM_ACT_SILU = 3  /* y / (1 + exp(-y))                       */
} fp8gemm_activation;

/* ------------------------------------------------------------------------- */
/* Quantisation: fp32 -> e4m3fn codes + scales.                                */
/*                                                                           */
/* Computes the scale and codes the JAX/Triton Blackwell FP8 GEMM post asks for  */
/* (E4M3 operands with per-block scale factors, fine-grained against            */
/* underflow) under these rules:                                              */
/*   TENSOR : amax over all rows*k elements, s = fl32(amax/448) (1 if amax=0),   */
/*            q = RNE_sat(fl32(x/s)); scales -> float[1].                        */
/*   ROWWISE: the same per row (reduction over k); scales -> float[rows].        */
/*            Quantise A with rows=M; quantise a column-major B with rows=N, so */
/*            this gives one scale per column of B.                             */
/*   MX32   : per (row, 32-element block): e = floor(log2 amax) - 8, code =     */
/*            clamp(e+127, 0, 254) (127 if amax = 0), q = RNE_sat(x * 2^-e);    */
/*            scales -> uint8 [rows][k/32], row-major, k/32 bytes per row.     */
/* RNE_sat rounds to the nearest e4m3fn value, ties to even, and saturates to   */
/* +-448; the sign of zero is kept.  Results are bit-exact (deterministic).     */
/*                                                                           */
/* x      : device fp32, element (r,i) at x[r*ldx+i]; ldx >= k, ldx*4 % 16 == 0.  */
/* q      : device uint8 codes, element (r,i) at q[r*ldq+i]; ldq >= k, ldq % 16 == 0.*/
/* k      : > 0, multiple of 16 (of 32 for MX32).  rows >= 0 (0: no work).       */
/* workspace: device memory of fp8gemm_quantize_workspace_size() bytes, 16-byte  */
/*          aligned (NULL allowed when the size is 0).  Contents are scratch.    */
/* Errors : INVALID_VALUE, MISALIGNED, NOT_SUPPORTED, WORKSPACE, LAUNCH.        */
/* ------------------------------------------------------------------------- */
size_t fp8gemm_quantize_workspace_size(int64_t rows, int64_t k, int mode);

fp8gemm_status fp8gemm_quantize(const float* x, int64_t rows, int64_t k, int64_t ldx, int mode,
                                uint8_t* q, int64_t ldq, void* scales, void* workspace,
                                size_t workspace_bytes, void* stream);

/* The same for either element format (fp8gemm_format): with FP8GEMM_FORMAT_E5M2
   the rules above use 57344 in place of 448 (s = fl32(amax/57344), saturation
   to +-57344, never infinity) and 15 in place of 8 (MX32: e = floor(log2 amax)
   - 15).  With FP8GEMM_FORMAT_E2M1 (MX32 only, else NOT_SUPPORTED) they use 6
   and 2 (e = floor(log2 amax) - 2, q = RNE_sat(x * 2^-e) onto e2m1, saturating
   at +-6) and q holds two codes per byte: element (r,i) in byte q[r*ldq + i/2],
   low nibble for even i; ldq >= k/2 bytes, a multiple of 16.  With
   FP8GEMM_FORMAT_E2M3 / E3M2 (MX32 only) they use 7.5 and 2 / 28 and 4 (e =
   floor(log2 amax) - 2 or - 4, saturating at +-7.5 / +-28) and q holds a row of
   k 6-bit codes in 3k/4 bytes (the stream above); ldq >= 3k/4, a multiple of 16.
   fp8gemm_quantize is this call with FP8GEMM_FORMAT_E4M3.  Errors as above; an
   unknown format is INVALID_VALUE. */
fp8gemm_status fp8gemm_quantize_ex(const float* x, int64_t rows, int64_t k, int64_t ldx, int mode,
                                   int format, uint8_t* q, int64_t ldq, void* scales,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* Dense scaled GEMM: C[m,n] = cast( sum_k dq_a(m,k) * dq_b(k,n) ).             */
/*                                                                           */
/* The tiled fp32-accumulating GEMM of "Hopper/Blackwell architecture features"  */
/* §12.7 with FP8 operands and the scale applied in the epilogue (TENSOR,      */
/* ROWWISE) or inside the matrix instruction per 32-K block (MX32).             */
/*   TENSOR : scale_a, scale_b -> device float[1] each.                         */
/*   ROWWISE: scale_a -> device float[M], scale_b -> device float[N].          */
/*   MX32   : scale_a -> device uint8 [M][K/32], scale_b -> uint8 [N][K/32].   */
/* M, N >= 0 (either 0: SUCCESS, nothing enqueued).  K > 0, multiple of 16     */
/* (32 for MX32).  lda, ldb >= K and multiples of 16; ldc >= N with ldc*2 a     */
/* multiple of 16; A, B, C 16-byte aligned; scale arrays 4-byte aligned.        */
/* workspace: fp8gemm_workspace_size() bytes (may be 0 -> NULL allowed).  Its    */
/* first 4 KiB hold split-K arrival counters: zero-fill the workspace before    */
/* its first use; every call leaves the counters at zero (the rest is scratch), */
/* so one workspace serves calls of every shape, including fp8gemm_run_kn, as   */
/* long as they run one after another.  Calls that may run concurrently (on     */
/* different streams) need separate workspaces: the counters and the partial    */
/* tiles sit at fixed places, so two overlapping calls on one workspace race.   */
/* Accuracy: |C - C_ref| <= 1e-3 * sum_k|dq_a*dq_b| + 1 ulp of the output type. */
/* ------------------------------------------------------------------------- */
size_t fp8gemm_workspace_size(int64_t M, int64_t N, int64_t K, int mode);

fp8gemm_status fp8gemm_run(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                           const uint8_t* B, int64_t ldb, int mode, const void* scale_a,
                           const void* scale_b, void* C, int64_t ldc, int out_dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* Dense scaled GEMM with operand formats and a fused epilogue:                */
/*   y[m,n] = sum_k dq_a(m,k) * dq_b(k,n)  (as fp8gemm_run),                   */
/*   C[m,n] = cast( act( y[m,n] + bias[n] ) ).                                 */
/* a_format, b_format: fp8gemm_format of the A and B codes (any pair of e4m3   */
/*          and e5m2: e5m2 x e5m2 or mixed e4m3 x e5m2, the gradient-GEMM       */
/*          pairing), or E2M1 for both (MXFP4 x MXFP4: mode MX32 only, else     */
/*          NOT_SUPPORTED; A holds two codes per byte, element (m,k) in byte    */
/*          A[m*lda + k/2], likewise B[n*ldb + k/2]; lda, ldb >= K/2 bytes;     */
/*          K % 32 == 0; scales uint8 [M][K/32] and [N][K/32]; the workspace    */
/*          of fp8gemm_workspace_size(M, N, K, MX32), K in elements); or E2M3 /  */
/*          E3M2 for both, in any pairing (MXFP6: MX32 only; A and B rows hold   */
/*          K codes in 3K/4 bytes; lda, ldb >= 3K/4; K % 128 == 0, else         */
/*          NOT_SUPPORTED; no workspace).                                       */
/* bias   : device float[N], 4-byte aligned, or NULL (no bias).               */
/* activation: fp8gemm_activation, applied in fp32 after the scales and bias.   */
/* The scale modes, layouts, workspace and errors are those of fp8gemm_run      */
/* (the workspace size does not depend on formats or epilogue); an unknown      */
/* format or activation is INVALID_VALUE.  fp8gemm_run is this call with e4m3   */
/* operands, no bias and FP8GEMM_ACT_NONE.                                     */
/* Accuracy: |C - act(y_ref + bias)| <= L * (1e-3 * sum_k|dq_a*dq_b|           */
/*   + 2^-22 |y_ref + bias|) + 2^-20 (|act| + |y_ref + bias|) + 1 output ulp,   */
/*   with L the activation's Lipschitz bound (1 for none/ReLU, 1.13 for GELU,  */
/*   1.1 for SiLU) and the 2^-22 and 2^-20 terms the fp32 rounding of the       */
/*   scaled value, the bias add and the activation's math functions.            */
/* ------------------------------------------------------------------------- */
fp8gemm_status fp8gemm_run_ex(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                              int a_format, const uint8_t* B, int64_t ldb, int b_format, int mode,
                              const void* scale_a, const void* scale_b, const float* bias,
                              int activation, void* C, int64_t ldc, int out_dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* Dense scaled GEMM whose output is quantised again for the next layer: the    */
/* fused epilogue of fp8gemm_run_ex computes y = act(scaled GEMM + bias) in     */
/* fp32 and writes it as e4m3 codes with one E8M0 scale per 32 consecutive      */
/* columns of each row (the MX32 rule of fp8gemm_quantize: e = floor(log2 amax) */
/* - 8, code = clamp(e + 127, 0, 254), q = RNE_sat(y * 2^-e)).  The Cutlass-    */
/* named Triton FP8 post fuses epilogues to save a round trip of C through      */
/* memory; this one also saves the quantisation pass of the next FP8 GEMM.      */
/*   C       : device uint8 e4m3 codes, element (m,n) at C[m*ldc+n]; ldc >= N,  */
/*             a multiple of 16; 16-byte aligned.                               */
/*   c_scales: device uint8 E8M0 codes, block (m, n/32) at c_scales[m*ldcs +    */
/*             n/32]; ldcs >= N/32.                                             */
/*   N must be a multiple of 32 (else NOT_SUPPORTED).                           */
/* A, B, formats, mode, scales, bias, activation, workspace and errors as       */
/* fp8gemm_run_ex.  Accuracy: each output dequantises (code value times its    */
/* block's 2^e) to within the fp8gemm_run_ex bound of act(y_ref + bias) plus    */
/* half an e4m3 spacing at its magnitude and block exponent (and the saturation */
/* of block maxima in [448, 512) * 2^e to 448 * 2^e); a block exponent may      */
/* differ by one from the exact result's when its maximum lies within that      */
/* bound of a power of two.                                                     */
/* ------------------------------------------------------------------------- */
fp8gemm_status fp8gemm_run_mxout(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                                 int a_format, const uint8_t* B, int64_t ldb, int b_format,
                                 int mode, const void* scale_a, const void* scale_b,
                                 const float* bias, int activation, uint8_t* C, int64_t ldc,
                                 uint8_t* c_scales, int64_t ldcs, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* Dense scaled GEMM whose output is quantised again for the next layer with a  */
/* fresh per-tensor or per-row scale (the Cutlass-named Triton FP8 post fuses    */
/* epilogues to save a round trip of C; the JAX/Triton Blackwell FP8 GEMM post's */
/* operands are E4M3 codes with their scale factors, the form this produces).    */
/* The layer's output C16 is the bf16 result fp8gemm_run_ex computes (scaled     */
/* GEMM + bias, activation, RNE to bf16); the codes are the rule of             */
/* fp8gemm_quantize_ex applied to C16's values:                                 */
/*   out_mode TENSOR : s = fl32(amax/fmax) over all of C16 (1 if amax = 0),      */
/*                     c_scales -> float[1];                                    */
/*   out_mode ROWWISE: the same per row, c_scales -> float[M] (the scale_a of a  */
/*                     row-wise GEMM that takes C as its A operand);            */
/*   q = RNE_sat(fl32(C16/s)), fmax = 448 (c_format E4M3) or 57344 (E5M2).      */
/* The result is bit-identical to fp8gemm_run_ex with bf16 output followed by   */
/* fp8gemm_quantize_ex on that output (as fp32).  The GEMM kernels store C16 to  */
/* the workspace and fold its magnitudes into per-row (or one) atomic maxima in */
/* their epilogue; a second, HBM-streaming kernel derives the scales and encodes */
/* (the maxima are zeroed by a small kernel first, so no memset node is        */
/* recorded under graph capture).                                               */
/*   C       : device uint8 codes, element (m,n) at C[m*ldc+n]; ldc >= N, a      */
/*             multiple of 16; 16-byte aligned.  N % 16 == 0 (else              */
/*             NOT_SUPPORTED).  c_scales 4-byte aligned.                         */
/*   c_format: E4M3 or E5M2 (another format is NOT_SUPPORTED); out_mode TENSOR   */
/*             or ROWWISE (else INVALID_VALUE).                                 */
/*   workspace: fp8gemm_qout_workspace_size(M, N, K, mode) bytes (M 4-byte      */
/*             maxima and C16, M x N bf16, after the GEMM's own workspace),     */
/*             16-byte aligned; zero-fill it before its first use (the GEMM's   */
/*             split-K counters, left at zero by every call).  One workspace    */
/*             serves calls of every shape one after another; calls that may    */
/*             overlap need their own.                                          */
/* A, B, formats (FP8, FP4 and FP6 pairs as fp8gemm_run_ex), mode, scales, bias, */
/* activation and the other errors as fp8gemm_run_ex.                          */
/* Accuracy: with tol the fp8gemm_run_ex bound plus half a bf16 ulp, s lies     */
/* between the scales of the largest |y_ref| minus and plus tol, and each code  */
/* dequantises (value times s) to within tol plus half a spacing of the format  */
/* at its magnitude (and the saturation of the maximum itself) of y_ref.        */
/* ------------------------------------------------------------------------- */
size_t fp8gemm_qout_workspace_size(int64_t M, int64_t N, int64_t K, int mode);

fp8gemm_status fp8gemm_run_qout(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                                int a_format, const uint8_t* B, int64_t ldb, int b_format,
                                int mode, const void* scale_a, const void* scale_b,
                                const float* bias, int activation, int out_mode, int c_format,
                                uint8_t* C, int64_t ldc, float* c_scales, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* Dense scaled GEMM with B in row-major [K,N] layout (N contiguous), the layout */
/* of the pages' Triton listings ("Hopper/Blackwell architecture features"      */
/* §12.7.1/§12.7.2 advance b_ptr by BLOCK_K * stride_bk).                        */
/*   B      : element (k,n) at B[k*ldb+n]; ldb >= N, a multiple of 16; 16-byte   */
/*            aligned.                                                           */
/*   scale_b: TENSOR float[1]; ROWWISE float[N]; MX32 uint8 [K/32][N] (row-major, */
/*            N codes per row).                                                 */
/*   E2M1 (MXFP4, both operands, MX32 only): B packs two codes per byte along N, */
/*            element (k,n) in byte B[k*ldb + n/2], low nibble for even n;       */
/*            ldb >= ceil(N/2) bytes, a multiple of 16.                          */
/* Everything else (A, C, formats, scale_a, bias, activation, accuracy, errors) */
/* as fp8gemm_run_ex; FP6 operands are NOT_SUPPORTED here.                     */
/* Two forms, chosen per call (fp8gemm_run_kn_path tells which):                 */
/*   in-kernel : the GEMM kernels read B row-major and form the K-major MFMA     */
/*               operand with transposing LDS reads (ds_read_b64_tr_b8, FP4:     */
/*               tr_b4; no extra pass over B).  Taken when K % 128 == 0 (MX: K % */
/*               512 == 0 and N % 16 == 0) and the operand spans fit 32-bit      */
/*               offsets (K * ldb < 2^31 - 256).                                 */
/*               Workspace: fp8gemm_workspace_size(M, N, K, mode) bytes (NULL    */
/*               when that is 0).                                                */
/*   transposing: otherwise the call first copies B and its MX codes into the   */
/*               K-contiguous layout in the workspace (one HBM pass over B; FP4  */
/*               codes by a nibble transpose), then runs the GEMM.  Workspace    */
/*               never NULL: the copy lives there.                               */
/* fp8gemm_workspace_size_kn() bytes, 16-byte aligned and zero-filled before    */
/* its first use, serve either form.  Its first 4 KiB are the counters of       */
/* fp8gemm_run (left at zero); the copies come after the GEMM's own workspace,  */
/* so the two entry points may share one.                                       */
/* ------------------------------------------------------------------------- */
size_t fp8gemm_workspace_size_kn(int64_t M, int64_t N, int64_t K, int mode);

fp8gemm_status fp8gemm_run_kn(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                              int a_format, const uint8_t* B, int64_t ldb, int b_format, int mode,
                              const void* scale_a, const void* scale_b, const float* bias,
                              int activation, void* C, int64_t ldc, int out_dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* Grouped (mixture-of-experts) GEMM, the grouped form in the MoE paragraph of   */
/* the JAX/Triton Blackwell FP8 GEMM post: rows of A are sorted by expert and    */
/* expert g owns rows [offsets[g], offsets[g+1]):                               */
/*   C[m,:] = cast( dq_a(m,:) . dq_{B_g} )  for offsets[g] <= m < offsets[g+1]. */
/* offsets: DEVICE int32[num_groups+1], offsets[0] = 0, non-decreasing,          */
/*          offsets[num_groups] = total_m.  The host never reads it (no sync);   */
/*          rows outside [0, total_m) are never touched, but values violating    */
/*          these rules give unspecified C.  Empty experts are allowed.          */
/* B_g = B + g*stride_b (column-major N x K per expert, ldb >= K), stride_b >=   */
/*          N*ldb and a multiple of 16.                                         */
/*   TENSOR : scale_a float[1], scale_b float[num_groups].                      */
/*   ROWWISE: scale_a float[total_m], scale_b float[num_groups*N] (expert-major).*/
/*   MX32   : scale_a uint8 [total_m][K/32], scale_b uint8 [num_groups][N][K/32]. */
/* 1 <= num_groups <= 1024 (more: NOT_SUPPORTED; the persistent kernel keeps   */
/* per-expert tables in LDS), total_m >= 0, other rules as fp8gemm_run.        */
/* ------------------------------------------------------------------------- */
size_t fp8gemm_grouped_workspace_size(int32_t num_groups, int64_t total_m, int64_t N, int64_t K,
                                      int mode);

fp8gemm_status fp8gemm_grouped_run(int32_t num_groups, int64_t total_m, int64_t N, int64_t K,
                                   const uint8_t* A, int64_t lda, const int32_t* offsets,
                                   const uint8_t* B, int64_t ldb, int64_t stride_b, int mode,
                                   const void* scale_a, const void* scale_b, void* C,
                                   int64_t ldc, int out_dtype, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* The same with operand formats: a_format and b_format both FP8GEMM_FORMAT_E4M3
   (fp8gemm_grouped_run), or both FP8GEMM_FORMAT_E2M1 with MX32 scales (MXFP4
   activations and experts; A holds two codes per byte, element (m,k) in byte
   A[m*lda + k/2], expert g's element (k,n) in byte B[g*stride_b + n*ldb + k/2];
   lda, ldb >= K/2 bytes; K % 32 == 0; E8M0 codes as above).  Other pairings are
   NOT_SUPPORTED. */
fp8gemm_status fp8gemm_grouped_run_ex(int32_t num_groups, int64_t total_m, int64_t N, int64_t K,
                                      const uint8_t* A, int64_t lda, int a_format,
                                      const int32_t* offsets, const uint8_t* B, int64_t ldb,
                                      int b_format, int64_t stride_b, int mode,
                                      const void* scale_a, const void* scale_b, void* C,
                                      int64_t ldc, int out_dtype, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- */
/* fp8gemm_run_ex without a workspace, for callers that cannot allocate device  */
/* memory (code under HIP graph capture, serving loops or harnesses that forbid */
/* allocation).  The call allocates nothing: the split-K counters and partial   */
/* tiles go to a static device array of FP8GEMM_NOALLOC_SCRATCH_BYTES that every */
/* device the library runs on holds until the process ends.  The first call on */
/* a device (with it current) looks the array's address up and zeroes its       */
/* counters with a kernel on `stream`; every call leaves them at zero again.    */
/* Arguments, results, accuracy and errors as fp8gemm_run_ex, except:           */
/*   - a shape whose fp8gemm_workspace_size() exceeds                           */
/*     FP8GEMM_NOALLOC_SCRATCH_BYTES returns FP8GEMM_ERROR_WORKSPACE, checked    */
/*     before any HIP call (every shape with at most 512 split workgroups fits,  */
/*     the M = 128, N = K = 4096 decode shape among them);                      */
/*   - FP8GEMM_ERROR_LAUNCH also reports a failed look-up of the scratch.       */
/* All calls on one device share its scratch, which keeps the last call's       */
/* contents: calls that may overlap on one device (different streams or host    */
/* threads) race and must be ordered by the caller.                             */
/* ------------------------------------------------------------------------- */
#define FP8GEMM_NOALLOC_SCRATCH_BYTES (8 * 1024 * 1024 + 4096)

fp8gemm_status fp8gemm_run_noalloc(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda,
                                   int a_format, const uint8_t* B, int64_t ldb, int b_format,
                                   int mode, const void* scale_a, const void* scale_b,
                                   const float* bias, int activation, void* C, int64_t ldc,
                                   int out_dtype, void* stream);

/* ------------------------------------------------------------------------- */
/* Which kernel a dense GEMM call of this shape runs (no HIP call, no launch):   */
/* the tiling and persistence choices of "Hopper/Blackwell architecture          */
/* features" §12.7 (tile size per shape, persistent kernels in §12.7.3) and the  */
/* split along K for shapes with too few output tiles (the M = 128 shape of       */
/* §12.2.4).  The arguments are those of fp8gemm_run_ex / fp8gemm_run_mxout: K   */
/* in elements, lda / ldb in bytes; fused is nonzero when a bias or activation  */
/* is fused or the output is quantised (fp8gemm_run_mxout).                      */
/*   FP8GEMM_PATH_NONE       : nothing is launched (M or N is 0) or the formats   */
/*                             or mode are invalid or not offered together.      */
/*   FP8GEMM_PATH_SPLITK     : few output tiles: 64 x 64 tiles, K split over     */
/*                             workgroups, fp32 partials in the workspace.       */
/*   FP8GEMM_PATH_TILE128    : 128 x 128 tiles, one per workgroup.               */
/*   FP8GEMM_PATH_TILE256    : 256 x 256 tiles, one per workgroup.               */
/*   FP8GEMM_PATH_PERSISTENT : 256 x 256 tiles, one workgroup per compute unit   */
/*                             walking its tiles as one copy stream.             */
/* ------------------------------------------------------------------------- */
typedef enum fp8gemm_path {
  FP8GEMM_PATH_NONE = 0,
  FP8GEMM_PATH_SPLITK = 1,
  FP8GEMM_PATH_TILE128 = 2,
  FP8GEMM_PATH_TILE256 = 3,
  FP8GEMM_PATH_PERSISTENT = 4
} fp8gemm_path;

int fp8gemm_run_path(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int a_format,
                     int b_format, int mode, int fused);

/* The kernel path fp8gemm_run_kn takes in its in-kernel form (ldb: bytes      */
/* between the K-rows of the row-major B), or FP8GEMM_PATH_NONE when the call   */
/* makes B K-contiguous first (or would launch nothing).  Never PERSISTENT.     */
int fp8gemm_run_kn_path(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                        int a_format, int b_format, int mode);

/* Human-readable name of a status code (static string, never NULL). */
const char* fp8gemm_status_string(int status);

/* FP8GEMM_VERSION of the built library. */
int fp8gemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8GEMM_H_ */
