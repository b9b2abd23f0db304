/*
 * igc.h -- C ABI of libigc.so: tiled dense GEMM (fp16 -> fp32 and u8 x i8 ->
 * int32 with zero points and a fused quantization epilogue) and conv2d lowered
 * to an implicit GEMM (fp16, and u8 x i8 with zero points), for AMD Instinct
 * MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *  [GEMM-TVM]  CSDN article "TVM在CUDA GPU上跑GEMM的全套张量化实现：WMMA/DP4A/IMMA
 *              + TensorIR调度 + INT8/FP16多精度支持".
 *  [CONV-TC]   TVM tutorial (Chinese docs, segmentfault) on a conv2d schedule
 *              with TensorCores.
 *
 * Conventions shared by every entry point
 *  - All buffers are device memory owned by the caller: inputs, outputs,
 *    per-channel vectors and the optional workspace.  The library never
 *    allocates, frees or copies device memory.  Its only state is a
 *    per-device cache of the architecture and compute-unit count and the
 *    process-wide tuning overrides of igc_set_tuning.
 *  - Workspace.  A call may split the K loop of some output tiles between
 *    workgroups (stream-K) and sum their partial tiles through a caller-owned
 *    workspace.  <entry>_workspace_size() returns the bytes a call of that
 *    shape needs on the current device (0: none).  Pass a 16-byte aligned
 *    device buffer of at least that size, zero-filled before its first use;
 *    every call leaves it zero-filled again in the part that must start at
 *    zero.  With workspace == NULL the call runs without the split (same
 *    results, possibly slower).  A non-NULL workspace smaller than needed is
 *    rejected with IGC_EINVAL.  Calls that overlap in time (different
 *    streams) must not share a workspace.
 *  - Argument validation is synchronous and happens before any HIP call,
 *    except the workspace-size check, which needs the device's compute-unit
 *    count; a rejected call has no side effects.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without waiting.  The caller synchronizes.
 *  - Outputs must not alias inputs.  Calls on different streams that write the
 *    same output race.
 *  - The functions are thread-safe.  igc_last_error() is per thread.
 *  - Sizes are element counts; leading dimensions (ld*) are in elements.
 *  - M == 0 or N == 0 is a valid empty problem: nothing is launched.
 *    K == 0 is valid: every output is computed from an all-zero accumulator.
 */
#ifndef IGC_H
#define IGC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
#define IGC_OK 0
#define IGC_EINVAL (-1)       /* null pointer, negative size, ld too small, zero point out of range */
#define IGC_EUNSUPPORTED (-2) /* a shape / stride combination no kernel variant handles             */
#define IGC_EOVERFLOW (-3)    /* u8 x i8 with K > 33025: the int32 result could overflow              */
#define IGC_EHIP (-4)         /* HIP runtime or launch error; detail in igc_last_error()              */
#define IGC_ENODEV (-5)       /* the current HIP device is not a gfx950 GPU, or there is no device    */

/*
 * gemm_f16f32 -- C = A * B with fp16 operands and fp32 accumulation and output.
 *
 * Definition: [GEMM-TVM] §4.1 (C[i,j] = sum_k A[i,k] * B[k,j]); fp16 inputs
 * with an fp32 accumulator as in the TensorCore introduction of [CONV-TC].
 *
 *   A  fp16 (binary16), M x K, row-major:     A[m*lda + k],  lda >= K
 *   B  fp16, K x N, column-major (N rows of K): B[n*ldb + k], ldb >= K
 *   C  fp32, M x N, row-major:                C[m*ldc + n],  ldc >= N
 *
 * Every product of two fp16 values is exact in fp32; the K-sum is accumulated
 * in fp32 (summation order is unspecified).  Any alignment and any lda/ldb is
 * accepted; 16-byte aligned A/B with lda, ldb and K multiples of 8 take the
 * fast path.  workspace / ws_bytes: the optional caller-owned workspace of
 * the conventions above (NULL / 0 for none).
 * Errors: IGC_EINVAL (negative size, NULL pointer with a non-empty operand,
 * lda < K, ldb < K, ldc < N, workspace too small or misaligned), IGC_ENODEV,
 * IGC_EHIP.
 */
int gemm_f16f32(int M, int N, int K,
                const void* A, int lda,
                const void* B, int ldb,
                float* C, int ldc,
                void* workspace, size_t ws_bytes,
                void* stream);

/*
 * gemm_f16f32_workspace_size -- *bytes = the workspace gemm_f16f32 needs for
 * an M x N x K problem on the current device (0 when it never splits a tile;
 * an upper bound: a call whose operands take the element-wise path needs
 * none).  Errors: IGC_EINVAL (negative size, bytes NULL), IGC_ENODEV.
 */
int gemm_f16f32_workspace_size(int M, int N, int K, size_t* bytes);

/*
 * gemm_f16f32_noalloc -- gemm_f16f32 for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, layouts and results as gemm_f16f32
 * without the workspace: where the call splits tiles between workgroups its
 * workspace is a static device array of 32 MiB (33554432 bytes) per GPU,
 * which each GPU the library runs on holds until the process ends.  The call
 * allocates nothing and clears the array's counters with a kernel on
 * `stream` before using it.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (different streams) race.
 * Errors: as gemm_f16f32, plus IGC_EUNSUPPORTED when the split this call
 * makes needs more workspace than the 32 MiB the array holds (512 KiB per
 * workgroup sharing tiles; gemm_f16f32_workspace_size gives the amount, and
 * a shape for which it returns 0 never fails this way).
 */
int gemm_f16f32_noalloc(int M, int N, int K,
                        const void* A, int lda,
                        const void* B, int ldb,
                        float* C, int ldc,
                        void* stream);

/*
 * Outputs of gemm_u8i8_zp.  Any non-empty subset may be requested in one call;
 * a NULL pointer means "not requested".
 *
 *   C_i32, ldc      int32 M x N row-major: the exact zero-point-corrected
 *                   product  C = sum_k (A[m,k] - zA) * (B[k,n] - zB).
 *   D_f32, ldd      fp32 M x N row-major: dequantized  D = fl32(fl32(C) * dq_scale).
 *                   dq_scale is one fp32 multiplier (pass fl32(sA * sB) for
 *                   per-tensor scales sA, sB).
 *   Q_i8, ldq       int8 M x N row-major: requantized per output channel n:
 *                   t = fl32(fl32(C) * scale_n[n]); y = fl32(t + bias_n[n]);
 *                   Q = clamp(round_half_even(y), -128, 127).
 *                   scale_n and bias_n are fp32 device vectors of length N and
 *                   are required when Q_i8 is requested.
 *
 *   workspace,      optional caller-owned workspace (see the conventions above
 *   ws_bytes        and gemm_u8i8_zp_workspace_size); NULL / 0 for none.
 *
 *   colsum_B        optional int32 device vector of length N holding
 *                   colsum(B)[n] = sum_k B[k,n] (the weights' column sums,
 *                   for static weights computed once with u8i8_colsum), 4-byte
 *                   aligned; NULL to have the kernel form the sums it needs
 *                   itself.  Where a launch can use it (zA != 128, whole
 *                   tiles, Q_i8 the only output, no split) the K loop forms
 *                   no column sums; elsewhere it is not read.  The results
 *                   are those of the definition either way, provided the
 *                   vector holds the column sums of this call's B.
 *
 * Int -> fp32 conversions round to nearest even; the two fp32 operations of
 * the requantize step are separately rounded (no fused multiply-add).
 */
typedef struct igc_u8i8_epilogue {
  int32_t* C_i32;
  int ldc;
  float* D_f32;
  int ldd;
  float dq_scale;
  int8_t* Q_i8;
  int ldq;
  const float* scale_n;
  const float* bias_n;
  void* workspace;
  size_t ws_bytes;
  const int32_t* colsum_B;
} igc_u8i8_epilogue;

/*
 * gemm_u8i8_zp -- u8 x i8 GEMM with input zero points, int32 accumulation and
 * a fused epilogue.
 *
 * Definition: [GEMM-TVM] §2.3: the quantized product is
 * C = (A_q - zp_A) * (B_q - zp_B), followed by dequantize and add-bias in the
 * same kernel ("4-term fusion").  The zero-point terms are applied in the
 * epilogue through the four-term expansion
 *   C = sum_k A*B - zA*colsum(B)[n] - zB*rowsum(A)[m] + K*zA*zB,
 * which equals the definition exactly in int32.
 *
 *   A   uint8, M x K row-major: A[m*lda + k], lda >= K;   zA in [0, 255]
 *   B   int8,  K x N column-major: B[n*ldb + k], ldb >= K; zB in [-128, 127]
 *   ep  host pointer to the output description above (read during the call).
 *
 * Errors: IGC_EINVAL (negative size, NULL pointer with a non-empty operand,
 * ld too small, zero point out of range, ep NULL or requesting no output,
 * Q_i8 without scale_n/bias_n, workspace too small), IGC_EOVERFLOW (K > 33025, where
 * 255*255*K can exceed the int32 range), IGC_ENODEV, IGC_EHIP.
 */
int gemm_u8i8_zp(int M, int N, int K,
                 const uint8_t* A, int lda, int zA,
                 const int8_t* B, int ldb, int zB,
                 const igc_u8i8_epilogue* ep,
                 void* stream);

/* gemm_u8i8_zp_workspace_size -- as gemm_f16f32_workspace_size, for gemm_u8i8_zp. */
int gemm_u8i8_zp_workspace_size(int M, int N, int K, size_t* bytes);

/*
 * u8i8_colsum -- the column sums of an int8 B operand, for the colsum_B
 * field of igc_u8i8_epilogue: colsum[n] = sum_k B[n*ldb + k] for n < N, in
 * int32 (exact for K <= 33025 * 2, far beyond the K the GEMM accepts).
 *
 * Definition: [GEMM-TVM] §2.3: the zero-point term zA * colsum(B) of the
 * four-term expansion; B is the weight operand, fixed across calls, so its
 * sums can be formed once.  For the convolution B is the KRSC weight tensor
 * (N = Kout rows of K = R*S*C, ldb = K).
 *
 *   B       int8, N rows of K (column-major K x N): B[n*ldb + k], ldb >= K.
 *   colsum  int32 device vector of length N, written on `stream`.
 *
 * Errors: IGC_EINVAL (negative size, ldb < K, NULL pointer with N > 0),
 * IGC_EOVERFLOW (K > 33025), IGC_ENODEV, IGC_EHIP.
 */
int u8i8_colsum(int N, int K, const int8_t* B, int ldb, int32_t* colsum, void* stream);

/*
 * conv2d_implicit_gemm -- 2-D convolution (cross-correlation, no filter flip),
 * fp16 in, fp32 accumulation and output, lowered to a GEMM whose A operand is
 * the im2col matrix, formed on the fly and never materialized.
 *
 * Definition: [CONV-TC] "Preparation and algorithm": the input is read through
 * a zero-padded view and
 *   y[n,p,q,k] = sum_{r,s,c} xpad[n, p*stride_h + r, q*stride_w + s, c] * w[k,r,s,c]
 * with xpad = x inside the input and 0 in the padding.  Dilation 1, groups 1.
 *
 *   x  fp16 NHWC [Nb][H][W][C]
 *   w  fp16 KRSC [Kout][R][S][C]
 *   y  fp32 NHWC [Nb][P][Q][Kout], P = (H + 2*pad_h - R)/stride_h + 1,
 *      Q = (W + 2*pad_w - S)/stride_w + 1
 *
 * GEMM view: M = Nb*P*Q rows (n,p,q), N = Kout, K = R*S*C with
 * k = (r*S + s)*C + c; the weight tensor is the column-major B operand.
 * 16-byte aligned x/w with C a multiple of 8 take the fast path.
 * workspace / ws_bytes: optional, as for gemm_f16f32.
 * Errors: IGC_EINVAL (non-positive dimension or stride, negative padding,
 * NULL pointer, P or Q < 1, workspace too small), IGC_EUNSUPPORTED (an index
 * of x, w or y that does not fit in 32 bits; H, W, R, S, pad_h or pad_w of
 * 32768 or more), IGC_ENODEV, IGC_EHIP.
 */
int conv2d_implicit_gemm(int Nb, int H, int W, int C, int Kout, int R, int S,
                         int stride_h, int stride_w, int pad_h, int pad_w,
                         const void* x, const void* w, float* y,
                         void* workspace, size_t ws_bytes,
                         void* stream);

/* conv2d_implicit_gemm_workspace_size -- as gemm_f16f32_workspace_size, for
 * conv2d_implicit_gemm (the convolution's arguments are validated as there). */
int conv2d_implicit_gemm_workspace_size(int Nb, int H, int W, int C, int Kout, int R, int S,
                                        int stride_h, int stride_w, int pad_h, int pad_w,
                                        size_t* bytes);

/*
 * conv2d_implicit_gemm_nhwcnc -- the same convolution as conv2d_implicit_gemm
 * (fp16 in, fp32 accumulation and output, cross-correlation, dilation 1,
 * groups 1) on tensors in the blocked NHWCnc layout of [CONV-TC]
 * "Preparation and algorithm" (block size 16):
 *
 *   x  fp16 [Nb/16][H][W][C/16][16 (n % 16)][16 (c % 16)]        (data_shape)
 *   w  fp16 [R][S][C/16][Kout/16][16 (c % 16)][16 (k % 16)]      (kernel_shape)
 *   y  fp32 [Nb/16][P][Q][Kout/16][16 (n % 16)][16 (k % 16)]     (output_shape)
 *
 *   y[n,p,q,k] = sum_{r,s,c} xpad[n, p*stride_h + r, q*stride_w + s, c] * w[r,s,c,k]
 *
 * with the logical indices placed in the blocks as shown.  Nb, C and Kout
 * must be multiples of 16.  GEMM view: M = Nb*P*Q rows ordered
 * ((n/16, p, q), n % 16), N = Kout, K = R*S*C.  The weights keep the output
 * channels innermost, while the matrix cores read both operands with the
 * reduction contiguous, so each call first writes the weights in K-contiguous
 * order into the workspace (Kout*R*S*C*2 bytes); the workspace is therefore
 * required: conv2d_implicit_gemm_nhwcnc_workspace_size gives its size, which
 * also covers the stream-K part (zero-filled before first use, as for the
 * other entry points).  16-byte aligned x with C a multiple of 64 and
 * R*S <= 31 take the uniform-tap path.
 * Errors: as conv2d_implicit_gemm, plus IGC_EINVAL when Nb, C or Kout is not
 * a multiple of 16, when the workspace is NULL, misaligned or too small, or
 * w is not 16-byte aligned.
 */
int conv2d_implicit_gemm_nhwcnc(int Nb, int H, int W, int C, int Kout, int R, int S,
                                int stride_h, int stride_w, int pad_h, int pad_w,
                                const void* x, const void* w, float* y,
                                void* workspace, size_t ws_bytes,
                                void* stream);

/* conv2d_implicit_gemm_nhwcnc_workspace_size -- the workspace bytes
 * conv2d_implicit_gemm_nhwcnc needs for these sizes on the current device
 * (never 0).  Errors: as the convolution's argument checks, IGC_ENODEV. */
int conv2d_implicit_gemm_nhwcnc_workspace_size(int Nb, int H, int W, int C, int Kout, int R, int S,
                                               int stride_h, int stride_w, int pad_h, int pad_w,
                                               size_t* bytes);

/*
 * conv2d_u8i8_zp -- quantized 2-D convolution: u8 activations x i8 weights
 * with input zero points, int32 accumulation and the same fused outputs as
 * gemm_u8i8_zp (int32, dequantized fp32, requantized int8 per output
 * channel).
 *
 * Definition: the quantized product of [GEMM-TVM] §2.3,
 * (x_q - zp_x) * (w_q - zp_w), summed over the taps of the convolution of
 * [CONV-TC] "Preparation and algorithm":
 *   C[n,p,q,k] = sum_{r,s,c} (xpad[n, p*stride_h + r, q*stride_w + s, c] - zA)
 *                            * (w[k,r,s,c] - zB)
 * where the padding holds the real value 0, i.e. the code zA, so a padded
 * tap contributes nothing.  Dilation 1, groups 1, cross-correlation.
 *
 *   x  uint8 NHWC [Nb][H][W][C], zA in [0, 255]
 *   w  int8  KRSC [Kout][R][S][C], zB in [-128, 127]
 *   outputs (ep, as for gemm_u8i8_zp) row-major [Nb*P*Q][Kout] = NHWC, with
 *   the per-output-channel scale_n / bias_n indexed by k.
 *
 * GEMM view: M = Nb*P*Q, N = Kout, K = R*S*C (k = (r*S + s)*C + c).
 * 16-byte aligned x and w with C a multiple of 128 and R*S <= 31 take the
 * fast path; every other shape an element-wise one.
 * Errors: as conv2d_implicit_gemm, plus those of gemm_u8i8_zp for zA, zB,
 * the epilogue descriptor and K = R*S*C > 33025 (IGC_EOVERFLOW).
 */
int conv2d_u8i8_zp(int Nb, int H, int W, int C, int Kout, int R, int S,
                   int stride_h, int stride_w, int pad_h, int pad_w,
                   const uint8_t* x, int zA, const int8_t* w, int zB,
                   const igc_u8i8_epilogue* ep, void* stream);

/* conv2d_u8i8_zp_workspace_size -- as gemm_f16f32_workspace_size, for
 * conv2d_u8i8_zp. */
int conv2d_u8i8_zp_workspace_size(int Nb, int H, int W, int C, int Kout, int R, int S,
                                  int stride_h, int stride_w, int pad_h, int pad_w,
                                  size_t* bytes);

/* Diagnostics. */
const char* igc_status_string(int status); /* static string for a status code              */
const char* igc_last_error(void);          /* detail of this thread's last failure, or ""  */
int igc_device_check(void);                /* IGC_OK if the current device is gfx950       */

/*
 * igc_set_tuning -- process-wide overrides for tests and tuning sweeps (not
 * needed for normal use; the defaults are -1 and 1).  They apply to calls
 * made after it returns.
 *   force_variant  -1: the shape chooses the tile; 0: 256x256, 1: 128x128,
 *                  2: 64x64, 3: 256x128, 4: 224x256, 5: the fp16 LDS-bypass
 *                  kernel (32x32 tiles), 6: the same with 16x16 tiles.  A
 *                  tile the operands' path does not have falls back to the
 *                  nearest smaller one.
 *   streamk_mode   0: never split tiles; 1: split where it pays; 2: split
 *                  whenever the last round of tiles is partial.
 * Errors: IGC_EINVAL (value out of range).
 */
int igc_set_tuning(int force_variant, int streamk_mode);

#ifdef __cplusplus
}
#endif

#endif /* IGC_H */
