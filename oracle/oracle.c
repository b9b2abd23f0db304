/*
 * oracle.c -- plain, slow, obviously correct CPU oracle for the GEMM and
 * implicit-GEMM convolution path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may include,
 * link, load or call this file.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no source, header, helper or
 * constant with the HIP kernels: it has its own binary16 decoder, its own
 * loops and its own epilogue arithmetic.
 *
 * Build: gcc -std=c11 -O2 -fopenmp -ffp-contract=off -fno-fast-math
 *        -shared -fPIC oracle.c -o liboracle.so -lm
 * (-ffp-contract=off keeps every a*b+c as two separately rounded operations,
 * which the epilogue definitions below depend on.)
 *
 * Sources (the pages are cited by title and section):
 *  [GEMM-TVM]  CSDN article "TVM在CUDA GPU上跑GEMM的全套张量化实现：WMMA/DP4A/IMMA
 *              + TensorIR调度 + INT8/FP16多精度支持".
 *  [CONV-TC]   TVM tutorial (Chinese docs, segmentfault) on writing a conv2d
 *              schedule with TensorCores.
 *
 * Every function is the plain definition written out: one serial reduction per
 * output element in a fixed order (k ascending, or (r, s, c) ascending for the
 * convolution).  OpenMP only splits the independent outputs across threads, so
 * results do not depend on the thread count.
 *
 * Pins (what ties each function to something other than itself) live in the
 * CPU tests: exact rational brute force, numpy/scipy library routines,
 * algebraic identities and closed-form special cases.  No function here is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16 -> double.  Written from the format definition:          */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.                    */
/*   exponent 0      : subnormal, value = fraction * 2^-24                     */
/*   exponent 1..30  : normal,    value = (1024 + fraction) * 2^(exponent-25)  */
/*   exponent 31     : infinity (fraction 0) or NaN                            */
/* The fp16 operands of both GEMMs and the convolution are decoded with this.  */
/* ------------------------------------------------------------------------ */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1f;
  int frac = h & 0x3ff;
  double v;
  if (expo == 0) {
    v = ldexp((double)frac, -24);
  } else if (expo == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + frac), expo - 25);
  }
  return sign ? -v : v;
}

void oracle_f16_decode(const uint16_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(in[i]);
}

/* ------------------------------------------------------------------------ */
/* O1. fp16 GEMM, exact-ish reference.                                        */
/* Definition [GEMM-TVM] §4.1 (C[i,j] = sum over the reduce axis k of         */
/* A[i,k]*B[k,j]); the operands are widened before the multiply as in          */
/* [CONV-TC] "Preparation and algorithm" (astype float32 on both factors).    */
/* Here the widening is to double: products of two fp16 values are exact in   */
/* double, and the k-ascending double sum is within ~K*2^-53 of the exact sum. */
/*                                                                            */
/* Layout: A is M x K row-major, A[m*lda + k].                                */
/*         B is K x N column-major, i.e. stored as N rows of K: B[n*ldb + k]. */
/*         R is M x N row-major double, R[m*ldr + n].                         */
/* ------------------------------------------------------------------------ */
void oracle_gemm_f16(int64_t M, int64_t N, int64_t K,
                     const uint16_t* A, int64_t lda,
                     const uint16_t* B, int64_t ldb,
                     double* R, int64_t ldr) {
  /* Decode every operand element once; the sum below is unchanged by this. */
  double* a = (double*)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
  double* b = (double*)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
  for (int64_t m = 0; m < M; ++m)
    for (int64_t k = 0; k < K; ++k) a[m * K + k] = oracle_f16_to_f64(A[m * lda + k]);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) b[n * K + k] = oracle_f16_to_f64(B[n * ldb + k]);

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) acc += a[m * K + k] * b[n * K + k];
      R[m * ldr + n] = acc;
    }
  }
  free(a);
  free(b);
}

/* ------------------------------------------------------------------------ */
/* O2. u8 x i8 GEMM with input zero points, naive form.                       */
/* [GEMM-TVM] §2.3: the quantized product is C = (A_q - zp_A) * (B_q - zp_B). */
/* Exact in int64: every term is subtracted before the multiply.              */
/* Layout as O1: A[m*lda+k] uint8, B[n*ldb+k] int8, C[m*ldc+n] int64.         */
/* ------------------------------------------------------------------------ */
void oracle_gemm_u8i8_naive(int64_t M, int64_t N, int64_t K,
                            const uint8_t* A, int64_t lda, int64_t zA,
                            const int8_t* B, int64_t ldb, int64_t zB,
                            int64_t* C, int64_t ldc) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      int64_t acc = 0;
      for (int64_t k = 0; k < K; ++k)
        acc += ((int64_t)A[m * lda + k] - zA) * ((int64_t)B[n * ldb + k] - zB);
      C[m * ldc + n] = acc;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* O3. The same product through the four-term expansion, computed by a       */
/* separate loop nest (it must agree with O2 element for element):            */
/*   sum_k (a-zA)(b-zB) = sum_k a*b - zA*colsum(B)[n] - zB*rowsum(A)[m]       */
/*                        + K*zA*zB                                           */
/* [GEMM-TVM] §2.3 names the zero-point handling and the "4-term fusion";     */
/* the expansion itself is ordinary algebra.                                  */
/* ------------------------------------------------------------------------ */
void oracle_u8_rowsum(int64_t M, int64_t K, const uint8_t* A, int64_t lda, int64_t* out) {
  for (int64_t m = 0; m < M; ++m) {
    int64_t s = 0;
    for (int64_t k = 0; k < K; ++k) s += A[m * lda + k];
    out[m] = s;
  }
}

void oracle_i8_colsum(int64_t N, int64_t K, const int8_t* B, int64_t ldb, int64_t* out) {
  for (int64_t n = 0; n < N; ++n) {
    int64_t s = 0;
    for (int64_t k = 0; k < K; ++k) s += B[n * ldb + k];
    out[n] = s;
  }
}

void oracle_gemm_u8i8_closed(int64_t M, int64_t N, int64_t K,
                             const uint8_t* A, int64_t lda, int64_t zA,
                             const int8_t* B, int64_t ldb, int64_t zB,
                             int64_t* C, int64_t ldc) {
  int64_t* rowsum = (int64_t*)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
  int64_t* colsum = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
  oracle_u8_rowsum(M, K, A, lda, rowsum);
  oracle_i8_colsum(N, K, B, ldb, colsum);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      int64_t ab = 0;
      for (int64_t k = 0; k < K; ++k) ab += (int64_t)A[m * lda + k] * (int64_t)B[n * ldb + k];
      C[m * ldc + n] = ab - zA * colsum[n] - zB * rowsum[m] + K * zA * zB;
    }
  }
  free(rowsum);
  free(colsum);
}

/* ------------------------------------------------------------------------ */
/* O4. Dequantize to fp32 with per-tensor scales.                             */
/* [GEMM-TVM] §2.3 lists dequantize(C) after the integer product.  Reading    */
/* taken here: one fp32 multiplier s = fl32(sA*sB), then D = fl32(fl32(C)*s), */
/* the int -> fp32 conversion rounding to nearest even.                       */
/* ------------------------------------------------------------------------ */
float oracle_dequant_scale(float sA, float sB) {
  float s = sA * sB; /* one fp32 rounding */
  return s;
}

void oracle_dequant(int64_t M, int64_t N, const int64_t* C, int64_t ldc,
                    float sA, float sB, float* D, int64_t ldd) {
  float s = oracle_dequant_scale(sA, sB);
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      float c = (float)C[m * ldc + n]; /* RNE under the default rounding mode */
      D[m * ldd + n] = c * s;
    }
}

/* ------------------------------------------------------------------------ */
/* O5. Per-output-channel scale, bias, round-to-nearest-even requantize to    */
/* int8 with saturation ([GEMM-TVM] §2.3: dequantize(C), add_bias; the stage  */
/* order is the one the workload states: scale, then bias, then requantize).  */
/*   t = fl32(fl32(C) * scale[n]);  y = fl32(t + bias[n]);                    */
/*   q = clamp(round_half_even(y), -128, 127)                                 */
/* Two separately rounded fp32 operations (no fused multiply-add).            */
/* ------------------------------------------------------------------------ */
int8_t oracle_requant_one(int64_t c, float scale, float bias) {
  float cf = (float)c;
  float t = cf * scale;
  float y = t + bias;
  float r = nearbyintf(y); /* default mode: round half to even */
  if (r > 127.0f) r = 127.0f;
  if (r < -128.0f) r = -128.0f;
  return (int8_t)r;
}

void oracle_requant(int64_t M, int64_t N, const int64_t* C, int64_t ldc,
                    const float* scale, const float* bias, int8_t* Q, int64_t ldq) {
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n)
      Q[m * ldq + n] = oracle_requant_one(C[m * ldc + n], scale[n], bias[n]);
}

/* ------------------------------------------------------------------------ */
/* O6. Direct convolution, seven loops.                                       */
/* [CONV-TC] "Preparation and algorithm": the input is zero-padded (Apad      */
/* reads the input inside the bounds, 0 outside) and                          */
/*   Conv[n,h,w,o] = sum over (kh, kw, ic) of                                 */
/*                   Apad[n, h*stride_h + kh, w*stride_w + kw, ic] * W[kh,kw,ic,o] */
/* with both factors widened before the multiply.  Cross-correlation: the     */
/* filter is not flipped.                                                     */
/*                                                                            */
/* Logical layouts (plain, unblocked): x NHWC [Nb][H][W][C] fp16,             */
/* w KRSC [Kout][R][S][C] fp16, y NHWC [Nb][P][Q][Kout] double, with          */
/* P = (H + 2*pad_h - R)/stride_h + 1 and Q likewise.  Sum order r, s, c.     */
/* ------------------------------------------------------------------------ */
static double conv_one(int64_t H, int64_t W, int64_t C, int64_t R, int64_t S,
                       int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                       const double* x, const double* w,
                       int64_t n, int64_t p, int64_t q, int64_t ko) {
  double acc = 0.0;
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t s = 0; s < S; ++s) {
      int64_t h = p * sh + r - ph;
      int64_t ww = q * sw + s - pw;
      for (int64_t c = 0; c < C; ++c) {
        double xv = 0.0; /* padding contributes zero */
        if (h >= 0 && h < H && ww >= 0 && ww < W) xv = x[((n * H + h) * W + ww) * C + c];
        acc += xv * w[((ko * R + r) * S + s) * C + c];
      }
    }
  }
  return acc;
}

int64_t oracle_conv_out_dim(int64_t in, int64_t k, int64_t stride, int64_t pad) {
  return (in + 2 * pad - k) / stride + 1;
}

/* Direct convolution at a list of output pixels m = (n*P + p)*Q + q; writes
 * y[i*Kout + ko] for each listed pixel i and every output channel ko.  With the
 * list 0..Nb*P*Q-1 this is the whole NHWC output. */
void oracle_conv2d_direct_at(int64_t Nb, int64_t H, int64_t W, int64_t C, int64_t Kout,
                             int64_t R, int64_t S, int64_t sh, int64_t sw,
                             int64_t ph, int64_t pw,
                             const uint16_t* x16, const uint16_t* w16,
                             const int64_t* pix, int64_t npix, double* y) {
  int64_t P = oracle_conv_out_dim(H, R, sh, ph);
  int64_t Q = oracle_conv_out_dim(W, S, sw, pw);
  int64_t nx = Nb * H * W * C, nw = Kout * R * S * C;
  double* x = (double*)malloc(sizeof(double) * (size_t)(nx > 0 ? nx : 1));
  double* w = (double*)malloc(sizeof(double) * (size_t)(nw > 0 ? nw : 1));
  oracle_f16_decode(x16, x, nx);
  oracle_f16_decode(w16, w, nw);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < npix; ++i) {
    int64_t m = pix[i];
    int64_t n = m / (P * Q);
    int64_t p = (m / Q) % P;
    int64_t q = m % Q;
    for (int64_t ko = 0; ko < Kout; ++ko)
      y[i * Kout + ko] = conv_one(H, W, C, R, S, sh, sw, ph, pw, x, w, n, p, q, ko);
  }
  free(x);
  free(w);
}

void oracle_conv2d_direct(int64_t Nb, int64_t H, int64_t W, int64_t C, int64_t Kout,
                          int64_t R, int64_t S, int64_t sh, int64_t sw,
                          int64_t ph, int64_t pw,
                          const uint16_t* x16, const uint16_t* w16, double* y) {
  int64_t P = oracle_conv_out_dim(H, R, sh, ph);
  int64_t Q = oracle_conv_out_dim(W, S, sw, pw);
  int64_t npix = Nb * P * Q;
  int64_t* pix = (int64_t*)malloc(sizeof(int64_t) * (size_t)(npix > 0 ? npix : 1));
  for (int64_t i = 0; i < npix; ++i) pix[i] = i;
  oracle_conv2d_direct_at(Nb, H, W, C, Kout, R, S, sh, sw, ph, pw, x16, w16, pix, npix, y);
  free(pix);
}

/* ------------------------------------------------------------------------ */
/* O7. Explicit im2col (the lowering [GEMM-TVM] §1 and §2.2 name), followed by */
/* the O1 GEMM.  Acol[m][k] with m = (n*P + p)*Q + q and k = (r*S + s)*C + c  */
/* holds x[n, p*sh + r - ph, q*sw + s - pw, c] or 0 outside the input; the    */
/* weight operand is w itself, read as Kout rows of R*S*C (column-major B).   */
/* The im2col matrix holds fp16 bit patterns, so the GEMM that follows is     */
/* exactly O1.                                                                */
/* ------------------------------------------------------------------------ */
void oracle_im2col_f16(int64_t Nb, int64_t H, int64_t W, int64_t C,
                       int64_t R, int64_t S, int64_t sh, int64_t sw,
                       int64_t ph, int64_t pw, const uint16_t* x16, uint16_t* col) {
  int64_t P = oracle_conv_out_dim(H, R, sh, ph);
  int64_t Q = oracle_conv_out_dim(W, S, sw, pw);
  int64_t Kdim = R * S * C;
  for (int64_t n = 0; n < Nb; ++n)
    for (int64_t p = 0; p < P; ++p)
      for (int64_t q = 0; q < Q; ++q) {
        int64_t m = (n * P + p) * Q + q;
        for (int64_t r = 0; r < R; ++r)
          for (int64_t s = 0; s < S; ++s) {
            int64_t h = p * sh + r - ph;
            int64_t ww = q * sw + s - pw;
            for (int64_t c = 0; c < C; ++c) {
              uint16_t v = 0; /* +0.0 in binary16 */
              if (h >= 0 && h < H && ww >= 0 && ww < W) v = x16[((n * H + h) * W + ww) * C + c];
              col[m * Kdim + (r * S + s) * C + c] = v;
            }
          }
      }
}

void oracle_conv2d_im2col(int64_t Nb, int64_t H, int64_t W, int64_t C, int64_t Kout,
                          int64_t R, int64_t S, int64_t sh, int64_t sw,
                          int64_t ph, int64_t pw,
                          const uint16_t* x16, const uint16_t* w16, double* y) {
  int64_t P = oracle_conv_out_dim(H, R, sh, ph);
  int64_t Q = oracle_conv_out_dim(W, S, sw, pw);
  int64_t M = Nb * P * Q, Kdim = R * S * C;
  uint16_t* col = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(M * Kdim > 0 ? M * Kdim : 1));
  oracle_im2col_f16(Nb, H, W, C, R, S, sh, sw, ph, pw, x16, col);
  oracle_gemm_f16(M, Kout, Kdim, col, Kdim, w16, Kdim, y, Kout);
  free(col);
}

/* ------------------------------------------------------------------------ */
/* O8. Quantized convolution: u8 activations x i8 weights with zero points.   */
/* It joins the two definitions above: the quantized product of [GEMM-TVM]    */
/* §2.3, (x_q - zp_x) * (w_q - zp_w), summed over the taps of the             */
/* convolution of [CONV-TC] "Preparation and algorithm".  The padding holds    */
/* the real value 0, whose u8 code is zp_x (the reading taken here), so a     */
/* padded tap contributes (zp_x - zp_x) * (w - zp_w) = 0.                     */
/*   y[n,p,q,ko] = sum_{r,s,c} (x[n, p*sh+r-ph, q*sw+s-pw, c] - zA)           */
/*                             * (w[ko,r,s,c] - zB)                          */
/* over the taps inside the input.  Exact in int64.  Layouts as O6 (x NHWC     */
/* uint8, w KRSC int8, y NHWC int64); written at a list of output pixels.      */
/* ------------------------------------------------------------------------ */
void oracle_conv2d_u8i8_direct_at(int64_t Nb, int64_t H, int64_t W, int64_t C, int64_t Kout,
                                  int64_t R, int64_t S, int64_t sh, int64_t sw,
                                  int64_t ph, int64_t pw,
                                  const uint8_t* x, int64_t zA, const int8_t* w, int64_t zB,
                                  const int64_t* pix, int64_t npix, int64_t* y) {
  int64_t P = oracle_conv_out_dim(H, R, sh, ph);
  int64_t Q = oracle_conv_out_dim(W, S, sw, pw);
  (void)Nb;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < npix; ++i) {
    int64_t m = pix[i];
    int64_t n = m / (P * Q);
    int64_t p = (m / Q) % P;
    int64_t q = m % Q;
    for (int64_t ko = 0; ko < Kout; ++ko) {
      int64_t acc = 0;
      for (int64_t r = 0; r < R; ++r) {
        for (int64_t s = 0; s < S; ++s) {
          int64_t h = p * sh + r - ph;
          int64_t ww = q * sw + s - pw;
          if (h < 0 || h >= H || ww < 0 || ww >= W) continue; /* padding: x - zA = 0 */
          for (int64_t c = 0; c < C; ++c)
            acc += ((int64_t)x[((n * H + h) * W + ww) * C + c] - zA) *
                   ((int64_t)w[((ko * R + r) * S + s) * C + c] - zB);
        }
      }
      y[i * Kout + ko] = acc;
    }
  }
}

/* Explicit u8 im2col for O8: Acol[m][(r*S + s)*C + c] is the input byte, or  */
/* the zero point zA where the tap falls in the padding.  Followed by O2 on   */
/* (Acol, zA) and (w, zB) it must reproduce O8.                               */
void oracle_im2col_u8(int64_t Nb, int64_t H, int64_t W, int64_t C,
                      int64_t R, int64_t S, int64_t sh, int64_t sw,
                      int64_t ph, int64_t pw, const uint8_t* x, int64_t zA, uint8_t* col) {
  int64_t P = oracle_conv_out_dim(H, R, sh, ph);
  int64_t Q = oracle_conv_out_dim(W, S, sw, pw);
  int64_t Kdim = R * S * C;
  for (int64_t n = 0; n < Nb; ++n)
    for (int64_t p = 0; p < P; ++p)
      for (int64_t q = 0; q < Q; ++q) {
        int64_t m = (n * P + p) * Q + q;
        for (int64_t r = 0; r < R; ++r)
          for (int64_t s = 0; s < S; ++s) {
            int64_t h = p * sh + r - ph;
            int64_t ww = q * sw + s - pw;
            int inside = h >= 0 && h < H && ww >= 0 && ww < W;
            for (int64_t c = 0; c < C; ++c)
              col[m * Kdim + (r * S + s) * C + c] =
                  inside ? x[((n * H + h) * W + ww) * C + c] : (uint8_t)zA;
          }
      }
}

/* ------------------------------------------------------------------------ */
/* O9. Direct convolution in the blocked NHWCnc layout of [CONV-TC]            */
/* "Preparation and algorithm" (block size 16):                               */
/*   input   A[n/16][h][w][c/16][n%16][c%16]      (data_shape)                */
/*   weights W[kh][kw][c/16][o/16][c%16][o%16]    (kernel_shape)              */
/*   output  Conv[n/16][p][q][o/16][n%16][o%16]   (output_shape)              */
/* and Conv[nb,p,q,ob,nn,oo] = sum over (kh, kw, ic, ii) of                   */
/*   Apad[nb, p*sh+kh, q*sw+kw, ic, nn, ii] * W[kh, kw, ic, ob, ii, oo]        */
/* with Apad = A inside the input and 0 in the padding, both factors widened  */
/* before the multiply.  The sum runs over (kh, kw, ic, ii), i.e. the same    */
/* (r, s, c) order as O6, so the two agree bit for bit on the same logical    */
/* tensors.  Nb, C and Kout must be multiples of 16.  fp16 in, double out.     */
/* ------------------------------------------------------------------------ */
void oracle_conv2d_nhwcnc_direct(int64_t Nb, int64_t H, int64_t W, int64_t C, int64_t Kout,
                                 int64_t R, int64_t S, int64_t sh, int64_t sw,
                                 int64_t ph, int64_t pw,
                                 const uint16_t* x16, const uint16_t* w16, double* y) {
  int64_t P = oracle_conv_out_dim(H, R, sh, ph);
  int64_t Q = oracle_conv_out_dim(W, S, sw, pw);
  int64_t NB = Nb / 16, CB = C / 16, OB = Kout / 16;
  int64_t nx = Nb * H * W * C, nw = Kout * R * S * C;
  double* x = (double*)malloc(sizeof(double) * (size_t)(nx > 0 ? nx : 1));
  double* w = (double*)malloc(sizeof(double) * (size_t)(nw > 0 ? nw : 1));
  oracle_f16_decode(x16, x, nx);
  oracle_f16_decode(w16, w, nw);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t nb = 0; nb < NB; ++nb)
    for (int64_t p = 0; p < P; ++p)
      for (int64_t q = 0; q < Q; ++q)
        for (int64_t ob = 0; ob < OB; ++ob)
          for (int64_t nn = 0; nn < 16; ++nn)
            for (int64_t oo = 0; oo < 16; ++oo) {
              double acc = 0.0;
              for (int64_t kh = 0; kh < R; ++kh)
                for (int64_t kw = 0; kw < S; ++kw) {
                  int64_t h = p * sh + kh - ph;
                  int64_t ww = q * sw + kw - pw;
                  int inside = h >= 0 && h < H && ww >= 0 && ww < W;
                  for (int64_t ic = 0; ic < CB; ++ic)
                    for (int64_t ii = 0; ii < 16; ++ii) {
                      double a = 0.0; /* padding */
                      if (inside) a = x[((((nb * H + h) * W + ww) * CB + ic) * 16 + nn) * 16 + ii];
                      acc += a * w[((((kh * S + kw) * CB + ic) * OB + ob) * 16 + ii) * 16 + oo];
                    }
                }
              y[((((nb * P + p) * Q + q) * OB + ob) * 16 + nn) * 16 + oo] = acc;
            }
  free(x);
  free(w);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
