/*
 * oracle_sanitize_main.c -- exercises every function of oracle/oracle.c on
 * small, ragged and empty problems so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (gcc, host code only) reports any out-of-bounds
 * access, leak, signed overflow or invalid shift in the oracle.  It also
 * checks the oracle's two u8 x i8 forms and its two convolution forms against
 * each other, so the run does real work.  Built and run by
 * tests/test_oracle_sanitize.py; exits non-zero on a mismatch.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_f16_to_f64(uint16_t h);
void oracle_f16_decode(const uint16_t* in, double* out, int64_t n);
void oracle_gemm_f16(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda, const uint16_t* B,
                     int64_t ldb, double* R, int64_t ldr);
void oracle_gemm_u8i8_naive(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, int64_t zA,
                            const int8_t* B, int64_t ldb, int64_t zB, int64_t* C, int64_t ldc);
void oracle_gemm_u8i8_closed(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, int64_t zA,
                             const int8_t* B, int64_t ldb, int64_t zB, int64_t* C, int64_t ldc);
void oracle_u8_rowsum(int64_t M, int64_t K, const uint8_t* A, int64_t lda, int64_t* out);
void oracle_i8_colsum(int64_t N, int64_t K, const int8_t* B, int64_t ldb, int64_t* out);
float oracle_dequant_scale(float sA, float sB);
void oracle_dequant(int64_t M, int64_t N, const int64_t* C, int64_t ldc, float sA, float sB, float* D,
                    int64_t ldd);
int8_t oracle_requant_one(int64_t c, float scale, float bias);
void oracle_requant(int64_t M, int64_t N, const int64_t* C, int64_t ldc, const float* scale,
                    const float* bias, int8_t* Q, int64_t ldq);
int64_t oracle_conv_out_dim(int64_t in, int64_t k, int64_t stride, int64_t pad);
void oracle_conv2d_direct(int64_t Nb, int64_t H, int64_t W, int64_t C, int64_t Kout, int64_t R, int64_t S,
                          int64_t sh, int64_t sw, int64_t ph, int64_t pw, const uint16_t* x16,
                          const uint16_t* w16, double* y);
void oracle_conv2d_im2col(int64_t Nb, int64_t H, int64_t W, int64_t C, int64_t Kout, int64_t R, int64_t S,
                          int64_t sh, int64_t sw, int64_t ph, int64_t pw, const uint16_t* x16,
                          const uint16_t* w16, double* y);
void oracle_conv2d_u8i8_direct_at(int64_t Nb, int64_t H, int64_t W, int64_t C, int64_t Kout, int64_t R,
                                  int64_t S, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                                  const uint8_t* x, int64_t zA, const int8_t* w, int64_t zB,
                                  const int64_t* pix, int64_t npix, int64_t* y);
void oracle_im2col_u8(int64_t Nb, int64_t H, int64_t W, int64_t C, int64_t R, int64_t S, int64_t sh,
                      int64_t sw, int64_t ph, int64_t pw, const uint8_t* x, int64_t zA, uint8_t* col);
void oracle_conv2d_nhwcnc_direct(int64_t Nb, int64_t H, int64_t W, int64_t C, int64_t Kout, int64_t R,
                                 int64_t S, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                                 const uint16_t* x16, const uint16_t* w16, double* y);
int oracle_num_threads(void);

static uint32_t state = 12345u;
static uint32_t next(void) {
  state = state * 1664525u + 1013904223u;
  return state >> 8;
}
/* finite fp16 bit patterns with small integer values -8..8 (exact sums) */
static uint16_t small_f16(void) {
  static const uint16_t tab[17] = {0xc800, 0xc700, 0xc600, 0xc500, 0xc400, 0xc200, 0xc000, 0xbc00, 0x0000,
                                   0x3c00, 0x4000, 0x4200, 0x4400, 0x4500, 0x4600, 0x4700, 0x4800};
  return tab[next() % 17];
}

static int fails = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++fails;                                                        \
    }                                                                 \
  } while (0)

static void gemm_cases(void) {
  const int64_t shapes[][3] = {{5, 7, 13}, {1, 1, 1}, {0, 4, 4}, {4, 0, 4}, {3, 3, 0}, {9, 2, 33}};
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
    const int64_t M = shapes[s][0], N = shapes[s][1], K = shapes[s][2];
    const int64_t lda = K + 3, ldb = K + 1, ldc = N + 2;
    uint16_t* A = malloc(sizeof(uint16_t) * (size_t)(M * lda + 1));
    uint16_t* B = malloc(sizeof(uint16_t) * (size_t)(N * ldb + 1));
    uint8_t* A8 = malloc((size_t)(M * lda + 1));
    int8_t* B8 = malloc((size_t)(N * ldb + 1));
    double* R = malloc(sizeof(double) * (size_t)(M * ldc + 1));
    int64_t* C1 = malloc(sizeof(int64_t) * (size_t)(M * ldc + 1));
    int64_t* C2 = malloc(sizeof(int64_t) * (size_t)(M * ldc + 1));
    float* D = malloc(sizeof(float) * (size_t)(M * ldc + 1));
    int8_t* Q = malloc((size_t)(M * ldc + 1));
    float* sc = malloc(sizeof(float) * (size_t)(N + 1));
    float* bi = malloc(sizeof(float) * (size_t)(N + 1));
    int64_t* rs = malloc(sizeof(int64_t) * (size_t)(M + 1));
    int64_t* cs = malloc(sizeof(int64_t) * (size_t)(N + 1));
    for (int64_t i = 0; i < M * lda; ++i) {
      A[i] = small_f16();
      A8[i] = (uint8_t)next();
    }
    for (int64_t i = 0; i < N * ldb; ++i) {
      B[i] = small_f16();
      B8[i] = (int8_t)(next() & 0xff);
    }
    for (int64_t n = 0; n < N; ++n) {
      sc[n] = 0.001f * (float)(1 + n);
      bi[n] = 0.5f * (float)n - 1.0f;
    }
    oracle_gemm_f16(M, N, K, A, lda, B, ldb, R, ldc);
    const int64_t zps[][2] = {{0, 0}, {128, 3}, {255, -128}, {37, 127}};
    for (int z = 0; z < 4; ++z) {
      oracle_gemm_u8i8_naive(M, N, K, A8, lda, zps[z][0], B8, ldb, zps[z][1], C1, ldc);
      oracle_gemm_u8i8_closed(M, N, K, A8, lda, zps[z][0], B8, ldb, zps[z][1], C2, ldc);
      for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) CHECK(C1[m * ldc + n] == C2[m * ldc + n]);
    }
    oracle_u8_rowsum(M, K, A8, lda, rs);
    oracle_i8_colsum(N, K, B8, ldb, cs);
    oracle_dequant(M, N, C1, ldc, 0.02f, 0.01f, D, ldc);
    oracle_requant(M, N, C1, ldc, sc, bi, Q, ldc);
    free(A); free(B); free(A8); free(B8); free(R); free(C1); free(C2); free(D); free(Q);
    free(sc); free(bi); free(rs); free(cs);
  }
  CHECK(oracle_requant_one(255, 0.5f, 0.0f) == 127);
  CHECK(oracle_requant_one(-257, 0.5f, 0.0f) == -128);
  CHECK(oracle_requant_one(INT64_C(2147483647), 1.0f, 0.0f) == 127);
  CHECK(oracle_dequant_scale(0.5f, 0.25f) == 0.125f);
}

static void conv_cases(void) {
  /* Nb, H, W, C, Kout, R, S, sh, sw, ph, pw */
  const int64_t shapes[][11] = {{2, 5, 4, 3, 2, 3, 3, 1, 1, 1, 1}, {1, 3, 7, 2, 3, 2, 3, 2, 1, 0, 2},
                                {1, 1, 1, 1, 1, 1, 1, 1, 1, 0, 0}, {1, 4, 4, 5, 2, 4, 4, 3, 3, 2, 2}};
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s) {
    const int64_t* d = shapes[s];
    const int64_t Nb = d[0], H = d[1], W = d[2], C = d[3], Kout = d[4], R = d[5], S = d[6];
    const int64_t P = oracle_conv_out_dim(H, R, d[7], d[9]), Qo = oracle_conv_out_dim(W, S, d[8], d[10]);
    const int64_t nx = Nb * H * W * C, nw = Kout * R * S * C, ny = Nb * P * Qo * Kout;
    uint16_t* x = malloc(sizeof(uint16_t) * (size_t)nx);
    uint16_t* w = malloc(sizeof(uint16_t) * (size_t)nw);
    uint8_t* x8 = malloc((size_t)nx);
    int8_t* w8 = malloc((size_t)nw);
    for (int64_t i = 0; i < nx; ++i) {
      x[i] = small_f16();
      x8[i] = (uint8_t)next();
    }
    for (int64_t i = 0; i < nw; ++i) {
      w[i] = small_f16();
      w8[i] = (int8_t)(next() & 0xff);
    }
    double* y1 = malloc(sizeof(double) * (size_t)ny);
    double* y2 = malloc(sizeof(double) * (size_t)ny);
    oracle_conv2d_direct(Nb, H, W, C, Kout, R, S, d[7], d[8], d[9], d[10], x, w, y1);
    oracle_conv2d_im2col(Nb, H, W, C, Kout, R, S, d[7], d[8], d[9], d[10], x, w, y2);
    for (int64_t i = 0; i < ny; ++i) CHECK(y1[i] == y2[i]);
    const int64_t npix = Nb * P * Qo, Kd = R * S * C;
    int64_t* pix = malloc(sizeof(int64_t) * (size_t)npix);
    for (int64_t i = 0; i < npix; ++i) pix[i] = i;
    int64_t* q1 = malloc(sizeof(int64_t) * (size_t)ny);
    int64_t* q2 = malloc(sizeof(int64_t) * (size_t)ny);
    uint8_t* col = malloc((size_t)(npix * Kd));
    oracle_conv2d_u8i8_direct_at(Nb, H, W, C, Kout, R, S, d[7], d[8], d[9], d[10], x8, 77, w8, -3, pix, npix, q1);
    oracle_im2col_u8(Nb, H, W, C, R, S, d[7], d[8], d[9], d[10], x8, 77, col);
    oracle_gemm_u8i8_naive(npix, Kout, Kd, col, Kd, 77, w8, Kd, -3, q2, Kout);
    for (int64_t i = 0; i < ny; ++i) CHECK(q1[i] == q2[i]);
    free(x); free(w); free(x8); free(w8); free(y1); free(y2); free(pix); free(q1); free(q2); free(col);
  }
}

/* the blocked layout against the plain one on the same logical tensors */
static void blocked_case(void) {
  const int64_t Nb = 16, H = 3, W = 4, C = 32, Kout = 16, R = 3, S = 2, sh = 1, sw = 2, ph = 1, pw = 1;
  const int64_t P = oracle_conv_out_dim(H, R, sh, ph), Qo = oracle_conv_out_dim(W, S, sw, pw);
  const int64_t nx = Nb * H * W * C, nw = Kout * R * S * C, ny = Nb * P * Qo * Kout;
  uint16_t* xb = malloc(sizeof(uint16_t) * (size_t)nx);
  uint16_t* wb = malloc(sizeof(uint16_t) * (size_t)nw);
  uint16_t* x = malloc(sizeof(uint16_t) * (size_t)nx);
  uint16_t* w = malloc(sizeof(uint16_t) * (size_t)nw);
  double* yb = malloc(sizeof(double) * (size_t)ny);
  double* y = malloc(sizeof(double) * (size_t)ny);
  for (int64_t i = 0; i < nx; ++i) xb[i] = small_f16();
  for (int64_t i = 0; i < nw; ++i) wb[i] = small_f16();
  for (int64_t n = 0; n < Nb; ++n)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t ww = 0; ww < W; ++ww)
        for (int64_t c = 0; c < C; ++c)
          x[((n * H + h) * W + ww) * C + c] = xb[((((n / 16) * H + h) * W + ww) * (C / 16) + c / 16) * 256 + (n % 16) * 16 + c % 16];
  for (int64_t k = 0; k < Kout; ++k)
    for (int64_t r = 0; r < R; ++r)
      for (int64_t s = 0; s < S; ++s)
        for (int64_t c = 0; c < C; ++c)
          w[((k * R + r) * S + s) * C + c] = wb[(((r * S + s) * (C / 16) + c / 16) * (Kout / 16) + k / 16) * 256 + (c % 16) * 16 + k % 16];
  oracle_conv2d_nhwcnc_direct(Nb, H, W, C, Kout, R, S, sh, sw, ph, pw, xb, wb, yb);
  oracle_conv2d_direct(Nb, H, W, C, Kout, R, S, sh, sw, ph, pw, x, w, y);
  for (int64_t n = 0; n < Nb; ++n)
    for (int64_t p = 0; p < P; ++p)
      for (int64_t q = 0; q < Qo; ++q)
        for (int64_t k = 0; k < Kout; ++k)
          CHECK(y[((n * P + p) * Qo + q) * Kout + k] ==
                yb[((((n / 16) * P + p) * Qo + q) * (Kout / 16) + k / 16) * 256 + (n % 16) * 16 + k % 16]);
  free(xb); free(wb); free(x); free(w); free(yb); free(y);
}

int main(void) {
  for (uint32_t h = 0; h < 65536; ++h) (void)oracle_f16_to_f64((uint16_t)h);
  uint16_t bits[4] = {0x0001, 0x7bff, 0xfc00, 0x3c00};
  double out[4];
  oracle_f16_decode(bits, out, 4);
  CHECK(out[3] == 1.0);
  gemm_cases();
  conv_cases();
  blocked_case();
  CHECK(oracle_num_threads() >= 1);
  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("oracle sanitizer run: ok\n");
  return 0;
}
