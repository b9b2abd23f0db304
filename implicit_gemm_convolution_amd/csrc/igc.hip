// igc.hip -- the C ABI of libigc.so (declared in include/igc.h): argument
// validation, device check, and the host state of the launches (error
// detail, compute-unit counts, stream-K workspaces).  Variant choice and the
// launches themselves are in igc_host.hpp, instantiated in igc_launch.hip;
// all arithmetic happens in the kernels of igc_kernels.hpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <map>
#include <mutex>
#include <utility>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/igc.h"
#include "igc_host.hpp"
namespace igc_host {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

// Per-device architecture cache: 0 unknown, 1 gfx950, -1 other.
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device(int* dev_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(IGC_ENODEV, "no HIP device: %s", hipGetErrorString(e));
  }
  if (dev >= kMaxDevices) return fail(IGC_ENODEV, "device index %d out of range", dev);
  int st = g_arch_ok[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(IGC_ENODEV, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    }
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_arch_ok[dev].store(st, std::memory_order_release);
    if (st < 0) return fail(IGC_ENODEV, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  }
  if (st < 0) return fail(IGC_ENODEV, "device %d is not gfx950", dev);
  *dev_out = dev;
  return IGC_OK;
}

// Per-device compute-unit count (0 = not read yet).
std::atomic<int> g_cus[kMaxDevices];

int device_cus(int dev) {
  int n = g_cus[dev].load(std::memory_order_acquire);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    g_cus[dev].store(n, std::memory_order_release);
  }
  return n;
}

// Stream-K workspace, one per (device, stream) so that launches on different
// streams never share it: partial tiles and per-tile arrival counters (zeroed
// once when allocated; the kernel leaves them at zero).  It grows on demand
// and is kept until the process ends.
struct SkWorkspace {
  void* ws = nullptr;
  size_t ws_bytes = 0;
  int* cnt = nullptr;
  size_t cnt_n = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, SkWorkspace> g_ws;

int sk_workspace(int dev, hipStream_t stream, size_t ws_bytes, size_t cnt_n, float** ws, int** cnt) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  SkWorkspace& w = g_ws[std::make_pair(dev, stream)];
  if (w.ws_bytes < ws_bytes || w.cnt_n < cnt_n) {
    if (w.ws || w.cnt) {
      // earlier launches on this stream may still use the old buffers
      if (hipStreamSynchronize(stream) != hipSuccess) {
        (void)hipGetLastError();
        return fail(IGC_EHIP, "hipStreamSynchronize failed before growing the stream-K workspace");
      }
      (void)hipFree(w.ws);
      (void)hipFree(w.cnt);
      w = SkWorkspace();
    }
    const size_t nb = std::max(ws_bytes, w.ws_bytes), nc = std::max(cnt_n, w.cnt_n);
    if (hipMalloc(&w.ws, nb) != hipSuccess || hipMalloc(reinterpret_cast<void**>(&w.cnt), nc * sizeof(int)) != hipSuccess ||
        hipMemsetAsync(w.cnt, 0, nc * sizeof(int), stream) != hipSuccess) {
      (void)hipGetLastError();
      if (w.ws) (void)hipFree(w.ws);
      if (w.cnt) (void)hipFree(w.cnt);
      w = SkWorkspace();
      return fail(IGC_EHIP, "cannot allocate the stream-K workspace (%zu bytes)", nb);
    }
    w.ws_bytes = nb;
    w.cnt_n = nc;
  }
  *ws = static_cast<float*>(w.ws);
  *cnt = w.cnt;
  return IGC_OK;
}

igc::Params zero_params() {
  igc::Params p;
  std::memset(&p, 0, sizeof(p));
  return p;
}

// Validation shared by the two convolutions; fills the im2col part of p.
int conv_params(int Nb, int H, int W, int C, int Kout, int R, int S, int stride_h, int stride_w,
                int pad_h, int pad_w, igc::Params& p, long long* nx_out) {
  if (Nb <= 0 || H <= 0 || W <= 0 || C <= 0 || Kout <= 0 || R <= 0 || S <= 0)
    return fail(IGC_EINVAL, "non-positive dimension");
  if (stride_h <= 0 || stride_w <= 0 || pad_h < 0 || pad_w < 0)
    return fail(IGC_EINVAL, "bad stride or padding");
  const long long P = ((long long)H + 2LL * pad_h - R) / stride_h + 1;
  const long long Q = ((long long)W + 2LL * pad_w - S) / stride_w + 1;
  if ((long long)H + 2LL * pad_h < R || (long long)W + 2LL * pad_w < S || P < 1 || Q < 1)
    return fail(IGC_EINVAL, "filter larger than the padded input");
  const long long M = (long long)Nb * P * Q;
  const long long K = (long long)R * S * C;
  const long long nx = (long long)Nb * H * W * C;
  if (M > 0x7fffffffLL || K > 0x7fffffffLL || nx > 0x7fffffffLL ||
      (long long)Kout * K > 0x7fffffffLL || M * Kout > (1LL << 62))
    return fail(IGC_EUNSUPPORTED, "tensor index exceeds 32 bits");
  p.M = (int)M; p.N = Kout; p.K = (int)K;
  p.Nb = Nb; p.H = H; p.W = W; p.C = C; p.R = R; p.S = S;
  p.sh = stride_h; p.sw = stride_w; p.ph = pad_h; p.pw = pad_w;
  p.P = (int)P; p.Q = (int)Q;
  *nx_out = nx;
  return IGC_OK;
}

// The zero-point sums are compiled only into the kernels that need them:
// rowsum(A') when zB != 0, colsum(B) when zA != 128.
template <int KIND>
int launch_u8i8(const igc::Params& p, bool fast, hipStream_t stream, int dev) {
  const int sums = (p.zB != 0 ? igc::SUM_ROWS : 0) | (p.zAp != 0 ? igc::SUM_COLS : 0);
  switch (sums) {
    case 0: return launch<KIND, 0>(p, fast, stream, dev);
    case 1: return launch<KIND, 1>(p, fast, stream, dev);
    case 2: return launch<KIND, 2>(p, fast, stream, dev);
    default: return launch<KIND, 3>(p, fast, stream, dev);
  }
}

}  // namespace igc_host

using namespace igc_host;

extern "C" {

const char* igc_status_string(int status) {
  switch (status) {
    case IGC_OK: return "IGC_OK";
    case IGC_EINVAL: return "IGC_EINVAL: invalid argument";
    case IGC_EUNSUPPORTED: return "IGC_EUNSUPPORTED: shape not supported";
    case IGC_EOVERFLOW: return "IGC_EOVERFLOW: K too large for an exact int32 result";
    case IGC_EHIP: return "IGC_EHIP: HIP runtime error";
    case IGC_ENODEV: return "IGC_ENODEV: no gfx950 device";
    default: return "unknown status";
  }
}

const char* igc_last_error(void) { return g_last_error; }

int igc_device_check(void) {
  int dev;
  return check_device(&dev);
}

int gemm_f16f32(int M, int N, int K, const void* A, int lda, const void* B, int ldb, float* C,
                int ldc, void* stream) {
  g_last_error[0] = 0;
  if (M < 0 || N < 0 || K < 0) return fail(IGC_EINVAL, "negative size M=%d N=%d K=%d", M, N, K);
  if (M == 0 || N == 0) return IGC_OK;
  if (!C) return fail(IGC_EINVAL, "C is NULL");
  if (ldc < N) return fail(IGC_EINVAL, "ldc=%d < N=%d", ldc, N);
  if (K > 0) {
    if (!A || !B) return fail(IGC_EINVAL, "A or B is NULL");
    if (lda < K || ldb < K) return fail(IGC_EINVAL, "lda=%d / ldb=%d < K=%d", lda, ldb, K);
  }
  int dev;
  if (int s = check_device(&dev)) return s;
  igc::Params p = zero_params();
  p.M = M; p.N = N; p.K = K;
  p.A = static_cast<const uint8_t*>(A); p.lda = lda;
  p.B = static_cast<const uint8_t*>(B); p.ldb = ldb;
  p.Cf = C; p.ldcf = ldc;
  p.vec_c = aligned16(C) && ldc % 4 == 0;  // 16-byte stores of 4 consecutive columns
  // Buffer descriptors of the fast path cover one tile of rows and must stay below 2^31 bytes.
  const bool fast = aligned16(A) && aligned16(B) && lda % 8 == 0 && ldb % 8 == 0 && K % 8 == 0 &&
                    256LL * lda * 2 < (1LL << 31) && 256LL * ldb * 2 < (1LL << 31);
  return launch<igc::KIND_F16_GEMM, 0>(p, fast, static_cast<hipStream_t>(stream), dev);
}

int gemm_u8i8_zp(int M, int N, int K, const uint8_t* A, int lda, int zA, const int8_t* B, int ldb,
                 int zB, const igc_u8i8_epilogue* ep, void* stream) {
  g_last_error[0] = 0;
  if (M < 0 || N < 0 || K < 0) return fail(IGC_EINVAL, "negative size M=%d N=%d K=%d", M, N, K);
  if (zA < 0 || zA > 255) return fail(IGC_EINVAL, "zA=%d outside [0, 255]", zA);
  if (zB < -128 || zB > 127) return fail(IGC_EINVAL, "zB=%d outside [-128, 127]", zB);
  if (!ep) return fail(IGC_EINVAL, "epilogue descriptor is NULL");
  if (!ep->C_i32 && !ep->D_f32 && !ep->Q_i8) return fail(IGC_EINVAL, "no output requested");
  if (K > 33025) return fail(IGC_EOVERFLOW, "K=%d > 33025 can overflow int32", K);
  if (M == 0 || N == 0) return IGC_OK;
  if (ep->C_i32 && ep->ldc < N) return fail(IGC_EINVAL, "ldc=%d < N=%d", ep->ldc, N);
  if (ep->D_f32 && ep->ldd < N) return fail(IGC_EINVAL, "ldd=%d < N=%d", ep->ldd, N);
  if (ep->Q_i8) {
    if (ep->ldq < N) return fail(IGC_EINVAL, "ldq=%d < N=%d", ep->ldq, N);
    if (!ep->scale_n || !ep->bias_n) return fail(IGC_EINVAL, "Q_i8 needs scale_n and bias_n");
  }
  if (K > 0) {
    if (!A || !B) return fail(IGC_EINVAL, "A or B is NULL");
    if (lda < K || ldb < K) return fail(IGC_EINVAL, "lda=%d / ldb=%d < K=%d", lda, ldb, K);
  }
  int dev;
  if (int s = check_device(&dev)) return s;
  igc::Params p = zero_params();
  p.M = M; p.N = N; p.K = K;
  p.A = A; p.lda = lda;
  p.B = reinterpret_cast<const uint8_t*>(B); p.ldb = ldb;
  p.zAp = zA - 128; p.zB = zB;
  p.Ci = ep->C_i32; p.ldci = ep->ldc;
  p.D = ep->D_f32; p.ldd = ep->ldd; p.dq = ep->dq_scale;
  p.Qo = ep->Q_i8; p.ldq = ep->ldq; p.scale = ep->scale_n; p.bias = ep->bias_n;
  p.vec_c = aligned16(ep->C_i32) && ep->ldc % 4 == 0;
  p.vec_d = aligned16(ep->D_f32) && ep->ldd % 4 == 0;
  p.vec_q = (reinterpret_cast<uintptr_t>(ep->Q_i8) & 3u) == 0 && ep->ldq % 4 == 0;
  const bool fast = aligned16(A) && aligned16(B) && lda % 16 == 0 && ldb % 16 == 0 &&
                    K % 16 == 0 && 256LL * lda < (1LL << 31) && 256LL * ldb < (1LL << 31);
  return launch_u8i8<igc::KIND_U8I8_GEMM>(p, fast, static_cast<hipStream_t>(stream), dev);
}

int conv2d_u8i8_zp(int Nb, int H, int W, int C, int Kout, int R, int S, int stride_h, int stride_w,
                   int pad_h, int pad_w, const uint8_t* x, int zA, const int8_t* w, int zB,
                   const igc_u8i8_epilogue* ep, void* stream) {
  g_last_error[0] = 0;
  igc::Params p = zero_params();
  long long nx = 0;
  if (int st = conv_params(Nb, H, W, C, Kout, R, S, stride_h, stride_w, pad_h, pad_w, p, &nx)) return st;
  if (!x || !w) return fail(IGC_EINVAL, "x or w is NULL");
  if (zA < 0 || zA > 255) return fail(IGC_EINVAL, "zA=%d outside [0, 255]", zA);
  if (zB < -128 || zB > 127) return fail(IGC_EINVAL, "zB=%d outside [-128, 127]", zB);
  if (!ep) return fail(IGC_EINVAL, "epilogue descriptor is NULL");
  if (!ep->C_i32 && !ep->D_f32 && !ep->Q_i8) return fail(IGC_EINVAL, "no output requested");
  if (p.K > 33025) return fail(IGC_EOVERFLOW, "K=R*S*C=%d > 33025 can overflow int32", p.K);
  const int N = Kout;
  if (ep->C_i32 && ep->ldc < N) return fail(IGC_EINVAL, "ldc=%d < Kout=%d", ep->ldc, N);
  if (ep->D_f32 && ep->ldd < N) return fail(IGC_EINVAL, "ldd=%d < Kout=%d", ep->ldd, N);
  if (ep->Q_i8) {
    if (ep->ldq < N) return fail(IGC_EINVAL, "ldq=%d < Kout=%d", ep->ldq, N);
    if (!ep->scale_n || !ep->bias_n) return fail(IGC_EINVAL, "Q_i8 needs scale_n and bias_n");
  }
  int dev;
  if (int s = check_device(&dev)) return s;
  p.A = x; p.lda = 0;
  p.B = reinterpret_cast<const uint8_t*>(w); p.ldb = p.K;
  p.zAp = zA - 128; p.zB = zB;
  p.Ci = ep->C_i32; p.ldci = ep->ldc;
  p.D = ep->D_f32; p.ldd = ep->ldd; p.dq = ep->dq_scale;
  p.Qo = ep->Q_i8; p.ldq = ep->ldq; p.scale = ep->scale_n; p.bias = ep->bias_n;
  p.vec_c = aligned16(ep->C_i32) && ep->ldc % 4 == 0;
  p.vec_d = aligned16(ep->D_f32) && ep->ldd % 4 == 0;
  p.vec_q = (reinterpret_cast<uintptr_t>(ep->Q_i8) & 3u) == 0 && ep->ldq % 4 == 0;
  // whole 128-channel K tiles within one tap: the uniform-tap loader
  const bool fast = aligned16(x) && aligned16(w) && C % 128 == 0 && (long long)R * S <= 31 &&
                    nx < (1LL << 31) && 256LL * p.K < (1LL << 31);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launch_u8i8<igc::KIND_U8I8_CONV>(p, fast, st, dev);
}

int conv2d_implicit_gemm(int Nb, int H, int W, int C, int Kout, int R, int S, int stride_h,
                         int stride_w, int pad_h, int pad_w, const void* x, const void* w, float* y,
                         void* stream) {
  g_last_error[0] = 0;
  igc::Params p = zero_params();
  long long nx = 0;
  if (int st = conv_params(Nb, H, W, C, Kout, R, S, stride_h, stride_w, pad_h, pad_w, p, &nx)) return st;
  if (!x || !w || !y) return fail(IGC_EINVAL, "x, w or y is NULL");
  int dev;
  if (int s = check_device(&dev)) return s;
  p.A = static_cast<const uint8_t*>(x); p.lda = 0;
  p.B = static_cast<const uint8_t*>(w); p.ldb = p.K;
  p.Cf = y; p.ldcf = Kout;
  p.vec_c = aligned16(y) && Kout % 4 == 0;
  const bool fast = aligned16(x) && aligned16(w) && C % 8 == 0 && nx * 2 < (1LL << 31) &&
                    256LL * p.K * 2 < (1LL << 31);
  // whole 64-channel K tiles within one tap: the uniform-tap loader
  if (fast && C % 64 == 0 && (long long)R * S <= 31)
    return launch<igc::KIND_F16_CONV_C64, 0>(p, true, static_cast<hipStream_t>(stream), dev);
  return launch<igc::KIND_F16_CONV, 0>(p, fast, static_cast<hipStream_t>(stream), dev);
}

}  // extern "C"
