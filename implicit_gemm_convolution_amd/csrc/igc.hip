// igc.hip -- the C ABI of libigc.so (declared in include/igc.h): argument
// validation, device check, workspace checks and the library's host state
// (error detail, per-device architecture and compute-unit counts, tuning
// overrides).  The launch plan and the launches themselves are in
// igc_host.hpp, instantiated in igc_launch.hip; all arithmetic happens in the
// kernels of igc_kernels.hpp.  The library allocates no device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <mutex>
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

std::atomic<int> g_force_variant{V_AUTO};
std::atomic<int> g_streamk_mode{1};

// The caller's workspace against the plan: none needed, or one large enough.
int check_workspace(const Plan& pl, const void* ws, size_t ws_bytes) {
  if (!pl.ws_bytes) return IGC_OK;
  if (ws_bytes < pl.ws_bytes)
    return fail(IGC_EINVAL, "workspace of %zu bytes < the %zu bytes this call needs", ws_bytes, pl.ws_bytes);
  if (!aligned16(ws)) return fail(IGC_EINVAL, "workspace not 16-byte aligned");
  return IGC_OK;
}

igc::Params zero_params() {
  igc::Params p;
  std::memset(&p, 0, sizeof(p));
  return p;
}

// Validation shared by the two convolutions; fills the im2col part of p.
// The im2col loaders keep a row's top-left input coordinate in two signed
// 16-bit halves of one register, so H, W, R, S and the paddings must stay
// below 2^15.
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
  if (H >= 32768 || W >= 32768 || R >= 32768 || S >= 32768 || pad_h >= 32768 || pad_w >= 32768)
    return fail(IGC_EUNSUPPORTED, "H, W, R, S, pad_h and pad_w must be below 32768");
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
  p.fd_pq = make_fastdiv(P * Q);
  p.fd_q = make_fastdiv(Q);
  p.fd_c = make_fastdiv(C);
  p.fd_s = make_fastdiv(S);
  *nx_out = nx;
  return IGC_OK;
}

// Validation of a u8 x i8 output descriptor for an M x N product.
int check_epilogue(const igc_u8i8_epilogue* ep, int N, int K) {
  if (!ep) return fail(IGC_EINVAL, "epilogue descriptor is NULL");
  if (!ep->C_i32 && !ep->D_f32 && !ep->Q_i8) return fail(IGC_EINVAL, "no output requested");
  if (K > 33025) return fail(IGC_EOVERFLOW, "K=%d > 33025 can overflow int32", K);
  if (ep->C_i32 && ep->ldc < N) return fail(IGC_EINVAL, "ldc=%d < N=%d", ep->ldc, N);
  if (ep->D_f32 && ep->ldd < N) return fail(IGC_EINVAL, "ldd=%d < N=%d", ep->ldd, N);
  if (ep->Q_i8) {
    if (ep->ldq < N) return fail(IGC_EINVAL, "ldq=%d < N=%d", ep->ldq, N);
    if (!ep->scale_n || !ep->bias_n) return fail(IGC_EINVAL, "Q_i8 needs scale_n and bias_n");
  }
  if ((reinterpret_cast<uintptr_t>(ep->colsum_B) & 3u) != 0) return fail(IGC_EINVAL, "colsum_B is not 4-byte aligned");
  return IGC_OK;
}

void epilogue_params(igc::Params& p, const igc_u8i8_epilogue* ep) {
  p.Ci = ep->C_i32; p.ldci = ep->ldc;
  p.D = ep->D_f32; p.ldd = ep->ldd; p.dq = ep->dq_scale;
  p.Qo = ep->Q_i8; p.ldq = ep->ldq; p.scale = ep->scale_n; p.bias = ep->bias_n;
  p.colsum = ep->colsum_B;
  p.vec_c = aligned16(ep->C_i32) && ep->ldc % 4 == 0;
  p.vec_d = aligned16(ep->D_f32) && ep->ldd % 4 == 0;
  p.vec_q = (reinterpret_cast<uintptr_t>(ep->Q_i8) & 3u) == 0 && ep->ldq % 4 == 0;
}

// Plans a launch on the current device, checks the caller's workspace
// against it and launches.
template <int KIND, int SUMS>
int plan_and_launch(igc::Params& p, bool fast, void* ws, size_t ws_bytes, hipStream_t stream) {
  int dev;
  if (int s = check_device(&dev)) return s;
  const Plan pl = make_plan(KIND, p.M, p.N, p.K, fast, device_cus(dev), ws != nullptr);
  if (int s = check_workspace(pl, ws, ws_bytes)) return s;
  apply_plan(p, pl, ws);
  if constexpr (KIND == igc::KIND_U8I8_GEMM || KIND == igc::KIND_U8I8_CONV) {
    if (req_tiles(p, pl, fast)) {
      // the caller's column sums replace the K loop's
      if constexpr ((SUMS & igc::SUM_COLS) != 0)
        if (p.colsum)
          return launch<KIND, (SUMS & igc::SUM_ROWS) | igc::REQ_TILES | igc::COLS_IN>(p, pl, fast, stream);
      return launch<KIND, SUMS | igc::REQ_TILES>(p, pl, fast, stream);
    }
    if (pl.sk_wgs == 0 && fast && (pl.variant == V_64x64 || pl.variant == V_128x128))
      return launch<KIND, SUMS | igc::NO_SPLIT>(p, pl, fast, stream);
  }
  if constexpr (KIND == igc::KIND_F16_GEMM || KIND == igc::KIND_F16_CONV || KIND == igc::KIND_F16_CONV_C64)
    if (pl.sk_wgs == 0) return launch<KIND, SUMS | igc::NO_SPLIT>(p, pl, fast, stream);
  return launch<KIND, SUMS>(p, pl, fast, stream);
}

// The zero-point sums are compiled only into the kernels that need them:
// rowsum(A') when zB != 0, colsum(B) when zA != 128.
template <int KIND>
int launch_u8i8(igc::Params& p, bool fast, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int sums = (p.zB != 0 ? igc::SUM_ROWS : 0) | (p.zAp != 0 ? igc::SUM_COLS : 0);
  switch (sums) {
    case 0: return plan_and_launch<KIND, 0>(p, fast, ws, ws_bytes, stream);
    case 1: return plan_and_launch<KIND, 1>(p, fast, ws, ws_bytes, stream);
    case 2: return plan_and_launch<KIND, 2>(p, fast, ws, ws_bytes, stream);
    default: return plan_and_launch<KIND, 3>(p, fast, ws, ws_bytes, stream);
  }
}

// Scratch of gemm_f16f32_noalloc: the stream-K workspace as a static device
// array, one per GPU, held until the process ends.  In host code `scratch`
// only names the symbol; its device address comes from hipGetSymbolAddress,
// taken once per device with that device current and kept in
// g_scratch_ptr.
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return fail(IGC_EHIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return IGC_OK;
}

// Zero-fills n 32-bit words (a kernel, not a memset, so that a caller's HIP
// graph capture records an ordinary kernel node).
__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* p, int n) {
  const int i = (int)(blockIdx.x * 256 + threadIdx.x);
  if (i < n) p[i] = 0u;
}

// Column sums of an int8 operand stored as N rows of K ([GEMM-TVM] §2.3, the
// zA * colsum(B) term): one wave per row, each lane summing every 64th
// 16-byte chunk (aligned rows) or every 64th byte, then a reduction across
// the wave.
__global__ void __launch_bounds__(256) i8_colsum_kernel(const int8_t* __restrict__ B, int ldb, int N, int K,
                                                        int32_t* __restrict__ out) {
  const int n = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= N) return;
  const int8_t* row = B + (long long)n * ldb;
  int s = 0;
  if ((reinterpret_cast<uintptr_t>(row) & 15u) == 0 && K % 16 == 0) {
    for (int k = lane * 16; k < K; k += 64 * 16) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + k);
      s = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, s, false);
      s = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, s, false);
      s = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, s, false);
      s = __builtin_amdgcn_sdot4((int)v.w, 0x01010101, s, false);
    }
  } else {
    for (int k = lane; k < K; k += 64) s += row[k];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) out[n] = s;
}

// ---------------------------------------------------------------------------
// Weights of the blocked NHWCnc convolution ([CONV-TC] "Preparation and
// algorithm": W[kh][kw][c/16][k/16][c%16][k%16], output channels innermost)
// rewritten in the GEMM's K-contiguous order [k][kh][kw][c] (the column-major
// B operand), so both MFMA operands read 16 consecutive bytes of K per lane.
// Each group of 32 threads transposes one 16 x 16 block through LDS: thread t
// loads channel t/2, output channels 8(t%2) .. +7 (16 bytes) and stores
// output channel t/2, channels 8(t%2) .. +7 (16 bytes).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) nhwcnc_weights_kernel(const uint16_t* __restrict__ wb,
                                                             uint16_t* __restrict__ krsc, int RS, int C,
                                                             int Kout, int nblocks) {
  __shared__ uint16_t t16[8][16][17];
  const int grp = threadIdx.x >> 5, t = threadIdx.x & 31;
  const int bi = (int)blockIdx.x * 8 + grp;
  const bool live = bi < nblocks;
  if (live) {
    const uint4 v = *reinterpret_cast<const uint4*>(wb + (long long)bi * 256 + (t >> 1) * 16 + (t & 1) * 8);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) t16[grp][t >> 1][(t & 1) * 8 + e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
  }
  __syncthreads();
  if (live) {
    const int CB = C >> 4, KB = Kout >> 4;
    const int kb = bi % KB;
    const int rc = bi / KB;  // rs * CB + cb
    const int cb = rc % CB;
    const int rs = rc / CB;
    const int k = kb * 16 + (t >> 1);
    const int c0 = cb * 16 + (t & 1) * 8;
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (uint32_t)t16[grp][(t & 1) * 8 + 2 * e][t >> 1] | ((uint32_t)t16[grp][(t & 1) * 8 + 2 * e + 1][t >> 1] << 16);
    *reinterpret_cast<uint4*>(krsc + (long long)k * RS * C + (long long)rs * C + c0) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Workspace of the blocked-layout convolution: the stream-K part (if any)
// first, so that its counters sit where the caller's zero fill put them,
// then the weights in K-contiguous order, rewritten by every call.
inline size_t nhwcnc_ws_offset(size_t sk_bytes) { return (sk_bytes + 255) / 256 * 256; }
inline size_t nhwcnc_weight_bytes(const igc::Params& p) { return (size_t)p.N * (size_t)p.K * 2; }

// Workspace bytes of the plan for an M x N x K problem of this kind on the
// current device, with the aligned operand path (the one that may split).
int query_workspace(int kind, int M, int N, int K, size_t* bytes) {
  if (!bytes) return fail(IGC_EINVAL, "bytes is NULL");
  *bytes = 0;
  if (M == 0 || N == 0) return IGC_OK;
  int dev;
  if (int s = check_device(&dev)) return s;
  *bytes = make_plan(kind, M, N, K, true, device_cus(dev), true).ws_bytes;
  return IGC_OK;
}

}  // namespace igc_host

using namespace igc_host;

// The uniform-tap conv loaders address x through a 2^31-byte buffer whose
// base is x moved back by the padding's offset ((ph*W + pw) pixels), with
// the K tile's tap and channel position as a scalar offset: x plus the
// padding's offset, and the largest scalar offset (a filter row past the
// last, for the tiles prefetched beyond K), must both stay below 2^31 bytes.
static bool uniform_taps_fit(const igc::Params& p, long long x_bytes, int eb, bool blocked) {
  const long long sc = (long long)eb * (blocked ? 16 : 1);
  const long long pad_off = ((long long)p.ph * p.W + p.pw) * p.C * sc;
  const long long max_off = ((long long)(p.R + 1) * p.W + p.S) * p.C * sc;
  return x_bytes + pad_off < (1LL << 31) && max_off < (1LL << 31);
}

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

int igc_set_tuning(int force_variant, int streamk_mode) {
  g_last_error[0] = 0;
  if (force_variant < V_AUTO || force_variant >= V_COUNT)
    return fail(IGC_EINVAL, "force_variant=%d outside [-1, %d]", force_variant, V_COUNT - 1);
  if (streamk_mode < 0 || streamk_mode > 2) return fail(IGC_EINVAL, "streamk_mode=%d outside [0, 2]", streamk_mode);
  g_force_variant.store(force_variant, std::memory_order_relaxed);
  g_streamk_mode.store(streamk_mode, std::memory_order_relaxed);
  return IGC_OK;
}

int gemm_f16f32_workspace_size(int M, int N, int K, size_t* bytes) {
  g_last_error[0] = 0;
  if (M < 0 || N < 0 || K < 0) return fail(IGC_EINVAL, "negative size M=%d N=%d K=%d", M, N, K);
  return query_workspace(igc::KIND_F16_GEMM, M, N, K, bytes);
}

int gemm_f16f32(int M, int N, int K, const void* A, int lda, const void* B, int ldb, float* C,
                int ldc, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (M < 0 || N < 0 || K < 0) return fail(IGC_EINVAL, "negative size M=%d N=%d K=%d", M, N, K);
  if (M == 0 || N == 0) return IGC_OK;
  if (!C) return fail(IGC_EINVAL, "C is NULL");
  if (ldc < N) return fail(IGC_EINVAL, "ldc=%d < N=%d", ldc, N);
  if (K > 0) {
    if (!A || !B) return fail(IGC_EINVAL, "A or B is NULL");
    if (lda < K || ldb < K) return fail(IGC_EINVAL, "lda=%d / ldb=%d < K=%d", lda, ldb, K);
  }
  igc::Params p = zero_params();
  p.M = M; p.N = N; p.K = K;
  p.A = static_cast<const uint8_t*>(A); p.lda = lda;
  p.B = static_cast<const uint8_t*>(B); p.ldb = ldb;
  p.Cf = C; p.ldcf = ldc;
  p.vec_c = aligned16(C) && ldc % 4 == 0;  // 16-byte stores of 4 consecutive columns
  // Buffer descriptors of the fast path cover one tile of rows and must stay below 2^31 bytes.
  const bool fast = aligned16(A) && aligned16(B) && lda % 8 == 0 && ldb % 8 == 0 && K % 8 == 0 &&
                    256LL * lda * 2 < (1LL << 31) && 256LL * ldb * 2 < (1LL << 31);
  return plan_and_launch<igc::KIND_F16_GEMM, 0>(p, fast, workspace, ws_bytes, static_cast<hipStream_t>(stream));
}

int gemm_f16f32_noalloc(int M, int N, int K, const void* A, int lda, const void* B, int ldb, float* C,
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
  p.vec_c = aligned16(C) && ldc % 4 == 0;
  const bool fast = aligned16(A) && aligned16(B) && lda % 8 == 0 && ldb % 8 == 0 && K % 8 == 0 &&
                    256LL * lda * 2 < (1LL << 31) && 256LL * ldb * 2 < (1LL << 31);
  const Plan pl = make_plan(igc::KIND_F16_GEMM, M, N, K, fast, device_cus(dev), true);
  void* ws = nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (pl.ws_bytes) {
    if (pl.ws_bytes > kNoallocScratchBytes)
      return fail(IGC_EUNSUPPORTED, "this call needs %zu bytes of stream-K workspace; the static scratch holds %zu",
                  pl.ws_bytes, kNoallocScratchBytes);
    if (int s = scratch_address(dev, &ws)) return s;
    // the arrival counters must start at zero whatever an earlier call left
    const int words = (int)(pl.cnt_bytes / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st,
                       static_cast<uint32_t*>(ws), words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(IGC_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  }
  apply_plan(p, pl, ws);
  if (pl.sk_wgs == 0) return launch<igc::KIND_F16_GEMM, igc::NO_SPLIT>(p, pl, fast, st);
  return launch<igc::KIND_F16_GEMM, 0>(p, pl, fast, st);
}

int gemm_u8i8_zp_workspace_size(int M, int N, int K, size_t* bytes) {
  g_last_error[0] = 0;
  if (M < 0 || N < 0 || K < 0) return fail(IGC_EINVAL, "negative size M=%d N=%d K=%d", M, N, K);
  return query_workspace(igc::KIND_U8I8_GEMM, M, N, K, bytes);
}

int u8i8_colsum(int N, int K, const int8_t* B, int ldb, int32_t* colsum, void* stream) {
  g_last_error[0] = 0;
  if (N < 0 || K < 0) return fail(IGC_EINVAL, "negative size N=%d K=%d", N, K);
  if (ldb < K) return fail(IGC_EINVAL, "ldb=%d < K=%d", ldb, K);
  if (K > 33025) return fail(IGC_EOVERFLOW, "K=%d > 33025", K);
  if (N == 0) return IGC_OK;
  if (!colsum || (!B && K > 0)) return fail(IGC_EINVAL, "B or colsum is NULL");
  int dev;
  if (int s = check_device(&dev)) return s;
  hipLaunchKernelGGL(i8_colsum_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     B, ldb, N, K, colsum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(IGC_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return IGC_OK;
}

int gemm_u8i8_zp(int M, int N, int K, const uint8_t* A, int lda, int zA, const int8_t* B, int ldb,
                 int zB, const igc_u8i8_epilogue* ep, void* stream) {
  g_last_error[0] = 0;
  if (M < 0 || N < 0 || K < 0) return fail(IGC_EINVAL, "negative size M=%d N=%d K=%d", M, N, K);
  if (zA < 0 || zA > 255) return fail(IGC_EINVAL, "zA=%d outside [0, 255]", zA);
  if (zB < -128 || zB > 127) return fail(IGC_EINVAL, "zB=%d outside [-128, 127]", zB);
  if (int s = check_epilogue(ep, N, K)) return s;
  if (M == 0 || N == 0) return IGC_OK;
  if (K > 0) {
    if (!A || !B) return fail(IGC_EINVAL, "A or B is NULL");
    if (lda < K || ldb < K) return fail(IGC_EINVAL, "lda=%d / ldb=%d < K=%d", lda, ldb, K);
  }
  igc::Params p = zero_params();
  p.M = M; p.N = N; p.K = K;
  p.A = A; p.lda = lda;
  p.B = reinterpret_cast<const uint8_t*>(B); p.ldb = ldb;
  p.zAp = zA - 128; p.zB = zB;
  epilogue_params(p, ep);
  const bool fast = aligned16(A) && aligned16(B) && lda % 16 == 0 && ldb % 16 == 0 &&
                    K % 16 == 0 && 256LL * lda < (1LL << 31) && 256LL * ldb < (1LL << 31);
  return launch_u8i8<igc::KIND_U8I8_GEMM>(p, fast, ep->workspace, ep->ws_bytes, static_cast<hipStream_t>(stream));
}

int conv2d_u8i8_zp_workspace_size(int Nb, int H, int W, int C, int Kout, int R, int S, int stride_h,
                                  int stride_w, int pad_h, int pad_w, size_t* bytes) {
  g_last_error[0] = 0;
  igc::Params p = zero_params();
  long long nx = 0;
  if (int st = conv_params(Nb, H, W, C, Kout, R, S, stride_h, stride_w, pad_h, pad_w, p, &nx)) return st;
  return query_workspace(igc::KIND_U8I8_CONV, p.M, p.N, p.K, bytes);
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
  if (int s = check_epilogue(ep, Kout, p.K)) return s;
  p.A = x; p.lda = 0;
  p.B = reinterpret_cast<const uint8_t*>(w); p.ldb = p.K;
  p.zAp = zA - 128; p.zB = zB;
  epilogue_params(p, ep);
  // whole 128-channel K tiles within one tap: the uniform-tap loader
  const bool fast = aligned16(x) && aligned16(w) && C % 128 == 0 && (long long)R * S <= 31 &&
                    nx < (1LL << 31) && 256LL * p.K < (1LL << 31) && uniform_taps_fit(p, nx, 1, false);
  return launch_u8i8<igc::KIND_U8I8_CONV>(p, fast, ep->workspace, ep->ws_bytes, static_cast<hipStream_t>(stream));
}

int conv2d_implicit_gemm_workspace_size(int Nb, int H, int W, int C, int Kout, int R, int S, int stride_h,
                                        int stride_w, int pad_h, int pad_w, size_t* bytes) {
  g_last_error[0] = 0;
  igc::Params p = zero_params();
  long long nx = 0;
  if (int st = conv_params(Nb, H, W, C, Kout, R, S, stride_h, stride_w, pad_h, pad_w, p, &nx)) return st;
  return query_workspace(igc::KIND_F16_CONV, p.M, p.N, p.K, bytes);
}

int conv2d_implicit_gemm(int Nb, int H, int W, int C, int Kout, int R, int S, int stride_h,
                         int stride_w, int pad_h, int pad_w, const void* x, const void* w, float* y,
                         void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  igc::Params p = zero_params();
  long long nx = 0;
  if (int st = conv_params(Nb, H, W, C, Kout, R, S, stride_h, stride_w, pad_h, pad_w, p, &nx)) return st;
  if (!x || !w || !y) return fail(IGC_EINVAL, "x, w or y is NULL");
  p.A = static_cast<const uint8_t*>(x); p.lda = 0;
  p.B = static_cast<const uint8_t*>(w); p.ldb = p.K;
  p.Cf = y; p.ldcf = Kout;
  p.vec_c = aligned16(y) && Kout % 4 == 0;
  const bool fast = aligned16(x) && aligned16(w) && C % 8 == 0 && nx * 2 < (1LL << 31) &&
                    256LL * p.K * 2 < (1LL << 31);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // whole 64-channel K tiles within one tap: the uniform-tap loader
  if (fast && C % 64 == 0 && (long long)R * S <= 31 && uniform_taps_fit(p, nx * 2, 2, false))
    return plan_and_launch<igc::KIND_F16_CONV_C64, 0>(p, true, workspace, ws_bytes, st);
  return plan_and_launch<igc::KIND_F16_CONV, 0>(p, fast, workspace, ws_bytes, st);
}

int conv2d_implicit_gemm_nhwcnc_workspace_size(int Nb, int H, int W, int C, int Kout, int R, int S,
                                               int stride_h, int stride_w, int pad_h, int pad_w, size_t* bytes) {
  g_last_error[0] = 0;
  igc::Params p = zero_params();
  long long nx = 0;
  if (int st = conv_params(Nb, H, W, C, Kout, R, S, stride_h, stride_w, pad_h, pad_w, p, &nx)) return st;
  if (Nb % 16 || C % 16 || Kout % 16) return fail(IGC_EINVAL, "Nb, C and Kout must be multiples of 16");
  if (!bytes) return fail(IGC_EINVAL, "bytes is NULL");
  size_t sk = 0;
  if (int s = query_workspace(igc::KIND_F16_CONV, p.M, p.N, p.K, &sk)) return s;
  *bytes = nhwcnc_ws_offset(sk) + nhwcnc_weight_bytes(p);
  return IGC_OK;
}

int conv2d_implicit_gemm_nhwcnc(int Nb, int H, int W, int C, int Kout, int R, int S, int stride_h,
                                int stride_w, int pad_h, int pad_w, const void* x, const void* w, float* y,
                                void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  igc::Params p = zero_params();
  long long nx = 0;
  if (int st = conv_params(Nb, H, W, C, Kout, R, S, stride_h, stride_w, pad_h, pad_w, p, &nx)) return st;
  if (Nb % 16 || C % 16 || Kout % 16) return fail(IGC_EINVAL, "Nb, C and Kout must be multiples of 16");
  if (!x || !w || !y) return fail(IGC_EINVAL, "x, w or y is NULL");
  if (!workspace) return fail(IGC_EINVAL, "the blocked layout needs a workspace (conv2d_implicit_gemm_nhwcnc_workspace_size)");
  if (!aligned16(w) || !aligned16(workspace)) return fail(IGC_EINVAL, "w and the workspace must be 16-byte aligned");
  int dev;
  if (int s = check_device(&dev)) return s;
  p.A = static_cast<const uint8_t*>(x); p.lda = 0;
  p.ldb = p.K;
  p.Cf = y; p.ldcf = Kout;
  p.blk = 1;
  p.vec_c = aligned16(y);
  const bool fast = aligned16(x) && nx * 2 < (1LL << 31) && 256LL * p.K * 2 < (1LL << 31);
  const int kind = (fast && C % 64 == 0 && (long long)R * S <= 31 && uniform_taps_fit(p, nx * 2, 2, true))
                       ? igc::KIND_F16_CONV_C64 : igc::KIND_F16_CONV;
  const Plan pl = make_plan(kind, p.M, p.N, p.K, fast, device_cus(dev), true);
  const size_t woff = nhwcnc_ws_offset(pl.ws_bytes), wbytes = nhwcnc_weight_bytes(p);
  if (ws_bytes < woff + wbytes)
    return fail(IGC_EINVAL, "workspace of %zu bytes < the %zu bytes this call needs", ws_bytes, woff + wbytes);
  uint8_t* const wk = static_cast<uint8_t*>(workspace) + woff;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the weights in the GEMM's K-contiguous order, then the GEMM on them
  const int nblocks = R * S * (C / 16) * (Kout / 16);
  hipLaunchKernelGGL(nhwcnc_weights_kernel, dim3((unsigned)((nblocks + 7) / 8)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(w), reinterpret_cast<uint16_t*>(wk), R * S, C, Kout, nblocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(IGC_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  p.B = wk;
  apply_plan(p, pl, workspace);
  constexpr int WHOLE = igc::BLK_OUT | igc::NO_SPLIT;
  if (kind == igc::KIND_F16_CONV_C64)
    return pl.sk_wgs == 0 ? launch<igc::KIND_F16_CONV_C64, WHOLE>(p, pl, true, st)
                          : launch<igc::KIND_F16_CONV_C64, igc::BLK_OUT>(p, pl, true, st);
  return pl.sk_wgs == 0 ? launch<igc::KIND_F16_CONV, WHOLE>(p, pl, fast, st)
                        : launch<igc::KIND_F16_CONV, igc::BLK_OUT>(p, pl, fast, st);
}

}  // extern "C"
