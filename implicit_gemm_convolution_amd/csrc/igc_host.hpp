// igc_host.hpp -- host side of a launch, shared by the C ABI (igc.hip) and
// the launch units (igc_launch.hip): tile-variant choice, the stream-K split
// and the kernel launch on the caller's stream.  launch<KIND, SUMS> is
// instantiated in igc_launch.hip, once per kernel kind, so that the kinds
// compile in parallel; igc.hip only calls it.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <cstdlib>

#include "../../include/igc.h"
#include "igc_kernels.hpp"

namespace igc_host {

constexpr int kMaxDevices = 64;

// Defined in igc.hip: the thread's error detail, the per-device compute-unit
// count and the per-(device, stream) stream-K workspace.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int device_cus(int dev);
int sk_workspace(int dev, hipStream_t stream, size_t ws_bytes, size_t cnt_n, float** ws, int** cnt);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Tile variants.  The large tile keeps the most MFMA work per LDS byte; the
// smaller ones exist so that small problems still spread over the 256 CUs
// (the multi-kernel-per-shape dispatch of [GEMM-TVM] §4.3, done at run time).
enum Variant {
  V_AUTO = -1,
  V_256x256 = 0,
  V_128x128 = 1,
  V_64x64 = 2,
  V_256x128 = 3,
  V_224x256 = 4,
  V_BYPASS = 5,  // fp16 GEMM, aligned operands: 32x32 tiles, one wave each, no LDS
  V_COUNT = 6
};

inline int forced_variant() {
  const char* s = std::getenv("IGC_FORCE_VARIANT");
  if (!s || !*s) return V_AUTO;
  int v = std::atoi(s);
  return (v >= 0 && v < V_COUNT) ? v : V_AUTO;
}

inline long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

// Large problems run on one workgroup per compute unit, in rounds of `cus`
// tiles, so their time goes as (rounds) x (tile area).  224 x 256 tiles are
// taken over 256 x 256 when that cost is lower: e.g. M = 50176, N = 512
// (the 256 x 14 x 14 conv) needs 392 tiles of 256 rows, two rounds with the
// second 53% full, but 448 tiles of 224 rows, two rounds of 7/8 the work.
inline int choose_variant(int M, int N, int cus) {
  int f = forced_variant();
  if (f != V_AUTO) return f;
  const long long t256 = ceil_div(M, 256) * ceil_div(N, 256);
  if (t256 >= 192) {
    const long long t224 = ceil_div(M, 224) * ceil_div(N, 256);
    const long long c256 = ceil_div(t256, cus) * 256, c224 = ceil_div(t224, cus) * 224;
    return c224 < c256 ? V_224x256 : V_256x256;
  }
  if (ceil_div(M, 128) * ceil_div(N, 128) >= 192) return V_128x128;
  return V_64x64;
}

// Stream-K (shared tiles): when the 256x256 tiles do not fill the last
// round of compute units, the whole rounds run as whole tiles and the rest
// of the tiles' K-tile iterations are split evenly over up to one workgroup
// per compute unit (at least 4 iterations each).  fp16 GEMM and conv only.
// It pays only when the idle part of the last round is worth more than the
// cost of publishing and summing the partial tiles, measured on MI355X at
// about 26 K-tile iterations (4096^2 conv tiles: 392 tiles on 256 CUs, 36
// iterations each, ran 12% slower split).  IGC_STREAMK=0 never splits,
// IGC_STREAMK=2 splits whenever the last round is partial (tests).
inline int streamk_mode() {
  const char* s = std::getenv("IGC_STREAMK");
  if (s && s[0] == '0') return 0;
  if (s && s[0] == '2') return 2;
  return 1;
}
constexpr long long kStreamKFixupIters = 26;

template <int KIND, int BM, int BN, int WM, int WN, bool FAST, int SUMS, int DEPTH = 2>
int launch_one(igc::Params p, hipStream_t stream) {
  p.tiles_m = (int)ceil_div(p.M, BM);
  p.tiles_n = (int)ceil_div(p.N, BN);
  long long grid = (long long)p.tiles_m * p.tiles_n;
  if (grid > 0x7fffffffLL) return fail(IGC_EUNSUPPORTED, "too many tiles (%lld)", grid);
  p.dp_tiles = (int)grid;
  {
    int d = 0;
    const long long cus = (hipGetDevice(&d) == hipSuccess && d >= 0 && d < kMaxDevices) ? device_cus(d) : 256;
    p.xcd_regroup = grid > cus;  // several rounds of workgroups per compute unit
  }
  p.sk_wgs = 0;
  p.sk_iters = 0;
  if constexpr (BM == 256 && BN == 256 && FAST && SUMS == 0 && KIND != igc::KIND_U8I8_GEMM && KIND != igc::KIND_U8I8_CONV) {
    int dev = 0;
    const int mode = streamk_mode();
    if (mode && hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
      const long long cus = device_cus(dev);
      const long long nk = ceil_div((long long)p.K * 2, igc::KT_BYTES);
      // iterations the last round leaves idle, per compute unit
      const long long idle = (cus - grid % cus) * nk / cus;
      if (grid > cus && grid % cus != 0 && nk >= 4 && (mode == 2 || idle > kStreamKFixupIters)) {
        const long long dp = grid / cus * cus;
        const long long iters = (grid - dp) * nk;
        const long long wgs = std::min(cus, std::max(1LL, iters / 4));
        float* ws = nullptr;
        int* cnt = nullptr;
        if (int st = sk_workspace(dev, stream, (size_t)(2 * wgs * BM * BN * 4), (size_t)(grid - dp), &ws, &cnt))
          return st;
        p.dp_tiles = (int)dp;
        p.sk_wgs = (int)wgs;
        p.sk_iters = iters;
        p.ws = ws;
        p.cnt = cnt;
        grid = dp + wgs;
      }
    }
  }
  hipLaunchKernelGGL((igc::gemm_kernel<KIND, BM, BN, WM, WN, FAST, SUMS, DEPTH>), dim3((unsigned)grid),
                     dim3(64 * WM * WN), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(IGC_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return IGC_OK;
}

template <int KIND, bool FAST, int SUMS>
int launch_variant(int v, const igc::Params& p, hipStream_t stream) {
  switch (v) {
    case V_224x256:
      if constexpr (FAST) return launch_one<KIND, 224, 256, 2, 2, FAST, SUMS>(p, stream);
      [[fallthrough]];
    case V_256x256:
      if constexpr (FAST) return launch_one<KIND, 256, 256, 2, 2, FAST, SUMS>(p, stream);
      [[fallthrough]];
    case V_256x128:
      if constexpr (FAST) return launch_one<KIND, 256, 128, 2, 2, FAST, SUMS>(p, stream);
      [[fallthrough]];
    case V_128x128: return launch_one<KIND, 128, 128, 2, 2, FAST, SUMS>(p, stream);
    default: return launch_one<KIND, 64, 64, 2, 2, FAST, SUMS>(p, stream);
  }
}

inline int launch_bypass(igc::Params p, hipStream_t stream) {
  p.tiles_m = (int)ceil_div(p.M, 32);
  p.tiles_n = (int)ceil_div(p.N, 32);
  const long long grid = (long long)p.tiles_m * p.tiles_n;
  if (grid > 0x7fffffffLL) return fail(IGC_EUNSUPPORTED, "too many tiles (%lld)", grid);
  hipLaunchKernelGGL((igc::gemm_f16_bypass_kernel<8>), dim3((unsigned)grid), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(IGC_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return IGC_OK;
}

template <int KIND, int SUMS>
int launch(const igc::Params& p, bool fast, hipStream_t stream, int dev) {
  if constexpr (KIND == igc::KIND_F16_GEMM) {
    // The LDS-bypass kernel wins only where the whole problem is one short
    // round: measured on MI355X, 256^3 3.6 us against 4.1 (64x64 tiles), 512^3
    // 4.8 against 4.9, but 1024^3 16.4 against 6.6 and 256x256x4096 23.5
    // against 14.2 (a single wave then walks a long K loop alone).
    const int fv = forced_variant();
    const bool small = ceil_div(p.M, 32) * ceil_div(p.N, 32) <= device_cus(dev) && p.K <= 512;
    if (fast && (fv == V_BYPASS || (fv == V_AUTO && small))) return launch_bypass(p, stream);
  }
  const int cus = device_cus(dev);
  int v = choose_variant(p.M, p.N, cus);
  if (v == V_BYPASS) v = V_64x64;  // (forced, for a kind or shape without the bypass kernel)
  // The element-wise (unaligned) loaders need more registers; they stop at 128x128.
  if (!fast && (v == V_256x256 || v == V_256x128 || v == V_224x256)) v = V_128x128;
  if constexpr (KIND == igc::KIND_F16_CONV_C64) {
    return launch_variant<KIND, true, SUMS>(v, p, stream);  // dispatched only with aligned operands
  } else {
    return fast ? launch_variant<KIND, true, SUMS>(v, p, stream)
                : launch_variant<KIND, false, SUMS>(v, p, stream);
  }
}

// The (kind, zero-point sums) pairs the C ABI launches: the fp16 kinds
// without sums, the u8 x i8 kinds with each subset of SUM_ROWS | SUM_COLS.
#define IGC_LAUNCH_KINDS(X)         \
  X(0, igc::KIND_F16_GEMM, 0)       \
  X(1, igc::KIND_F16_CONV, 0)       \
  X(2, igc::KIND_F16_CONV_C64, 0)   \
  X(3, igc::KIND_U8I8_GEMM, 0)      \
  X(4, igc::KIND_U8I8_GEMM, 1)      \
  X(5, igc::KIND_U8I8_GEMM, 2)      \
  X(6, igc::KIND_U8I8_GEMM, 3)      \
  X(7, igc::KIND_U8I8_CONV, 0)      \
  X(8, igc::KIND_U8I8_CONV, 1)      \
  X(9, igc::KIND_U8I8_CONV, 2)      \
  X(10, igc::KIND_U8I8_CONV, 3)

#define IGC_EXTERN_LAUNCH(n, K, S) \
  extern template int launch<K, S>(const igc::Params&, bool, hipStream_t, int);
IGC_LAUNCH_KINDS(IGC_EXTERN_LAUNCH)
#undef IGC_EXTERN_LAUNCH

}  // namespace igc_host
