// igc_host.hpp -- host side of a launch, shared by the C ABI (igc.hip) and
// the launch units (igc_launch.hip): the launch plan (tile variant, stream-K
// split, workspace bytes) and the kernel launch on the caller's stream.
// launch<KIND, SUMS> is instantiated in igc_launch.hip, once per kernel kind,
// so that the kinds compile in parallel; igc.hip plans and calls it.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstddef>
#include <cstdint>

#include "../../include/igc.h"
#include "igc_kernels.hpp"

namespace igc_host {

constexpr int kMaxDevices = 64;

// Defined in igc.hip: the thread's error detail.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

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
  V_BYPASS = 5,    // fp16 GEMM, aligned operands: 32x32 tiles, one wave each, no LDS
  V_BYPASS16 = 6,  // the same with 16x16 tiles (four times the waves)
  V_COUNT = 7
};

// Process-wide tuning overrides set by igc_set_tuning (tests and sweeps):
// a forced variant (V_AUTO: the shape decides) and the stream-K mode
// (0 never split, 1 split where it pays, 2 split whenever a round is partial).
extern std::atomic<int> g_force_variant;
extern std::atomic<int> g_streamk_mode;

inline long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

inline void variant_tile(int v, int& bm, int& bn) {
  switch (v) {
    case V_256x256: bm = 256; bn = 256; return;
    case V_224x256: bm = 224; bn = 256; return;
    case V_256x128: bm = 256; bn = 128; return;
    case V_128x128: bm = 128; bn = 128; return;
    case V_BYPASS: bm = 32; bn = 32; return;
    case V_BYPASS16: bm = 16; bn = 16; return;
    default: bm = 64; bn = 64; return;
  }
}

// Large problems run on one workgroup per compute unit, in rounds of `cus`
// tiles, so their time goes as (rounds) x (tile area).  224 x 256 tiles are
// taken over 256 x 256 when that cost is lower: e.g. M = 50176, N = 512
// (the 256 x 14 x 14 conv) needs 392 tiles of 256 rows, two rounds with the
// second 53% full, but 448 tiles of 224 rows, two rounds of 7/8 the work.
inline int choose_variant(int M, int N, int cus) {
  const long long t256 = ceil_div(M, 256) * ceil_div(N, 256);
  if (t256 >= 192) {
    const long long t224 = ceil_div(M, 224) * ceil_div(N, 256);
    const long long c256 = ceil_div(t256, cus) * 256, c224 = ceil_div(t224, cus) * 224;
    return c224 < c256 ? V_224x256 : V_256x256;
  }
  if (ceil_div(M, 128) * ceil_div(N, 128) >= 192) return V_128x128;
  return V_64x64;
}

// Stream-K (shared tiles): when the tiles do not fill the last round of
// compute units (or a grid smaller than one round leaves most of them idle),
// the whole rounds run as whole tiles and the rest of the tiles' K-tile
// iterations are split evenly over up to one workgroup per compute unit (at
// least 4 iterations each).  Compiled for every fp16 tile and for the u8 x i8
// tiles of at most 128 rows.  It pays only when the idle part of the last
// round is worth more than the cost of publishing and summing the partial
// tiles, measured on MI355X at about 26 K-tile iterations per compute unit
// (4096^2 conv tiles: 392 tiles of 256x256 on 256 CUs, 36 iterations each,
// ran 12% slower split).
constexpr long long kStreamKFixupIters = 26;

inline bool streamk_compiled(bool int8, int v) {
  return int8 ? (v == V_128x128 || v == V_64x64) : (v != V_BYPASS && v != V_BYPASS16);
}

// Everything a launch needs to know before it enqueues anything; a pure
// function of the problem, the device's compute-unit count and the tuning
// overrides, so the workspace-size queries and the launches agree.
struct Plan {
  int variant = V_64x64;
  int bm = 64, bn = 64;
  int tiles_m = 0, tiles_n = 0;
  long long grid = 0;     // workgroups launched
  int dp_tiles = 0;       // whole-tile workgroups
  int sk_wgs = 0;         // stream-K workgroups after them
  long long sk_iters = 0; // K-tile iterations they share
  int xcd_regroup = 0;
  size_t cnt_bytes = 0;   // arrival counters at the start of the workspace (256-byte multiple)
  size_t ws_bytes = 0;    // total workspace the launch uses (0: none)
};

// kind: igc::Kind; fast: the aligned (direct-to-LDS) loaders apply; ws_ok:
// a workspace may be used (the caller passed one).  EB = bytes per element.
inline Plan make_plan(int kind, int M, int N, int K, bool fast, int cus, bool ws_ok) {
  Plan pl;
  const int fv = g_force_variant.load(std::memory_order_relaxed);
  const bool int8 = kind == igc::KIND_U8I8_GEMM || kind == igc::KIND_U8I8_CONV;
  int v;
  if (kind == igc::KIND_F16_GEMM && fast &&
      (fv == V_BYPASS || fv == V_BYPASS16 ||
       (fv == V_AUTO && ceil_div(M, 16) * ceil_div(N, 16) <= cus && K <= 512))) {
    // The LDS-bypass kernel wins only where its 16x16 tiles, one wave each,
    // fit one round of compute units and K is short: measured on MI355X
    // (graph replays, per launch) 256x256x512 2.82 us against 3.69 us on
    // 64x64 LDS tiles.  Where they do not fit, the 64x64 whole-tile kernel
    // matches or beats both bypass forms: 512^3 3.77 us against 4.52 (32x32
    // bypass) and 5.25 (16x16, two rounds), 384^3 3.46 against 4.15 and 4.00,
    // 512x256x512 3.72 against 4.43 and 3.63.  The 32x32 form is taken only
    // when forced.
    v = fv == V_AUTO ? V_BYPASS16 : fv;
  } else {
    v = fv == V_AUTO ? choose_variant(M, N, cus) : fv;
    if (v == V_BYPASS || v == V_BYPASS16) v = V_64x64;  // (forced, for a kind or shape without the bypass kernel)
    // The element-wise (unaligned) loaders need more registers; they stop at 128x128.
    if (!fast && (v == V_256x256 || v == V_256x128 || v == V_224x256)) v = V_128x128;
    // The uniform-tap u8 convolution keeps two registers per fragment row (its
    // rows' tap masks and conversion constants) beside the accumulators: at
    // 256x256 the K loop would spill, so its 256-row tile is the 224-row one.
    if (kind == igc::KIND_U8I8_CONV && fast && v == V_256x256) v = V_224x256;
  }
  pl.variant = v;
  variant_tile(v, pl.bm, pl.bn);
  pl.tiles_m = (int)ceil_div(M, pl.bm);
  pl.tiles_n = (int)ceil_div(N, pl.bn);
  const long long grid = (long long)pl.tiles_m * pl.tiles_n;
  pl.grid = grid;
  pl.dp_tiles = (int)std::min(grid, 0x7fffffffLL);
  pl.xcd_regroup = grid > cus;  // several rounds of workgroups per compute unit
  const int mode = g_streamk_mode.load(std::memory_order_relaxed);
  if (streamk_compiled(int8, v) && fast && ws_ok && mode != 0) {
    const long long nk = ceil_div((long long)K * (int8 ? 1 : 2), igc::KT_BYTES);
    // iterations the last round leaves idle, per compute unit
    const long long idle = (cus - grid % cus) * nk / cus;
    if (grid % cus != 0 && nk >= 4 && (mode == 2 || idle > kStreamKFixupIters)) {
      const long long dp = grid / cus * cus;
      const long long iters = (grid - dp) * nk;
      const long long wgs = std::min((long long)cus, std::max(1LL, iters / 4));
      pl.dp_tiles = (int)dp;
      pl.sk_wgs = (int)wgs;
      pl.sk_iters = iters;
      pl.grid = dp + wgs;
      pl.cnt_bytes = (size_t)ceil_div((grid - dp) * 4, 256) * 256;
      pl.ws_bytes = pl.cnt_bytes + (size_t)(2 * wgs) * (size_t)(pl.bm * pl.bn * 4);
    }
  }
  return pl;
}

// The reciprocal of d for igc::FastDiv (1 <= d < 2^31).
inline igc::FastDiv make_fastdiv(long long d) {
  igc::FastDiv f;
  f.d = (uint32_t)d;
  f.m = d <= 1 ? 0u : (uint32_t)((1ULL << 32) / (unsigned long long)d + 1);
  return f;
}

// Fills the split and workspace fields of p from the plan; ws is the
// caller's workspace (used only when the plan needs one).
inline void apply_plan(igc::Params& p, const Plan& pl, void* ws) {
  p.tiles_m = pl.tiles_m;
  p.tiles_n = pl.tiles_n;
  p.fd_group = make_fastdiv(8LL * pl.tiles_n);
  p.fd_glast = make_fastdiv(pl.tiles_m % 8 ? pl.tiles_m % 8 : 8);
  p.dp_tiles = pl.dp_tiles;
  p.xcd_regroup = pl.xcd_regroup;
  p.sk_wgs = pl.sk_wgs;
  p.sk_iters = pl.sk_iters;
  if (pl.ws_bytes) {
    p.cnt = static_cast<int*>(ws);
    p.ws = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + pl.cnt_bytes);
  } else {
    p.cnt = nullptr;
    p.ws = nullptr;
  }
}

template <int KIND, int BM, int BN, int WM, int WN, bool FAST, int SUMS, int DEPTH = 2>
int launch_one(const igc::Params& p, const Plan& pl, hipStream_t stream) {
  if (pl.grid > 0x7fffffffLL) return fail(IGC_EUNSUPPORTED, "too many tiles (%lld)", pl.grid);
  hipLaunchKernelGGL((igc::gemm_kernel<KIND, BM, BN, WM, WN, FAST, SUMS, DEPTH>), dim3((unsigned)pl.grid),
                     dim3(64 * WM * WN), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(IGC_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return IGC_OK;
}

template <int KIND, bool FAST, int SUMS>
int launch_variant(const igc::Params& p, const Plan& pl, hipStream_t stream) {
  constexpr bool INT8 = KIND == igc::KIND_U8I8_GEMM || KIND == igc::KIND_U8I8_CONV;
  if constexpr (INT8 && (SUMS & igc::NO_SPLIT) != 0) {
    // whole tiles of the integer kinds without the split code: the aligned
    // tiles that have it (the wider ones never split)
    if constexpr (FAST) {
      if (pl.variant == V_128x128) return launch_one<KIND, 128, 128, 2, 2, FAST, SUMS>(p, pl, stream);
      if (pl.variant == V_64x64) return launch_one<KIND, 64, 64, 2, 2, FAST, SUMS>(p, pl, stream);
    }
    return fail(IGC_EUNSUPPORTED, "internal: variant %d has no whole-tile integer kernel", pl.variant);
  } else if constexpr ((SUMS & igc::REQ_TILES) != 0) {
    // whole requantize-only tiles: compiled for the 256-column integer tiles
    if constexpr (FAST) {
      if (pl.variant == V_224x256) return launch_one<KIND, 224, 256, 2, 2, FAST, SUMS>(p, pl, stream);
      if constexpr (KIND != igc::KIND_U8I8_CONV)
        if (pl.variant == V_256x256) return launch_one<KIND, 256, 256, 2, 2, FAST, SUMS>(p, pl, stream);
    }
    return fail(IGC_EUNSUPPORTED, "internal: variant %d has no whole-tile requantize-only kernel", pl.variant);
  } else {
    switch (pl.variant) {
      case V_224x256:
        if constexpr (FAST) return launch_one<KIND, 224, 256, 2, 2, FAST, SUMS>(p, pl, stream);
        break;
      case V_256x256:  // (not for the uniform-tap u8 convolution, see make_plan)
        if constexpr (FAST && KIND != igc::KIND_U8I8_CONV) return launch_one<KIND, 256, 256, 2, 2, FAST, SUMS>(p, pl, stream);
        break;
      case V_256x128:
        if constexpr (FAST) return launch_one<KIND, 256, 128, 2, 2, FAST, SUMS>(p, pl, stream);
        break;
      case V_128x128: return launch_one<KIND, 128, 128, 2, 2, FAST, SUMS>(p, pl, stream);
      case V_64x64: return launch_one<KIND, 64, 64, 2, 2, FAST, SUMS>(p, pl, stream);
      default: break;
    }
    return fail(IGC_EUNSUPPORTED, "internal: variant %d not compiled for this operand form", pl.variant);
  }
}

inline int launch_bypass(const igc::Params& p, const Plan& pl, hipStream_t stream) {
  if (pl.grid > 0x7fffffffLL) return fail(IGC_EUNSUPPORTED, "too many tiles (%lld)", pl.grid);
  if (pl.variant == V_BYPASS16)
    hipLaunchKernelGGL((igc::gemm_f16_bypass_kernel<8, 16>), dim3((unsigned)pl.grid), dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL((igc::gemm_f16_bypass_kernel<8, 32>), dim3((unsigned)pl.grid), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(IGC_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
  return IGC_OK;
}

// p carries the problem, its outputs and the plan's split (apply_plan).
template <int KIND, int SUMS>
int launch(const igc::Params& p, const Plan& pl, bool fast, hipStream_t stream) {
  if constexpr (KIND == igc::KIND_F16_GEMM) {
    if (pl.variant == V_BYPASS || pl.variant == V_BYPASS16) return launch_bypass(p, pl, stream);
  }
  constexpr bool INT8 = KIND == igc::KIND_U8I8_GEMM || KIND == igc::KIND_U8I8_CONV;
  if constexpr (KIND == igc::KIND_F16_CONV_C64 || (SUMS & igc::REQ_TILES) != 0 || (INT8 && (SUMS & igc::NO_SPLIT) != 0)) {
    return launch_variant<KIND, true, SUMS>(p, pl, stream);  // dispatched only with aligned operands
  } else {
    return fast ? launch_variant<KIND, true, SUMS>(p, pl, stream)
                : launch_variant<KIND, false, SUMS>(p, pl, stream);
  }
}

// Whole requantize-only tiles (REQ_TILES): every tile whole, requantized
// int8 the only output, no split, a 256-column integer tile.
inline bool req_tiles(const igc::Params& p, const Plan& pl, bool fast) {
  return fast && p.Qo && !p.Ci && !p.D && p.vec_q && pl.sk_wgs == 0 &&
         (pl.variant == V_256x256 || pl.variant == V_224x256) && p.M % pl.bm == 0 && p.N % pl.bn == 0;
}

// The (kind, variant) pairs the C ABI launches: the fp16 kinds without
// sums (the convolutions also with BLK_OUT), the u8 x i8 kinds with each
// subset of SUM_ROWS | SUM_COLS, alone and with REQ_TILES, and REQ_TILES
// with the caller's column sums (COLS_IN, with or without SUM_ROWS); every
// kind also as NO_SPLIT, for launches whose tiles are all whole (the integer
// kinds only at the aligned 64x64 and 128x128 tiles, the ones that can split).
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
  X(10, igc::KIND_U8I8_CONV, 3)     \
  X(11, igc::KIND_U8I8_GEMM, 4)     \
  X(12, igc::KIND_U8I8_GEMM, 5)     \
  X(13, igc::KIND_U8I8_GEMM, 6)     \
  X(14, igc::KIND_U8I8_GEMM, 7)     \
  X(15, igc::KIND_U8I8_CONV, 4)     \
  X(16, igc::KIND_U8I8_CONV, 5)     \
  X(17, igc::KIND_U8I8_CONV, 6)     \
  X(18, igc::KIND_U8I8_CONV, 7)     \
  X(19, igc::KIND_F16_CONV, 8)      \
  X(20, igc::KIND_F16_CONV_C64, 8)  \
  X(21, igc::KIND_U8I8_GEMM, 20)    \
  X(22, igc::KIND_U8I8_GEMM, 21)    \
  X(23, igc::KIND_U8I8_CONV, 20)    \
  X(24, igc::KIND_U8I8_CONV, 21)    \
  X(25, igc::KIND_F16_GEMM, 32)     \
  X(26, igc::KIND_F16_CONV, 32)     \
  X(27, igc::KIND_F16_CONV_C64, 32) \
  X(28, igc::KIND_F16_CONV, 40)     \
  X(29, igc::KIND_F16_CONV_C64, 40) \
  X(30, igc::KIND_U8I8_GEMM, 32)    \
  X(31, igc::KIND_U8I8_GEMM, 33)    \
  X(32, igc::KIND_U8I8_GEMM, 34)    \
  X(33, igc::KIND_U8I8_GEMM, 35)    \
  X(34, igc::KIND_U8I8_CONV, 32)    \
  X(35, igc::KIND_U8I8_CONV, 33)    \
  X(36, igc::KIND_U8I8_CONV, 34)    \
  X(37, igc::KIND_U8I8_CONV, 35)

#define IGC_EXTERN_LAUNCH(n, K, S) \
  extern template int launch<K, S>(const igc::Params&, const Plan&, bool, hipStream_t);
IGC_LAUNCH_KINDS(IGC_EXTERN_LAUNCH)
#undef IGC_EXTERN_LAUNCH

}  // namespace igc_host
