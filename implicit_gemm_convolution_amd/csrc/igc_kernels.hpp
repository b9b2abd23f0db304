// igc_kernels.hpp -- MFMA GEMM mainloop for gfx950 (CDNA4) and its three
// users: fp16 GEMM, fp16 implicit-GEMM convolution and u8 x i8 GEMM with the
// zero-point / dequantize / requantize epilogue.
//
// Sources (cited by page title and section):
//  [GEMM-TVM]  CSDN article "TVM在CUDA GPU上跑GEMM的全套张量化实现：WMMA/DP4A/IMMA
//              + TensorIR调度 + INT8/FP16多精度支持".
//  [TIR-PRACTICE] "TVM TensorIR 自动化算子优化工程实践：从调度原语到硬件原生性能".
//  [CONV-TC]   TVM tutorial (Chinese docs, segmentfault) on a conv2d schedule
//              with TensorCores.
//  [TIR-COMPILER] article on the MLIR-based "TensorIR-Compiler".
//
// Design (gfx950, wave64):
//  * Each workgroup owns one BM x BN tile of C and walks K in tiles of 128
//    bytes per row (64 fp16 or 128 int8 elements): the block / warp / fragment
//    hierarchy of [GEMM-TVM] §4.2 and [CONV-TC] "Scheduling the computation",
//    re-derived for 64-wide waves and 32x32 MFMA tiles.
//  * Both operands are K-contiguous (A row-major, B column-major), so a tile
//    row is one 128-byte run: every load request is a whole cache line.
//  * The K loop is software-pipelined two tiles deep ([TIR-COMPILER] §2.2 and
//    §4.4): one operand goes from HBM straight into one of three LDS stages
//    with buffer loads that write LDS; the other goes through one of two
//    register staging sets into one of two LDS stages.  Loads for tile kt+2
//    are issued while tile kt is computed (three plus two stages fill the
//    160 KiB LDS at 256x256).  Out-of-range buffer offsets read as zeros:
//    ragged tiles, K tails and the convolution's zero padding need no
//    branches.
//  * LDS rows are 128 bytes; the 16-byte chunk c of row r sits in slot
//    c ^ ((r >> 1) & 7), so fragment reads and tile writes are free of bank
//    conflicts on the 64-bank LDS (see swz()).  This replaces the padding
//    offsets of [GEMM-TVM] §3.2 and storage_align of [TIR-PRACTICE] §2.2 with
//    the swizzle named in [TIR-COMPILER] §2.2.
//  * MFMA: v_mfma_f32_32x32x16_f16 and v_mfma_i32_32x32x32_i8.  Each lane
//    feeds 16 bytes of one row of A and 16 bytes of one column of B per
//    instruction (lane l: row/column l % 32, K half l / 32).  A and B use the
//    same (lane, element) -> k assignment, so the K order inside one MFMA
//    never matters.  Fragments are read one k-step ahead; the last k-step's
//    MFMAs of a tile run after the barrier, hiding the next tile's reads.
//  * u8 activations on the signed i8 MFMA: A' = A - 128 = A xor 0x80 per byte,
//    applied on the way into LDS (the u8 A takes the register path); the
//    epilogue then uses zA' = zA - 128 in the four-term identity of
//    [GEMM-TVM] §2.3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>
#include <type_traits>

namespace igc {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

enum Kind : int { KIND_F16_GEMM = 0, KIND_F16_CONV = 1, KIND_U8I8_GEMM = 2 };

constexpr int KT_BYTES = 128;    // bytes of K per tile row
constexpr int CHUNK_BYTES = 16;  // one vector load
constexpr int CPR = KT_BYTES / CHUNK_BYTES;  // chunks per tile row

struct Params {
  // GEMM view: M x N output, K reduction.
  int M, N, K;
  int tiles_m, tiles_n;
  const uint8_t* A;  // fp16 or uint8 rows of K (for the conv: the input x)
  long long lda;     // elements
  const uint8_t* B;  // fp16 or int8 rows of K (column-major B)
  long long ldb;     // elements
  // implicit im2col view of an NHWC input
  int Nb, H, W, C, R, S, sh, sw, ph, pw, P, Q;
  // fp32 output (fp16 GEMM and conv)
  float* Cf;
  long long ldcf;
  // u8 x i8 epilogue
  int zAp;  // zA - 128
  int zB;
  int32_t* Ci;
  long long ldci;
  float* D;
  long long ldd;
  float dq;
  int8_t* Qo;
  long long ldq;
  const float* scale;
  const float* bias;
  // 16-byte (int8: 4-byte) vector stores allowed for each output
  int vec_c, vec_d, vec_q;
};

// ---------------------------------------------------------------------------
// Tile scheduling.  The dispatcher hands workgroups to the 8 XCDs round-robin
// (workgroup b runs on XCD b % 8).  When the tile count divides by 8, logical
// tile ids are regrouped so that each XCD owns a contiguous run of them, and
// the run is laid out in groups of GROUP_M tile-rows, so the workgroups that
// share an XCD's L2 also share A and B panels.
// ---------------------------------------------------------------------------
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(const Params& p, int& tm, int& tn) {
  const int total = p.tiles_m * p.tiles_n;
  int bid = blockIdx.x;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  const int per_group = GROUP_M * p.tiles_n;
  const int group = bid / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(p.tiles_m - first_m, GROUP_M);
  const int in_group = bid - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// LDS has 64 banks of 4 bytes and serves a 16-byte-per-lane access 16 lanes
// at a time.  A 128-byte row covers half the banks, so rows r and r+1 use
// different halves, and the chunk XOR (r >> 1) & 7 spreads the 8 rows of each
// parity over the 8 chunk slots: 16 consecutive rows reading one chunk
// column, and 2 rows written by 16 consecutive lanes, are conflict-free.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * KT_BYTES + ((chunk ^ ((row >> 1) & 7)) << 4);
}

__device__ __forceinline__ uint4 lds_read16(const uint8_t* base, int off) {
  return *reinterpret_cast<const uint4*>(base + off);
}

__device__ __forceinline__ void lds_write16(uint8_t* base, int off, uint4 v) {
  *reinterpret_cast<uint4*>(base + off) = v;
}

// Output stores bypass the caches' retention (non-temporal): the results are
// not read again by the kernel, and streaming them measured ~20% faster.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16_nt(void* dst, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(dst));
}
__device__ __forceinline__ void store4_nt(void* dst, uint32_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(dst));
}

// ---------------------------------------------------------------------------
// Buffer descriptors and direct-to-LDS loads.
// ---------------------------------------------------------------------------
constexpr uint32_t OOB = 0x80000000u;  // descriptors are limited to < 2^31 bytes

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // word 3 = 0x00020000: raw (untyped) 32-bit-dword buffer on gfx9-family GPUs.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// One wave-wide 16-byte-per-lane load written to LDS: lane l's 16 bytes land
// at lds + 16*l (lds is uniform across the wave).  An offset past the
// descriptor's extent writes zeros.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, (int)off, 0, 0, 0);
}

// Direct-to-LDS tiles of ROWS rows x 128 bytes.  Wave-instruction q fills
// rows 8q .. 8q+7 (1 KB of LDS); lane l covers row 8q + l/8 and fetches the
// global chunk that belongs in its LDS slot l % 8, i.e. chunk
// (l % 8) ^ ((4q + l/16) % 8).  Instruction q = i*NWAVES + wave, i < NQ; with
// an even wave count q % 2 = wave % 2, so each lane's chunk is fixed.
// Index of the calling wave in its workgroup, as a scalar (wave-uniform) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

template <int NT, int ROWS>
struct DmaShape {
  static constexpr int NWAVES = NT / 64;
  static constexpr int NQ = ROWS / 8 / NWAVES;  // instructions per wave per tile
  static_assert(ROWS % (8 * NWAVES) == 0 && NWAVES % 2 == 0, "tile rows must split over the waves");
  __device__ static __forceinline__ int lane_row() {  // + i * 8 * NWAVES
    return (threadIdx.x >> 6) * 8 + ((threadIdx.x & 63) >> 3);
  }
  __device__ static __forceinline__ int lane_chunk() {
    const int l = threadIdx.x & 63;
    return (l & 7) ^ ((4 * ((threadIdx.x >> 6) & 1) + (l >> 4)) & 7);
  }
  __device__ static __forceinline__ uint8_t* dst(uint8_t* tile, int i) {
    return tile + (i * NWAVES + wave_id()) * 1024;
  }
};

// Operand loaded straight into LDS (A of the fp16 GEMM; the i8 B of the
// u8 x i8 GEMM): rows of K.
//  FAST: 16-byte aligned rows, K a multiple of the chunk: direct-to-LDS loads.
//  else: element-wise loads, written to LDS with the same layout.
template <int NT, int ROWS, int EB, bool FAST>
struct RowDmaLoader {
  typedef DmaShape<NT, ROWS> Sh;
  const uint8_t* base;  // row 0 of this tile
  long long ld_bytes;
  int rows_valid;       // rows of this tile that exist
  int K;
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t lane_off;    // byte offset of this lane's first row and chunk
  uint32_t row_step;    // bytes between this lane's rows (uniform)

  __device__ __forceinline__ void init(const uint8_t* ptr, long long ld, int r0, int nrows, int k) {
    ld_bytes = ld * EB;
    base = ptr + (long long)r0 * ld_bytes;
    rows_valid = nrows - r0;
    K = k;
    if (FAST) {
      const long long extent = (long long)min(rows_valid, ROWS) * ld_bytes;
      rsrc = make_rsrc(base, (uint32_t)extent);
      lane_off = (uint32_t)(Sh::lane_row() * ld_bytes) + (uint32_t)(Sh::lane_chunk() * CHUNK_BYTES);
      row_step = (uint32_t)(8 * Sh::NWAVES * ld_bytes);
    }
  }

  // Fill `tile` (ROWS x 128 bytes, swizzled) with K tile kt; rows past the
  // operand and k past K read as zero bytes.
  __device__ __forceinline__ void load(uint8_t* tile, int kt) const {
    if (FAST) {
      const bool kin = kt * KT_BYTES + Sh::lane_chunk() * CHUNK_BYTES < K * EB;
#pragma unroll
      for (int i = 0; i < Sh::NQ; ++i)
        dma16(rsrc, Sh::dst(tile, i), kin ? lane_off + (uint32_t)(i * row_step + kt * KT_BYTES) : OOB);
    } else {
      constexpr int EPC = CHUNK_BYTES / EB;
      const int c = threadIdx.x & 7;  // thread t: chunk t%8 of rows t/8 + (NT/8)*j
      const int k0 = kt * (KT_BYTES / EB) + c * EPC;
#pragma unroll
      for (int j = 0; j < ROWS * CPR / NT; ++j) {
        const int row = (threadIdx.x >> 3) + j * (NT / 8);
        const uint8_t* rp = base + (long long)row * ld_bytes;
        uint8_t bytes[16];
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const int k = k0 + e;
          const bool ok = row < rows_valid && k < K;
#pragma unroll
          for (int b = 0; b < EB; ++b) bytes[e * EB + b] = ok ? rp[(long long)k * EB + b] : (uint8_t)0;
        }
        uint4 v;
        __builtin_memcpy(&v, bytes, 16);
        lds_write16(tile, swz(row, c), v);
      }
    }
  }
};

// Operand staged through registers (B of the fp16 GEMM and the conv weight;
// the u8 A of the u8 x i8 GEMM): thread t holds chunk t%8 of rows
// t/8 + (NT/8)*j, so each group of 8 lanes fetches one whole 128-byte line.
template <int NT, int ROWS, int EB, bool FAST, bool XOR80 = false>
struct RowRegLoader {
  static constexpr int NCH = ROWS * CPR / NT;  // chunks per thread
  const uint8_t* base;
  long long ld_bytes;
  int rows_valid;
  int K;
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t lane_off;  // byte offset of this thread's first row and chunk
  uint32_t row_step;  // bytes between its rows (uniform)

  __device__ __forceinline__ void init(const uint8_t* ptr, long long ld, int r0, int nrows, int k) {
    ld_bytes = ld * EB;
    base = ptr + (long long)r0 * ld_bytes;
    rows_valid = nrows - r0;
    K = k;
    if (FAST) {
      const long long extent = (long long)min(rows_valid, ROWS) * ld_bytes;
      rsrc = make_rsrc(base, (uint32_t)extent);
      lane_off = (uint32_t)((threadIdx.x >> 3) * ld_bytes) + (uint32_t)((threadIdx.x & 7) * CHUNK_BYTES);
      row_step = (uint32_t)((NT / 8) * ld_bytes);
    }
  }

  __device__ __forceinline__ void load(uint4 (&r)[NCH], int kt) const {
    constexpr int EPC = CHUNK_BYTES / EB;
    const int c = threadIdx.x & 7;
    if (FAST) {
      const bool kin = kt * KT_BYTES + c * CHUNK_BYTES < K * EB;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        auto v = __builtin_amdgcn_raw_buffer_load_b128(
            rsrc, (int)(kin ? lane_off + (uint32_t)(j * row_step + kt * KT_BYTES) : OOB), 0, 0);
        r[j] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    } else {
      const int k0 = kt * (KT_BYTES / EB) + c * EPC;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int row = (threadIdx.x >> 3) + j * (NT / 8);
        const uint8_t* rp = base + (long long)row * ld_bytes;
        uint8_t bytes[16];
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const int k = k0 + e;
          const bool ok = row < rows_valid && k < K;
#pragma unroll
          for (int b = 0; b < EB; ++b) bytes[e * EB + b] = ok ? rp[(long long)k * EB + b] : (uint8_t)0;
        }
        uint4 v;
        __builtin_memcpy(&v, bytes, 16);
        r[j] = v;
      }
    }
  }

  // XOR80: u8 -> s8 operand, A' = A - 128 = A xor 0x80 per byte, applied on
  // the way into LDS (padding bytes 0 become A' = 0).
  __device__ __forceinline__ void store(uint8_t* tile, const uint4 (&r)[NCH]) const {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      uint4 v = r[j];
      if constexpr (XOR80) {
        v.x ^= 0x80808080u; v.y ^= 0x80808080u; v.z ^= 0x80808080u; v.w ^= 0x80808080u;
      }
      lds_write16(tile, swz((threadIdx.x >> 3) + j * (NT / 8), threadIdx.x & 7), v);
    }
  }
};

// Implicit im2col view of an NHWC fp16 input (the conv's A operand): row
// m = (n, p, q), column k = (r*S + s)*C + c holds
// x[n, p*sh + r - ph, q*sw + s - pw, c], or 0 where that position lies in the
// zero padding ([CONV-TC] "Preparation and algorithm": Apad is inlined, the
// padding predicate is evaluated inside the shared-memory fill).  (n, p, q)
// is decoded once per row at kernel start.  FAST (C % 8 == 0): the 8 channels
// of a chunk share one tap (r, s); each lane tracks the (r, s, c) of its chunk
// and advances it by the 64 channels of one K tile.
template <int NT, int ROWS, bool FAST>
struct Im2colLoader {
  typedef DmaShape<NT, ROWS> Sh;
  static constexpr int NR = FAST ? Sh::NQ : ROWS * CPR / NT;  // rows per lane
  const uint8_t* x;
  int pix[NR];  // pixel index in x of (n, p*sh - ph, q*sw - pw), i.e. of tap (0, 0)
  int hw[NR];   // (p*sh - ph) << 16 | (q*sw - pw) & 0xffff; INT32_MIN for rows past M
  int H, W, C, S, K;
  __amdgpu_buffer_rsrc_t rsrc;
  // tap of this lane's chunk for the next K tile to be loaded (FAST)
  mutable int cur_r, cur_s, cur_c;

  __device__ __forceinline__ int row_h(int j) const { return hw[j] >> 16; }
  __device__ __forceinline__ int row_w(int j) const { return (int)(int16_t)(hw[j] & 0xffff); }

  __device__ __forceinline__ void init(const Params& p, int m0) {
    x = p.A;
    H = p.H; W = p.W; C = p.C; S = p.S; K = p.K;
    if (FAST) rsrc = make_rsrc(x, (uint32_t)((long long)p.Nb * H * W * C * 2));
    const int PQ = p.P * p.Q;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int r = FAST ? Sh::lane_row() + j * 8 * Sh::NWAVES : (int)(threadIdx.x >> 3) + j * (NT / 8);
      const int m = m0 + r;
      if (m < p.M) {
        const int n = m / PQ;
        const int pq = m - n * PQ;
        const int pp = pq / p.Q;
        const int qq = pq - pp * p.Q;
        const int h0 = pp * p.sh - p.ph;
        const int w0 = qq * p.sw - p.pw;
        pix[j] = n * H * W + h0 * W + w0;
        hw[j] = (int)(((uint32_t)h0 << 16) | ((uint32_t)w0 & 0xffffu));
      } else {
        pix[j] = 0;
        hw[j] = INT32_MIN;
      }
    }
    // tap of k = chunk*8 (K tile 0)
    const int k0 = FAST ? Sh::lane_chunk() * 8 : 0;
    const int rs = k0 / C;
    cur_c = k0 - rs * C;
    cur_r = rs / S;
    cur_s = rs - cur_r * S;
  }

  __device__ __forceinline__ uint16_t elem(int j, int k) const {
    if (hw[j] == INT32_MIN || k >= K) return 0;
    const int rs = k / C;
    const int c = k - rs * C;
    const int r = rs / S;
    const int s = rs - r * S;
    const int h = row_h(j) + r;
    const int w = row_w(j) + s;
    if ((unsigned)h >= (unsigned)H || (unsigned)w >= (unsigned)W) return 0;
    return reinterpret_cast<const uint16_t*>(x)[(long long)(pix[j] + r * W + s) * C + c];
  }

  // FAST: K tiles must be requested in order 0, 1, 2, ... (the tap advances).
  __device__ __forceinline__ void load(uint8_t* tile, int kt) const {
    if (FAST) {
      const bool kin = kt * 64 + Sh::lane_chunk() * 8 < K;
      const int tap = cur_r * W + cur_s;
#pragma unroll
      for (int j = 0; j < Sh::NQ; ++j) {
        const int h = row_h(j) + cur_r;  // rows past M have h < -16000: never in range
        const int w = row_w(j) + cur_s;
        const bool ok = kin && (unsigned)h < (unsigned)H && (unsigned)w < (unsigned)W;
        const uint32_t off = ((uint32_t)(pix[j] + tap) * (uint32_t)C + (uint32_t)cur_c) * 2u;
        dma16(rsrc, Sh::dst(tile, j), ok ? off : OOB);
      }
      // advance this lane's tap by the 64 channels of one K tile
      cur_c += 64;
      while (cur_c >= C) {
        cur_c -= C;
        if (++cur_s == S) {
          cur_s = 0;
          ++cur_r;
        }
      }
    } else {
      const int c = threadIdx.x & 7;
      const int k0 = kt * 64 + c * 8;
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const int row = (threadIdx.x >> 3) + j * (NT / 8);
        uint16_t e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = elem(j, k0 + i);
        uint4 v;
        __builtin_memcpy(&v, e, 16);
        lds_write16(tile, swz(row, c), v);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA wrappers.  One call = one 32 x 32 output tile, 32 bytes of K per row.
// ---------------------------------------------------------------------------
template <int KIND>
struct Mfma;

template <>
struct Mfma<KIND_F16_GEMM> {
  typedef f32x16 acc_t;
  __device__ __forceinline__ static void run(acc_t& c, uint4 a, uint4 b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                               __builtin_bit_cast(half8, b), c, 0, 0, 0);
  }
};
template <>
struct Mfma<KIND_F16_CONV> : Mfma<KIND_F16_GEMM> {};
template <>
struct Mfma<KIND_U8I8_GEMM> {
  typedef i32x16 acc_t;
  __device__ __forceinline__ static void run(acc_t& c, uint4 a, uint4 b) {
    c = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                              __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
  }
};

__device__ __forceinline__ int sum_bytes(uint4 v, int acc) {
  acc = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, acc, false);
  acc = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, acc, false);
  acc = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, acc, false);
  acc = __builtin_amdgcn_sdot4((int)v.w, 0x01010101, acc, false);
  return acc;
}

// s_waitcnt until at most N vector-memory operations of this wave are
// outstanding and all of its LDS operations are done.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// ---------------------------------------------------------------------------
// The kernel.
//  SUMS (u8 x i8 only): accumulate rowsum(A') / colsum(B) for the zero-point
//  correction; not compiled when zA == 128 and zB == 0.
// ---------------------------------------------------------------------------
template <int KIND, int BM, int BN, int WM, int WN, bool FAST, bool SUMS = false>
__global__ void __launch_bounds__(64 * WM * WN, 1) gemm_kernel(const Params p) {
  constexpr int NT = 64 * WM * WN;
  constexpr int EB = (KIND == KIND_U8I8_GEMM) ? 1 : 2;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int SA = BM * KT_BYTES, SB = BN * KT_BYTES;  // stage sizes
  constexpr bool INT8 = KIND == KIND_U8I8_GEMM;
  // Operand roles: one operand streams straight into a 3-stage LDS ring (X),
  // the other goes through 2 register staging sets into a 2-stage ring (Y).
  // The u8 A of the integer GEMM takes the register path so that its
  // u8 -> s8 conversion happens once, on the way into LDS, rather than on
  // every fragment read.
  constexpr bool A_IN_X = !INT8;
  constexpr int SX = A_IN_X ? SA : SB, SY = A_IN_X ? SB : SA;
  typedef typename std::conditional<
      KIND == KIND_F16_CONV, Im2colLoader<NT, BM, FAST>,
      typename std::conditional<A_IN_X, RowDmaLoader<NT, BM, EB, FAST>,
                                RowRegLoader<NT, BM, EB, FAST, true>>::type>::type ALoader;
  typedef typename std::conditional<A_IN_X, RowRegLoader<NT, BN, EB, FAST>,
                                    RowDmaLoader<NT, BN, EB, FAST>>::type BLoader;
  typedef typename std::conditional<A_IN_X, BLoader, ALoader>::type YLoader;  // register path
  constexpr int NCH_Y = YLoader::NCH;
  // vector-memory instructions per K tile per lane (the X loads count only on
  // the direct-to-LDS path; element-wise loads are waited for by the compiler
  // before they are used)
  constexpr int NLX = FAST ? DmaShape<NT, A_IN_X ? BM : BN>::NQ : 0;
  constexpr int NVM = NLX + (FAST ? NCH_Y : 0);
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(FM <= 4 && BM >= BN, "epilogue staging reuses the stage arrays");
  static_assert(NVM < 64, "vmcnt range");
  typedef typename Mfma<KIND>::acc_t acc_t;

  // One LDS array per stage: the compiler then knows which stage each
  // direct-to-LDS load writes and waits for exactly that one.
  __shared__ __attribute__((aligned(16))) uint8_t sx0[SX];
  __shared__ __attribute__((aligned(16))) uint8_t sx1[SX];
  __shared__ __attribute__((aligned(16))) uint8_t sx2[SX];
  __shared__ __attribute__((aligned(16))) uint8_t sy0[SY];
  __shared__ __attribute__((aligned(16))) uint8_t sy1[SY];
  auto stX = [&](auto U) -> uint8_t* {
    constexpr int u = decltype(U)::value % 3;
    if constexpr (u == 0) return sx0;
    if constexpr (u == 1) return sx1;
    return sx2;
  };
  auto stY = [&](auto U) -> uint8_t* {
    constexpr int u = decltype(U)::value % 2;
    if constexpr (u == 0) return sy0;
    return sy1;
  };
  auto stA = [&](auto U) -> uint8_t* {
    if constexpr (A_IN_X) return stX(U); else return stY(U);
  };
  auto stB = [&](auto U) -> uint8_t* {
    if constexpr (A_IN_X) return stY(U); else return stX(U);
  };

  int tm, tn;
  tile_coords<8>(p, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id();
  const int wm = wave / WN, wn = wave % WN;

  ALoader la;
  if constexpr (KIND == KIND_F16_CONV) {
    la.init(p, m0);
  } else {
    la.init(p.A, p.lda, m0, p.M, p.K);
  }
  BLoader lb;
  lb.init(p.B, p.ldb, n0, p.N, p.K);

  acc_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  // Per-lane partial sums of A' rows / B columns (u8 x i8 with zero points).
  int rsum[FM], csum[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) rsum[i] = 0;
#pragma unroll
  for (int j = 0; j < FN; ++j) csum[j] = 0;
  const bool want_rsum = SUMS && p.zB != 0 && wn == 0;
  const bool want_csum = SUMS && p.zAp != 0 && wm == 0;

  const int nk = (p.K * EB + KT_BYTES - 1) / KT_BYTES;

  // Fragments, double-buffered in registers: lane l reads row l % 32 of its
  // 32-row block, 16-byte chunk 2*ks + l/32 (k-step ks covers 32 bytes of K).
  const int frow = lane & 31;
  const int fhalf = lane >> 5;
  uint4 fa[2][FM], fb[2][FN];
  auto read_frags = [&](const uint8_t* As, const uint8_t* Bs, int ks, uint4 (&a)[FM], uint4 (&b)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i) a[i] = lds_read16(As, swz(wm * TM + i * 32 + frow, ks * 2 + fhalf));
#pragma unroll
    for (int j = 0; j < FN; ++j) b[j] = lds_read16(Bs, swz(wn * TN + j * 32 + frow, ks * 2 + fhalf));
  };
  auto mfmas = [&](const uint4 (&a)[FM], const uint4 (&b)[FN]) {
    if constexpr (SUMS) {
#pragma unroll
      for (int i = 0; i < FM; ++i) rsum[i] = sum_bytes(a[i], rsum[i]);
#pragma unroll
      for (int j = 0; j < FN; ++j) csum[j] = sum_bytes(b[j], csum[j]);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) Mfma<KIND>::run(acc[i][j], a[i], b[j]);
  };
  constexpr int NMF = FM * FN;  // MFMAs per k-step
  constexpr int NRD = FM + FN;  // fragment reads per k-step
  constexpr int KSTEPS = KT_BYTES / 32;

  // The two operand paths: X straight into LDS, Y through registers.
  auto x_load = [&](uint8_t* st, int kt) {
    if constexpr (A_IN_X) la.load(st, kt); else lb.load(st, kt);
  };
  auto y_load = [&](uint4 (&r)[NCH_Y], int kt) {
    if constexpr (A_IN_X) lb.load(r, kt); else la.load(r, kt);
  };
  auto y_store = [&](uint8_t* st, const uint4 (&r)[NCH_Y]) {
    if constexpr (A_IN_X) lb.store(st, r); else la.store(st, r);
  };
  uint4 ry[2][NCH_Y];  // register staging sets

  // Prologue: tiles 0 and 1 in flight; tile 0 in LDS.
  x_load(sx0, 0);
  y_load(ry[0], 0);
  x_load(sx1, 1);
  y_load(ry[1], 1);
  y_store(sy0, ry[0]);
  wait_vmcnt_lgkm0<NVM>();
  __builtin_amdgcn_s_barrier();
  read_frags(stA(std::integral_constant<int, 0>()), stB(std::integral_constant<int, 0>()), 0, fa[0], fb[0]);

  // K tile kt: X operand in stage kt % 3 (the stage of tile kt+2 is the one
  // tile kt-1 used), Y operand in stage kt % 2, Y of tile kt+2 in staging set
  // kt % 2.  Region 1: loads of tile kt+2, k-steps 0..KSTEPS-2 of tile kt,
  // staging set of tile kt+1 -> Y stage (kt+1) % 2.  Then wait until every
  // load issued before this iteration has landed (X of tile kt+1 included)
  // and every LDS access of this wave is done, and barrier.  Region 2: the
  // last k-step's MFMAs run over the reads of the next tile's first
  // fragments.  The instruction scheduler is asked to spread the memory
  // instructions between the MFMAs, so the in-order wave never stalls behind
  // a burst of them.
  auto tile = [&](int kt, auto U) {
    constexpr int u = decltype(U)::value;
    const uint8_t* As = stA(U);
    const uint8_t* Bs = stB(U);
    x_load(stX(std::integral_constant<int, u + 2>()), kt + 2);
    y_load(ry[u % 2], kt + 2);
    int buf = 0;
#pragma unroll
    for (int ks = 0; ks < KSTEPS - 1; ++ks) {
      read_frags(As, Bs, ks + 1, fa[buf ^ 1], fb[buf ^ 1]);
      mfmas(fa[buf], fb[buf]);
      buf ^= 1;
    }
    y_store(stY(std::integral_constant<int, u + 1>()), ry[(u + 1) % 2]);
    {
      int rd = 0, vm = 0, wr = 0;
#pragma unroll
      for (int m = 0; m < (KSTEPS - 1) * NMF; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if ((m & 1) == 0 && rd < (KSTEPS - 1) * NRD) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
          ++rd;
        }
        if (m % 3 == 0 && vm < NLX + NCH_Y) {
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global load
          ++vm;
        }
        if (m % 3 == 1 && m >= NMF && wr < NCH_Y) {
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // LDS write
          ++wr;
        }
      }
    }
    wait_vmcnt_lgkm0<NVM>();
    __builtin_amdgcn_s_barrier();
    read_frags(stA(std::integral_constant<int, u + 1>()), stB(std::integral_constant<int, u + 1>()), 0,
               fa[buf ^ 1], fb[buf ^ 1]);
    mfmas(fa[buf], fb[buf]);
#pragma unroll
    for (int q = 0; q < NMF; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (q < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };
  static_assert(KSTEPS % 2 == 0, "the fragment double buffer returns to set 0 after a tile");
  for (int kt = 0; kt < nk; kt += 6) {
    tile(kt, std::integral_constant<int, 0>());
    if (kt + 1 < nk) tile(kt + 1, std::integral_constant<int, 1>());
    if (kt + 2 < nk) tile(kt + 2, std::integral_constant<int, 2>());
    if (kt + 3 < nk) tile(kt + 3, std::integral_constant<int, 3>());
    if (kt + 4 < nk) tile(kt + 4, std::integral_constant<int, 4>());
    if (kt + 5 < nk) tile(kt + 5, std::integral_constant<int, 5>());
  }
  // Loads past the last tile may still be writing (zeros): drain them before
  // the epilogue reuses the stage arrays.
  wait_vmcnt_lgkm0<0>();
  __builtin_amdgcn_s_barrier();

  // ------------------------------------------------------------------ epilogue
  // The accumulators are staged through LDS one wave-row at a time (TM rows;
  // rows 32i..32i+31 in stage array i, BN*4 bytes per row, 16-byte chunk q
  // in slot q ^ (8 * ((row >> 2) & 1)) so that the two row groups written by
  // one staging store land in different bank halves).  Then every thread
  // takes 4 consecutive columns of a row: the int8 corrections and
  // quantization run element-wise on them, and results leave in 16-byte
  // (fp32/int32) or 4-byte (int8) stores.
  //
  // Accumulator layout of a 32x32 MFMA tile: lane l holds column l % 32 and,
  // in register e, row 8*(e/4) + 4*(l/32) + e%4.
  const int ccol = lane & 31;
  const int rbase = 4 * (lane >> 5);
  // Staging arrays for 32-row blocks: the three X stages and the first Y
  // stage (each holds 32 x BN x 4 bytes since BN <= BM); the zero-point sums
  // go to the second Y stage.
  auto stage_rt = [&](int u) -> uint8_t* {  // u is a constant after unrolling
    return u == 0 ? sx0 : u == 1 ? sx1 : u == 2 ? sx2 : sy0;
  };
  static_assert(32 * BN * 4 <= SB && (BM + BN) * 4 <= SB, "staging and sums fit in the stages");
  int* const sums = reinterpret_cast<int*>(sy1);
  auto stage_off = [](int rl, int c) {  // rl: row within a 32-row array; c: column
    return rl * (BN * 4) + (((c >> 2) ^ (8 * ((rl >> 2) & 1))) << 4) + (c & 3) * 4;
  };

  uint32_t kzz = 0;
  if constexpr (SUMS) {
    // Complete the row / column sums (the two K halves live in lanes l, l^32)
    // and publish them through LDS.
    if (want_rsum) {
      // K-tail padding loads as byte 0 and is stored as A' = -128: add those
      // terms back.
      const int pad_fix = 128 * (nk * KT_BYTES - p.K);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int t = rsum[i] + __shfl_xor(rsum[i], 32) + pad_fix;
        if (lane < 32) sums[wm * TM + i * 32 + lane] = t;
      }
    }
    if (want_csum) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int t = csum[j] + __shfl_xor(csum[j], 32);
        if (lane < 32) sums[BM + wn * TN + j * 32 + lane] = t;
      }
    }
  }
  if constexpr (INT8) kzz = (uint32_t)p.K * (uint32_t)p.zAp * (uint32_t)p.zB;

  constexpr int GPR = BN / 4;    // 4-column groups per row
  constexpr int RPP = NT / GPR;  // rows per pass of the whole workgroup
  static_assert(NT % GPR == 0 && 32 % RPP == 0, "a pass must cover whole rows of one array");
  const int lcol = (tid % GPR) * 4;
  const int col = n0 + lcol;
  const int rr0 = tid / GPR;

#pragma unroll
  for (int h = 0; h < WM; ++h) {
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        uint8_t* arr = stage_rt(i);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            // copy the element out first: bit-casting a vector-element lvalue
            // directly reads element 0 with this compiler
            const auto val = acc[i][j][e];
            const int off = stage_off(8 * (e >> 2) + rbase + (e & 3), wn * TN + j * 32 + ccol);
            *reinterpret_cast<int32_t*>(arr + off) = __builtin_bit_cast(int32_t, val);
          }
      }
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < TM / RPP; ++pass) {
      const int rr = rr0 + pass * RPP;         // row within the wave-row
      const uint8_t* arr = stage_rt((pass * RPP) / 32);
      const int lrow = h * TM + rr;
      const int row = m0 + lrow;
      if (row < p.M && col < p.N) {
        const uint4 v = *reinterpret_cast<const uint4*>(arr + stage_off(rr & 31, lcol));
        const bool full = col + 3 < p.N;
        if constexpr (!INT8) {
          float* dst = p.Cf + (long long)row * p.ldcf + col;
          if (full && p.vec_c) {
            store16_nt(dst, v);
          } else {
            const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (col + q < p.N) dst[q] = __builtin_bit_cast(float, vv[q]);
          }
        } else {
          // C = acc' - zA'*colsum(B) - zB*rowsum(A') + K*zA'*zB in wrapping
          // 32-bit arithmetic; the true value fits in int32 (K <= 33025).
          uint32_t rcorr = 0;
          if constexpr (SUMS) rcorr = p.zB != 0 ? (uint32_t)p.zB * (uint32_t)sums[lrow] : 0u;
          const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
          int32_t c[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t ccorr = 0;
            if constexpr (SUMS)
              ccorr = p.zAp != 0 ? (uint32_t)p.zAp * (uint32_t)sums[BM + min(lcol + q, BN - 1)] : 0u;
            c[q] = (int32_t)(vv[q] - ccorr - rcorr + kzz);
          }
          if (p.Ci) {
            int32_t* dst = p.Ci + (long long)row * p.ldci + col;
            if (full && p.vec_c) {
              store16_nt(dst, make_uint4((uint32_t)c[0], (uint32_t)c[1], (uint32_t)c[2], (uint32_t)c[3]));
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (col + q < p.N) dst[q] = c[q];
            }
          }
          float cf[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) cf[q] = (float)c[q];  // round to nearest even
          if (p.D) {
            float* dst = p.D + (long long)row * p.ldd + col;
            float d[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) d[q] = cf[q] * p.dq;
            if (full && p.vec_d) {
              store16_nt(dst, make_uint4(__builtin_bit_cast(uint32_t, d[0]), __builtin_bit_cast(uint32_t, d[1]),
                                         __builtin_bit_cast(uint32_t, d[2]), __builtin_bit_cast(uint32_t, d[3])));
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (col + q < p.N) dst[q] = d[q];
            }
          }
          if (p.Qo) {
            int8_t* dst = p.Qo + (long long)row * p.ldq + col;
            uint32_t packed = 0;
            int8_t qv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int cc = min(col + q, p.N - 1);
              const float t = cf[q] * p.scale[cc];  // separately rounded: built with -ffp-contract=off
              const float y = t + p.bias[cc];
              float r = __builtin_rintf(y);         // half to even
              r = fminf(fmaxf(r, -128.f), 127.f);
              qv[q] = (int8_t)(int)r;
              packed |= (uint32_t)(uint8_t)qv[q] << (8 * q);
            }
            if (full && p.vec_q) {
              store4_nt(dst, packed);
            } else {
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (col + q < p.N) dst[q] = qv[q];
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace igc
