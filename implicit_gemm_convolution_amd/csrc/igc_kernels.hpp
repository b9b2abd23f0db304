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
//  * Both operands are K-contiguous (A row-major, B column-major), so every
//    tile row is one 128-byte run: eight 16-byte vector loads, coalesced
//    ([CONV-TC] vectorizes the shared-memory fill the same way).
//  * LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at chunk
//    slot c ^ (r & 7).  A fragment read (32 rows, one chunk column) then hits
//    eight distinct slots per eight lanes: no bank conflicts.  This replaces
//    the padding offsets of [GEMM-TVM] §3.2 and storage_align of
//    [TIR-PRACTICE] §2.2 with the swizzle named in [TIR-COMPILER] §2.2.
//  * Two LDS stages: the global loads for tile k+1 are issued before the
//    MFMAs of tile k and written to the other stage afterwards; one barrier
//    per K tile (software pipelining, [TIR-COMPILER] §2.2 and §4.4).
//  * MFMA: v_mfma_f32_32x32x16_f16 and v_mfma_i32_32x32x32_i8.  Each lane
//    feeds 16 bytes of one row of A and 16 bytes of one column of B per
//    instruction (lane l: row/column l % 32, K half l / 32).  A and B use the
//    same (lane, element) -> k assignment, so the K order inside one MFMA
//    never matters.
//  * u8 activations on the signed i8 MFMA: A' = A - 128 = A xor 0x80 per byte,
//    applied to the fragment after it is read from LDS; the epilogue then uses
//    zA' = zA - 128 in the four-term identity of [GEMM-TVM] §2.3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace igc {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

enum Kind : int { KIND_F16_GEMM = 0, KIND_F16_CONV = 1, KIND_U8I8_GEMM = 2 };

constexpr int ROW_BYTES = 128;  // bytes of K per tile row
constexpr int CHUNK_BYTES = 16; // one vector load

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

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * ROW_BYTES + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ uint4 lds_read16(const uint8_t* base, int off) {
  return *reinterpret_cast<const uint4*>(base + off);
}

__device__ __forceinline__ void lds_write16(uint8_t* base, int off, uint4 v) {
  *reinterpret_cast<uint4*>(base + off) = v;
}

// ---------------------------------------------------------------------------
// Operand loaders.  Thread t owns chunk column (t % 8) of rows
// t/8 + (NT/8)*j, j = 0..NCH-1 of its tile.  Padding (rows past M/N, k past K,
// and the zero padding of the convolution) reads as zero bytes.
//
// The fast path uses raw buffer loads: the buffer descriptor bounds the tile's
// rows, and an offset of OOB (past every descriptor's extent) makes the
// hardware return zeros, so the loads carry no branches.
// ---------------------------------------------------------------------------
constexpr uint32_t OOB = 0x80000000u;  // descriptors are limited to < 2^31 bytes

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // word 3 = 0x00020000: raw (untyped) 32-bit-dword buffer on gfx9-family GPUs.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Plain row-major operand (A of a GEMM, or B / the conv weight).
template <int NT, int NCH, int EB, bool FAST>
struct RowLoader {
  const uint8_t* base;  // row 0 of this tile
  long long ld_bytes;
  int rows_valid;       // rows of this tile that exist
  int K;
  int chunk;            // this thread's chunk column
  int row0;             // this thread's first row
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t row_off[NCH];

  __device__ __forceinline__ void init(const uint8_t* ptr, long long ld, int r0, int nrows, int k,
                                       int tile_rows) {
    ld_bytes = ld * EB;
    base = ptr + (long long)r0 * ld_bytes;
    rows_valid = nrows - r0;
    K = k;
    chunk = threadIdx.x & 7;
    row0 = threadIdx.x >> 3;
    if (FAST) {
      const long long extent = (long long)min(rows_valid, tile_rows) * ld_bytes;
      rsrc = make_rsrc(base, (uint32_t)extent);
#pragma unroll
      for (int j = 0; j < NCH; ++j)
        row_off[j] = (uint32_t)((row0 + j * (NT / 8)) * ld_bytes) + (uint32_t)(chunk * CHUNK_BYTES);
    }
  }

  __device__ __forceinline__ void load(uint4 (&r)[NCH], int kt) const {
    constexpr int EPC = CHUNK_BYTES / EB;
    const int k0 = kt * (ROW_BYTES / EB) + chunk * EPC;
    if (FAST) {
      // K % EPC == 0 here, so a chunk is either wholly inside K or wholly past it.
      const bool kin = k0 < K;
      const uint32_t koff = (uint32_t)(kt * ROW_BYTES);
#pragma unroll
      for (int j = 0; j < NCH; ++j) r[j] = buf_load16(rsrc, kin ? row_off[j] + koff : OOB);
    } else {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int row = row0 + j * (NT / 8);
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
};

// Implicit im2col view of an NHWC fp16 input: row m = (n, p, q), column
// k = (r*S + s)*C + c holds x[n, p*sh + r - ph, q*sw + s - pw, c], or 0 where
// that position lies in the zero padding ([CONV-TC] "Preparation and
// algorithm": Apad is inlined, the padding predicate is evaluated inside the
// shared-memory fill).  (n, p, q) is decoded once per row at kernel start;
// (r, s, c) once per K tile.
template <int NT, int NCH, bool FAST>
struct Im2colLoader {
  const uint8_t* x;
  int img[NCH];  // n*H*W (pixel index of the image), or -1 for rows past M
  int hb[NCH];   // p*sh - ph
  int wb[NCH];   // q*sw - pw
  int H, W, C, S, K;
  int chunk;
  __amdgpu_buffer_rsrc_t rsrc;

  __device__ __forceinline__ void init(const Params& p, int m0) {
    x = p.A;
    H = p.H; W = p.W; C = p.C; S = p.S; K = p.K;
    chunk = threadIdx.x & 7;
    if (FAST) rsrc = make_rsrc(x, (uint32_t)((long long)p.Nb * H * W * C * 2));
    const int PQ = p.P * p.Q;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int m = m0 + (threadIdx.x >> 3) + j * (NT / 8);
      if (m < p.M) {
        const int n = m / PQ;
        const int pq = m - n * PQ;
        const int pp = pq / p.Q;
        const int qq = pq - pp * p.Q;
        img[j] = n * H * W;
        hb[j] = pp * p.sh - p.ph;
        wb[j] = qq * p.sw - p.pw;
      } else {
        img[j] = -1;
        hb[j] = 0;
        wb[j] = 0;
      }
    }
  }

  __device__ __forceinline__ uint16_t elem(int j, int k) const {
    if (img[j] < 0 || k >= K) return 0;
    const int rs = k / C;
    const int c = k - rs * C;
    const int r = rs / S;
    const int s = rs - r * S;
    const int h = hb[j] + r;
    const int w = wb[j] + s;
    if ((unsigned)h >= (unsigned)H || (unsigned)w >= (unsigned)W) return 0;
    return reinterpret_cast<const uint16_t*>(x)[(long long)(img[j] + h * W + w) * C + c];
  }

  __device__ __forceinline__ void load(uint4 (&r)[NCH], int kt) const {
    const int k0 = kt * 64 + chunk * 8;  // 64 fp16 per K tile, 8 per chunk
    if (FAST) {
      // C % 8 == 0: the 8 channels of a chunk share one (r, s).
      int rr = 0, ss = 0, cc = 0;
      const bool kin = k0 < K;
      if (kin) {
        const int rs = k0 / C;
        cc = k0 - rs * C;
        rr = rs / S;
        ss = rs - rr * S;
      }
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int h = hb[j] + rr;
        const int w = wb[j] + ss;
        const bool ok = kin && img[j] >= 0 && (unsigned)h < (unsigned)H && (unsigned)w < (unsigned)W;
        const uint32_t off = ((uint32_t)(img[j] + h * W + w) * (uint32_t)C + (uint32_t)cc) * 2u;
        r[j] = buf_load16(rsrc, ok ? off : OOB);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        uint16_t e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = elem(j, k0 + i);
        uint4 v;
        __builtin_memcpy(&v, e, 16);
        r[j] = v;
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

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <int KIND, int BM, int BN, int WM, int WN, bool FAST>
__global__ void __launch_bounds__(64 * WM * WN, 1) gemm_kernel(const Params p) {
  constexpr int NT = 64 * WM * WN;
  constexpr int EB = (KIND == KIND_U8I8_GEMM) ? 1 : 2;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int A_CH = BM * 8 / NT, B_CH = BN * 8 / NT;
  constexpr int STAGE = (BM + BN) * ROW_BYTES;
  constexpr bool INT8 = KIND == KIND_U8I8_GEMM;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert((BM * 8) % NT == 0 && (BN * 8) % NT == 0, "tile rows must split evenly");
  typedef typename Mfma<KIND>::acc_t acc_t;

  constexpr int PITCH = BN + 8;  // dwords per row of the epilogue staging buffer
  constexpr int SMEM = (2 * STAGE > TM * PITCH * 4) ? 2 * STAGE : TM * PITCH * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ int sums[INT8 ? (BM + BN) : 1];

  int tm, tn;
  tile_coords<8>(p, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  typedef typename std::conditional<KIND == KIND_F16_CONV, Im2colLoader<NT, A_CH, FAST>,
                                    RowLoader<NT, A_CH, EB, FAST>>::type ALoader;
  ALoader la;
  if constexpr (KIND == KIND_F16_CONV) {
    la.init(p, m0);
  } else {
    la.init(p.A, p.lda, m0, p.M, p.K, BM);
  }
  RowLoader<NT, B_CH, EB, FAST> lb;
  lb.init(p.B, p.ldb, n0, p.N, p.K, BN);

  acc_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  // Per-lane partial sums of A' rows / B columns (u8 x i8 only).
  int rsum[FM], csum[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) rsum[i] = 0;
#pragma unroll
  for (int j = 0; j < FN; ++j) csum[j] = 0;
  const bool want_rsum = INT8 && p.zB != 0 && wn == 0;
  const bool want_csum = INT8 && p.zAp != 0 && wm == 0;

  const int nk = (p.K + (ROW_BYTES / EB) - 1) / (ROW_BYTES / EB);
  uint4 ra[A_CH], rb[B_CH];

  const int st_row = tid >> 3, st_chunk = tid & 7;
  auto store_stage = [&](int s) {
    uint8_t* As = smem + s * STAGE;
    uint8_t* Bs = As + BM * ROW_BYTES;
#pragma unroll
    for (int j = 0; j < A_CH; ++j) lds_write16(As, swz(st_row + j * (NT / 8), st_chunk), ra[j]);
#pragma unroll
    for (int j = 0; j < B_CH; ++j) lds_write16(Bs, swz(st_row + j * (NT / 8), st_chunk), rb[j]);
  };

  if (nk > 0) {
    la.load(ra, 0);
    lb.load(rb, 0);
    store_stage(0);
  }
  __syncthreads();

  const int frow = lane & 31;
  const int fhalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(ra, kt + 1);
      lb.load(rb, kt + 1);
    }
    const uint8_t* As = smem + cur * STAGE;
    const uint8_t* Bs = As + BM * ROW_BYTES;
#pragma unroll
    for (int ks = 0; ks < ROW_BYTES / 32; ++ks) {
      uint4 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        af[i] = lds_read16(As, swz(wm * TM + i * 32 + frow, ks * 2 + fhalf));
        if constexpr (INT8) {
          af[i].x ^= 0x80808080u; af[i].y ^= 0x80808080u;
          af[i].z ^= 0x80808080u; af[i].w ^= 0x80808080u;
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[j] = lds_read16(Bs, swz(wn * TN + j * 32 + frow, ks * 2 + fhalf));
      if constexpr (INT8) {
        if (want_rsum) {
#pragma unroll
          for (int i = 0; i < FM; ++i) rsum[i] = sum_bytes(af[i], rsum[i]);
        }
        if (want_csum) {
#pragma unroll
          for (int j = 0; j < FN; ++j) csum[j] = sum_bytes(bf[j], csum[j]);
        }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mfma<KIND>::run(acc[i][j], af[i], bf[j]);
    }
    if (kt + 1 < nk) store_stage(cur ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------------ epilogue
  // The accumulators are staged through LDS one wave-row at a time (row-major,
  // PITCH dwords per row), then every thread takes 4 consecutive columns of a
  // row: the int8 corrections and quantization run element-wise on them and
  // the results leave in 16-byte (fp32/int32) or 4-byte (int8) stores.
  //
  // Accumulator layout of a 32x32 MFMA tile: lane l holds column l % 32 and,
  // in register e, row 8*(e/4) + 4*(l/32) + e%4.
  const int ccol = lane & 31;
  const int rbase = 4 * (lane >> 5);
  int32_t* stage = reinterpret_cast<int32_t*>(smem);

  uint32_t kzz = 0;
  if constexpr (INT8) {
    // Complete the row / column sums (the two K halves live in lanes l, l^32)
    // and publish them through LDS.
    if (want_rsum) {
      // K-tail padding reads as byte 0, i.e. A' = -128: add those terms back.
      const int pad_fix = 128 * (nk * ROW_BYTES - p.K);
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
    kzz = (uint32_t)p.K * (uint32_t)p.zAp * (uint32_t)p.zB;
  }

  constexpr int GPR = BN / 4;           // 4-column groups per row
  constexpr int RPP = NT / GPR;         // rows per pass of the whole workgroup
  static_assert(NT % GPR == 0, "a pass must cover whole rows");
  const int lcol = (tid % GPR) * 4;
  const int col = n0 + lcol;

#pragma unroll
  for (int h = 0; h < WM; ++h) {
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            // copy the element out first: bit-casting a vector-element lvalue
            // directly reads element 0 with this compiler
            const auto val = acc[i][j][e];
            stage[(i * 32 + 8 * (e >> 2) + rbase + (e & 3)) * PITCH + wn * TN + j * 32 + ccol] =
                __builtin_bit_cast(int32_t, val);
          }
    }
    __syncthreads();
    for (int rr = tid / GPR; rr < TM; rr += RPP) {
      const int lrow = h * TM + rr;
      const int row = m0 + lrow;
      if (row < p.M && col < p.N) {
        const uint4 v = *reinterpret_cast<const uint4*>(stage + rr * PITCH + lcol);
        const bool full = col + 3 < p.N;
        if constexpr (!INT8) {
          float* dst = p.Cf + (long long)row * p.ldcf + col;
          if (full && p.vec_c) {
            *reinterpret_cast<uint4*>(dst) = v;
          } else {
            const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (col + q < p.N) dst[q] = __builtin_bit_cast(float, vv[q]);
          }
        } else {
          // C = acc' - zA'*colsum(B) - zB*rowsum(A') + K*zA'*zB in wrapping
          // 32-bit arithmetic; the true value fits in int32 (K <= 33025).
          const uint32_t rcorr = p.zB != 0 ? (uint32_t)p.zB * (uint32_t)sums[lrow] : 0u;
          const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
          int32_t c[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t ccorr =
                p.zAp != 0 ? (uint32_t)p.zAp * (uint32_t)sums[BM + min(lcol + q, BN - 1)] : 0u;
            c[q] = (int32_t)(vv[q] - ccorr - rcorr + kzz);
          }
          if (p.Ci) {
            int32_t* dst = p.Ci + (long long)row * p.ldci + col;
            if (full && p.vec_c) {
              *reinterpret_cast<int4*>(dst) = make_int4(c[0], c[1], c[2], c[3]);
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
              *reinterpret_cast<float4*>(dst) = make_float4(d[0], d[1], d[2], d[3]);
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
              *reinterpret_cast<uint32_t*>(dst) = packed;
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
