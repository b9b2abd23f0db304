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
//    re-derived for 64-wide waves and 16x16 MFMA blocks.
//  * Both operands are K-contiguous (A row-major, B column-major), so a tile
//    row is one 128-byte run: every load request is a whole cache line.
//  * Both operands go from HBM straight into LDS with buffer loads that write
//    LDS (no register staging).  The K loop is software-pipelined
//    ([TIR-COMPILER] §2.2 and §4.4): A has three LDS stages and its tile kt+2
//    is loaded during the first k-step of tile kt; B has two and its tile
//    kt+2 is loaded during the last k-step, right after the barrier that frees
//    tile kt's stage (3 x 32 + 2 x 32 KiB fill the 160 KiB LDS at 256x256).
//    The loads are spread one per MFMA row over the k-steps in program order,
//    so the address unit's queues never fill and stall the wave.  Out-of-range
//    buffer offsets read as zeros: ragged tiles, K tails and the
//    convolution's zero padding need no branches.
//  * LDS rows are 128 bytes; the 16-byte chunk c of row r sits in slot
//    c ^ ((r >> 1) & 7), so fragment reads and tile writes are free of bank
//    conflicts on the 64-bank LDS (see swz()).  This replaces the padding
//    offsets of [GEMM-TVM] §3.2 and storage_align of [TIR-PRACTICE] §2.2 with
//    the swizzle named in [TIR-COMPILER] §2.2.
//  * MFMA: v_mfma_f32_16x16x32_f16 and v_mfma_i32_16x16x64_i8.  Each lane
//    feeds 16 bytes of one row of A and 16 bytes of one column of B per
//    instruction (lane l: row/column l % 16, 16-byte chunk l / 16 of the
//    64-byte k-step).  A and B use the same (lane, element) -> k assignment,
//    so the K order inside one MFMA never matters.  On MI355X the 16x16 forms
//    hold a higher clock under the power limit than the 32x32 forms with the
//    same work per cycle.  Fragments are read one k-step ahead; the last
//    k-step's MFMAs of a tile run after the barrier, hiding the next tile's
//    reads.
//  * u8 activations on the signed i8 MFMA: A' = A - 128 = A xor 0x80 per
//    byte, applied to each A fragment just before use; the epilogue then uses
//    zA' = zA - 128 in the four-term identity of [GEMM-TVM] §2.3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>
#include <type_traits>
#include <utility>

namespace igc {

// f(std::integral_constant<int, i>()) for i = 0 .. N-1, in order.
template <class F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>()), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>());
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#ifndef IGC_MFMA_DIM
#define IGC_MFMA_DIM 16
#endif

// KIND_F16_CONV_C64: the convolution when C % 64 == 0 and R*S <= 31, so a
// K tile (64 channels) never straddles two taps and the tap is uniform.
// KIND_U8I8_CONV: the quantized convolution (u8 activations x i8 weights
// with zero points); with FAST it needs C % 128 == 0 and R*S <= 31 (uniform
// taps of 128 channels), else the element-wise im2col loader.
enum Kind : int {
  KIND_F16_GEMM = 0,
  KIND_F16_CONV = 1,
  KIND_U8I8_GEMM = 2,
  KIND_F16_CONV_C64 = 3,
  KIND_U8I8_CONV = 4
};

constexpr int KT_BYTES = 128;    // bytes of K per tile row
constexpr int CHUNK_BYTES = 16;  // one vector load
constexpr int CPR = KT_BYTES / CHUNK_BYTES;  // chunks per tile row

// n / d for 0 <= n < 2^31 and 1 <= d < 2^31 with a reciprocal formed on the
// host: m = floor(2^32 / d) + 1 (0 for d = 1).  umulhi(n, m) is n / d or one
// more; one compare corrects it.  A runtime division costs a few dozen
// instructions on the GPU, and the tile and im2col set-up of every workgroup
// needs several.
struct FastDiv {
  uint32_t d, m;
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    const uint32_t q = __umulhi(n, m);
    return m == 0 ? n : q - (q * d > n ? 1u : 0u);
  }
};

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
  FastDiv fd_pq, fd_q, fd_c, fd_s;  // divisions by P*Q, Q, C and S
  // blocked NHWCnc layout (block 16) of the conv input and output: GEMM row
  // m = ((n/16 * P + p) * Q + q) * 16 + n % 16; x[n/16][h][w][c/16][n%16][c%16],
  // y[n/16][p][q][k/16][n%16][k%16]
  int blk;
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
  const int32_t* colsum;  // optional precomputed colsum(B) (length N)
  // 16-byte (int8: 4-byte) vector stores allowed for each output
  int vec_c, vec_d, vec_q;
  // Work split.  Workgroups [0, dp_tiles) each compute one whole tile.  The
  // remaining tiles_m*tiles_n - dp_tiles tiles are shared by sk_wgs
  // workgroups as one range of sk_iters K-tile iterations (stream-K):
  // workgroup dp_tiles + g runs iterations [sk_start(g), sk_start(g+1)).  A
  // tile split between workgroups is summed through ws (two partial-tile
  // slots per stream-K workgroup) by whichever contributor finishes last, as
  // counted in cnt (one counter per stream-K tile, zero between launches).
  int dp_tiles;
  int xcd_regroup;  // regroup whole tiles by XCD (see dp_tile)
  FastDiv fd_group, fd_glast;  // tile_coords: by 8 * tiles_n, and by the last group's tile rows
  int sk_wgs;
  long long sk_iters;
  float* ws;
  int* cnt;
};

// NARROW: sk_iters * sk_wgs < 2^32 (the integer kernels: K <= 33025 keeps
// sk_iters below 2^17), so 32-bit unsigned division serves; its lowering
// uses no fused multiply-add, which the requantize epilogue must not contain.
template <bool NARROW = false>
__device__ __forceinline__ long long sk_start(const Params& p, int g) {
  if constexpr (NARROW) return (long long)((uint32_t)g * (uint32_t)p.sk_iters / (uint32_t)p.sk_wgs);
  return (long long)g * p.sk_iters / p.sk_wgs;
}
// the stream-K workgroup whose range holds iteration x
template <bool NARROW = false>
__device__ __forceinline__ int sk_owner(const Params& p, long long x) {
  if constexpr (NARROW) return (int)(((uint32_t)(x + 1) * (uint32_t)p.sk_wgs - 1u) / (uint32_t)p.sk_iters);
  return (int)(((x + 1) * p.sk_wgs - 1) / p.sk_iters);
}

// ---------------------------------------------------------------------------
// Tile scheduling.  The dispatcher hands workgroups to the 8 XCDs round-robin
// (workgroup b runs on XCD b % 8).  When the whole-tile count divides by 8
// and the grid takes more than one round of compute units,
// logical tile ids are regrouped so that each XCD owns a contiguous run of
// them, and logical tiles are laid out in groups of GROUP_M tile-rows, so the
// workgroups that share an XCD's L2 also share A and B panels.
// ---------------------------------------------------------------------------
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(const Params& p, int t, int& tm, int& tn) {
  static_assert(GROUP_M == 8, "the host forms the reciprocals for groups of 8 tile rows");
  const int group = (int)p.fd_group.div((uint32_t)t);  // t / (GROUP_M * tiles_n)
  const int first_m = group * GROUP_M;
  const int in_group = t - group * GROUP_M * p.tiles_n;
  if (p.tiles_m - first_m >= GROUP_M) {
    tm = first_m + (in_group & (GROUP_M - 1));
    tn = in_group / GROUP_M;
  } else {  // the last, partial group of tile rows
    const int q = (int)p.fd_glast.div((uint32_t)in_group);
    tm = first_m + in_group - q * (p.tiles_m - first_m);
    tn = q;
  }
}
// logical tile of whole-tile workgroup b
// (the regrouping is applied when the grid takes several rounds of compute
// units: measured on MI355X, 8192^3 int8 (four rounds) 440 -> 410-420 us
// with it, but 4096^3 fp16 (one round) 105 -> 108 us)
__device__ __forceinline__ int dp_tile(const Params& p, int b) {
  return (p.xcd_regroup && (p.dp_tiles & 7) == 0) ? (b & 7) * (p.dp_tiles >> 3) + (b >> 3) : b;
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
// Cache policy of a buffer access at device ("agent") scope: sc1.  The
// stream-K partial tiles are written and read with it; it does not by itself
// make them visible across XCDs (each has its own L2): the arrival count is
// an acquire-release atomic at device scope, which writes the L2 back before
// it and invalidates after it.
constexpr int CPOL_DEV = 16;

// A buffer descriptor, both as the compiler's resource type (for the
// compiler-visible loads) and as the four raw words (for the inline-assembly
// direct-to-LDS loads).
struct Rsrc {
  __amdgpu_buffer_rsrc_t r;
  i32x4 d;
};
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  // word 3 = 0x00020000: raw (untyped) 32-bit-dword buffer on gfx9-family GPUs.
  Rsrc x;
  x.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
  const uint64_t a = (uint64_t)(uintptr_t)base;
  x.d = i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
  return x;
}
// The direct-to-LDS load is issued from inline assembly: the compiler then
// neither reorders it (program order is the schedule) nor inserts its own,
// conservative vmcnt waits before later LDS reads (it cannot tell the stage
// arrays apart across the loop's back edge).  Every wait for these loads is
// explicit in the kernel, and so are the wait states before the load (see
// dma16s).  IGC_DMA_ASM=0 selects the compiler builtin instead.
#ifndef IGC_DMA_ASM
#define IGC_DMA_ASM 1
#endif
// Direct-to-LDS load at byte offset off + soff (both range-checked against
// the descriptor's size: past it, the lanes read zeros).
// One wait state: the compiler writes M0 with a scalar instruction right
// before the asm, and an LDS-DMA load may read M0 one wait state after a
// scalar write.  A vector memory instruction may read an SGPR written by a
// VALU instruction (v_readfirstlane, v_readlane) only five wait states
// later; the compiler cannot see that this asm reads its operands, so
// tests/test_isa.py checks every shipped kernel's assembly for a VALU write
// of an operand SGPR (descriptor, offset, M0) within the five wait states
// before each of these loads.  Each wait state costs the wave an issue slot
// (4 clocks): with five, the load sequence outlasted the 16-clock MFMA it
// sits between and the matrix pipe idled.
// The loads of the main loop take NOPS = 0 (one wait state); the prologue's,
// where the compiler restores spilled scalar registers with v_readlane right
// before them, take NOPS = 4 (five).
constexpr int NOPS_LOOP = 0, NOPS_SAFE = 4;
template <int NOPS>
__device__ __forceinline__ void dma16s(const Rsrc& r, uint8_t* lds, uint32_t off, uint32_t soff) {
  static_assert(NOPS == NOPS_LOOP || NOPS == NOPS_SAFE, "wait states");
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  if constexpr (NOPS == NOPS_SAFE)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 : : "v"(off), "s"(r.d), "s"(soff), "{m0}"(m0) : "memory");
  else
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 : : "v"(off), "s"(r.d), "s"(soff), "{m0}"(m0) : "memory");
}
template <int NOPS>
__device__ __forceinline__ void dma16(const Rsrc& r, uint8_t* lds, uint32_t off) {
  static_assert(NOPS == NOPS_LOOP || NOPS == NOPS_SAFE, "wait states");
  if constexpr (IGC_DMA_ASM) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
    if constexpr (NOPS == NOPS_SAFE)
      asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(off), "s"(r.d), "{m0}"(m0) : "memory");
    else
      asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(off), "s"(r.d), "{m0}"(m0) : "memory");
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r.r, (__attribute__((address_space(3))) void*)lds, 16, (int)off, 0, 0, 0);
  }
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
  // the same with the wave's offset (wave_id() * 1024) computed once
  __device__ static __forceinline__ uint8_t* dst(uint8_t* tile, int i, uint32_t wofs) {
    return tile + i * NWAVES * 1024 + wofs;
  }
  __device__ static __forceinline__ uint32_t wave_offset() { return (uint32_t)wave_id() * 1024u; }
};

// Operand loaded straight into LDS (A of the fp16 GEMM; the i8 B of the
// u8 x i8 GEMM): rows of K.
//  FAST: 16-byte aligned rows, K a multiple of the chunk: direct-to-LDS loads.
//  else: element-wise loads, written to LDS with the same layout.
//  TAIL_FIRST (FAST only): the partial K tile, if any, is tile 0 -- it holds
//  bytes [0, t) of each row, t = K*EB - 128*(nk-1) -- and tile kt >= 1 holds
//  bytes [t + 128*(kt-1), t + 128*kt).  Only tile 0 then needs a per-lane K
//  bound; every later load is one scalar offset (the K position) away from
//  one of this lane's fixed offsets (one per row group), with no vector
//  arithmetic.  Otherwise tile kt holds bytes
//  [128*kt, 128*kt + 128) and the K tail is masked in the last tile.  The
//  two operands of a kernel must use the same order.
//  WHOLE_K (FAST, K tiles walked in order, K * EB a multiple of 128: no
//  partial tile): like TAIL_FIRST, every load is one of this lane's fixed
//  offsets plus a scalar K offset.
template <int NT, int ROWS, int EB, bool FAST, bool TAIL_FIRST = false, bool WHOLE_K = false>
struct RowDmaLoader {
  static_assert(!(TAIL_FIRST && WHOLE_K), "one K walk");
  static constexpr bool SCALAR_K = FAST && (TAIL_FIRST || WHOLE_K);
  typedef DmaShape<NT, ROWS> Sh;
  const uint8_t* base;  // row 0 of this tile
  long long ld_bytes;
  int rows_valid;       // rows of this tile that exist
  int K;
  Rsrc rsrc;
  uint32_t lane_off;    // byte offset of this lane's first row and chunk
  uint32_t lane_off0;   // same, or OOB past the K bound of tile 0 (TAIL_FIRST)
  uint32_t row_step;    // bytes between this lane's rows (uniform)
  int kpad;             // 128 * nk - K * EB: zero bytes in the partial tile
  int nk;               // K tiles
  uint32_t voff[SCALAR_K ? Sh::NQ : 1];  // lane_off + i * row_step (scalar K offsets)
  uint32_t wofs;        // this wave's offset in a tile's LDS rows

  __device__ __forceinline__ void init(const uint8_t* ptr, long long ld, int r0, int nrows, int k) {
    wofs = Sh::wave_offset();
    ld_bytes = ld * EB;
    base = ptr + (long long)r0 * ld_bytes;
    rows_valid = nrows - r0;
    K = k;
    if (FAST) {
      const long long extent = (long long)min(rows_valid, ROWS) * ld_bytes;
      rsrc = make_rsrc(base, (uint32_t)extent);
      lane_off = (uint32_t)(Sh::lane_row() * ld_bytes) + (uint32_t)(Sh::lane_chunk() * CHUNK_BYTES);
      row_step = (uint32_t)(8 * Sh::NWAVES * ld_bytes);
      nk = max(1, (K * EB + KT_BYTES - 1) / KT_BYTES);
      kpad = nk * KT_BYTES - K * EB;
      lane_off0 = Sh::lane_chunk() * CHUNK_BYTES < KT_BYTES - kpad ? lane_off : OOB;
      if constexpr (SCALAR_K) {
#pragma unroll
        for (int i = 0; i < Sh::NQ; ++i) voff[i] = lane_off + (uint32_t)(i * row_step);
      }
    }
  }

  // Loading K tile kt into `tile` (ROWS x 128 bytes, swizzled) takes NPART
  // calls part(tile, kt, i), i = 0..NPART-1, then advance(); rows past the
  // operand and k past K read as zero bytes.  FAST: part i is one
  // direct-to-LDS load of 8 rows per wave; else part 0 does it all.
  // TAIL_FIRST: part() serves tiles kt >= 1 and part0() tile 0.
  static constexpr int NPART = FAST ? Sh::NQ : 1;
  __device__ __forceinline__ void advance() const {}
  template <int NOPS = NOPS_LOOP>
  __device__ __forceinline__ void load(uint8_t* tile, int kt) const {
#pragma unroll
    for (int i = 0; i < NPART; ++i) {
      if (TAIL_FIRST && kt == 0)
        part0<NOPS>(tile, i);
      else
        part<NOPS>(tile, kt, i);
    }
  }
  template <int NOPS = NOPS_LOOP>
  __device__ __forceinline__ void part0(uint8_t* tile, int i) const {
    dma16s<NOPS>(rsrc, Sh::dst(tile, i, wofs), lane_off0, (uint32_t)(i * row_step));
  }
  template <int NOPS = NOPS_LOOP>
  __device__ __forceinline__ void part(uint8_t* tile, int kt, int i) const {
    if constexpr (SCALAR_K) {
      // tiles past K (prefetched by the pipeline, never multiplied) read
      // out of range: zeros, no memory traffic (kpad = 0 without a tail)
      dma16s<NOPS>(rsrc, Sh::dst(tile, i, wofs), voff[i], kt < nk ? (uint32_t)(kt * KT_BYTES - kpad) : OOB);
    } else if (FAST) {
      const bool kin = kt * KT_BYTES + Sh::lane_chunk() * CHUNK_BYTES < K * EB;
      dma16<NOPS>(rsrc, Sh::dst(tile, i, wofs), kin ? lane_off + (uint32_t)(i * row_step + kt * KT_BYTES) : OOB);
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

// Implicit im2col view of an NHWC fp16 input (the conv's A operand): row
// m = (n, p, q), column k = (r*S + s)*C + c holds
// x[n, p*sh + r - ph, q*sw + s - pw, c], or 0 where that position lies in the
// zero padding ([CONV-TC] "Preparation and algorithm": Apad is inlined, the
// padding predicate is evaluated inside the shared-memory fill).  (n, p, q)
// is decoded once per row at kernel start.  FAST (C % 8 == 0): the 8 channels
// of a chunk share one tap (r, s); each lane tracks the (r, s, c) of its chunk
// and advances it by the 64 channels of one K tile.
// EB = 1 (u8 activations, element-wise only): the padding holds the zero
// point zA, the code of the real value 0, instead of 0.
template <int NT, int ROWS, bool FAST, int EB = 2>
struct Im2colLoader {
  static_assert(EB == 2 || !FAST, "u8 activations take the element-wise or the uniform-tap loader");
  typedef DmaShape<NT, ROWS> Sh;
  static constexpr int NR = FAST ? Sh::NQ : ROWS * CPR / NT;  // rows per lane
  const uint8_t* x;
  int pix[NR];  // pixel index in x of (n, p*sh - ph, q*sw - pw), i.e. of tap (0, 0)
  int hw[NR];   // (p*sh - ph) << 16 | (q*sw - pw) & 0xffff; INT32_MIN for rows past M
  int H, W, C, S, K;
  FastDiv fd_c, fd_s;
  uint8_t padv;  // u8 padding value (zA)
  Rsrc rsrc;
  // tap of this lane's chunk for the next K tile to be loaded (FAST)
  mutable int cur_r, cur_s, cur_c;

  __device__ __forceinline__ int row_h(int j) const { return hw[j] >> 16; }
  __device__ __forceinline__ int row_w(int j) const { return (int)(int16_t)(hw[j] & 0xffff); }

  // blocked layout (fp16 only): element (pixel, channel c) of row j sits at
  // pixel * 16C + (c / 16) * 256 + nn_j * 16 + c % 16 (nnoff[j] = nn_j * 16)
  static constexpr bool BLK_OK = EB == 2;
  int blk;
  int nnoff[BLK_OK ? NR : 1];
  __device__ __forceinline__ long long elem_index(int j, int pixel, int c) const {
    if constexpr (BLK_OK) {
      if (blk) return (long long)pixel * (16 * C) + ((c >> 4) << 8) + nnoff[j] + (c & 15);
    }
    return (long long)pixel * C + c;
  }

  uint32_t wofs;  // this wave's offset in a tile's LDS rows

  __device__ __forceinline__ void init(const Params& p, int m0, int kt0) {
    x = p.A;
    wofs = Sh::wave_offset();
    H = p.H; W = p.W; C = p.C; S = p.S; K = p.K;
    blk = BLK_OK ? p.blk : 0;
    padv = (uint8_t)(p.zAp + 128);
    if (FAST) rsrc = make_rsrc(x, (uint32_t)((long long)p.Nb * H * W * C * 2));
    const int PQ = p.P * p.Q;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int r = FAST ? Sh::lane_row() + j * 8 * Sh::NWAVES : (int)(threadIdx.x >> 3) + j * (NT / 8);
      const int m = m0 + r;
      if constexpr (BLK_OK) nnoff[j] = 0;
      if (m < p.M) {
        // NHWC: m = (n*P + p)*Q + q; blocked: m = ((n16*P + p)*Q + q)*16 + nn, the
        // pixel index then counting 16-image groups
        const int g = blk ? (m >> 4) : m;
        if constexpr (BLK_OK) {
          if (blk) nnoff[j] = (m & 15) << 4;
        }
        const int n = (int)p.fd_pq.div((uint32_t)g);
        const int pq = g - n * PQ;
        const int pp = (int)p.fd_q.div((uint32_t)pq);
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
    // tap of k = chunk*8 of K tile kt0
    const int k0 = FAST ? kt0 * 64 + Sh::lane_chunk() * 8 : 0;
    const int rs = (int)p.fd_c.div((uint32_t)k0);
    cur_c = k0 - rs * C;
    cur_r = (int)p.fd_s.div((uint32_t)rs);
    cur_s = rs - cur_r * S;
    fd_c = p.fd_c;
    fd_s = p.fd_s;
  }

  __device__ __forceinline__ uint16_t elem(int j, int k) const {
    if (hw[j] == INT32_MIN || k >= K) return 0;
    const int rs = (int)fd_c.div((uint32_t)k);
    const int c = k - rs * C;
    const int r = (int)fd_s.div((uint32_t)rs);
    const int s = rs - r * S;
    const int h = row_h(j) + r;
    const int w = row_w(j) + s;
    if ((unsigned)h >= (unsigned)H || (unsigned)w >= (unsigned)W) return 0;
    return reinterpret_cast<const uint16_t*>(x)[elem_index(j, pix[j] + r * W + s, c)];
  }
  // u8: past K (and rows past M) 0, like the row operands' K tail; padding zA
  __device__ __forceinline__ uint8_t elem8(int j, int k) const {
    if (hw[j] == INT32_MIN || k >= K) return 0;
    const int rs = (int)fd_c.div((uint32_t)k);
    const int c = k - rs * C;
    const int r = (int)fd_s.div((uint32_t)rs);
    const int s = rs - r * S;
    const int h = row_h(j) + r;
    const int w = row_w(j) + s;
    if ((unsigned)h >= (unsigned)H || (unsigned)w >= (unsigned)W) return padv;
    return x[elem_index(j, pix[j] + r * W + s, c)];
  }

  // Loading K tile kt takes NPART calls part(tile, kt, j) and then
  // advance().  FAST: K tiles must be loaded in order 0, 1, 2, ... (advance()
  // moves this lane's tap on by the 64 channels of one K tile); part j is one
  // direct-to-LDS load of 8 rows per wave.  Else part 0 does it all.
  static constexpr int NPART = FAST ? Sh::NQ : 1;
  template <int NOPS = NOPS_LOOP>
  __device__ __forceinline__ void load(uint8_t* tile, int kt) const {
#pragma unroll
    for (int j = 0; j < NPART; ++j) part<NOPS>(tile, kt, j);
    advance();
  }
  __device__ __forceinline__ void advance() const {
    if (FAST) {
      cur_c += 64;
      while (cur_c >= C) {
        cur_c -= C;
        if (++cur_s == S) {
          cur_s = 0;
          ++cur_r;
        }
      }
    }
  }
  template <int NOPS = NOPS_LOOP>
  __device__ __forceinline__ void part(uint8_t* tile, int kt, int j) const {
    if (FAST) {
      const bool kin = kt * 64 + Sh::lane_chunk() * 8 < K;
      const int tap = cur_r * W + cur_s;
      const int h = row_h(j) + cur_r;  // rows past M have h < -16000: never in range
      const int w = row_w(j) + cur_s;
      const bool ok = kin && (unsigned)h < (unsigned)H && (unsigned)w < (unsigned)W;
      // (a chunk's 8 channels lie in one 16-channel block: cur_c % 8 == 0)
      const uint32_t off = (uint32_t)elem_index(j, pix[j] + tap, cur_c) * 2u;
      dma16<NOPS>(rsrc, Sh::dst(tile, j, wofs), ok ? off : OOB);
    } else if constexpr (EB == 2) {
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
    } else {
      const int c = threadIdx.x & 7;
      const int k0 = kt * 128 + c * 16;
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const int row = (threadIdx.x >> 3) + j * (NT / 8);
        uint8_t e[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) e[i] = elem8(j, k0 + i);
        uint4 v;
        __builtin_memcpy(&v, e, 16);
        lds_write16(tile, swz(row, c), v);
      }
    }
  }
};

// Convolution output row g = (n, p, q): its image n and the input position
// (h0, w0) of tap (0, 0).
__device__ __forceinline__ void conv_row(const Params& p, int g, int& n, int& h0, int& w0) {
  n = (int)p.fd_pq.div((uint32_t)g);
  const int pq = g - n * (p.P * p.Q);
  const int pp = (int)p.fd_q.div((uint32_t)pq);
  const int qq = pq - pp * p.Q;
  h0 = pp * p.sh - p.ph;
  w0 = qq * p.sw - p.pw;
}
// One bit at r*S for every filter row r.
__device__ __forceinline__ uint32_t conv_tap_rows(const Params& p) {
  uint32_t rep = 0;
  for (int r = 0; r < p.R; ++r) rep |= 1u << (r * p.S);
  return rep;
}
// Bit r*S + s set where tap (r, s) of the output row whose tap (0, 0) is at
// (h0, w0) lies inside the image (R*S <= 31): r in [r_lo, r_hi], s in
// [s_lo, s_hi], the product of a column run (bits s_lo .. s_hi) and one bit
// at r*S per row of the row run (no carries).
__device__ __forceinline__ uint32_t conv_tap_mask(const Params& p, int h0, int w0, uint32_t rep) {
  const int r_lo = max(0, -h0), r_hi = min(p.R - 1, p.H - 1 - h0);
  const int s_lo = max(0, -w0), s_hi = min(p.S - 1, p.W - 1 - w0);
  // (shift counts clamped to 31: a window wholly in the padding has
  // r_lo > r_hi or s_lo > s_hi, and its mask is 0)
  const uint32_t cols = (2u << min(max(s_hi, 0), 30)) - (1u << min(s_lo, 31));
  const uint32_t rows = rep & ((2u << min(max(r_hi, 0) * p.S, 30)) - (1u << min(r_lo * p.S, 31)));
  return (r_lo <= r_hi && s_lo <= s_hi) ? rows * cols : 0u;
}

// The implicit-im2col A operand when a K tile (128 bytes: 64 fp16 or 128 u8
// channels) always lies in one tap: C a multiple of it and R*S <= 31 (FAST
// only).  The tap (r, s) is then the same for all lanes, so the tap walk is
// scalar.  A row's input pixel is a fixed per-lane offset from a fixed
// buffer base (x moved back by the padding's offset, so every offset is
// non-negative); the K tile's position, ((r*W + s)*C + c) elements, is the
// load's scalar offset.  In NHWC that position grows by 128 bytes per K tile
// (tap (r, s+1) channel 0 follows tap (r, s) channel C-1 in memory), plus
// (W - S)*C elements when the walk moves to the next filter row, so a K tile
// costs a few scalar additions.  Each row keeps a bit mask of its taps that
// fall in the zero padding; once per tap the per-lane offset
// becomes OOB where the tap is padding, so that lane's load reads zeros.
// The buffer spans 2^31 bytes (OOB): valid offsets stay below it (the host
// checks that x plus the padding's offset, and the largest scalar offset, fit
// in 2^31 bytes).  u8 activations: the padding must hold the zero point zA;
// the kernel turns the zero rows into zA - 128 when it converts fragments to
// signed bytes (see gemm_kernel).
template <int NT, int ROWS, int EB = 2>
struct Im2colC64Loader {
  typedef DmaShape<NT, ROWS> Sh;
  static constexpr int NPART = Sh::NQ;
  static constexpr int CPT = KT_BYTES / EB;  // channels per K tile
  Rsrc rsrc;            // x moved back by the padding's offset, 2^31 bytes
  int C, S, RS;
  uint32_t pixb[Sh::NQ];  // (pixel of tap (0,0) + ph*W + pw) * C * EB + chunk * 16
  uint32_t pad[Sh::NQ];   // bit r*S+s: tap (r, s) of this row is padding (all set past M)
  mutable uint32_t vo[Sh::NQ];  // pixb, or OOB where the current tap is padding
  mutable int vo_tap;           // the tap vo[] was formed for
  mutable int cur_tap, cur_s, cur_c;  // tap r*S + s, s and channel of the next K tile
  mutable uint32_t soff;        // scalar offset of the next K tile: ((r*W + s)*C + c)*EB
  uint32_t step, row_jump;      // soff per K tile; extra soff when s wraps
  // blocked NHWCnc input (fp16 only): every pixel and channel offset is 16
  // times its NHWC value (16 images interleaved), plus the row's image within
  // its group of 16 and the chunk's place in a 16-channel block
  int blk_shift;                // 4 blocked, 0 NHWC
  uint32_t wofs;                // this wave's offset in a tile's LDS rows

  // Output row m's entry in the tile's row table: the byte offset of its
  // tap (0, 0) pixel from the buffer base, and its tap mask; zeros past M
  // (no tap inside: every load of the row reads zeros).  rep: conv_tap_rows.
  // Branch-free: the values it reads from the parameters must not become
  // results of a divergent branch (the scalar K walk uses them).
  __device__ static __forceinline__ uint2 row_entry(const Params& p, int m, uint32_t rep) {
    const bool in = m < p.M;
    m = in ? m : p.M - 1;
    const int bs = (EB == 2 && p.blk) ? 4 : 0;
    int n, h0, w0;
    conv_row(p, bs ? (m >> 4) : m, n, h0, w0);
    const int p0 = p.ph * p.W + p.pw;
    const uint32_t nn_off = bs ? (uint32_t)((m & 15) * 16 * EB) : 0u;
    const uint32_t pix = ((uint32_t)((n * p.H * p.W + h0 * p.W + w0 + p0) * p.C * EB) << bs) + nn_off;
    const uint32_t mk = conv_tap_mask(p, h0, w0, rep);
    return make_uint2(in ? pix : 0u, in ? mk : 0u);
  }
  // rows: the tile's row table (row_entry of rows m0 .. m0 + ROWS - 1)
  __device__ __forceinline__ void init(const Params& p, const uint2* rows, int kt0) {
    wofs = Sh::wave_offset();
    C = p.C; S = p.S; RS = p.R * p.S;
    const int p0 = p.ph * p.W + p.pw;
    blk_shift = (EB == 2 && p.blk) ? 4 : 0;
    rsrc = make_rsrc((const void*)((uintptr_t)p.A - ((uintptr_t)p0 * C * EB << blk_shift)), OOB);
    step = (uint32_t)(KT_BYTES << blk_shift);
    row_jump = (uint32_t)(((long long)(p.W - S) * C * EB) << blk_shift);
    // chunk c of a 128-byte K-tile row (channels 8c .. 8c+7 of the tile):
    // byte 16c (NHWC), or 512 (c / 2) + 16 (c % 2) in the blocked layout
    const int ch = Sh::lane_chunk();
    const uint32_t chunk_off = blk_shift ? (uint32_t)((ch >> 1) * 512 + (ch & 1) * 16) : (uint32_t)(ch * CHUNK_BYTES);
#pragma unroll
    for (int j = 0; j < Sh::NQ; ++j) {
      const uint2 e = rows[Sh::lane_row() + j * 8 * Sh::NWAVES];
      pixb[j] = e.x + chunk_off;
      pad[j] = ~e.y;
    }
    const int k = kt0 * CPT;
    const int rs = (int)p.fd_c.div((uint32_t)k);
    cur_c = k - rs * C;
    cur_tap = rs;
    const int r = (int)p.fd_s.div((uint32_t)rs);
    cur_s = rs - r * S;
    soff = (uint32_t)((((long long)(r * p.W + cur_s) * C + cur_c) * EB) << blk_shift);
    vo_tap = -1;
  }
  __device__ __forceinline__ void advance() const {
    cur_c += CPT;
    soff += step;
    if (cur_c == C) {
      cur_c = 0;
      ++cur_tap;
      if (++cur_s == S) {
        cur_s = 0;
        soff += row_jump;
      }
    }
  }
  // the per-row offsets of the current tap, formed once per tap (a tap
  // spans C / CPT K tiles) instead of once per load
  __device__ __forceinline__ void retap(int tap) const {
    if (tap != vo_tap) {
      // tiles past the last tap (prefetch beyond K) use bit 31, never set
      const int bit = tap < RS ? tap : 31;
#pragma unroll
      for (int j = 0; j < Sh::NQ; ++j) {
        // m = -1 where the tap is padding, 0 inside; then a bit-field insert.
        // (The compare-and-select form serialized the rows on VCC, with the
        // matrix pipe idle, once per tap.)
        const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)pad[j], bit, 1);
        vo[j] = (pixb[j] & ~m) | (OOB & m);
      }
      vo_tap = tap;
    }
  }
  template <int NOPS = NOPS_LOOP>
  __device__ __forceinline__ void load(uint8_t* tile, int kt) const {
#pragma unroll
    for (int j = 0; j < NPART; ++j) part<NOPS>(tile, kt, j);
    advance();
  }
  template <int NOPS = NOPS_LOOP>
  __device__ __forceinline__ void part(uint8_t* tile, int, int j) const {
    retap(cur_tap);
    dma16s<NOPS>(rsrc, Sh::dst(tile, j, wofs), vo[j], soff);
  }
};

// ---------------------------------------------------------------------------
// MFMA wrappers.  One call = one 32 x 32 output tile, 32 bytes of K per row.
// ---------------------------------------------------------------------------
template <int KIND, int MB>
struct Mfma;

template <>
struct Mfma<KIND_F16_GEMM, 32> {
  typedef f32x16 acc_t;
  __device__ __forceinline__ static void run(acc_t& c, uint4 a, uint4 b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                               __builtin_bit_cast(half8, b), c, 0, 0, 0);
  }
};
template <>
struct Mfma<KIND_F16_GEMM, 16> {
  typedef f32x4 acc_t;
  __device__ __forceinline__ static void run(acc_t& c, uint4 a, uint4 b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                               __builtin_bit_cast(half8, b), c, 0, 0, 0);
  }
};
template <int MB>
struct Mfma<KIND_F16_CONV, MB> : Mfma<KIND_F16_GEMM, MB> {};
template <int MB>
struct Mfma<KIND_F16_CONV_C64, MB> : Mfma<KIND_F16_GEMM, MB> {};
template <int MB>
struct Mfma<KIND_U8I8_CONV, MB> : Mfma<KIND_U8I8_GEMM, MB> {};
template <>
struct Mfma<KIND_U8I8_GEMM, 32> {
  typedef i32x16 acc_t;
  __device__ __forceinline__ static void run(acc_t& c, uint4 a, uint4 b) {
    c = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                              __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
  }
};
template <>
struct Mfma<KIND_U8I8_GEMM, 16> {
  typedef i32x4 acc_t;
  __device__ __forceinline__ static void run(acc_t& c, uint4 a, uint4 b) {
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                              __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
  }
};

// The requantize step's rounding and saturation of y to int8: clamping y to
// [-128, 127] first gives the same result (the bounds are integers and
// rounding is monotonic); adding 1.5 * 2^23 then rounds in fp32 to the
// nearest integer, ties to even, and leaves that integer in two's
// complement in the low mantissa bits: the int8 value is the low byte of
// the sum's bit pattern.  (Two operations instead of a rounding, a clamp and
// a conversion.)
__device__ __forceinline__ uint32_t requant_bits(float y) {
  const float v = fminf(fmaxf(y, -128.f), 127.f);
  return __builtin_bit_cast(uint32_t, v + 12582912.0f);
}

// requant_bits with the int8 code written straight into byte Q of `packed`:
// the rounding add as an SDWA instruction whose destination select takes the
// sum's low byte (byte 0 zeroes the other bytes, bytes 1-3 keep them), so
// four codes are packed by their own rounding adds, without byte permutes.
template <int Q>
__device__ __forceinline__ void requant_byte(uint32_t& packed, float y) {
  static_assert(Q >= 0 && Q < 4, "byte");
  const float v = fminf(fmaxf(y, -128.f), 127.f);
  const float magic = 12582912.0f;
  if constexpr (Q == 0)
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD"
        : "=v"(packed) : "v"(magic), "v"(v));
  else if constexpr (Q == 1)
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(packed) : "v"(magic), "v"(v));
  else if constexpr (Q == 2)
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(packed) : "v"(magic), "v"(v));
  else
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(packed) : "v"(magic), "v"(v));
}

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
  // The waitcnt and barrier builtins do not order memory accesses for the
  // compiler (they are "no memory" intrinsics): empty asm statements with a
  // memory clobber keep LDS reads and writes on their side of them.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

// Workgroup barrier without a memory fence (a fence would wait for every
// direct-to-LDS load in flight); pair it with wait_vmcnt_lgkm0.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One scalar load per 64-byte line of the kernel's parameters, issued
// together at entry: the later loads of them (set-up, epilogue) then hit the
// scalar cache instead of waiting out one miss after another (measured on
// the 1024^3 u8 x i8 GEMM: 6.85 -> 6.44 us).
__device__ __forceinline__ void touch_params(const Params& p) {
  constexpr int NL = (int)((sizeof(Params) + 63) / 64);
  const uint32_t* const w = reinterpret_cast<const uint32_t*>(&p);
  uint32_t t[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) t[i] = w[16 * i];
#pragma unroll
  for (int i = 0; i < NL; ++i) asm volatile("" : : "s"(t[i]));
}

// ---------------------------------------------------------------------------
// The kernel.
//  VAR (u8 x i8 only): the zero-point sums the mainloop accumulates, a mask
//  of SUM_ROWS (rowsum(A'), needed when zB != 0) and SUM_COLS (colsum(B),
//  needed when zA != 128), each compiled only into the kernels that use it;
//  plus REQ_TILES when every tile of the launch is whole, requantized int8
//  is the only output and no tile is split: the epilogue is then compiled
//  with its requantize-in-registers path alone (with the staged path beside
//  it, the 256-column integer tiles spill registers).  fp16 convolution:
//  BLK_OUT writes the output in the blocked NHWCnc layout (the launch's
//  p.blk), so the row-major kernels carry no blocked code.  u8 x i8:
//  COLS_IN (with REQ_TILES) takes colsum(B) from p.colsum instead of forming
//  it in the K loop (SUM_COLS then not set).  NO_SPLIT compiles the kernel
//  without the stream-K code, for launches whose tiles are all whole (the
//  split code, never run there, cost them 1-12%: the 4096^3 fp16 GEMM
//  104.9 -> 103.6 us, the 256x14x14 conv 109.5 -> 105.6 us, the 1024^3
//  u8 x i8 GEMM 6.44 -> 5.67 us).
//  DEPTH: K tiles in flight ahead of the one being multiplied.  A has
//  DEPTH + 1 LDS stages; B has 2 at DEPTH 2 (the 160 KiB of LDS at 256 x 256)
//  and DEPTH + 1 otherwise.  Every launch uses DEPTH 2: deeper rings for the
//  small tiles of short K loops (up to 7 tiles ahead) measured no faster on
//  MI355X, whose small launches are bound by fixed costs and a low clock,
//  not by load latency.
// ---------------------------------------------------------------------------
constexpr int SUM_ROWS = 1, SUM_COLS = 2, REQ_TILES = 4, BLK_OUT = 8, COLS_IN = 16, NO_SPLIT = 32;
template <int KIND, int BM, int BN, int WM, int WN, bool FAST, int VAR = 0, int DEPTH = 2>
__global__ void __launch_bounds__(64 * WM * WN, 1) gemm_kernel(const Params p) {
  touch_params(p);
  constexpr int SUMS = VAR & (SUM_ROWS | SUM_COLS);
  constexpr bool REQ = (VAR & REQ_TILES) != 0;
  constexpr bool BLKO = (VAR & BLK_OUT) != 0;
  constexpr bool CIN = (VAR & COLS_IN) != 0;
  constexpr int NT = 64 * WM * WN;
  constexpr bool INT8 = KIND == KIND_U8I8_GEMM || KIND == KIND_U8I8_CONV;
  constexpr int EB = INT8 ? 1 : 2;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int MB = IGC_MFMA_DIM;          // MFMA output block: MB x MB
  constexpr int FM = TM / MB, FN = TN / MB;
  constexpr int NE = MB * MB / 64;          // accumulator elements per lane
  constexpr int LPR = 64 / MB;              // lanes sharing one row of a fragment
  constexpr int SA = BM * KT_BYTES, SB = BN * KT_BYTES;  // stage sizes
  // The A stage arrays also stage 32 output rows of BN fp32/int32 each in
  // the epilogue, so a tile with BM < BN allocates them at that size.
  constexpr int SA_ALLOC = SA > 32 * BN * 4 ? SA : 32 * BN * 4;
  // stream-K (shared tiles): compiled for the fp16 kinds and for the integer
  // kinds' aligned tiles of at most 128 rows (the wider integer tiles use
  // every register); the host splits only where it is compiled
  constexpr bool SK = (VAR & NO_SPLIT) == 0 && (INT8 ? (BM <= 128 && FAST && !REQ) : (SUMS == 0));
  static_assert(!REQ || (INT8 && FAST), "whole requantize-only tiles: the aligned integer kernels");
  static_assert(!BLKO || !INT8, "blocked output: the fp16 convolution");
  static_assert(!CIN || (REQ && (SUMS & SUM_COLS) == 0), "precomputed column sums: whole requantize-only tiles");
  // (the im2col operand walks K in order, so the conv's B does too)
  constexpr bool CONV = KIND == KIND_F16_CONV || KIND == KIND_F16_CONV_C64 || KIND == KIND_U8I8_CONV;
  // u8 activations through the uniform-tap loader (padded rows arrive as
  // zeros and become zA - 128 in the fragment conversion)
  constexpr bool U8_UNIFORM_TAPS = KIND == KIND_U8I8_CONV && FAST;
  // the uniform-tap loaders read their rows' im2col data from a table
  constexpr bool ROW_TABLE = KIND == KIND_F16_CONV_C64 || U8_UNIFORM_TAPS;
  constexpr bool TAIL_FIRST = FAST && !CONV;
  typedef typename std::conditional<
      KIND == KIND_F16_CONV_C64 || U8_UNIFORM_TAPS, Im2colC64Loader<NT, BM, EB>,
      typename std::conditional<KIND == KIND_F16_CONV || KIND == KIND_U8I8_CONV, Im2colLoader<NT, BM, FAST, EB>,
                                RowDmaLoader<NT, BM, EB, FAST, TAIL_FIRST>>::type>::type ALoader;
  static_assert(KIND != KIND_F16_CONV_C64 || FAST, "the uniform-tap conv loader needs aligned operands");
  // the uniform-tap convolutions walk K in order with whole K tiles (C a
  // multiple of the tile's channels)
  constexpr bool WHOLE_K = KIND == KIND_F16_CONV_C64 || U8_UNIFORM_TAPS;
  typedef RowDmaLoader<NT, BN, EB, FAST, TAIL_FIRST, WHOLE_K> BLoader;
  // direct-to-LDS loads per K tile per wave (counted by vmcnt); the
  // element-wise path of unaligned operands is waited for as it goes
  constexpr int NLA = FAST ? ALoader::NPART : 0;
  constexpr int NLB = FAST ? BLoader::NPART : 0;
  static_assert(TM % MB == 0 && TM % 16 == 0 && TN % 32 == 0, "wave tile must be whole MFMA blocks");
  static_assert(TM <= 128, "epilogue staging reuses the stage arrays (at most four 32-row arrays)");
  static_assert(DEPTH >= 2 && (DEPTH == 2 || FAST), "deep pipelines need the direct-to-LDS loaders");
  static_assert((DEPTH - 1) * (NLA + NLB) < 64, "vmcnt range");
  typedef typename Mfma<KIND, MB>::acc_t acc_t;

  // LDS stage rings (DEPTH 2: A in 3 stages, B in 2, 160 KiB at 256 x 256);
  // the loop below is unrolled over UNR tiles so every stage is a
  // compile-time LDS address.
  constexpr int RA = DEPTH + 1, RB = DEPTH == 2 ? 2 : DEPTH + 1;
  constexpr int UNR = RA == RB ? RA : RA * RB;
  static_assert(RA >= 3 && RB >= 2, "the epilogue stages through A stages 0-2 and B stages 0-1");
  __shared__ __attribute__((aligned(16))) uint8_t sa_ring[RA][SA_ALLOC];
  __shared__ __attribute__((aligned(16))) uint8_t sb_ring[RB][SB];
  uint8_t* const sa0 = sa_ring[0];
  uint8_t* const sa1 = sa_ring[1];
  uint8_t* const sa2 = sa_ring[2];
  uint8_t* const sb0 = sb_ring[0];
  uint8_t* const sb1 = sb_ring[1];
  auto stA = [&](auto U) -> uint8_t* { return sa_ring[decltype(U)::value % RA]; };
  auto stB = [&](auto U) -> uint8_t* { return sb_ring[decltype(U)::value % RB]; };

  // (K = 0 still runs one all-zero K tile, so the outputs are written)
  const int nk = max(1, (p.K * EB + KT_BYTES - 1) / KT_BYTES);

  // This workgroup's K-tile iterations: one whole tile, or a stream-K range
  // that may start and end inside tiles.  It is walked in segments of one
  // tile each.
  long long it, it_end;
  const bool whole = (int)blockIdx.x < p.dp_tiles;
  const int t_whole = whole ? dp_tile(p, blockIdx.x) : 0;
  if (whole) {
    it = (long long)t_whole * nk;
    it_end = it + nk;
  } else {
    const int g = blockIdx.x - p.dp_tiles;
    const long long base = (long long)p.dp_tiles * nk;
    it = base + sk_start<INT8>(p, g);
    it_end = base + sk_start<INT8>(p, g + 1);
  }
  bool first_seg = true;
  while (it < it_end) {
  // The thread and wave indices pass through an empty asm each segment, so
  // the compiler cannot hoist the many lane-dependent LDS addresses (fragment
  // reads, epilogue staging) out of this loop and keep them live across the
  // whole K loop.
  int tid_v = threadIdx.x;
  asm volatile("" : "+v"(tid_v));
  int wave_s = wave_id();
  asm volatile("" : "+s"(wave_s));
  const int tid = tid_v;
  const int lane = tid & 63;
  const int wave = wave_s;
  const int wm = wave / WN, wn = wave % WN;
  // (a whole-tile workgroup's one segment is its tile; no division)
  const int t = (!SK || whole) ? t_whole : (int)(it / nk);
  const int k0 = (!SK || whole) ? 0 : (int)(it - (long long)t * nk);
  const int k1 = (int)min((long long)nk, (long long)k0 + (it_end - it));
  int tm, tn;
  tile_coords<8>(p, t, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // The uniform-tap conv loaders: each row's pixel offset and tap mask
  // (integer divisions and a mask, some 50 instructions, a quarter of them
  // quarter-rate multiplies) are formed once per tile, one row per thread,
  // into a table in the last A stage, where every lane that loads or
  // converts the row reads them (formed per lane, 7-14 rows each, they took
  // 1.6-2.2 us per tile).  That stage's first loads are issued after the
  // prologue's wait and barrier, so the table's reads are done by then.
  const uint2* rows = nullptr;
  if constexpr (ROW_TABLE) {
    // (every thread writes an entry, rows m0 .. m0 + NT - 1: no branch)
    static_assert(NT * (int)sizeof(uint2) <= SA_ALLOC && BM <= NT, "the row table fits one stage, one row per thread");
    uint2* const tab = reinterpret_cast<uint2*>(sa_ring[RA - 1]);
    if (!first_seg) __syncthreads();  // the previous segment's epilogue may still read LDS
    tab[tid] = ALoader::row_entry(p, m0 + tid, conv_tap_rows(p));
    __syncthreads();
    rows = tab;
  }
  ALoader la;
  if constexpr (ROW_TABLE) {
    la.init(p, rows, k0);
  } else if constexpr (CONV) {
    la.init(p, m0, k0);
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
      for (int e = 0; e < NE; ++e) acc[i][j][e] = 0;

  // Per-lane partial sums of A' rows / B columns (u8 x i8 with zero points).
  int rsum[FM], csum[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) rsum[i] = 0;
#pragma unroll
  for (int j = 0; j < FN; ++j) csum[j] = 0;
  // With 16 x 16 blocks the sums run on the matrix cores instead: onehot[j]
  // is a fragment of ones in row j (the lanes with l % 16 == j) and zeros
  // elsewhere.  MFMA(B block j, onehot[j]) adds colsum(B block j) into
  // column j of one shared 16 x 16 accumulator (cacc), MFMA(onehot[i],
  // A' block i) adds rowsum(A' block i) into row i of another (racc); every
  // other entry gets zeros, so one accumulator holds all the blocks' sums.
  // One MFMA per block and k-step: 1/FN more matrix work per sum, where the
  // v_dot4 form cost over a third of the main loop's time.  The two extra
  // accumulators must fit beside the tile's in the 256 accumulator
  // registers: at 256 x 256 (all 256 taken) the sums stay on v_dot4.
  constexpr bool MSUMS = SUMS != 0 && MB == 16 && FM <= 16 && FN <= 16 && FM * FN * NE + 2 * NE <= 256;
  acc_t racc, cacc;
  uint4 onehot[MSUMS ? (FM > FN ? FM : FN) : 1];
  if constexpr (MSUMS) {
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      racc[e] = 0;
      cacc[e] = 0;
    }
#pragma unroll
    for (int j = 0; j < (FM > FN ? FM : FN); ++j) {
      const uint32_t v = (lane & 15) == j ? 0x01010101u : 0u;
      onehot[j] = make_uint4(v, v, v, v);
    }
  }
  const bool want_rsum = (SUMS & SUM_ROWS) && p.zB != 0 && wn == 0;
  const bool want_csum = (SUMS & SUM_COLS) && p.zAp != 0 && wm == 0;

  // Fragments, double-buffered in registers: lane l reads row l % MB of its
  // MB-row block, 16-byte chunk LPR * ks + l / MB (a k-step is 16 * LPR bytes
  // of K: 64 for 16 x 16 blocks, 32 for 32 x 32).
  const int frow = lane % MB;
  const int fhalf = lane / MB;
  // The u8 convolution through the uniform-tap loader: a padded row's K tile
  // lands as zero bytes, and the conversion to signed bytes (A xor 0x80 =
  // A - 128) xors each fragment row with xk[i]: 0x80808080 where the current
  // tap is inside the image, 0x80808080 xor (zA in every byte) where it is
  // padding, so a padded row becomes zA - 128 like an input byte equal to
  // zA.  xk follows the tap of the K tile being multiplied (a tap spans
  // C / 128 tiles); row 0's constant moves to the next tile's tap when the
  // last k-step begins (its last chunk converts the next tile's first
  // fragment), the others at the end of the tile.
  constexpr uint32_t X80 = 0x80808080u;
  uint32_t fpad[U8_UNIFORM_TAPS ? FM : 1];  // padding-tap bits of this lane's fragment rows
  uint32_t xk[U8_UNIFORM_TAPS ? FM : 1];
  uint32_t xz = X80;
  // fragment row i's constant for tap t: X80, xor zA in every byte where t is
  // padding (a bit-field extract and two bit operations; no compare)
  auto xk_for = [&](int i, int t) -> uint32_t {
    const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)fpad[i], t, 1);
    return X80 ^ ((xz ^ X80) & m);
  };
  int xtap = 0, xleft = 1, xtpt = 1;  // tap of the K tile in use, its tiles left, tiles per tap
  if constexpr (U8_UNIFORM_TAPS) {
    xz = X80 ^ ((uint32_t)(uint8_t)(p.zAp + 128) * 0x01010101u);
#pragma unroll
    for (int i = 0; i < FM; ++i) fpad[i] = ~rows[wm * TM + i * MB + frow].y;
    const int k = k0 * KT_BYTES;  // u8: one byte per channel
    xtap = (int)p.fd_c.div((uint32_t)k);
    xtpt = p.C / KT_BYTES;
    xleft = xtpt - (k - xtap * p.C) / KT_BYTES;
#pragma unroll
    for (int i = 0; i < FM; ++i) xk[i] = xk_for(i, xtap);
  }
  // the conversion constant of fragment row i
  auto xconst = [&](int i) -> uint32_t {
    if constexpr (U8_UNIFORM_TAPS) return xk[i];
    else return X80;
  };
  uint4 fa[2][FM], fb[2][FN];
  auto read_a = [&](const uint8_t* As, int ks, int i, uint4& a) {
    a = lds_read16(As, swz(wm * TM + i * MB + frow, ks * LPR + fhalf));
  };
  auto read_b = [&](const uint8_t* Bs, int ks, int j, uint4& b) {
    b = lds_read16(Bs, swz(wn * TN + j * MB + frow, ks * LPR + fhalf));
  };
  constexpr int KSTEPS = KT_BYTES / (16 * LPR);
  static_assert(KSTEPS % 2 == 0, "the fragment double buffer returns to set 0 after a tile");

  // One chunk of a k-step: the FN MFMAs of fragment row c, with its share of
  // the reads of the next k-step's fragments and the direct-to-LDS loads given
  // by `issue`.  Program order is the issue order: the first MFMA goes before the
  // loads so the matrix pipe is busy while they issue, and the compiler may
  // not move anything across a chunk boundary.  The u8 A operand becomes
  // A' = A xor 0x80 (A - 128 as a signed byte) one chunk ahead of use: `ax`
  // carries row c's converted fragment in, and `a_up` (the next chunk's raw
  // fragment) is converted between this chunk's MFMAs.
  uint4 ax = make_uint4(0, 0, 0, 0);
  auto chunk = [&](int c, const uint4 (&a)[FM], const uint4 (&b)[FN], const uint8_t* As_n,
                   const uint8_t* Bs_n, int ks_n, uint4 (&an)[FM], uint4 (&bn)[FN], const uint4& a_up,
                   auto issue) {
    __builtin_amdgcn_sched_barrier(0);
    const uint4 ac = INT8 ? ax : a[c];
    // B's fragment goes in the instruction's first operand slot and A's in
    // the second: the block comes out transposed, so each lane holds 4
    // consecutive columns of one row (see the epilogue).
    Mfma<KIND, MB>::run(acc[c][0], b[0], ac);
    __builtin_amdgcn_sched_barrier(0);
    issue();
    __builtin_amdgcn_sched_barrier(0);
    // next k-step's fragments: all B first (the next k-step's first chunk
    // uses every one of them), then A in row order
    int nrd = 0;
#pragma unroll
    for (int r = 0; r < FN + FM; ++r)
      if (r * FM / (FN + FM) == c) {
        if (r < FN)
          read_b(Bs_n, ks_n, r, bn[r]);
        else
          read_a(As_n, ks_n, r - FN, an[r - FN]);
        ++nrd;
      }
    constexpr int NV = (INT8 ? 4 : 0) + ((!MSUMS && (SUMS & SUM_ROWS)) ? 4 : 0) +
                       ((!MSUMS && (SUMS & SUM_COLS)) ? 4 * ((FN + FM - 1) / FM) : 0);
    // u8 without v_dot4 sums: the conversion of the next chunk's fragment
    // goes before the row's last two MFMAs (fenced), so the reads issued
    // early in the chunk have it to land before the conversion waits for
    // them, and two MFMAs cover the conversion's latency before the next
    // chunk reads it.  (Left to the scheduler, the conversion followed the
    // first read, behind an LDS wait two MFMAs into the chunk.)
    constexpr bool LATE_X = INT8 && NV == 4 && FN >= 4 && FN - 2 > 2;
    uint4 axn = a_up;
    auto convert = [&]() {
      if constexpr (INT8) {
        const uint32_t xc = xconst((c + 1) % FM);  // a_up is fragment row (c + 1) % FM
        axn.x ^= xc;
        axn.y ^= xc;
        axn.z ^= xc;
        axn.w ^= xc;
      }
    };
    if constexpr (LATE_X) {
#pragma unroll
      for (int j = 1; j < FN - 2; ++j) Mfma<KIND, MB>::run(acc[c][j], b[j], ac);
#pragma unroll
      for (int q = 1; q < FN - 2; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if (q <= nrd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      }
      __builtin_amdgcn_sched_barrier(0);
      convert();
      __builtin_amdgcn_sched_barrier(0);
      Mfma<KIND, MB>::run(acc[c][FN - 2], b[FN - 2], ac);
      Mfma<KIND, MB>::run(acc[c][FN - 1], b[FN - 1], ac);
    } else {
      convert();
#pragma unroll
      for (int j = 1; j < FN; ++j) Mfma<KIND, MB>::run(acc[c][j], b[j], ac);
    }
    if constexpr (MSUMS) {
      if constexpr ((SUMS & SUM_ROWS) != 0) Mfma<KIND, MB>::run(racc, onehot[c], ac);
      if constexpr ((SUMS & SUM_COLS) != 0) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
          if (j * FM / FN == c) Mfma<KIND, MB>::run(cacc, b[j], onehot[j]);
      }
    } else {
      if constexpr ((SUMS & SUM_ROWS) != 0) rsum[c] = sum_bytes(ac, rsum[c]);
      if constexpr ((SUMS & SUM_COLS) != 0) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
          if (j * FM / FN == c) csum[j] = sum_bytes(b[j], csum[j]);
      }
    }
    // between the MFMAs: the reads first, then the vector ALU work
    int nv = 0;
#pragma unroll
    for (int q = 1; q < (LATE_X ? 1 : FN); ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (q <= nrd) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      } else if (nv < NV) {
        const int k = (NV - nv + (FN - 1 - q)) / (FN - q);  // spread evenly
#pragma unroll
        for (int t = 0; t < k; ++t) __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);  // vector ALU
        nv += k;
      }
    }
    if constexpr (INT8) ax = axn;
  };

  // Prologue: tiles 0 .. DEPTH-1 in flight, tile 0 landed, its first
  // fragments read.
  static_for<DEPTH>([&](auto D) {
    la.template load<NOPS_SAFE>(stA(D), k0 + decltype(D)::value);
    lb.template load<NOPS_SAFE>(stB(D), k0 + decltype(D)::value);
  });
  wait_vmcnt_lgkm0<(DEPTH - 1) * (NLA + NLB)>();
  lds_barrier();
#pragma unroll
  for (int i = 0; i < FM; ++i) read_a(sa0, 0, i, fa[0][i]);
#pragma unroll
  for (int j = 0; j < FN; ++j) read_b(sb0, 0, j, fb[0][j]);
  if constexpr (INT8) {
    const uint32_t xc = xconst(0);
    ax = fa[0][0];
    ax.x ^= xc;
    ax.y ^= xc;
    ax.z ^= xc;
    ax.w ^= xc;
  }

  // K tile kt (D = DEPTH): A in stage kt % RA, B in stage kt % RB.  On entry
  // tiles kt+1 .. kt+D-1 are in flight.  Region 1: k-steps 0..KSTEPS-2 of
  // tile kt, issuing the loads of A tile kt+D into the stage tile kt-1 used.
  // Then wait until A and B of tile kt+1 have landed (only the loads issued
  // after them, of tiles kt+2 .. kt+D, may still be in flight) and every LDS
  // access of this wave is done, and barrier: every wave is then past its
  // reads of tile kt.  Region 2: the last k-step of tile kt, issuing the
  // loads of B tile kt+D into stage (kt+D) % RB (tile kt's own at RB = D,
  // tile kt-1's at RB = D+1) and reading tile kt+1's first fragments.
  // [TIR-COMPILER] §2.2/§4.4 pipeline; at D = 2 two tiles deep for A, one
  // and a half for B.
  constexpr int NS1 = (KSTEPS - 1) * FM;  // chunks in region 1
  auto tile = [&](int kt, auto U) {
    constexpr int u = decltype(U)::value;
    const uint8_t* As = stA(U);
    const uint8_t* Bs = stB(U);
    uint8_t* const An = stA(std::integral_constant<int, u + DEPTH>());
    uint8_t* const Bn = stB(std::integral_constant<int, u + DEPTH>());
    int buf = 0;
#pragma unroll
    for (int ks = 0; ks < KSTEPS - 1; ++ks) {
#pragma unroll
      for (int c = 0; c < FM; ++c) {
        const int slot = ks * FM + c;
        chunk(c, fa[buf], fb[buf], As, Bs, ks + 1, fa[buf ^ 1], fb[buf ^ 1],
              c + 1 < FM ? fa[buf][c + 1 < FM ? c + 1 : 0] : fa[buf ^ 1][0], [&]() {
#pragma unroll
          for (int i = 0; i < ALoader::NPART; ++i)
            if (i * NS1 / ALoader::NPART == slot) la.part(An, kt + DEPTH, i);
        });
      }
      buf ^= 1;
    }
    la.advance();
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt_lgkm0<(DEPTH - 2) * (NLA + NLB) + NLA>();
    lds_barrier();
    const uint8_t* As1 = stA(std::integral_constant<int, u + 1>());
    const uint8_t* Bs1 = stB(std::integral_constant<int, u + 1>());
    // row 0's conversion constant now serves the next tile's first fragment
    if constexpr (U8_UNIFORM_TAPS) xk[0] = xk_for(0, xleft == 1 ? xtap + 1 : xtap);
#pragma unroll
    for (int c = 0; c < FM; ++c) {
      chunk(c, fa[buf], fb[buf], As1, Bs1, 0, fa[buf ^ 1], fb[buf ^ 1],
            c + 1 < FM ? fa[buf][c + 1 < FM ? c + 1 : 0] : fa[buf ^ 1][0], [&]() {
#pragma unroll
        for (int i = 0; i < BLoader::NPART; ++i)
          if (i * FM / BLoader::NPART == c) lb.part(Bn, kt + DEPTH, i);
      });
    }
    lb.advance();
    if constexpr (U8_UNIFORM_TAPS) {
      if (--xleft == 0) {
        ++xtap;
        xleft = xtpt;
#pragma unroll
        for (int i = 1; i < FM; ++i) xk[i] = xk_for(i, xtap);
      }
    }
  };
  for (int kt = k0; kt < k1; kt += UNR) {
    tile(kt, std::integral_constant<int, 0>());
    static_for<UNR - 1>([&](auto J) {
      constexpr int j = decltype(J)::value + 1;
      if (kt + j < k1) tile(kt + j, std::integral_constant<int, j>());
    });
  }
  // Loads past the segment's last tile may still be writing: drain them before
  // the epilogue reuses the stage arrays.
  wait_vmcnt_lgkm0<0>();
  lds_barrier();

  // ------------------------------------------------------------------ epilogue
  // Accumulator layout of an output block (the MFMA computes it transposed,
  // B x A): lane l holds row l % MB and, in register e, column
  // acc_col(e) = 4*(l/16) + e of a 16 x 16 block, or 8*(e/4) + 4*(l/32) + e%4
  // of a 32 x 32 block: every 4 registers are 4 consecutive columns, staged
  // with one 16-byte LDS store.
  //
  // The accumulators are staged through LDS one wave-row at a time (TM rows;
  // rows 32i..32i+31 in stage array i, BN*4 bytes per row, the 16-byte chunk
  // q of row r in slot q ^ (r % 16), so the 16 rows of one staging store hit
  // distinct banks).  Then every thread takes 4 consecutive columns of a
  // row: the int8 corrections and quantization run element-wise on them, and
  // a wave's stores cover whole rows, 16 bytes (fp32/int32) or 4 (int8) per
  // thread.  (Storing straight from the registers instead -- 16 rows x 16-64
  // bytes per store instruction -- measured slower on MI355X: 8192^2 int8
  // requantize 449 -> 508 us.)
  const int arow = lane % MB;
  auto acc_col = [&](int e) { return MB == 16 ? 4 * (lane >> 4) + e : 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); };
  // registers 4*g4 .. 4*g4+3 of block (i, j) as raw bits (each element is
  // copied out first: bit-casting a vector-element lvalue directly reads
  // element 0 with this compiler)
  auto acc_quad = [&](int i, int j, int g4) {
    const auto v0 = acc[i][j][4 * g4], v1 = acc[i][j][4 * g4 + 1];
    const auto v2 = acc[i][j][4 * g4 + 2], v3 = acc[i][j][4 * g4 + 3];
    return make_uint4(__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                      __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3));
  };
  // Staging arrays for 32-row blocks: the three A stages and the first B
  // stage (each holds 32 x BN x 4 bytes since BN <= BM); the zero-point sums
  // go to the second B stage.
  auto stage_rt = [&](int u) -> uint8_t* {  // u is a constant after unrolling
    return u == 0 ? sa0 : u == 1 ? sa1 : u == 2 ? sa2 : sb0;
  };
  static_assert(32 * BN * 4 <= SB && 32 * BN * 4 <= SA_ALLOC && (BM + BN) * 4 <= SB,
                "staging and sums fit in the stages");
  int* const sums = reinterpret_cast<int*>(sb1);
  // rl: row within a 32-row array; c: column.  The 16-byte chunk index is
  // XOR-ed with rl % 16 (within its aligned group of 16 chunks, BN >= 64), so
  // a staging store (16 rows, one chunk column each) is free of bank
  // conflicts and a row read is a permutation of its chunks.
  static_assert(BN >= 64, "chunk swizzle within groups of 16");
  auto stage_off = [](int rl, int c) {
    return rl * (BN * 4) + (((c >> 2) ^ (rl & 15)) << 4) + (c & 3) * 4;
  };

  uint32_t kzz = 0;
  if constexpr (SUMS != 0) {
    // Complete the row / column sums (the K parts of one row live in lanes
    // l, l + MB, ...) and publish them through LDS.
    auto lane_total = [&](int v) {
      v += __shfl_xor(v, 32);
      if constexpr (MB == 16) v += __shfl_xor(v, 16);
      return v;
    };
    // K-tail padding loads as byte 0 and is stored as A' = -128: add those
    // terms back (in the segment that multiplied the partial K tile: the
    // first with the tail-first order, else the last).
    const bool has_tail = TAIL_FIRST ? k0 == 0 : k1 == nk;
    const int pad_fix = has_tail ? 128 * (nk * KT_BYTES - p.K) : 0;
    if constexpr (MSUMS) {
      // racc: lane l, register e holds the sum of row l % 16 of A' block
      // 4*(l/16) + e; cacc: lane l (l % 16 = j < FN), register e holds the
      // sum of column 4*(l/16) + e of B block j.
      if (want_rsum) {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const int i = 4 * (lane >> 4) + e;
          const int v = racc[e];
          if (i < FM) sums[wm * TM + i * MB + (lane & 15)] = v + pad_fix;
        }
      }
      if (want_csum && (lane & 15) < FN) {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const int v = cacc[e];
          sums[BM + wn * TN + (lane & 15) * MB + 4 * (lane >> 4) + e] = v;
        }
      }
    } else {
      if (want_rsum) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int t = lane_total(rsum[i]) + pad_fix;
          if (lane < MB) sums[wm * TM + i * MB + lane] = t;
        }
      }
      if (want_csum) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int t = lane_total(csum[j]);
          if (lane < MB) sums[BM + wn * TN + j * MB + lane] = t;
        }
      }
    }
  }
  // (nonzero only when both zA' and zB are, i.e. with both sums in use)
  if constexpr (INT8 && (SUMS & SUM_ROWS) != 0 && ((SUMS & SUM_COLS) != 0 || CIN))
    kzz = (uint32_t)p.K * (uint32_t)p.zAp * (uint32_t)p.zB;

  constexpr int GPR = BN / 4;    // 4-column groups per row
  constexpr int RPP = NT / GPR;  // rows per pass of the whole workgroup
  static_assert(NT % GPR == 0 && 32 % RPP == 0, "a pass must cover whole rows of one array");
  const int lcol = (tid % GPR) * 4;
  const int col = n0 + lcol;
  const int rr0 = tid / GPR;
  // A thread's 4 columns are the same in every row it emits: their
  // requantize scale and bias are loaded once, before the rows (loaded per
  // row, each pass waited for its own loads behind the previous pass's
  // stores, which may alias them).
  // (loaded at the start of the staged path below)
  float q_scale[4] = {0.f, 0.f, 0.f, 0.f}, q_bias[4] = {0.f, 0.f, 0.f, 0.f};

  // Stream-K.  A segment that is only part of its tile first publishes the
  // tile's partial sums (mode 1: the staged tile, row-major, in this
  // workgroup's slot of ws) and counts itself in; the contributor that
  // counts last runs the epilogue again in mode 2, adding the others'
  // partials as each group of 4 columns leaves LDS: own + other for two
  // contributors (one add, the same either way round), else every partial in
  // workgroup order.  Mode 0: a whole tile, straight to the outputs.
  int mode = (!SK || (k0 == 0 && k1 == nk)) ? 0 : 1;
  const int g = (int)blockIdx.x - p.dp_tiles;
  const int j_sk = t - p.dp_tiles;
  const long long xs = (long long)j_sk * nk;  // tile start in the stream-K range
  int g_lo = 0, g_hi = 0;
  if (mode) {
    g_lo = sk_owner<INT8>(p, xs);
    g_hi = sk_owner<INT8>(p, xs + nk - 1);
  }
  constexpr int SLOT = BM * BN * 4;  // bytes per partial tile
  auto slot_of = [&](int gg) { return (2 * gg + (sk_start<INT8>(p, gg) >= xs ? 0 : 1)) * SLOT; };
  const __amdgpu_buffer_rsrc_t wsr =
      __builtin_amdgcn_make_buffer_rsrc(p.ws, (short)0, 2 * p.sk_wgs * SLOT, 0x00020000);
  // One group of 4 columns of one row leaves for the outputs.
  // corrected: v already holds the zero-point-corrected sum without the
  // K*zA'*zB term (the shared tiles of the integer kernels)
  // lc: the thread's first column within the tile (lcol but for blocked
  // output passes)
  auto emit = [&](uint4 v, int lrow, bool corrected, int lc) {
    const int row = m0 + lrow;
    const int col = n0 + lc;
      if (row < p.M && col < p.N) {
        const bool full = col + 3 < p.N;
        if constexpr (!INT8) {
          // (blocked output: 16-column block col/16 of 16-row group row/16 is
          // one 16 x 16 array; 4 consecutive columns stay inside it)
          float* dst = BLKO ? p.Cf + ((long long)(row >> 4) * (p.N >> 4) + (col >> 4)) * 256 + (row & 15) * 16 + (col & 15)
                            : p.Cf + (long long)row * p.ldcf + col;
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
          if constexpr ((SUMS & SUM_ROWS) != 0)
            rcorr = (p.zB != 0 && !corrected) ? (uint32_t)p.zB * (uint32_t)sums[lrow] : 0u;
          const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
          int32_t c[4];
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t ccorr = 0;
            if constexpr ((SUMS & SUM_COLS) != 0)
              ccorr = (p.zAp != 0 && !corrected) ? (uint32_t)p.zAp * (uint32_t)sums[BM + min(lcol + q, BN - 1)] : 0u;
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
              const float t = cf[q] * q_scale[q];  // separately rounded: built with -ffp-contract=off
              const float y = t + q_bias[q];
              const uint32_t r = requant_bits(y);  // half to even, saturated
              qv[q] = (int8_t)(uint8_t)r;
              packed |= (r & 0xffu) << (8 * q);
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
  };
  // Requantized int8 as the only output of a whole tile: requantize in the
  // registers (a lane's 4 accumulators of a block are 4 consecutive columns
  // of one row), stage the packed int8 tile once (BM x BN bytes, the 16-byte
  // chunk q of row r in slot q ^ (r % (BN/16)), so a staging store of 16
  // rows and a row read are free of bank conflicts), and write it out in
  // 16-byte rows.  Other tiles and outputs take the staged int32 path below.
  bool qonly = false;
  if constexpr (INT8) qonly = REQ || (mode == 0 && p.Qo && !p.Ci && !p.D && p.vec_q && m0 + BM <= p.M && n0 + BN <= p.N);
  if (qonly) {
    if constexpr (INT8) {
      static_assert(BM * BN <= RA * SA_ALLOC, "the int8 tile fits in the A stages");
      constexpr int CQ = BN / 16;  // 16-byte chunks per int8 row
      uint8_t* const qs = sa0;     // the A stage arrays are contiguous
      auto qoff = [](int r, int c) { return r * BN + ((((c >> 4) ^ (r & (CQ - 1)))) << 4) + (c & 15); };
      if constexpr (SUMS != 0) __syncthreads();  // the published row / column sums
      // Each group of 4 columns needs its scale and bias (and the caller's
      // column sums) from memory: they are loaded one group ahead, so the
      // loads of group t+1 are in flight while group t is requantized
      // (loaded where used, every group waited out a load's full latency;
      // loaded for all groups at once they spill registers).
      constexpr int NG = FN * (NE / 4);  // column groups of a lane
      auto group_col = [&](int t) { return wn * TN + (t / (NE / 4)) * MB + acc_col(4 * (t % (NE / 4))); };
      float nsc[4], nbi[4];
      int32_t ncs[4];
      auto fetch = [&](int t) {
        const int lc = group_col(t);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          nsc[q] = p.scale[n0 + lc + q];
          nbi[q] = p.bias[n0 + lc + q];
          if constexpr (CIN) ncs[q] = p.colsum[n0 + lc + q];
        }
      };
      // (kernels that keep both epilogue paths load each group's where it is
      // used and form the row terms per row: the prefetched values and the
      // row terms held across the groups made them spill more)
      if constexpr (REQ) fetch(0);
      // C = acc' - zA'*colsum(B) - zB*rowsum(A') + K*zA'*zB (wrapping; the
      // true value fits in int32) as acc' + a row term + a column term: the
      // row terms -zB*rowsum(A') once per fragment row, the column terms
      // K*zA'*zB - zA'*colsum(B) once per group of 4 columns, so each value
      // takes one three-operand add (formed per value, the terms and their
      // row sums' LDS reads took a third of the epilogue's instructions).
      auto row_term = [&](int i) -> uint32_t {
        return ((SUMS & SUM_ROWS) != 0 && p.zB != 0) ? 0u - (uint32_t)p.zB * (uint32_t)sums[wm * TM + i * MB + arow] : 0u;
      };
      uint32_t rterm[REQ ? FM : 1];
      if constexpr (REQ) {
#pragma unroll
        for (int i = 0; i < FM; ++i) rterm[i] = row_term(i);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int g4 = 0; g4 < NE / 4; ++g4) {
          // (a scheduling fence per group keeps its loads one group ahead)
          __builtin_amdgcn_sched_barrier(0);
          const int t = j * (NE / 4) + g4;
          const int lc = group_col(t);  // tile column of the first of the 4
          if constexpr (!REQ) fetch(t);
          uint32_t cterm[4];
          float sc[4], bi[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t ccorr;
            if constexpr (CIN)
              ccorr = (uint32_t)p.zAp * (uint32_t)ncs[q];
            else
              ccorr = ((SUMS & SUM_COLS) != 0 && p.zAp != 0) ? (uint32_t)p.zAp * (uint32_t)sums[BM + lc + q] : 0u;
            cterm[q] = kzz - ccorr;
            sc[q] = nsc[q];
            bi[q] = nbi[q];
          }
          if constexpr (REQ)
            if (t + 1 < NG) fetch(t + 1);
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const uint4 v = acc_quad(i, j, g4);
            const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
            float y[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              // the corrected C, then the requantize steps
              const int32_t c = (int32_t)(vv[q] + cterm[q] + (REQ ? rterm[i] : row_term(i)));
              const float t = (float)c * sc[q];  // separately rounded: built with -ffp-contract=off
              y[q] = t + bi[q];
            }
            uint32_t packed;  // half to even, saturated, byte q = column q
            requant_byte<0>(packed, y[0]);
            requant_byte<1>(packed, y[1]);
            requant_byte<2>(packed, y[2]);
            requant_byte<3>(packed, y[3]);
            *reinterpret_cast<uint32_t*>(qs + qoff(wm * TM + i * MB + arow, lc)) = packed;
          }
        }
      __syncthreads();
      constexpr int RPQ = NT / CQ;  // rows per pass
      static_assert(NT % CQ == 0 && BM % RPQ == 0, "int8 passes cover whole rows");
      const int qc = (tid % CQ) * 16;
#pragma unroll 4
      for (int r = tid / CQ; r < BM; r += RPQ)
        store16_nt(p.Qo + (long long)(m0 + r) * p.ldq + n0 + qc, lds_read16(qs, qoff(r, qc)));
    }
  } else if constexpr (!REQ) {
    if constexpr (INT8) {
      if (p.Qo) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cc = min(col + q, p.N - 1);
          q_scale[q] = p.scale[cc];
          q_bias[q] = p.bias[cc];
        }
      }
    }
    // (one wave-row of the tile per step; not unrolled in the 256x256 u8 x i8
    // kernels with in-loop column sums, where the optimizer cannot)
    constexpr int UNR_H = (INT8 && BM == 256 && BN == 256 && (SUMS & SUM_COLS) != 0) ? 1 : WM;
  #pragma unroll UNR_H
    for (int h = 0; h < WM; ++h) {
      if (wm == h) {
  #pragma unroll
        for (int i = 0; i < FM; ++i) {
          uint8_t* arr = stage_rt((i * MB) / 32);
  #pragma unroll
          for (int j = 0; j < FN; ++j)
  #pragma unroll
            for (int g4 = 0; g4 < NE / 4; ++g4) {
              const int off = stage_off((i * MB) % 32 + arow, wn * TN + j * MB + acc_col(4 * g4));
              lds_write16(arr, off, acc_quad(i, j, g4));
            }
        }
      }
      __syncthreads();
      // A whole tile into the blocked layout (fp16 convolution, NHWCnc
      // output): each wave stores one 16 x 16 block per pass, lane l taking
      // row l % 16 and columns 4 (l / 16) .. +3 of it, so one store
      // instruction writes the block's 1 KB of y; the 16 rows of a pass read
      // distinct LDS banks.  Otherwise (below) a wave stores one row per pass.
      if (BLKO && mode == 0) {
        if constexpr (BLKO) {
          constexpr int PB = BN / 64;  // passes per 16-row band
          static_assert(NT == 256 && MB == 16, "blocked passes: 4 waves x 16 columns of 16 x 16 blocks");
  #pragma unroll
          for (int pass = 0; pass < TM / RPP; ++pass) {
            const int rr = (pass / PB) * 16 + (lane & 15);  // row within the wave-row
            const int lc = (pass % PB) * 64 + wave * 16 + 4 * (lane >> 4);
            const uint8_t* arr = stage_rt((pass / PB) / 2);
            emit(*reinterpret_cast<const uint4*>(arr + stage_off(rr & 31, lc)), h * TM + rr, false, lc);
          }
        }
      } else {
  #pragma unroll
      for (int pass = 0; pass < TM / RPP; ++pass) {
        const int rr = rr0 + pass * RPP;         // row within the wave-row
        const uint8_t* arr = stage_rt((pass * RPP) / 32);
        const int lrow = h * TM + rr;
        uint4 v = *reinterpret_cast<const uint4*>(arr + stage_off(rr & 31, lcol));
        const int voff = (lrow * BN + lcol) * 4;
        if constexpr (SK) {
          if (mode == 1) {
            if constexpr (INT8) {
              // this segment's share of acc' - zA'*colsum(B) - zB*rowsum(A'),
              // from its own K range's sums (wrapping; the shares add up to
              // the exact int32 total)
              uint32_t rcorr = 0;
              if constexpr ((SUMS & SUM_ROWS) != 0) rcorr = p.zB != 0 ? (uint32_t)p.zB * (uint32_t)sums[lrow] : 0u;
              uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                uint32_t ccorr = 0;
                if constexpr ((SUMS & SUM_COLS) != 0)
                  ccorr = p.zAp != 0 ? (uint32_t)p.zAp * (uint32_t)sums[BM + lcol + q] : 0u;
                vv[q] = vv[q] - ccorr - rcorr;
              }
              v = make_uint4(vv[0], vv[1], vv[2], vv[3]);
            }
            // (the slot in the vector offset, scalar offset 0: with a
            // register there the compiler keeps no wait states between this
            // 16-byte store and a following write of its data registers, and
            // on this GPU that write reached the store: the first of the four
            // values became the next store's offset)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), wsr,
                                                   voff + (2 * g + (first_seg ? 0 : 1)) * SLOT, 0, CPOL_DEV);
            continue;
          }
        }
        if (mode == 0) emit(v, lrow, false, lcol);
      }
      }
      __syncthreads();
    }
  }
  if constexpr (SK) if (mode == 1) {
    // the partial is out (its device-coherent stores acknowledged): count
    // this contributor in
    wait_vmcnt_lgkm0<0>();
    __syncthreads();
    // (the flag lives in the idle second B stage; read as a wave-uniform
    // value so the segment loop stays scalar)
    volatile int* const s_last = reinterpret_cast<volatile int*>(sb1);
    if (tid == 0) {
      // Release and acquire at device scope: the sc1 policy alone does not
      // carry the partials past an XCD's L2 (a last contributor on another
      // XCD then read a zero-filled slot: one contributor's sums missing).
      // The count follows a write-back of this XCD's L2 (every wave has
      // waited for its stores above) that has completed (the explicit wait:
      // the compiler dropped its own between the write-back and the atomic),
      // and a last contributor invalidates before its loads below.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      wait_vmcnt_lgkm0<0>();
      const int before = __hip_atomic_fetch_add(p.cnt + j_sk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      const int last = before == g_hi - g_lo;
      if (last) __hip_atomic_store(p.cnt + j_sk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // for the next launch
      *s_last = last;
    }
    __syncthreads();
    const bool last = __builtin_amdgcn_readfirstlane(*s_last) != 0;
    __syncthreads();
    if (last) {
      // every partial, this one included, in workgroup order (device-coherent
      // loads: they read past this XCD's L2)
      // rows in batches of RB, every load of a batch in flight at once
      constexpr int NROW = BM / RPP;
      constexpr int RB = NROW % 16 == 0 ? 16 : NROW % 8 == 0 ? 8 : NROW % 4 == 0 ? 4 : NROW < 16 ? NROW : 1;
      static_assert((BM / RPP) % RB == 0, "row batches");
      auto load_rows = [&](int slot, int lrow0, uint4 (&x)[RB]) {
#pragma unroll
        for (int b = 0; b < RB; ++b)
          x[b] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                               wsr, ((lrow0 + b * RPP) * BN + lcol) * 4, slot, CPOL_DEV));
      };
      for (int lrow0 = rr0; lrow0 < BM; lrow0 += RB * RPP) {
        uint4 v[RB], w[RB];
        load_rows(slot_of(g_lo), lrow0, v);
        for (int gg = g_lo + 1; gg <= g_hi; ++gg) {
          load_rows(slot_of(gg), lrow0, w);
#pragma unroll
          for (int b = 0; b < RB; ++b) {
            if constexpr (INT8) {
              v[b] = make_uint4(v[b].x + w[b].x, v[b].y + w[b].y, v[b].z + w[b].z, v[b].w + w[b].w);
            } else {
              const float4 f = __builtin_bit_cast(float4, v[b]), e = __builtin_bit_cast(float4, w[b]);
              v[b] = __builtin_bit_cast(uint4, make_float4(f.x + e.x, f.y + e.y, f.z + e.z, f.w + e.w));
            }
          }
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) emit(v[b], lrow0 + b * RPP, true, lcol);
      }
    }
  }
  if constexpr (!SK) break;  // one whole tile per workgroup: no loop
  it += k1 - k0;
  first_seg = false;
  // Every access of this segment is complete before the next one: the
  // compiler then carries no load of the fix-up (mode 2) round this loop as
  // outstanding (it did in some integer kernels, and waited for it inside
  // the next segment's K loop, where the wait also drained the operand
  // loads in flight every K tile).
  wait_vmcnt_lgkm0<0>();
  }  // segments
}

// ---------------------------------------------------------------------------
// LDS-bypass fp16 GEMM for small, latency-bound problems ([GEMM-TVM] §3.4:
// operands loaded from global memory straight into the tensor-core operand
// registers, no shared-memory staging).  One wave per T x T output tile
// (T = 32: 2 x 2 blocks of 16 x 16; T = 16: one block, four times as many
// waves, so a 256^3 problem spreads over 256 compute units instead of 64);
// lane l loads, for each 16-row block of A and of B, row l % 16 and the
// 16-byte chunk l / 16 of each 64-byte k-step, i.e. exactly its MFMA operand.
// KC k-steps of loads are issued before the first MFMA that needs them.  No
// LDS, no barriers.  Needs the aligned operands of the fast path (rows
// 16-byte aligned, K % 8 == 0).  The MFMA takes B first (transposed block:
// lane l holds row l % 16, columns 4*(l/16) .. +3), so each block leaves in
// one 16-byte store per lane.
// ---------------------------------------------------------------------------
template <int KC, int T = 32>
__global__ void __launch_bounds__(64, 1) gemm_f16_bypass_kernel(const Params p) {
  static_assert(T == 16 || T == 32, "wave tile of one or two 16-row blocks per side");
  constexpr int FB = T / 16;  // 16 x 16 blocks per side
  const int lane = threadIdx.x & 63;
  const int tm = (int)blockIdx.x / p.tiles_n;
  const int tn = (int)blockIdx.x - tm * p.tiles_n;
  const int m0 = tm * T, n0 = tn * T;
  const long long lda2 = p.lda * 2, ldb2 = p.ldb * 2;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.A + m0 * lda2), (short)0, (int)(min(T, p.M - m0) * lda2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.B + n0 * ldb2), (short)0, (int)(min(T, p.N - n0) * ldb2), 0x00020000);
  const int frow = lane & 15;
  const uint32_t chunk = (uint32_t)(lane >> 4) * 16u;
  uint32_t oa[FB], ob[FB];
#pragma unroll
  for (int i = 0; i < FB; ++i) {
    oa[i] = (uint32_t)((frow + 16 * i) * lda2) + chunk;
    ob[i] = (uint32_t)((frow + 16 * i) * ldb2) + chunk;
  }
  const uint32_t kbytes = (uint32_t)p.K * 2u;
  const int nks = (p.K + 31) / 32;  // 64-byte k-steps
  f32x4 acc[FB][FB];
#pragma unroll
  for (int i = 0; i < FB; ++i)
#pragma unroll
    for (int j = 0; j < FB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto ld = [&](const __amdgpu_buffer_rsrc_t& r, uint32_t off, uint32_t kb) {
    // k past K reads out of range (zeros): K % 8 == 0, so a chunk is all in or all out
    const uint32_t o = kb + chunk < kbytes ? off + kb : OOB;
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)o, 0, 0));
  };
  for (int kb = 0; kb < nks; kb += KC) {
    uint4 a[KC][FB], b[KC][FB];
#pragma unroll
    for (int s = 0; s < KC; ++s) {
      const uint32_t k = (uint32_t)(kb + s) * 64u;
#pragma unroll
      for (int i = 0; i < FB; ++i) {
        a[s][i] = ld(ra, oa[i], k);
        b[s][i] = ld(rb, ob[i], k);
      }
    }
#pragma unroll
    for (int s = 0; s < KC; ++s)
#pragma unroll
      for (int i = 0; i < FB; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j) Mfma<KIND_F16_GEMM, 16>::run(acc[i][j], b[s][j], a[s][i]);
  }
#pragma unroll
  for (int i = 0; i < FB; ++i) {
    const int row = m0 + i * 16 + frow;
    if (row >= p.M) continue;
#pragma unroll
    for (int j = 0; j < FB; ++j) {
      const int col = n0 + j * 16 + (lane >> 4) * 4;
      float* dst = p.Cf + (long long)row * p.ldcf + col;
      const float v0 = acc[i][j][0], v1 = acc[i][j][1], v2 = acc[i][j][2], v3 = acc[i][j][3];
      if (col + 3 < p.N && p.vec_c) {
        store16_nt(dst, make_uint4(__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                                   __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3)));
      } else {
        const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (col + q < p.N) dst[q] = vv[q];
      }
    }
  }
}

}  // namespace igc
