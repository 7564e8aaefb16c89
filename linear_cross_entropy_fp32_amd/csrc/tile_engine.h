// Tile engine for the fused linear cross-entropy kernels (gfx950 / CDNA4).
//
// A workgroup of WM x WN waves of 64 accumulates a BM x BN fp32 tile of
// sum_k A(m, k) B(n, k) with bf16 MFMA (v_mfma_f32_32x32x16_bf16); each wave
// owns TM x TN blocks of 32 x 32 (TM = BM / WM / 32, TN = BN / WN / 32).  The
// kernels use 2 x 2 waves at two workgroups per CU and 4 x 2 or 2 x 4 waves
// at one, so that every SIMD holds two waves either way.
//
// Operands stream HBM -> LDS in K slices of 32 values through a ring of
// STAGES LDS stages that buffer loads write directly (buffer_load_dwordx4 ...
// lds, "LDS DMA"): no staging registers and no LDS store instructions.
// STAGES - 1 slices are in flight while one is multiplied, and a slice is
// consumed after an explicit "s_waitcnt vmcnt(loads of the later slices)" +
// s_barrier, so only that slice has to have landed (a fenced barrier would
// make the compiler drain every outstanding load).  Loads return in order, so the wait also holds
// when the caller's epilogue has issued other memory operations in between.
// The streamed loop (run_stream) barriers at the start of each slice; the
// single-tile loop (run) barriers in the middle of each slice, so that the
// LDS reads that follow a barrier overlap MFMAs of the same wave.
// Out-of-range rows and K values read zero through the buffer descriptor
// bound; no load is branched around.
//
// LDS layouts.  One LDS-DMA instruction writes 64 lanes x 16 bytes to 1 KB of
// consecutive LDS; each lane picks the global 16-byte chunk that belongs in
// its slot, which is how the layouts below are swizzled.
//  * K-major operand (K contiguous in memory: lm_head rows, hidden rows, dz
//    rows): one 64-byte row per M/N index; chunk c of row r sits at position
//    c ^ ((r / 4) % 4), which makes the fragment reads (8 consecutive K values
//    per lane, one ds_read_b128) free of bank conflicts.
//  * MN-major operand (M/N contiguous: lm_head read along the vocabulary,
//    hidden read along tokens, dz read along the vocabulary): one row per K
//    index holding the tile's M/N values; chunk c of K row k sits at position
//    c ^ (4 (k % 4)).  A fragment is two ds_read_b64_tr_b16: within every
//    16-lane group, lane j receives element j%4 of the 64-bit piece addressed
//    by lane 4e + j/4 as its element e, so lane 16g+i addresses K row
//    k0 + 8(g/2) + i/4 (+4 for the second read) at column m0 + 16(g%2) +
//    4(i%4), and holds the 8 consecutive K values of column m0 + lane%32.
//    The 32 lanes served in one LDS cycle then touch 8 distinct 32-byte
//    pieces of the 256-byte bank window.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define FLCE_HD __host__ __device__
#include "grid_order.h"

namespace flce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kBK = 32;        // K values per slice
constexpr int kStages = 3;     // LDS ring depth of the four-wave tiles
// Wave priority (s_setprio) while a tile's K loop runs; epilogues and result
// stores run at 0.  With two workgroups per CU, a SIMD holds one wave of
// each: when one is in its VALU-heavy epilogue and the other in its K loop,
// the arbiter then favours the MFMA and load issue of the K loop.  Measured
// on the 2048 x 640 x 262144 softcapped workload: -2% per step at 1, less
// at 2 and 3.
constexpr int kLoopPriority = 1;

// Row (within a 32x32 block) of accumulator register r of lane l for the
// 32x32x16 MFMA; the column is l % 32.
__device__ __forceinline__ int acc_row(int r, int lane) {
  return ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3);
}

// Operand descriptor.  K-major: element (row, k) at ptr[row * ld + k]; the row
// bound is exact, K is checked per 8-value chunk (callers keep K % 8 == 0 or
// zero padding).  MN-major: element (row, k) at ptr[k * ld + row]; rows are
// checked per group of 8 (callers keep the bound a multiple of 8), K exactly.
struct Operand {
  const uint16_t* ptr;
  int64_t ld;
  int row0;
  int row_bound;
  int k_bound;
};

constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset that reads as zero

// Buffer descriptor whose base is the tile's first element; loads past
// `bytes` return zero, which replaces per-load bounds branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int64_t bytes) {
  const int64_t b = bytes < 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)b, 0x00020000);
}

// `off` when `in_range`, else an offset that reads zero.  Written as bit
// arithmetic (kept opaque) so that the compiler does not split the load that
// uses it into two predicated copies.
__device__ __forceinline__ uint32_t offset_or_oob(bool in_range, uint32_t off) {
  uint32_t m = in_range ? 0u : kOutOfRange;
  asm("" : "+v"(m));
  return off | m;
}

// Buffer descriptor as four scalar registers (base, stride 0, size in bytes,
// the data format word of a raw buffer) for the LDS-DMA loads below.
__device__ __forceinline__ u32x4 dma_rsrc(const void* base, int64_t bytes) {
  const int64_t b = bytes < 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
  const uint64_t a = (uint64_t)(uintptr_t)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane((uint32_t)b);
  r[3] = 0x00020000u;
  return r;
}

// 16 bytes per lane from global memory into LDS: lane l of the wave writes
// bytes [16 l, 16 l + 16) of the 1 KB block at LDS byte address m0
// (wave-uniform); offsets at or past the descriptor size read zero.  Issued
// as inline assembly so that the compiler does not track the LDS writes: it
// would otherwise wait for every outstanding load before each transposing
// LDS read.  Completion is ordered by vm_barrier() alone; the waits the
// compiler places for its own loads stay sufficient, since loads return in
// order and these only add to the count.  Being volatile, the statement keeps
// its place between the barriers.  The s_nop covers the one wait state that
// GFX9 needs between an M0 write and an LDS-DMA instruction.  Callers form m0
// from the workgroup's LDS base (lds_addr) with scalar adds, so that no
// address conversion runs per load.
__device__ __forceinline__ void dma16_at(const u32x4& rs, uint32_t m0, uint32_t off) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(rs),
               "{m0}"(m0));
}

// 4 bytes per lane from global memory into LDS: lane l writes bytes
// [4 l, 4 l + 4) of the 256-byte block at LDS byte address m0 (wave-uniform).
// Same rules as dma16_at, with five wait states in front: the compiler does
// not look inside the statement for hazards, and where it reloads the
// descriptor from a spill lane (v_readlane, a VALU write of an SGPR) a vector
// memory instruction must not read those SGPRs for five wait states.  (One
// launch per tile, so the wait costs nothing measurable.)  The build scans the
// assembly of every kernel for this hazard at the other LDS-DMA sites.
__device__ __forceinline__ void dma4_at(const u32x4& rs, uint32_t m0, uint32_t off) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(off), "s"(rs),
               "{m0}"(m0));
}

// Per-row values of the A operand (an fp32 bias) for the epilogues of a
// streamed tile sequence (Tile::run_stream with ROWS): each wave loads the 64
// values of its slab of a tile's A rows (wave w: rows 64 (w % WM) + lane) by
// LDS DMA together with the tile's first slice, into its own 256-byte block
// of buffer t % STAGES.  Counted with that slice's loads, they have landed
// when the tile's last slice has, and the buffer is not loaded again before
// the tile's epilogue is done (the issue pointer runs STAGES - 1 slices
// ahead).
struct RowDma {
  u32x4 rsrc;      // 4-byte values per A row; rows past its size read zero
  uint32_t lds;    // LDS byte address of buffer 0 (row_dma_bytes(...))
  int row0;        // A row of the first tile
};
// Row-DMA buffers: one per ring stage (the issue pointer runs STAGES - 1
// slices ahead, so a one-slice tile's buffer is reloaded STAGES tiles later,
// after its epilogue), each one 256-byte block per wave.
constexpr int row_dma_bytes(int stages, int waves) { return stages * waves * 256; }

// LDS byte address of a pointer into the workgroup's LDS array.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p);
}

// Wait until at most N of this wave's vector memory operations are
// outstanding, then barrier the workgroup.
#define FLCE_VMB(n) \
  else if constexpr (N == n) asm volatile("s_waitcnt vmcnt(" #n ") lgkmcnt(0)\n\ts_barrier" ::: "memory");
template <int N>
__device__ __forceinline__ void vm_barrier() {
  static_assert(N >= 0 && N <= 24, "vmcnt immediate");
  // lgkmcnt(0): this wave's LDS reads of the stage about to be refilled are done
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  FLCE_VMB(1) FLCE_VMB(2) FLCE_VMB(3) FLCE_VMB(4) FLCE_VMB(5) FLCE_VMB(6) FLCE_VMB(7) FLCE_VMB(8)
  FLCE_VMB(9) FLCE_VMB(10) FLCE_VMB(11) FLCE_VMB(12) FLCE_VMB(13) FLCE_VMB(14) FLCE_VMB(15)
  FLCE_VMB(16) FLCE_VMB(17) FLCE_VMB(18) FLCE_VMB(19) FLCE_VMB(20) FLCE_VMB(21) FLCE_VMB(22)
  FLCE_VMB(23) FLCE_VMB(24)
}
#undef FLCE_VMB

// s_waitcnt lgkmcnt(0) in a form the compiler sees (vmcnt and expcnt left at
// their maxima), so that it knows the LDS reads issued so far have completed
// and places no waits of its own for them later; the waits inside the inline
// assembly above are invisible to it.
__device__ __forceinline__ void lds_reads_done() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier after this wave's LDS accesses have completed; loads
// into LDS that are still in flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// --------------------------------------------------------------- operands

template <int R, bool KMAJ, int NW>
struct Stage;

template <int R, int NW>
struct Stage<R, true, NW> {
  static constexpr int kRowBytes = kBK * 2;                 // 64
  static constexpr int kBytes = R * kRowBytes;
  static constexpr int kPerWave = R * (kBK / 8) / NW / 64;  // DMA instructions per wave
  static_assert(kPerWave >= 1 && kPerWave * NW * 64 == R * (kBK / 8), "K-major tile shape");
  __device__ static __forceinline__ int swz(int r) { return (r >> 2) & 3; }

  struct Src {
    u32x4 rsrc;
    uint32_t ld_bytes;
    int k_bound;
  };
  // rows past the operand's row bound fall outside the descriptor; chunks
  // past the K bound are sent out of range explicitly
  __device__ static __forceinline__ Src source(const Operand& op) {
    const int64_t rows = (int64_t)op.row_bound - op.row0;
    return Src{dma_rsrc(op.ptr + (int64_t)op.row0 * op.ld, rows * op.ld * 2),
               (uint32_t)(op.ld * 2), op.k_bound};
  }
  // m0: LDS byte address of the stage's operand block (wave-uniform)
  __device__ static __forceinline__ void issue(const Src& s, uint32_t m0, int k0) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int blk = wave * kPerWave + i;          // 1 KB block = 16 rows
      const int p = blk * 64 + lane;                // 16-byte slot this lane writes
      const int row = p >> 2, c = (p & 3) ^ swz(row);
      const int gk = k0 + c * 8;
      dma16_at(s.rsrc, m0 + blk * 1024, offset_or_oob(gk < s.k_bound, row * s.ld_bytes + gk * 2));
    }
  }
  // Per-lane load offsets of one tile, computed once: slice k0 adds 2 k0
  // bytes; a lane's chunk reads zero past the K bound (or when `live` is
  // false).
  struct Plan {
    u32x4 rsrc;
    uint32_t base[kPerWave];
    int c8[kPerWave];
    int k_bound;
  };
  __device__ static __forceinline__ Plan plan(const Operand& op) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t rows = (int64_t)op.row_bound - op.row0;
    Plan pl;
    pl.rsrc = dma_rsrc(op.ptr + (int64_t)op.row0 * op.ld, rows * op.ld * 2);
    pl.k_bound = op.k_bound;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int p = (wave * kPerWave + i) * 64 + lane;
      const int row = p >> 2, c = (p & 3) ^ swz(row);
      pl.base[i] = (uint32_t)(row * op.ld * 2) + c * 16;
      pl.c8[i] = c * 8;
    }
    return pl;
  }
  __device__ static __forceinline__ void issue(const Plan& pl, uint32_t m0, int k0, bool live) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i)
      dma16_at(pl.rsrc, m0 + (wave * kPerWave + i) * 1024,
               offset_or_oob(live && k0 + pl.c8[i] < pl.k_bound, pl.base[i] + k0 * 2));
  }
  // 8 consecutive K values (from 16 ks + 8 (lane / 32)) of row m0 + lane % 32
  __device__ static __forceinline__ bf16x8 frag(const char* lds, int m0, int ks) {
    const int lane = threadIdx.x & 63;
    const int r = m0 + (lane & 31), c = ks * 2 + (lane >> 5);
    return *reinterpret_cast<const bf16x8*>(lds + r * kRowBytes + ((c ^ swz(r)) << 4));
  }
};

template <int R, int NW>
struct Stage<R, false, NW> {
  static constexpr int kRowBytes = R * 2;                   // one K row
  static constexpr int kBytes = kBK * kRowBytes;
  static constexpr int kCPR = R / 8;                        // chunks per K row
  static constexpr int kPerWave = kBK * kCPR / NW / 64;
  static_assert(kPerWave >= 1 && kPerWave * NW * 64 == kBK * kCPR && kCPR >= 16 &&
                    kCPR % 16 == 0,
                "MN-major tile shape");
  __device__ static __forceinline__ int swz(int k) { return (k & 3) << 2; }

  struct Src {
    u32x4 rsrc;
    uint32_t ld_bytes;
    int rows;       // valid rows from row0
  };
  // K rows past the K bound fall outside the descriptor; chunks past the row
  // bound are sent out of range explicitly
  __device__ static __forceinline__ Src source(const Operand& op) {
    return Src{dma_rsrc(op.ptr + op.row0, ((int64_t)op.k_bound * op.ld - op.row0) * 2),
               (uint32_t)(op.ld * 2), op.row_bound - op.row0};
  }
  // m0: LDS byte address of the stage's operand block (wave-uniform)
  __device__ static __forceinline__ void issue(const Src& s, uint32_t m0, int k0) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int blk = wave * kPerWave + i;
      const int p = blk * 64 + lane;
      const int k = p / kCPR, c = (p % kCPR) ^ swz(k);
      dma16_at(s.rsrc, m0 + blk * 1024,
               offset_or_oob(c * 8 < s.rows, (uint32_t)(k0 + k) * s.ld_bytes + c * 16));
    }
  }
  // Per-lane load offsets of one tile, computed once: slice k0 adds k0 K
  // rows; K rows past the bound fall outside the descriptor, chunks past the
  // row bound (or every chunk when `live` is false) read zero.
  struct Plan {
    u32x4 rsrc;
    uint32_t base[kPerWave];
    bool ok[kPerWave];
    uint32_t ld_bytes;
  };
  __device__ static __forceinline__ Plan plan(const Operand& op) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    Plan pl;
    pl.rsrc = dma_rsrc(op.ptr + op.row0, ((int64_t)op.k_bound * op.ld - op.row0) * 2);
    pl.ld_bytes = (uint32_t)(op.ld * 2);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int p = (wave * kPerWave + i) * 64 + lane;
      const int k = p / kCPR, c = (p % kCPR) ^ swz(k);
      pl.base[i] = (uint32_t)k * pl.ld_bytes + c * 16;
      pl.ok[i] = c * 8 < op.row_bound - op.row0;
    }
    return pl;
  }
  __device__ static __forceinline__ void issue(const Plan& pl, uint32_t m0, int k0, bool live) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t koff = (uint32_t)k0 * pl.ld_bytes;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i)
      dma16_at(pl.rsrc, m0 + (wave * kPerWave + i) * 1024,
               offset_or_oob(live && pl.ok[i], pl.base[i] + koff));
  }
  // 8 consecutive K values (from 16 ks + 8 (lane / 32)) of column m0 + lane % 32
  __device__ static __forceinline__ bf16x8 frag(const char* lds, int m0, int ks) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, i = lane & 15;
    const int k = ks * 16 + ((g >> 1) << 3) + (i >> 2);     // k % 4 == (k + 4) % 4
    const int m = m0 + ((g & 1) << 4) + ((i & 3) << 2);
    const int pos = ((((m >> 3) ^ swz(k)) << 4) | ((m & 7) << 1));
    const char* p0 = lds + k * kRowBytes + pos;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p0 + 4 * kRowBytes));
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  }
};

// ------------------------------------------------------------------- tile

template <int BM, int BN, bool A_KMAJ, bool B_KMAJ, int WM = 2, int WN = 2, int STAGES = kStages>
struct Tile {
  static constexpr int kBM = BM, kBN = BN;
  static constexpr int kWM = WM, kWN = WN, kWaves = WM * WN, kThr = 64 * WM * WN;
  static constexpr int kRing = STAGES;
  static constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  static_assert(TM * WM * 32 == BM && TN * WN * 32 == BN, "wave grid");
  using SA = Stage<BM, A_KMAJ, WM * WN>;
  using SB = Stage<BN, B_KMAJ, WM * WN>;
  static constexpr int kLdsA = SA::kBytes;
  static constexpr int kStage = SA::kBytes + SB::kBytes;
  static constexpr int kLdsBytes = STAGES * kStage;
  static constexpr int kRowDmaBytes = row_dma_bytes(STAGES, WM * WN);
  static constexpr int kLoads = SA::kPerWave + SB::kPerWave;   // per wave per slice

  f32x16 acc[TM][TN];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }

  // One slice.  FIRST: the slice starts a tile, so its first MFMAs take a
  // zero accumulator input instead of the registers being cleared.
  template <bool FIRST = false>
  __device__ __forceinline__ void mma_stage(const char* lds) {
    const int wave = threadIdx.x >> 6;
    const int wm = wave % WM, wn = wave / WM;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8 fa[TM], fb[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = SB::frag(lds + kLdsA, wn * (BN / WN) + j * 32, ks);
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = SA::frag(lds, wm * (BM / WM) + i * 32, ks);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if (FIRST && ks == 0) {
            const f32x16 z = {};
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], z, 0, 0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
          }
        }
    }
  }

  // Fragments of K step ks (0 or 1) of the slice held in one LDS stage.
  __device__ __forceinline__ static void frags(const char* stage, int ks, bf16x8 (&fa)[TM],
                                               bf16x8 (&fb)[TN]) {
    const int wave = threadIdx.x >> 6;
    const int wm = wave % WM, wn = wave / WM;
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = SB::frag(stage + kLdsA, wn * (BN / WN) + j * 32, ks);
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = SA::frag(stage, wm * (BM / WM) + i * 32, ks);
  }
  __device__ __forceinline__ void mma(const bf16x8 (&fa)[TM], const bf16x8 (&fb)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  }

  // acc += the sum over k in [k_begin, k_end), read in whole slices: k_end -
  // k_begin must be a multiple of 32 unless k_end is the operands' K bound
  // (past which loads read zero).
  //
  // Schedule.  Slice kt lives in stage kt % S (S = STAGES).  The workgroup
  // barrier sits in the middle of each slice: after the MFMAs of its first K
  // step, a wave waits until slice kt+1 has landed (the loads of S - 2 later
  // slices may stay in flight) and until every wave has read slice kt, then
  // refills stage kt % S with slice kt+S, reads the first fragments of slice
  // kt+1, and multiplies the second K step of slice kt meanwhile.  So the LDS
  // reads after a barrier overlap MFMAs of the same wave, and S - 1 slices
  // stay in flight.
  // Loads past the last slice are issued as zero-reading loads, which keeps
  // the wait counts the same in every iteration.
  __device__ __forceinline__ void run(char* lds, const Operand a_op, const Operand b_op,
                                      int k_begin, int k_end) {
    const int kt_total = (k_end - k_begin + kBK - 1) / kBK;
    if (kt_total <= 0) return;
    const typename SA::Plan a = SA::plan(a_op);
    const typename SB::Plan b = SB::plan(b_op);
    const uint32_t l0 = lds_addr(lds);
    auto issue = [&](int kt, int stage) {
      const bool live = kt < kt_total;
      const int k0 = k_begin + (live ? kt : 0) * kBK;
      const uint32_t m0 = l0 + stage * kStage;
      SA::issue(a, m0, k0, live);
      SB::issue(b, m0 + kLdsA, k0, live);
    };
#pragma unroll
    for (int i = 0; i < STAGES; ++i) issue(i, i);
    bf16x8 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    __builtin_amdgcn_s_setprio(kLoopPriority);
    vm_barrier<(STAGES - 1) * kLoads>();  // slice 0 landed
    frags(lds, 0, fa0, fb0);
    int st = 0;                           // stage of slice kt
    for (int kt = 0; kt < kt_total; ++kt) {
      const int nst = st == STAGES - 1 ? 0 : st + 1;
      frags(lds + st * kStage, 1, fa1, fb1);
      mma(fa0, fb0);
      // keep the compiler from moving these MFMAs past the barrier, where the
      // wait for the reads above would then stand alone
      __builtin_amdgcn_sched_barrier(0);
      lds_reads_done();
      vm_barrier<(STAGES - 2) * kLoads>();  // slice kt+1 landed; slice kt read by every wave
      issue(kt + STAGES, st);
      if (kt + 1 < kt_total) frags(lds + nst * kStage, 0, fa0, fb0);
      mma(fa1, fb1);
      st = nst;
    }
    __builtin_amdgcn_s_setprio(0);
    vm_barrier<0>();
  }

  // Streams `ntiles` tiles that share the B operand and take A rows
  // a.row0 + t * BM (t = 0 .. ntiles-1), each summed over the K range
  // [0, k_end), with the prefetch running across tile boundaries.  After the
  // last slice of tile t, epi(t, *this, free) consumes acc (the next tile
  // starts from zero again); `free` is an LDS stage (kStage bytes) that no
  // wave reads or loads into until the epilogue returns, when Epi::kUsesLds
  // asks for it (one extra barrier per tile), else null.  ROWS: per-row values
  // of the A rows arrive by LDS DMA with each tile's first slice (see RowDma).
  template <bool ROWS, class Epi>
  __device__ __forceinline__ void run_stream(char* lds, const Operand a_op, const Operand b_op,
                                             int k_end, int ntiles, Epi& epi,
                                             const RowDma& rd = RowDma{}) {
    static_assert(!ROWS || BM == 64 * WM, "row values: 64 rows per wave");
    const int kt_tile = (k_end + kBK - 1) / kBK;
    if (kt_tile <= 0 || ntiles <= 0) return;
    const typename SB::Src b = SB::source(b_op);
    const int past = kt_tile;   // a slice index that reads zero
    // issue pointer: tile it, slice is, its A source, ring stage and row buffer
    int it = 0, is = 0, islot = 0, ibuf = 0;
    Operand ao = a_op;
    typename SA::Src a = SA::source(ao);
    const uint32_t l0 = lds_addr(lds);
    auto issue_next = [&]() {
      const int k0 = (it < ntiles ? is : past) * kBK;
      const uint32_t buf = l0 + islot * kStage;
      if constexpr (ROWS) {
        if (is == 0 && it < ntiles) {
          const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
          const int row = rd.row0 + it * BM + (wave % WM) * 64 + (int)(threadIdx.x & 63);
          dma4_at(rd.rsrc, rd.lds + ibuf * (kWaves * 256) + wave * 256, (uint32_t)row * 4);
          ibuf = ibuf == STAGES - 1 ? 0 : ibuf + 1;
        }
      }
      SA::issue(a, buf, k0);
      SB::issue(b, buf + kLdsA, k0);
      islot = islot == STAGES - 1 ? 0 : islot + 1;
      if (++is == kt_tile) {
        is = 0;
        if (++it < ntiles) {
          ao.row0 += BM;
          a = SA::source(ao);
        }
      }
    };
#pragma unroll
    for (int i = 0; i < STAGES - 1; ++i) issue_next();
    int cslot = 0;   // ring stage being multiplied
    constexpr int kAhead = (STAGES - 2) * kLoads;   // loads of later slices left in flight
    for (int ct = 0; ct < ntiles; ++ct) {
      // the first slice of a tile starts the accumulators from zero, so they
      // are dead between the previous epilogue and here
      vm_barrier<kAhead>();
      __builtin_amdgcn_s_setprio(kLoopPriority);
      issue_next();
      mma_stage<true>(lds + cslot * kStage);
      for (int cs = 1; cs < kt_tile; ++cs) {
        cslot = cslot == STAGES - 1 ? 0 : cslot + 1;
        vm_barrier<kAhead>();
        issue_next();
        mma_stage(lds + cslot * kStage);
      }
      __builtin_amdgcn_s_setprio(0);   // the epilogue yields issue slots to the other workgroup
      char* free_lds = nullptr;
      if constexpr (Epi::kUsesLds) {
        lds_barrier();                 // every wave is done reading this stage
        free_lds = lds + cslot * kStage;
      }
      epi(ct, *this, free_lds);
      cslot = cslot == STAGES - 1 ? 0 : cslot + 1;
    }
    vm_barrier<0>();
  }
};

}  // namespace flce
