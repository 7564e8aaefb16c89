// Tile engine for the fused linear cross-entropy kernels (gfx950 / CDNA4).
//
// A workgroup of 256 threads (4 waves of 64, a 2 x 2 wave grid) accumulates a
// BM x BN fp32 tile of sum_k A(m, k) B(n, k) with bf16 MFMA
// (v_mfma_f32_32x32x16_bf16); each wave owns TM x TN blocks of 32 x 32
// (TM = BM/64, TN = BN/64).
//
// Operands stream HBM -> LDS in K slices of 32 values through a ring of three
// LDS stages that buffer loads write directly (buffer_load_dwordx4 ... lds,
// "LDS DMA"): no staging registers and no LDS store instructions.  Slice kt+2 is issued while
// slice kt is multiplied, and slice kt is consumed after an explicit
// "s_waitcnt vmcnt(loads of one slice)" + s_barrier, so only that slice has to
// have landed (a fenced barrier would make the compiler drain every
// outstanding load).  Loads return in order, so the wait also holds when the
// caller's epilogue has issued other memory operations in between.
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

namespace flce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kBK = 32;        // K values per slice
constexpr int kStages = 3;     // LDS ring depth

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

// Segments of a streamed K loop (see Tile::run_stream): n in 1..3; bit s of a
// (b) selects the second A (B) operand for segment s.
struct SegPlan {
  int n, a, b;
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
// bytes [16 l, 16 l + 16) of the 1 KB block at `lds` (wave-uniform); offsets
// at or past the descriptor size read zero.  Issued as inline assembly so that
// the compiler does not track the LDS writes: it would otherwise wait for
// every outstanding load before each transposing LDS read.  Completion is
// ordered by vm_barrier() alone; the waits the compiler places for its own
// loads stay sufficient, since loads return in order and these only add to
// the count.  Being volatile, the statement keeps its place between the
// barriers.  The s_nop covers the one wait state that GFX9 needs between an
// M0 write and an LDS-DMA instruction.
__device__ __forceinline__ void dma16(const u32x4& rs, const char* lds, uint32_t off) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds);
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(rs),
               "{m0}"(m0));
}

// Wait until at most N of this wave's vector memory operations are
// outstanding, then barrier the workgroup.
template <int N>
__device__ __forceinline__ void vm_barrier() {
  static_assert(N >= 0 && N <= 12, "vmcnt immediate");
  // lgkmcnt(0): this wave's LDS reads of the stage about to be refilled are done
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 1) asm volatile("s_waitcnt vmcnt(1) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 3) asm volatile("s_waitcnt vmcnt(3) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 5) asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 7) asm volatile("s_waitcnt vmcnt(7) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 9) asm volatile("s_waitcnt vmcnt(9) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 10) asm volatile("s_waitcnt vmcnt(10) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 11) asm volatile("s_waitcnt vmcnt(11) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Workgroup barrier after this wave's LDS accesses have completed; loads
// into LDS that are still in flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// --------------------------------------------------------------- operands

template <int R, bool KMAJ>
struct Stage;

template <int R>
struct Stage<R, true> {
  static constexpr int kRowBytes = kBK * 2;                 // 64
  static constexpr int kBytes = R * kRowBytes;
  static constexpr int kPerWave = R * (kBK / 8) / 4 / 64;   // DMA instructions per wave
  static_assert(kPerWave >= 1 && R % 64 == 0, "K-major tile shape");
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
  __device__ static __forceinline__ void issue(const Src& s, char* lds, int k0) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int blk = wave * kPerWave + i;          // 1 KB block = 16 rows
      const int p = blk * 64 + lane;                // 16-byte slot this lane writes
      const int row = p >> 2, c = (p & 3) ^ swz(row);
      const int gk = k0 + c * 8;
      dma16(s.rsrc, lds + blk * 1024, offset_or_oob(gk < s.k_bound, row * s.ld_bytes + gk * 2));
    }
  }
  // 8 consecutive K values (from 16 ks + 8 (lane / 32)) of row m0 + lane % 32
  __device__ static __forceinline__ bf16x8 frag(const char* lds, int m0, int ks) {
    const int lane = threadIdx.x & 63;
    const int r = m0 + (lane & 31), c = ks * 2 + (lane >> 5);
    return *reinterpret_cast<const bf16x8*>(lds + r * kRowBytes + ((c ^ swz(r)) << 4));
  }
};

template <int R>
struct Stage<R, false> {
  static constexpr int kRowBytes = R * 2;                   // one K row
  static constexpr int kBytes = kBK * kRowBytes;
  static constexpr int kCPR = R / 8;                        // chunks per K row
  static constexpr int kPerWave = kBK * kCPR / 4 / 64;
  static_assert(kPerWave >= 1 && kCPR >= 16 && kCPR % 16 == 0, "MN-major tile shape");
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
  __device__ static __forceinline__ void issue(const Src& s, char* lds, int k0) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int blk = wave * kPerWave + i;
      const int p = blk * 64 + lane;
      const int k = p / kCPR, c = (p % kCPR) ^ swz(k);
      dma16(s.rsrc, lds + blk * 1024,
            offset_or_oob(c * 8 < s.rows, (uint32_t)(k0 + k) * s.ld_bytes + c * 16));
    }
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

template <int BM, int BN, bool A_KMAJ, bool B_KMAJ>
struct Tile {
  static constexpr int kBM = BM, kBN = BN;
  static constexpr int TM = BM / 64, TN = BN / 64;
  using SA = Stage<BM, A_KMAJ>;
  using SB = Stage<BN, B_KMAJ>;
  static constexpr int kLdsA = SA::kBytes;
  static constexpr int kStage = SA::kBytes + SB::kBytes;
  static constexpr int kLdsBytes = kStages * kStage;
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
    const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8 fa[TM], fb[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = SB::frag(lds + kLdsA, wn * (BN / 2) + j * 32, ks);
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = SA::frag(lds, wm * (BM / 2) + i * 32, ks);
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

  // Slice `kt` of a one- or two-segment K range [k_begin, k_begin + 32 kt_seg)
  // into LDS stage `buf`.  Segment 1 (the low half of a split fp32 operand)
  // reuses A and takes B from b1.  Slices past the end read zero.
  __device__ __forceinline__ static void issue(char* buf, const typename SA::Src& a,
                                               const typename SB::Src& b0,
                                               const typename SB::Src& b1, int kt_seg,
                                               int k_begin, int kt) {
    const int seg = kt >= kt_seg ? 1 : 0;
    const int k0 = k_begin + (kt - seg * kt_seg) * kBK;
    SA::issue(a, buf, k0);
    SB::issue(seg ? b1 : b0, buf + kLdsA, k0);
  }

  // acc = the sum over k in [k_begin, k_end), or twice over it when two_seg
  // is set (A against b0, then against b1); acc is overwritten (an empty
  // range leaves it untouched).  The range is read in whole slices:
  // k_end - k_begin must be a multiple of 32 unless k_end is the operands' K
  // bound (past which loads read zero).
  __device__ __forceinline__ void run(char* lds, const Operand a_op, const Operand b0_op,
                                      const Operand b1_op, bool two_seg, int k_begin, int k_end) {
    const int kt_seg = (k_end - k_begin + kBK - 1) / kBK;
    if (kt_seg <= 0) return;
    const int kt_total = kt_seg * (two_seg ? 2 : 1);
    const typename SA::Src a = SA::source(a_op);
    const typename SB::Src b0 = SB::source(b0_op);
    const typename SB::Src b1 = SB::source(two_seg ? b1_op : b0_op);
    const int past = 2 * kt_seg;       // a slice index that reads zero in both modes
    issue(lds, a, b0, b1, kt_seg, k_begin, 0);
    issue(lds + kStage, a, b0, b1, kt_seg, k_begin, kt_total > 1 ? 1 : past);
    int slot = 0, nslot = 2;
    // slice 0 starts the accumulators from zero
    vm_barrier<kLoads>();
    issue(lds + nslot * kStage, a, b0, b1, kt_seg, k_begin, kt_total > 2 ? 2 : past);
    mma_stage<true>(lds);
    slot = 1;
    nslot = 0;
    for (int kt = 1; kt < kt_total; ++kt) {
      vm_barrier<kLoads>();            // slice kt landed; slice kt-1 no longer read
      issue(lds + nslot * kStage, a, b0, b1, kt_seg, k_begin, kt + 2 < kt_total ? kt + 2 : past);
      mma_stage(lds + slot * kStage);
      slot = slot == kStages - 1 ? 0 : slot + 1;
      nslot = nslot == kStages - 1 ? 0 : nslot + 1;
    }
    vm_barrier<0>();
  }

  // Streams `ntiles` tiles that share the B operand and take A rows
  // a.row0 + t * BM (t = 0 .. ntiles-1), with the prefetch running across tile
  // boundaries.  Each tile sums sg.n segments of the K range [0, k_end): segment
  // s multiplies A operand (sg.a >> s) & 1 (a0 / a1) by B operand (sg.b >> s)
  // & 1 (b0 / b1), which is how split fp32 operands (bf16 high + low parts)
  // enter.  After the last slice of tile t, epi(t, *this, free) consumes acc
  // (the next tile starts from zero again); `free` is an LDS stage (kStage
  // bytes) that no wave reads or loads into until the epilogue returns, when
  // Epi::kUsesLds asks for it (one extra barrier per tile), else null.  A2:
  // whether the second A operand is used at all (compile time; without it
  // sg.a must be 0 and a1_op is ignored, and the loop is the one-A loop).
  template <bool A2, class Epi>
  __device__ __forceinline__ void run_stream(char* lds, const Operand a0_op, const Operand a1_op,
                                             const Operand b0_op, const Operand b1_op,
                                             const SegPlan sg, int k_end, int ntiles, Epi& epi) {
    const int kt_seg = (k_end + kBK - 1) / kBK;
    const int kt_tile = kt_seg * sg.n;
    if (kt_tile <= 0 || ntiles <= 0) return;
    const typename SB::Src b0 = SB::source(b0_op);
    const typename SB::Src b1 = SB::source(sg.b ? b1_op : b0_op);
    const int past = sg.n * kt_seg;   // a slice index that reads zero in every segment
    // issue pointer: tile it, slice is, its A sources and ring stage
    int it = 0, is = 0, islot = 0;
    Operand ao0 = a0_op, ao1 = a1_op;
    typename SA::Src a0 = SA::source(ao0);
    typename SA::Src a1 = a0;
    if constexpr (A2) a1 = SA::source(ao1);
    auto issue_next = [&]() {
      const int kt = it < ntiles ? is : past;
      const int seg = (kt >= kt_seg ? 1 : 0) + (sg.n > 2 && kt >= 2 * kt_seg ? 1 : 0);
      const int k0 = (kt - seg * kt_seg) * kBK;
      char* buf = lds + islot * kStage;
      if constexpr (A2)
        SA::issue(((sg.a >> seg) & 1) ? a1 : a0, buf, k0);
      else
        SA::issue(a0, buf, k0);
      SB::issue(((sg.b >> seg) & 1) ? b1 : b0, buf + kLdsA, k0);
      islot = islot == kStages - 1 ? 0 : islot + 1;
      if (++is == kt_tile) {
        is = 0;
        if (++it < ntiles) {
          ao0.row0 += BM;
          a0 = SA::source(ao0);
          if constexpr (A2) {
            ao1.row0 += BM;
            a1 = SA::source(ao1);
          }
        }
      }
    };
    issue_next();
    issue_next();
    int cslot = 0;   // ring stage being multiplied
    for (int ct = 0; ct < ntiles; ++ct) {
      // the first slice of a tile starts the accumulators from zero, so they
      // are dead between the previous epilogue and here
      vm_barrier<kLoads>();
      issue_next();
      mma_stage<true>(lds + cslot * kStage);
      for (int cs = 1; cs < kt_tile; ++cs) {
        cslot = cslot == kStages - 1 ? 0 : cslot + 1;
        vm_barrier<kLoads>();
        issue_next();
        mma_stage(lds + cslot * kStage);
      }
      char* free_lds = nullptr;
      if constexpr (Epi::kUsesLds) {
        lds_barrier();                 // every wave is done reading this stage
        free_lds = lds + cslot * kStage;
      }
      epi(ct, *this, free_lds);
      cslot = cslot == kStages - 1 ? 0 : cslot + 1;
    }
    vm_barrier<0>();
  }
};

// Order over a (token tile, vocabulary group) grid in windows of up to
// G groups x T token tiles (G = T = 8: 64 workgroups, what one XCD holds at
// two per CU).  Inside a window, consecutive workgroups share the operand
// that benefits most from being read by workgroups that run in step: the
// vocabulary group (token tile fastest) when all token tiles fit in L2
// anyway, else the token tile (group fastest).  Windows run over the token
// tiles of a band of G groups, then the next band; edge windows are
// narrower.  The map is a bijection onto the n_tt x n_grp grid.
struct GridPos {
  int tt, grp;
};
__device__ __forceinline__ GridPos grouped_order(int id, int n_tt, int n_grp, bool tt_fastest) {
  constexpr int G = 8, T = 8;
  const int b = id / (n_tt * G), r = id - b * (n_tt * G);
  const int gh = min(G, n_grp - b * G);              // groups in this band
  const int tb = r / (T * gh), j = r - tb * (T * gh);
  const int tw = min(T, n_tt - tb * T);              // token tiles in this window
  return tt_fastest ? GridPos{tb * T + j % tw, b * G + j / tw}
                    : GridPos{tb * T + j / gh, b * G + j % gh};
}

// Map a linear workgroup id so that ids adjacent in the logical order land on
// the same XCD (workgroups are dealt to the 8 XCDs round robin), keeping tiles
// that share an operand in one L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int full = nblocks - nblocks % kXcd;
  if (bid >= full) return bid;
  const int per = full / kXcd;
  return (bid % kXcd) * per + bid / kXcd;
}

}  // namespace flce
