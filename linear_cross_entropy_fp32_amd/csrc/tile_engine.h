// Tile engine for the fused linear cross-entropy kernels (gfx950 / CDNA4).
//
// A workgroup of 256 threads (4 waves of 64, a 2 x 2 wave grid) accumulates a
// BM x BN fp32 tile of sum_k A(m, k) B(n, k) with bf16 MFMA
// (v_mfma_f32_32x32x16_bf16); each wave owns TM x TN blocks of 32 x 32
// (TM = BM/64, TN = BN/64).
//
// Operands move HBM -> registers -> LDS in K slices of BK (32 or 64) values.
// Two register sets hold the next two slices while the current one is
// multiplied out of LDS, so a slice's global loads have two slices of MFMA
// work to land; LDS is double buffered.  In LDS each operand row (one M or N
// index) holds BK consecutive K values as 16-byte chunks whose positions are
// XOR-swizzled by the row, so that the MFMA fragment reads (eight consecutive
// rows, one chunk) and the staging stores are bank-conflict free.
//
// An operand whose K index is contiguous in memory is copied 16 bytes at a
// time and read back with one ds_read_b128 per MFMA fragment.  An operand whose
// M/N index is contiguous (the lm_head read along the vocabulary, the hidden
// states read along tokens) is stored in LDS as it lies in memory, one padded
// row per K index, and each fragment is read with two ds_read_b64_tr_b16:
// within every 16-lane group, lane j receives element j%4 of the 64-bit piece
// addressed by lane 4e + j/4 as its element e, so lane 16g+i addresses K row
// k0 + 8(g/2) + i/4 (+4 for the second read) at column m0 + 16(g%2) + 4(i%4)
// and ends up holding the 8 consecutive K values of column m0 + (lane % 32).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

// Row (within a 32x32 block) of accumulator register r of lane l for the
// 32x32x16 MFMA; the column is l % 32.
__device__ __forceinline__ int acc_row(int r, int lane) {
  return ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3);
}

// Operand descriptor.  K-major: element (row, k) at ptr[row * ld + k]; the row
// bound is exact and K is checked per 8-value chunk (callers keep K % 8 == 0
// or zero padding).  MN-major: element (row, k) at ptr[k * ld + row]; rows are
// checked per group of 8 (callers keep the bound a multiple of 8), K exactly.
struct Operand {
  const uint16_t* ptr;
  int64_t ld;
  int row0;
  int row_bound;
  int k_bound;
};

// Workgroup barrier that orders LDS only.  __syncthreads() also fences global
// memory, which makes the compiler drain every outstanding global load (the
// prefetched slices) at each barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr uint32_t kOutOfRange = 0x80000000u;   // buffer offset that reads as zero

// Buffer descriptor whose base is the tile's first element; loads past
// `bytes` return zero, which replaces per-load bounds branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int64_t bytes) {
  const int64_t b = bytes < 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)b, 0x00020000);
}

template <int BK>
struct LdsLayout {
  static constexpr int kChunks = BK / 8;       // 16-byte chunks per row
  static constexpr int kRowBytes = BK * 2;
  // Chunk swizzle chosen by measurement (SQ_LDS_BANK_CONFLICT): with 64-byte
  // rows the rows r and r+4 share banks, so the chunk is XORed with r/4.
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (BK == 64) return (r ^ (r >> 3)) & 7;
    else return (r >> 2) & 3;
  }
  __device__ static __forceinline__ int off(int r, int c) {
    return r * kRowBytes + ((c ^ swz(r)) << 4);
  }
};

template <int R, int BK, bool KMAJ>
struct Stage;

template <int R, int BK>
struct Stage<R, BK, true> {
  using L = LdsLayout<BK>;
  static constexpr int kN = R * L::kChunks / kThreads;
  static_assert(kN >= 1, "tile too small for the K-major loader");
  u32x4 reg[kN];

  // rows of the tile beyond the operand's row bound fall outside the
  // descriptor; chunks beyond the K bound are sent out of range explicitly.
  struct Src {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t ld_bytes;
    int k_bound;
  };
  __device__ static __forceinline__ Src source(const Operand& op) {
    const int64_t rows = (int64_t)op.row_bound - op.row0;
    return Src{tile_rsrc(op.ptr + (int64_t)op.row0 * op.ld, rows * op.ld * 2),
               (uint32_t)(op.ld * 2), op.k_bound};
  }
  __device__ __forceinline__ void load(const Src& s, int k0) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int q = threadIdx.x + i * kThreads;
      const int row = q / L::kChunks, c = q % L::kChunks;
      const int gk = k0 + c * 8;
      const uint32_t off = gk < s.k_bound ? row * s.ld_bytes + gk * 2 : kOutOfRange;
      reg[i] = __builtin_amdgcn_raw_buffer_load_b128(s.rsrc, off, 0, 0);
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int q = threadIdx.x + i * kThreads;
      *reinterpret_cast<u32x4*>(lds + L::off(q / L::kChunks, q % L::kChunks)) = reg[i];
    }
  }
};

template <int R, int BK>
struct Stage<R, BK, false> {
  static constexpr int kRowBytes = R * 2 + 32;        // padded: 4 K rows hit distinct banks
  static constexpr int kBytes = BK * kRowBytes;
  static constexpr int kCPR = R / 8;                  // 16-byte chunks per K row
  static constexpr int kN = BK * kCPR / kThreads;
  static_assert(kN >= 1 && (BK * kCPR) % kThreads == 0, "MN-major tile shape");
  u32x4 reg[kN];

  // k beyond the K bound falls outside the descriptor; chunks beyond the row
  // bound are sent out of range explicitly.
  struct Src {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t ld_bytes;
    int rows;       // valid rows from row0
  };
  __device__ static __forceinline__ Src source(const Operand& op) {
    return Src{tile_rsrc(op.ptr + op.row0, ((int64_t)op.k_bound * op.ld - op.row0) * 2),
               (uint32_t)(op.ld * 2), op.row_bound - op.row0};
  }
  __device__ __forceinline__ void load(const Src& s, int k0) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int q = threadIdx.x + i * kThreads;
      const int k = q / kCPR, c = q % kCPR;
      const uint32_t off = c * 8 < s.rows ? (uint32_t)(k0 + k) * s.ld_bytes + c * 16 : kOutOfRange;
      reg[i] = __builtin_amdgcn_raw_buffer_load_b128(s.rsrc, off, 0, 0);
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int q = threadIdx.x + i * kThreads;
      *reinterpret_cast<u32x4*>(lds + (q / kCPR) * kRowBytes + (q % kCPR) * 16) = reg[i];
    }
  }
};

// MFMA fragment (8 consecutive K values of row m0 + lane % 32, starting at K
// offset 16 ks + 8 (lane / 32)) from an LDS operand tile.
template <int R, int BK, bool KMAJ>
__device__ __forceinline__ bf16x8 read_frag(const char* lds, int m0, int ks) {
  const int lane = threadIdx.x & 63;
  if constexpr (KMAJ) {
    return *reinterpret_cast<const bf16x8*>(
        lds + LdsLayout<BK>::off(m0 + (lane & 31), ks * 2 + (lane >> 5)));
  } else {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    constexpr int kRowBytes = Stage<R, BK, false>::kRowBytes;
    const int g = lane >> 4, i = lane & 15;
    const int k = ks * 16 + ((g >> 1) << 3) + (i >> 2);
    const int m = m0 + ((g & 1) << 4) + ((i & 3) << 2);
    const char* p = lds + k * kRowBytes + m * 2;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p + 4 * kRowBytes));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  }
}

template <int BM, int BN, int BK, bool A_KMAJ, bool B_KMAJ>
struct Tile {
  static constexpr int kBM = BM, kBN = BN;
  static constexpr int TM = BM / 64, TN = BN / 64;
  using L = LdsLayout<BK>;
  static constexpr int kLdsA = A_KMAJ ? BM * L::kRowBytes : Stage<BM, BK, false>::kBytes;
  static constexpr int kLdsB = B_KMAJ ? BN * L::kRowBytes : Stage<BN, BK, false>::kBytes;
  static constexpr int kStage = kLdsA + kLdsB;
  static constexpr int kLdsBytes = 2 * kStage;

  f32x16 acc[TM][TN];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }

  __device__ __forceinline__ void mma_stage(const char* lds) {
    const int wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const char* la = lds;
    const char* lb = lds + kLdsA;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 fa[TM], fb[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[j] = read_frag<BN, BK, B_KMAJ>(lb, wn * (BN / 2) + j * 32, ks);
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = read_frag<BM, BK, A_KMAJ>(la, wm * (BM / 2) + i * 32, ks);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }

  using SA = Stage<BM, BK, A_KMAJ>;
  using SB = Stage<BN, BK, B_KMAJ>;

  __device__ static __forceinline__ void issue(SA& sa, SB& sb, const typename SA::Src& a,
                                               const typename SB::Src& b0,
                                               const typename SB::Src& b1, int kt_seg,
                                               int k_begin, int kt) {
    const int seg = kt >= kt_seg ? 1 : 0;
    const int k0 = k_begin + (kt - seg * kt_seg) * BK;
    sa.load(a, k0);
    if (seg) {
      sb.load(b1, k0);
    } else {
      sb.load(b0, k0);
    }
  }

  // Accumulate over k in [k_begin, k_end) for one K segment, or two when
  // two_seg is set: the second reuses A and takes B from b1 (the low half of
  // a split fp32 operand).
  __device__ __forceinline__ void run(char* lds, const Operand a_op, const Operand b0_op,
                                      const Operand b1_op, bool two_seg, int k_begin, int k_end) {
    const int kt_seg = (k_end - k_begin + BK - 1) / BK;
    if (kt_seg <= 0) return;
    const int kt_total = kt_seg * (two_seg ? 2 : 1);
    const typename SA::Src a = SA::source(a_op);
    const typename SB::Src b0 = SB::source(b0_op);
    const typename SB::Src b1 = SB::source(two_seg ? b1_op : b0_op);
    SA sa0, sa1;
    SB sb0, sb1;
    issue(sa0, sb0, a, b0, b1, kt_seg, k_begin, 0);
    issue(sa1, sb1, a, b0, b1, kt_seg, k_begin, 1);
    sa0.store(lds);
    sb0.store(lds + kLdsA);
    lds_barrier();
    int kt = 0;
    // Unrolled by two so each register set keeps a fixed name.
    for (; kt + 1 < kt_total; kt += 2) {
      // even step: compute buffer 0; set 0 is free, set 1 holds slice kt+1
      // past the last slice the loads fall out of range and read zeros; issuing
      // them unconditionally keeps the outstanding-load count static
      issue(sa0, sb0, a, b0, b1, kt_seg, k_begin, kt + 2);
      __builtin_amdgcn_sched_barrier(0);
      mma_stage(lds);
      sa1.store(lds + kStage);
      sb1.store(lds + kStage + kLdsA);
      lds_barrier();
      // odd step: compute buffer 1; set 1 is free, set 0 holds slice kt+2
      issue(sa1, sb1, a, b0, b1, kt_seg, k_begin, kt + 3);
      __builtin_amdgcn_sched_barrier(0);
      mma_stage(lds + kStage);
      if (kt + 2 < kt_total) {
        sa0.store(lds);
        sb0.store(lds + kLdsA);
      }
      lds_barrier();
    }
    if (kt < kt_total) {   // odd number of slices: the last one sits in buffer 0
      mma_stage(lds);
      lds_barrier();
    }
  }

  // Streams `ntiles` tiles that share the B operand and take A rows
  // a.row0 + t * BM (t = 0 .. ntiles-1), keeping the two-slice prefetch
  // running across tile boundaries.  After the last slice of tile t,
  // epi(t, *this) consumes acc, which is then cleared for the next tile.
  template <class Epi>
  __device__ __forceinline__ void run_stream(char* lds, const Operand a_op, const Operand b0_op,
                                             const Operand b1_op, bool two_seg, int k_end,
                                             int ntiles, Epi& epi) {
    const int kt_seg = (k_end + BK - 1) / BK;
    const int kt_tile = kt_seg * (two_seg ? 2 : 1);
    const int total = kt_tile * ntiles;
    if (total <= 0) return;
    const typename SB::Src b0 = SB::source(b0_op);
    const typename SB::Src b1 = SB::source(two_seg ? b1_op : b0_op);
    // issue pointer: tile it, slice is within the tile
    int it = 0, is = 0;
    auto issue_next = [&](SA& sa, SB& sb) {
      Operand o = a_op;
      o.row0 = a_op.row0 + (it < ntiles ? it : ntiles - 1) * BM;
      const int kt = it < ntiles ? is : kt_tile;       // past the end: out of range
      issue(sa, sb, SA::source(o), b0, b1, kt_seg, 0, kt);
      if (++is == kt_tile) {
        is = 0;
        ++it;
      }
    };
    SA sa0, sa1;
    SB sb0, sb1;
    zero();
    issue_next(sa0, sb0);
    issue_next(sa1, sb1);
    sa0.store(lds);
    sb0.store(lds + kLdsA);
    lds_barrier();
    int ct = 0, cs = 0;   // compute pointer
    for (int g = 0; g < total; g += 2) {
      issue_next(sa0, sb0);
      __builtin_amdgcn_sched_barrier(0);
      mma_stage(lds);
      if (g + 1 < total) {
        sa1.store(lds + kStage);
        sb1.store(lds + kStage + kLdsA);
      }
      lds_barrier();
      if (++cs == kt_tile) {
        epi(ct, *this);
        zero();
        cs = 0;
        ++ct;
      }
      if (g + 1 >= total) break;
      issue_next(sa1, sb1);
      __builtin_amdgcn_sched_barrier(0);
      mma_stage(lds + kStage);
      if (g + 2 < total) {
        sa0.store(lds);
        sb0.store(lds + kLdsA);
      }
      lds_barrier();
      if (++cs == kt_tile) {
        epi(ct, *this);
        zero();
        cs = 0;
        ++ct;
      }
    }
  }
};

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
