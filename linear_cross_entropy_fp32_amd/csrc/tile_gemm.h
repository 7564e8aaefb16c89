// Tile engine for the fused linear cross-entropy kernels (gfx950 / CDNA4).
//
// A workgroup of 256 threads (4 waves, wave64) computes a BM x BN fp32 tile
// C = A * B^T-style products with bf16 MFMA (v_mfma_f32_32x32x16_bf16).  The
// 4 waves form a 2 x 2 grid; each wave owns TM x TN blocks of 32 x 32.
//
// Operands are staged HBM -> registers -> LDS in 64-wide K slices, double
// buffered.  In LDS every operand is stored "K-major": one 128-byte row per
// M (or N) index holding 64 consecutive K values, split in eight 16-byte
// chunks whose positions are XOR-swizzled by the row so that the MFMA
// fragment reads (8 consecutive rows, same chunk) and the transposing stores
// below are free of bank conflicts.
//
// An operand whose K index is the contiguous one in memory (the lm_head rows
// and hidden rows for the logit tile) is copied 16 bytes at a time.  An
// operand whose M/N index is the contiguous one (lm_head read by vocabulary
// index for grad_hidden, hidden read by token for grad_weight) is read as
// 4 (K) x 8 (M/N) blocks and transposed in registers with byte permutes
// before it is written to LDS, so the MFMA always reads 8 consecutive K
// values per lane from one 16-byte LDS chunk.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kBK = 64;              // K values per LDS stage
constexpr int kRowBytes = kBK * 2;   // one LDS row: 64 bf16

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Byte offset of 16-byte chunk c (K values 8c..8c+7) of row r in an LDS tile.
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * kRowBytes + ((c ^ swz(r)) << 4);
}

// Row (within a 32x32 block) of accumulator register r of lane l for the
// 32x32x16 MFMA: the column is l % 32, rows come in groups of four.
__device__ __forceinline__ int acc_row(int r, int lane) {
  return ((r >> 2) << 3) + ((lane >> 5) << 2) + (r & 3);
}

// ---------------------------------------------------------------------------
// Operand descriptors.  `rows` counts M (or N) indices, `kdim` K indices.
// K-major: element (row, k) at ptr[row * ld + k].  Row bound is exact, K is
// checked per 8-value chunk (callers guarantee K % 8 == 0 or zero padding).
// MN-major: element (row, k) at ptr[k * ld + row].  Row bound is checked per
// 8 rows (callers guarantee a multiple of 8), K is exact.
struct Operand {
  const uint16_t* ptr;
  int64_t ld;
  int row0;        // first row of this tile
  int row_bound;   // rows >= row_bound read as zero
  int k_bound;     // k >= k_bound reads as zero
};

template <int R, bool KMAJ>
struct StageLoader;

template <int R>
struct StageLoader<R, true> {
  static constexpr int kN = R * 8 / kThreads;   // 16-byte chunks per thread
  u32x4 reg[kN];

  __device__ __forceinline__ void load(const Operand& op, int k0) {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int q = threadIdx.x + i * kThreads;
      const int row = q >> 3, c = q & 7;
      const int grow = op.row0 + row, gk = k0 + c * 8;
      if (grow < op.row_bound && gk < op.k_bound) {
        reg[i] = *reinterpret_cast<const u32x4*>(op.ptr + (int64_t)grow * op.ld + gk);
      } else {
        reg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int q = threadIdx.x + i * kThreads;
      *reinterpret_cast<u32x4*>(lds + lds_off(q >> 3, q & 7)) = reg[i];
    }
  }
};

template <int R>
struct StageLoader<R, false> {
  // blocks of 4 K values x 8 rows; (64/4) * (R/8) blocks per stage
  static constexpr int kRB = R / 8;
  static constexpr int kN = 16 * kRB / kThreads;
  u32x4 reg[kN][4];

  __device__ __forceinline__ void load(const Operand& op, int k0) {
#pragma unroll
    for (int b = 0; b < kN; ++b) {
      const int blk = threadIdx.x + b * kThreads;
      const int rb = blk % kRB, kb = blk / kRB;
      const int grow = op.row0 + rb * 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int gk = k0 + kb * 4 + j;
        if (grow < op.row_bound && gk < op.k_bound) {
          reg[b][j] = *reinterpret_cast<const u32x4*>(op.ptr + (int64_t)gk * op.ld + grow);
        } else {
          reg[b][j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
    for (int b = 0; b < kN; ++b) {
      const int blk = threadIdx.x + b * kThreads;
      const int rb = blk % kRB, kb = blk / kRB;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const int d = e >> 1;
        u32x2 v;
        v[0] = __builtin_amdgcn_perm(reg[b][1][d], reg[b][0][d], sel);
        v[1] = __builtin_amdgcn_perm(reg[b][3][d], reg[b][2][d], sel);
        *reinterpret_cast<u32x2*>(lds + lds_off(rb * 8 + e, kb >> 1) + ((kb & 1) << 3)) = v;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// The tile: TM x TN 32x32 blocks per wave, 2 x 2 waves.
template <int TM, int TN, bool A_KMAJ, bool B_KMAJ>
struct Tile {
  static constexpr int BM = 64 * TM;
  static constexpr int BN = 64 * TN;
  static constexpr int kLdsA = BM * kRowBytes;
  static constexpr int kLdsB = BN * kRowBytes;
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
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const char* la = lds;
    const char* lb = lds + kLdsA;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int c = ks * 2 + (lane >> 5);
      bf16x8 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(la + lds_off(wm * (BM / 2) + i * 32 + (lane & 31), c));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(lb + lds_off(wn * (BN / 2) + j * 32 + (lane & 31), c));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }

  // Accumulate sum over k of A(m, k) * B(n, k) for one or two K segments
  // (the second, when two_seg is set, serves the low half of a split fp32
  // operand: it reuses A and takes B from b1).  k runs over [k_begin, k_end) in each segment.
  __device__ __forceinline__ void run(char* lds, const Operand a, const Operand b0,
                                      const Operand b1, bool two_seg, int k_begin, int k_end) {
    StageLoader<BM, A_KMAJ> la;
    StageLoader<BN, B_KMAJ> lb;
    const int kt_seg = (k_end - k_begin + kBK - 1) / kBK;
    const int kt_total = kt_seg * (two_seg ? 2 : 1);
    if (kt_total <= 0) return;
    la.load(a, k_begin);
    lb.load(b0, k_begin);
    la.store(lds);
    lb.store(lds + kLdsA);
    __syncthreads();
    for (int kt = 0; kt < kt_total; ++kt) {
      const int nxt = kt + 1;
      if (nxt < kt_total) {
        const int seg = nxt / kt_seg;
        const int k0 = k_begin + (nxt - seg * kt_seg) * kBK;
        la.load(a, k0);
        if (seg) {
          lb.load(b1, k0);
        } else {
          lb.load(b0, k0);
        }
      }
      mma_stage(lds + (kt & 1) * kStage);
      if (nxt < kt_total) {
        char* dst = lds + (nxt & 1) * kStage;
        la.store(dst);
        lb.store(dst + kLdsA);
      }
      __syncthreads();
    }
  }
};

// Map a linear workgroup id so that ids that are adjacent in the logical
// order land on the same XCD (workgroups are dealt to the 8 XCDs round
// robin), keeping tiles that share an operand in one L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int full = nblocks - nblocks % kXcd;
  if (bid >= full) return bid;
  const int per = full / kXcd;
  return (bid % kXcd) * per + bid / kXcd;
}

}  // namespace flce
