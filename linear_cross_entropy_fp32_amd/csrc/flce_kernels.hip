// HIP kernels of the fused linear cross-entropy for gfx950.
//
// The method (TRL pull request "Add loss_type="cce", a fused linear
// cross-entropy loaded from the Hub", "What it supports" and the review's
// "Correctness" facts): the logits are the hidden x lm_head product
// accumulated in fp32, plus an fp32 bias, times logit_scale, then softcapped;
// the loss, the entropy (lse - sum p z) and the argmax all come from one pass
// over those logits, which are never stored.
//
// Units: inside the kernels a final logit z is carried as u = z * log2(e), so
// every exponential is one v_exp_f32 (2^x).  The forward keeps, per token, an
// online state (reference m, S = sum 2^(u-m), T = sum 2^(u-m) u, best value,
// best index, target value), all in base-2 units.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flce_internal.h"
#include "tile_engine.h"

namespace flce {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
// Value given to logits of rows past the vocabulary in the last tile: below
// every real logit, and 2^(it - m) is exactly 0 with 0 * it finite.
constexpr float kMasked = -3.0e38f;

static_assert(kSliceK == kBK, "slice depth");
// The two logit tile shapes (see kNarrowTileV / kWideTileV).  Both give a
// wave the same 64 x 128 block, so the epilogues are shared; both keep two
// waves on every SIMD (8 waves per CU).
using NarrowTile = Tile<kNarrowTileV, kLogitTileN, true, true, 2, 2, 3>;
using WideTile = Tile<kWideTileV, kLogitTileN, true, true, 4, 2, 4>;
// contraction tiles (see kGemmTileNNarrow / kGemmTileNWide)
using GhTile = Tile<kGemmTileM, kGemmTileNNarrow, true, false>;                  // dz . W
using GwTile = Tile<kGemmTileM, kGemmTileNNarrow, false, false>;                 // dz^T . h
using GhTileWide = Tile<kGemmTileM, kGemmTileNWide, true, false, 2, 4, 4>;
using GwTileWide = Tile<kGemmTileM, kGemmTileNWide, false, false, 2, 4, 4>;
constexpr int kColumns = NarrowTile::TN;     // token columns per lane
constexpr int kQ = NarrowTile::TM * 16;      // values per token column per lane
constexpr int kWaveRows = 64;                // vocabulary rows per wave
static_assert(WideTile::TM == NarrowTile::TM && WideTile::TN == NarrowTile::TN &&
                  kNarrowTileV / NarrowTile::kWM == kWaveRows &&
                  kWideTileV / WideTile::kWM == kWaveRows,
              "one wave block in both logit tile shapes");
static_assert(WideTile::kWaves * 32 * kWaveRows * 2 <= WideTile::kStage &&
                  NarrowTile::kWaves * 32 * kWaveRows * 2 <= NarrowTile::kStage,
              "dz transpose buffer fits one LDS stage");
template <class LT>
constexpr int wgs_per_cu() { return 8 / LT::kWaves; }
// workgroups one XCD (32 CUs) holds at once: the window of grouped_order
template <class LT>
constexpr int window_wgs() { return 32 * wgs_per_cu<LT>(); }

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Row offset, inside a wave's vocabulary rows, of value q (0..kQ-1) of a
// lane's token column (q = 16 * block + accumulator register), not counting
// the +4 of the lane's half-wave.
__host__ __device__ constexpr int q_row(int q) {
  return (q >> 4) * 32 + ((q & 15) >> 2) * 8 + (q & 3);
}

// Merge two online states.  Sums are rescaled to the larger reference; the
// argmax keeps the larger value and, on a tie, the lower vocabulary index; the
// target value is finite in at most one of the two states.
__device__ __forceinline__ PartState merge_state(PartState a, const PartState& b) {
  if (b.m == kNegInf) {
    a.zt = fmaxf(a.zt, b.zt);
    return a;
  }
  if (a.m == kNegInf) {
    PartState r = b;
    r.zt = fmaxf(a.zt, b.zt);
    return r;
  }
  const float m = fmaxf(a.m, b.m);
  const float fa = exp2f(a.m - m), fb = exp2f(b.m - m);
  PartState r;
  r.m = m;
  r.s = a.s * fa + b.s * fb;
  r.t = a.t * fa + b.t * fb;
  const bool take_b = (b.bu > a.bu) || (b.bu == a.bu && b.bi < a.bi);
  r.bu = take_b ? b.bu : a.bu;
  r.bi = take_b ? b.bi : a.bi;
  r.zt = fmaxf(a.zt, b.zt);
  return r;
}

__device__ __forceinline__ PartState shfl_xor_state(const PartState& s, int mask) {
  PartState o;
  o.m = __shfl_xor(s.m, mask);
  o.s = __shfl_xor(s.s, mask);
  o.t = __shfl_xor(s.t, mask);
  o.bu = __shfl_xor(s.bu, mask);
  o.zt = __shfl_xor(s.zt, mask);
  o.bi = __shfl_xor(s.bi, mask);
  return o;
}

// Final logit in base-2 units from the fp32 dot product x.  Without softcap:
// u = x * kx + bk with kx = s*log2e, bk = s*log2e*b.  With softcap c:
// c*tanh(y) = c - 2c / (1 + e^(2y)), y = s*(x+b)/c, so with kx = 2*s*log2e/c,
// bk = kx*b: e = 2^(x*kx + bk), r = 1/(1+e), u = c*log2e - 2c*log2e*r.
// `r` is also the backward's softcap slope: 1 - tanh^2 = 4 r (1 - r).
template <bool CAP>
__device__ __forceinline__ float final_u(float x, float kx, float bk, float c1, float c2,
                                         float& r) {
  if constexpr (CAP) {
    const float e = fast_exp2(fmaf(x, kx, bk));
    r = fast_rcp(e + 1.0f);
    return fmaf(-c2, r, c1);
  } else {
    r = 0.f;
    return fmaf(x, kx, bk);
  }
}

// Bias values of the rows q = 4a .. 4a+3 of a lane's token column (rows
// q_row(q) + 4 half of the wave's slab), read from the wave's row-DMA block of
// the tile (see RowDma): one 16-byte LDS read.  Rows past the vocabulary hold
// zero.
template <bool BIAS>
__device__ __forceinline__ void bias4(const float* blk, int a, int half, float (&b)[4]) {
  if constexpr (BIAS) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 v = *reinterpret_cast<const f32x4*>(blk + q_row(4 * a) + half * 4);
    b[0] = v[0];
    b[1] = v[1];
    b[2] = v[2];
    b[3] = v[3];
  } else {
    b[0] = b[1] = b[2] = b[3] = 0.f;
  }
}

// The wave's 64-value block of tile t in the row-DMA buffers at `rows`.
template <class LT>
__device__ __forceinline__ const float* bias_block(const float* rows, int t) {
  return rows + (t % LT::kRing) * (LT::kWaves * 64) + (threadIdx.x >> 6) * 64;
}

// ------------------------------------------- fp32 operands: rounded to bf16
// An fp32 hidden state or lm_head enters the MFMA products rounded to bf16
// (round to nearest even).  The logits then carry the operands' rounding
// (~1e-3 at H = 4096), which averages out in lse, entropy and the softmax,
// while the target logit, which the loss takes directly, is computed exactly
// from the unrounded operands (target_logit_kernel).  Eight values per
// thread (count is a multiple of 8), read and written 16 bytes at a time.
__global__ void round_bf16_kernel(const float* __restrict__ x, uint16_t* __restrict__ out,
                                  int64_t count) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i >= count) return;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const f32x4 x0 = *reinterpret_cast<const f32x4*>(x + i);
  const f32x4 x1 = *reinterpret_cast<const f32x4*>(x + i + 4);
  u32x4 o;
  o[0] = pack_bf16x2(x0[0], x0[1]);
  o[1] = pack_bf16x2(x0[2], x0[3]);
  o[2] = pack_bf16x2(x1[0], x1[1]);
  o[3] = pack_bf16x2(x1[2], x1[3]);
  *reinterpret_cast<u32x4*>(out + i) = o;
}

// The target logit of row n from the unrounded operands: one wave per row,
// lanes striding over H, products and sums in double, then a fixed xor tree;
// + bias, * scale, softcap in double, returned in base-2 units.
constexpr int kTargetRowsPerBlock = 4;
__global__ void __launch_bounds__(64 * kTargetRowsPerBlock)
target_logit_kernel(const TargetArgs a) {
  const int64_t n = (int64_t)blockIdx.x * kTargetRowsPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= a.n) return;
  const int64_t t = a.tgt[n];
  if (t == a.ignore_index || t < 0 || t >= a.v) {
    if (lane == 0) a.zt[n] = 0.f;
    return;
  }
  double acc = 0.0;
  for (int64_t k = lane; k < a.hdim; k += 64) {
    const int64_t hi = n * a.hdim + k, wi = t * a.hdim + k;
    const double hv = a.h_f32 ? (double)static_cast<const float*>(a.hidden)[hi]
                              : (double)__builtin_bit_cast(
                                    float, (uint32_t)static_cast<const uint16_t*>(a.hidden)[hi]
                                               << 16);
    const double wv = a.w_f32 ? (double)static_cast<const float*>(a.weight)[wi]
                              : (double)__builtin_bit_cast(
                                    float, (uint32_t)static_cast<const uint16_t*>(a.weight)[wi]
                                               << 16);
    acc = fma(hv, wv, acc);
  }
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (lane != 0) return;
  double z = acc;
  if (a.bias) z += (double)a.bias[t];
  z *= a.scale;
  if (a.softcap > 0.0) z = a.softcap * tanh(z / a.softcap);
  a.zt[n] = (float)(z * 1.4426950408889634);
}

// ------------------------------------------------------------ row compaction
// Optional (flce_problem.compact_valid): the rows that carry a loss (target in
// [0, V), not ignore_index) are listed first in perm, in row order, followed
// by the other rows in row order, so perm is a permutation of [0, N); the
// number of the former goes to cnt[0] and the number of out-of-range targets
// to cnt[1].  Every kernel then runs over compact row c with the original row
// perm[c], only for c < cnt[0].  Three passes: per-block counts, one block
// scans them, every block writes its rows' positions.
constexpr int kCompactBlock = 256;
constexpr int kScanThreads = 1024;

__device__ __forceinline__ void row_kind(const int64_t* tgt, int i, int n, int64_t ignore, int v,
                                         bool& valid, bool& bad) {
  valid = bad = false;
  if (i < n) {
    const int64_t t = tgt[i];
    const bool ig = (t == ignore);
    valid = !ig && t >= 0 && t < v;
    bad = !ig && !valid;
  }
}

__global__ void __launch_bounds__(kCompactBlock)
compact_count_kernel(const int64_t* __restrict__ tgt, int n, int64_t ignore, int v,
                     int* __restrict__ blk_valid, int* __restrict__ blk_bad) {
  bool valid, bad;
  row_kind(tgt, blockIdx.x * kCompactBlock + threadIdx.x, n, ignore, v, valid, bad);
  const uint64_t bv = __ballot(valid), bb = __ballot(bad);
  __shared__ int sv[kCompactBlock / 64], sb[kCompactBlock / 64];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[w] = __popcll(bv);
    sb[w] = __popcll(bb);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = 0, b = 0;
    for (int i = 0; i < kCompactBlock / 64; ++i) {
      a += sv[i];
      b += sb[i];
    }
    blk_valid[blockIdx.x] = a;
    blk_bad[blockIdx.x] = b;
  }
}

// One block: blk_valid becomes its exclusive prefix sum; cnt = {total valid,
// total out-of-range}.  Thread i scans a contiguous run of blocks.
__global__ void __launch_bounds__(kScanThreads)
compact_scan_kernel(int* __restrict__ blk_valid, const int* __restrict__ blk_bad, int nblk,
                    int* __restrict__ cnt) {
  const int per = (nblk + kScanThreads - 1) / kScanThreads;
  const int b0 = threadIdx.x * per, b1 = min(nblk, b0 + per);
  int sum = 0, bad = 0;
  for (int b = b0; b < b1; ++b) {
    sum += blk_valid[b];
    bad += blk_bad[b];
  }
  __shared__ int ss[kScanThreads], sb[kScanThreads];
  ss[threadIdx.x] = sum;
  sb[threadIdx.x] = bad;
  __syncthreads();
  // inclusive scan of the thread sums (Hillis-Steele); bad counts are summed
  for (int d = 1; d < kScanThreads; d <<= 1) {
    const int x = threadIdx.x >= d ? ss[threadIdx.x - d] : 0;
    const int y = threadIdx.x >= d ? sb[threadIdx.x - d] : 0;
    __syncthreads();
    ss[threadIdx.x] += x;
    sb[threadIdx.x] += y;
    __syncthreads();
  }
  int run = ss[threadIdx.x] - sum;
  for (int b = b0; b < b1; ++b) {
    const int c = blk_valid[b];
    blk_valid[b] = run;
    run += c;
  }
  if (threadIdx.x == kScanThreads - 1) {
    cnt[0] = ss[kScanThreads - 1];
    cnt[1] = sb[kScanThreads - 1];
  }
}

__global__ void __launch_bounds__(kCompactBlock)
compact_scatter_kernel(const int64_t* __restrict__ tgt, int n, int64_t ignore, int v,
                       const int* __restrict__ blk_off, const int* __restrict__ cnt,
                       int* __restrict__ perm) {
  const int i = blockIdx.x * kCompactBlock + threadIdx.x;
  bool valid, bad;
  row_kind(tgt, i, n, ignore, v, valid, bad);
  const bool other = (i < n) && !valid;
  const uint64_t bv = __ballot(valid), bo = __ballot(other);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  __shared__ int sv[kCompactBlock / 64], so[kCompactBlock / 64];
  if (lane == 0) {
    sv[w] = __popcll(bv);
    so[w] = __popcll(bo);
  }
  __syncthreads();
  int rv = __popcll(bv & below), ro = __popcll(bo & below);
  for (int k = 0; k < w; ++k) {
    rv += sv[k];
    ro += so[k];
  }
  if (i >= n) return;
  const int vbefore = blk_off[blockIdx.x];                       // valid rows in earlier blocks
  const int obefore = blockIdx.x * kCompactBlock - vbefore;      // other rows in earlier blocks
  perm[valid ? vbefore + rv : cnt[0] + obefore + ro] = i;
}

// Compact hidden rows: out[c] = h[perm[c]] for c < cnt[0], 8 bf16 per thread.
__global__ void gather_rows_kernel(const uint16_t* __restrict__ h, const int* __restrict__ perm,
                                   const int* __restrict__ cnt, int64_t hdim,
                                   uint16_t* __restrict__ out, int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = hdim / 8;
  const int64_t c = t / per_row, k = (t % per_row) * 8;
  if (c >= n || c >= cnt[0]) return;
  *reinterpret_cast<u32x4*>(out + c * hdim + k) =
      *reinterpret_cast<const u32x4*>(h + (int64_t)perm[c] * hdim + k);
}

// fp32 hidden: gather and round to bf16 in one pass.
__global__ void gather_round_kernel(const float* __restrict__ h, const int* __restrict__ perm,
                                    const int* __restrict__ cnt, int64_t hdim,
                                    uint16_t* __restrict__ out, int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_row = hdim / 8;
  const int64_t c = t / per_row, k = (t % per_row) * 8;
  if (c >= n || c >= cnt[0]) return;
  const float* src = h + (int64_t)perm[c] * hdim + k;
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(src[2 * i], src[2 * i + 1]);
  *reinterpret_cast<u32x4*>(out + c * hdim + k) = o;
}

// ------------------------------------------------------------- forward: K1
// Fold one token column (kQ values in a lane) of a finished logit tile into
// that token's state.  `val` holds the values in place of the accumulators.
//
// FIXED (softcap with 2c*log2e <= 120): every final logit is below c, so the
// sums use the fixed reference m = c*log2e and need no running max: the
// value kept is d = u - c*log2e = -2c*log2e*r.  Otherwise the two-pass online
// fold: tile max first, then the exponentials against the new reference.
template <bool CAP, bool FIXED>
__device__ __forceinline__ void fold_column(float (&val)[kQ], PartState& st, int tgt, int vw,
                                            int half) {
  float mt = val[0];
#pragma unroll
  for (int q = 1; q < kQ; ++q) mt = fmaxf(mt, val[q]);
  // argmax: the first (lowest-row) position holding the tile maximum
  if (mt > st.bu) {
    int row = 0;
#pragma unroll
    for (int q = kQ - 1; q >= 0; --q)
      if (val[q] == mt) row = q_row(q);
    st.bu = mt;
    st.bi = vw + half * 4 + row;
  }
  // target value: only in lanes whose target row is one of their rows
  {
    const int rel = tgt - vw - half * 4;
    if (rel >= 0 && rel < kWaveRows && (rel & 4) == 0) {
#pragma unroll
      for (int q = 0; q < kQ; ++q)
        if (q_row(q) == rel) st.zt = val[q];
    }
  }
  float s4[4] = {0.f, 0.f, 0.f, 0.f}, t4[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (FIXED) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const float p = fast_exp2(val[q]);
      s4[q & 3] += p;
      t4[q & 3] = fmaf(p, val[q], t4[q & 3]);
    }
    st.s += (s4[0] + s4[1]) + (s4[2] + s4[3]);
    st.t += (t4[0] + t4[1]) + (t4[2] + t4[3]);
  } else {
    // a lane that has only seen rows past the vocabulary keeps an empty state
    const float mn = fmaxf(st.m, mt);
    if (mn > kMasked) {
      const float alpha = fast_exp2(st.m - mn);
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const float p = fast_exp2(val[q] - mn);
        s4[q & 3] += p;
        t4[q & 3] = fmaf(p, val[q], t4[q & 3]);
      }
      st.s = fmaf(st.s, alpha, (s4[0] + s4[1]) + (s4[2] + s4[3]));
      st.t = fmaf(st.t, alpha, (t4[0] + t4[1]) + (t4[2] + t4[3]));
      st.m = mn;
    }
  }
}

template <class LT, bool CAP, bool FIXED, bool BIAS>
struct FwdEpilogue {
  static constexpr bool kUsesLds = false;
  const FwdArgs& a;
  PartState (&st)[kColumns];
  const int (&tgt)[kColumns];
  const float* rows;               // row-DMA buffers of the bias (BIAS)
  int vt_begin, wm, half;

  __device__ __forceinline__ void operator()(int t, LT& T, char*) {
    const int v0 = (vt_begin + t) * LT::kBM;
    const int vw = v0 + wm * kWaveRows;
    const bool tail = v0 + LT::kBM > a.v;
    const float* blk = BIAS ? bias_block<LT>(rows, t) : nullptr;
#pragma unroll
    for (int j = 0; j < kColumns; ++j) {
      // the bias values are read again for every column, four at a time, so
      // that they are never all live next to the accumulators
      if constexpr (BIAS) asm volatile("" ::: "memory");
      float val[kQ];
#pragma unroll
      for (int g = 0; g < kQ / 4; ++g) {
        float b[4];
        bias4<BIAS>(blk, g, half, b);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int q = 4 * g + e;
          // (x + b) * s in base-2 units: the product, then the bias, then the scale
          const float x = BIAS ? T.acc[q >> 4][j][q & 15] + b[e] : T.acc[q >> 4][j][q & 15];
          if constexpr (FIXED) {
            const float ex = fast_exp2(x * a.kx);
            val[q] = -a.c2 * fast_rcp(ex + 1.0f);
          } else {
            float r;
            val[q] = final_u<CAP>(x, a.kx, 0.f, a.c1, a.c2, r);
          }
        }
      }
      if (tail) {
#pragma unroll
        for (int q = 0; q < kQ; ++q)
          if (vw + half * 4 + q_row(q) >= a.v) val[q] = kMasked;
      }
      fold_column<CAP, FIXED>(val, st[j], tgt[j], vw, half);
    }
  }
};

// One workgroup = one token tile x one contiguous range ("split") of vocab
// tiles, streamed through the tile engine; each finished logit tile is folded
// into the per-token states held in registers.  At the end of the split the
// states of the two half-waves and of the waves sharing a token are merged
// and written as one partial state per (split, token).
template <class LT, bool CAP, bool FIXED, bool BIAS>
__global__ void __launch_bounds__(LT::kThr, wgs_per_cu<LT>())
fwd_stats_kernel(const FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[LT::kLdsBytes];
  const GridPos gp =
      grouped_order(xcd_remap(blockIdx.x, gridDim.x), a.n_tok_tiles, a.n_splits, a.win_tt,
                    a.tt_fastest, window_wgs<LT>());
  const int tt = gp.tt, sp = gp.grp;
  const int n0 = tt * kLogitTileN;
  const int n_rows = a.n_dev ? *a.n_dev : a.n;   // rows computed (compacted rows first)
  if (n0 >= n_rows) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % LT::kWM, wn = wave / LT::kWM;
  const int half = lane >> 5;

  int tgt[kColumns];
  PartState st[kColumns];
#pragma unroll
  for (int j = 0; j < kColumns; ++j) {
    const int n = n0 + wn * (kLogitTileN / LT::kWN) + j * 32 + (lane & 31);
    const int64_t t = (n < n_rows) ? a.tgt[a.perm ? a.perm[n] : n] : -1;
    tgt[j] = (t >= 0 && t < a.v) ? (int)t : -(1 << 30);
    st[j] = PartState{FIXED ? 0.f : kNegInf, 0.f, 0.f, kNegInf, kNegInf, 0x7fffffff};
  }
  const int vt_begin = sp * a.tiles_per_split;
  const int ntiles = min(a.n_voc_tiles, vt_begin + a.tiles_per_split) - vt_begin;
  const Operand opA{a.w, a.hdim, vt_begin * LT::kBM, a.v, a.hdim};
  const Operand opB{a.h0, a.hdim, n0, n_rows, a.hdim};
  __shared__ __attribute__((aligned(16))) float rows[BIAS ? LT::kRowDmaBytes / 4 : 4];
  RowDma rd{};
  if constexpr (BIAS)
    rd = RowDma{dma_rsrc(a.bias, (int64_t)a.v * 4), lds_addr(reinterpret_cast<char*>(rows)),
                vt_begin * LT::kBM};
  FwdEpilogue<LT, CAP, FIXED, BIAS> epi{a, st, tgt, rows, vt_begin, wm, half};
  LT T;
  T.template run_stream<BIAS>(lds, opA, opB, a.hdim, ntiles, epi, rd);

#pragma unroll
  for (int j = 0; j < kColumns; ++j) {
    if constexpr (FIXED) {
      // back from d = u - c*log2e to the reference m = c*log2e
      st[j].m = a.c1;
      st[j].t = fmaf(a.c1, st[j].s, st[j].t);
      st[j].bu += a.c1;
      st[j].zt += a.c1;
    }
    st[j] = merge_state(st[j], shfl_xor_state(st[j], 32));
  }
  // the waves wm = 1 .. kWM-1 of a token column hand their states to wave
  // wm = 0, which merges them in increasing wm (vocabulary) order
  PartState* sh = reinterpret_cast<PartState*>(lds);
  static_assert((LT::kWM - 1) * LT::kWN * kColumns * 32 * sizeof(PartState) <= LT::kLdsBytes,
                "merge buffer");
  if (wm > 0 && half == 0) {
#pragma unroll
    for (int j = 0; j < kColumns; ++j)
      sh[(((wm - 1) * LT::kWN + wn) * kColumns + j) * 32 + lane] = st[j];
  }
  __syncthreads();
  if (wm == 0 && half == 0) {
#pragma unroll
    for (int j = 0; j < kColumns; ++j) {
      PartState o = st[j];
#pragma unroll
      for (int w = 1; w < LT::kWM; ++w)
        o = merge_state(o, sh[(((w - 1) * LT::kWN + wn) * kColumns + j) * 32 + lane]);
      const int n = n0 + wn * (kLogitTileN / LT::kWN) + j * 32 + lane;
      if (n < n_rows) a.part[(int64_t)sp * a.n + n] = o;
    }
  }
}

// ------------------------------------------------------- forward: K2 merge
// 32 threads (half a wave) per token merge interleaved subsets of the splits
// (split sub, sub + 32, ...), then a fixed xor tree merges the 32 partial
// states; the first thread of each token derives lse, loss, entropy, argmax
// and hit.  Each block writes fixed-order partial sums for the reductions.
constexpr int kMergeLanes = 256 / kFinalTokens;
static_assert(kMergeLanes == 32, "a token's merge lanes are one half-wave");

__global__ void __launch_bounds__(256)
fwd_finalize_kernel(const FinalArgs a) {
  const int sub = threadIdx.x % kMergeLanes;
  const int n = blockIdx.x * kFinalTokens + threadIdx.x / kMergeLanes;   // compact row
  const int n_rows = a.n_dev ? *a.n_dev : a.n;
  PartState st{kNegInf, 0.f, 0.f, kNegInf, kNegInf, 0x7fffffff};
  if (n < n_rows) {
    int s = sub;
    // four loads in flight before they are merged, in split order
    for (; s + 3 * kMergeLanes < a.n_splits; s += 4 * kMergeLanes) {
      PartState q[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) q[i] = a.part[(int64_t)(s + i * kMergeLanes) * a.n + n];
#pragma unroll
      for (int i = 0; i < 4; ++i) st = merge_state(st, q[i]);
    }
    for (; s < a.n_splits; s += kMergeLanes) st = merge_state(st, a.part[(int64_t)s * a.n + n]);
  }
#pragma unroll
  for (int m = 1; m < kMergeLanes; m <<= 1) st = merge_state(st, shfl_xor_state(st, m));

  double l_sum = 0.0, e_sum = 0.0;
  int nv = 0, nc = 0, nb = 0;
  if (n < a.n && sub == 0 && n >= n_rows) {
    // a row left out by the row compaction: no loss, no statistics
    const int row = a.perm[n];
    a.loss[row] = 0.f;
    a.lse[row] = 0.f;
    a.entropy[row] = 0.f;
    a.hit[row] = 0;
    if (a.argmax) a.argmax[row] = -1;
  } else if (n < a.n && sub == 0) {
    const int row = a.perm ? a.perm[n] : n;
    const float lse2 = st.m + log2f(st.s);
    const int64_t t = a.tgt[row];
    const bool ignored = (t == a.ignore_index);
    const bool valid = !ignored && t >= 0 && t < a.v;
    float loss = 0.f, ent = 0.f;
    uint8_t hit = 0;
    if (valid) {
      const float zt = a.zt_exact ? a.zt_exact[row] : st.zt;
      loss = (lse2 - zt) * kLn2;
      ent = (lse2 - st.t / st.s) * kLn2;
      hit = (st.bi == (int)t) ? 1 : 0;
    }
    a.loss[row] = loss;
    a.lse[row] = lse2 * kLn2;
    a.entropy[row] = ent;
    a.hit[row] = hit;
    if (a.argmax) a.argmax[row] = st.bi;
    l_sum = loss;
    e_sum = ent;
    nv = valid;
    nc = hit;
    nb = (!ignored && !valid);
  }
  // the block's tokens in order (one value per token, from its first lane)
  __shared__ double sl[kFinalTokens], se[kFinalTokens];
  __shared__ int sv[kFinalTokens], sc[kFinalTokens], sb[kFinalTokens];
  if (sub == 0) {
    const int k = threadIdx.x / kMergeLanes;
    sl[k] = l_sum;
    se[k] = e_sum;
    sv[k] = nv;
    sc[k] = nc;
    sb[k] = nb;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    BlockSums r{0.0, 0.0, 0, 0, 0, 0};
    for (int k = 0; k < kFinalTokens; ++k) {
      r.loss += sl[k];
      r.entropy += se[k];
      r.n_valid += sv[k];
      r.n_correct += sc[k];
      r.n_bad += sb[k];
    }
    a.block_sums[blockIdx.x] = r;
  }
}

// The block sums in a fixed order: thread i adds blocks i, i + 256, ... in
// sequence, then a fixed tree adds the 256 thread sums.
constexpr int kReduceThreads = 256;

__global__ void __launch_bounds__(kReduceThreads)
fwd_reduce_kernel(const BlockSums* __restrict__ bs, int nblocks, float mean_divisor,
                  float* __restrict__ red_f32, int64_t* __restrict__ red_i64,
                  const int* __restrict__ n_bad_extra) {
  double l = 0.0, e = 0.0;
  int64_t nv = 0, nc = 0, nb = 0;
  for (int i = threadIdx.x; i < nblocks; i += kReduceThreads) {
    l += bs[i].loss;
    e += bs[i].entropy;
    nv += bs[i].n_valid;
    nc += bs[i].n_correct;
    nb += bs[i].n_bad;
  }
  __shared__ double sl[kReduceThreads], se[kReduceThreads];
  __shared__ int64_t sv[kReduceThreads], sc[kReduceThreads], sb[kReduceThreads];
  sl[threadIdx.x] = l;
  se[threadIdx.x] = e;
  sv[threadIdx.x] = nv;
  sc[threadIdx.x] = nc;
  sb[threadIdx.x] = nb;
  __syncthreads();
  for (int w = kReduceThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      sl[threadIdx.x] += sl[threadIdx.x + w];
      se[threadIdx.x] += se[threadIdx.x + w];
      sv[threadIdx.x] += sv[threadIdx.x + w];
      sc[threadIdx.x] += sc[threadIdx.x + w];
      sb[threadIdx.x] += sb[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
  l = sl[0];
  e = se[0];
  nv = sv[0];
  nc = sc[0];
  nb = sb[0] + (n_bad_extra ? *n_bad_extra : 0);
  const double div = mean_divisor > 0.f ? (double)mean_divisor : (double)nv;
  red_f32[0] = (float)l;
  red_f32[1] = div > 0.0 ? (float)(l / div) : 0.f;
  red_f32[2] = (float)e;
  red_i64[0] = nv;
  red_i64[1] = nc;
  red_i64[2] = nb;
}

// --------------------------------------------------- backward: dz recompute
// Recomputes logit tiles and writes the fp32 chain-ruled gradient w.r.t. the
// raw product, rounded to bf16, into a vocabulary chunk of the workspace:
// dz[n, v] = g_n * s * (p - [v == t_n]) * (softcap ? 1 - tanh^2 : 1).
__device__ __forceinline__ float row_grad(const DzArgs& a, int n, int64_t t) {
  if (n >= a.n) return 0.f;
  const bool valid = (t != a.ignore_index) && t >= 0 && t < a.v;
  if (!valid) return 0.f;
  float g;
  if (a.mode == 2) {
    g = a.grad_out[n];
  } else if (a.mode == 1) {
    g = a.grad_out[0];
  } else {
    const float div = a.mean_divisor > 0.f ? a.mean_divisor : (float)a.red_i64[0];
    g = div > 0.f ? a.grad_out[0] / div : 0.f;
  }
  return g * a.scale;
}

template <class LT, bool CAP, bool BIAS>
struct DzEpilogue {
  // The finished tile is transposed through a free LDS stage so that every
  // store covers whole 128-byte rows of dz (8 lanes per token).
  static constexpr bool kUsesLds = true;
  const DzArgs& a;
  const float (&gs)[kColumns];     // g_n * s (times 4 with softcap: the slope is 4 r (1-r))
  const float (&nl)[kColumns];     // -lse_n in base-2 units
  const int (&tgt)[kColumns];
  const float* rows;               // row-DMA buffers of the bias (BIAS)
  int vt_begin, wm, half, nbase;   // nbase: first token of the wave's columns

  __device__ __forceinline__ void operator()(int t, LT& T, char* free_lds) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int v0 = a.c0 + (vt_begin + t) * LT::kBM;
    const int vw = __builtin_amdgcn_readfirstlane(v0 + wm * kWaveRows);
    const bool tail = v0 + LT::kBM > a.v;
    const float* blk = BIAS ? bias_block<LT>(rows, t) : nullptr;
    // [32 tokens][64 vocabulary rows] bf16 of this wave; the 8-byte piece p of
    // token row tl is stored at piece p ^ (tl / 2), which keeps both the
    // 8-byte writes and the 16-byte reads below free of bank conflicts
    char* buf = free_lds + wave * (32 * kWaveRows * 2);
    // stores: base at row nbase of the chunk, bounded by the end of row N-1,
    // so stores of rows >= N are dropped
    const uint32_t ld_bytes = (uint32_t)a.ldz * 2;
    const __amdgpu_buffer_rsrc_t out =
        tile_rsrc(a.dz + (int64_t)nbase * a.ldz, (int64_t)(a.n - nbase) * ld_bytes);
    // kRowLanes lanes store one token's kWaveRows values, 16 bytes each
    constexpr int kRowLanes = kWaveRows * 2 / 16, kPassRows = 64 / kRowLanes;
    const uint32_t voff = (uint32_t)(lane / kRowLanes) * ld_bytes + (lane % kRowLanes) * 16 +
                          (vw - a.c0) * 2;
    // grad_bias: this wave's column sums of the stored (bf16) dz over its 128
    // tokens; lane l sums vocabulary rows 8 (l % 8) .. 8 (l % 8) + 7 of the slab
    // over the token rows it stores
    const bool cs = BIAS && a.cs_part != nullptr;
    float csum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kColumns; ++j) {
      // the bias values are read again for every column, four at a time, so
      // that they are never all live next to the accumulators
      if constexpr (BIAS) asm volatile("" ::: "memory");
      float d[kQ];
#pragma unroll
      for (int g = 0; g < kQ / 4; ++g) {
        float b[4];
        // with a bias, one group's reads at a time (the scheduler would
        // otherwise hoist all eight and spill)
        if constexpr (BIAS) __builtin_amdgcn_sched_barrier(0);
        bias4<BIAS>(blk, g, half, b);
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int q = 4 * g + e4;
          const float x = BIAS ? T.acc[q >> 4][j][q & 15] + b[e4] : T.acc[q >> 4][j][q & 15];
          if constexpr (CAP) {
            const float e = fast_exp2(x * a.kx);
            const float r = fast_rcp(e + 1.0f);
            const float p = fast_exp2(fmaf(-a.c2, r, a.c1 + nl[j]));
            d[q] = p * (fmaf(-r, r, r) * gs[j]);     // g s p (1 - tanh^2), gs carries the 4
          } else {
            d[q] = fast_exp2(fmaf(x, a.kx, nl[j])) * gs[j];
          }
        }
      }
      // one-hot term, only in lanes whose target row is one of their rows
      {
        const int rel = tgt[j] - vw - half * 4;
        if (rel >= 0 && rel < kWaveRows && (rel & 4) == 0) {
          const float bt = BIAS ? blk[rel + half * 4] : 0.f;
#pragma unroll
          for (int q = 0; q < kQ; ++q)
            if (q_row(q) == rel) {
              if constexpr (CAP) {
                const float x = BIAS ? T.acc[q >> 4][j][q & 15] + bt : T.acc[q >> 4][j][q & 15];
                const float e = fast_exp2(x * a.kx);
                const float r = fast_rcp(e + 1.0f);
                d[q] -= fmaf(-r, r, r) * gs[j];
              } else {
                d[q] -= gs[j];
              }
            }
        }
      }
      if (tail) {
#pragma unroll
        for (int q = 0; q < kQ; ++q)
          if (vw + half * 4 + q_row(q) >= a.v) d[q] = 0.f;
      }
      {
        const int tl = lane & 31;
        char* trow = buf + tl * (kWaveRows * 2);
#pragma unroll
        for (int g4 = 0; g4 < kQ / 4; ++g4) {
          u32x2 pk;
          pk[0] = pack_bf16x2(d[g4 * 4 + 0], d[g4 * 4 + 1]);
          pk[1] = pack_bf16x2(d[g4 * 4 + 2], d[g4 * 4 + 3]);
          const int piece = q_row(g4 * 4) / 4 + half;
          *reinterpret_cast<u32x2*>(trow + ((piece ^ (tl >> 1)) << 3)) = pk;
        }
      }
#pragma unroll
      for (int pass = 0; pass < 32 / kPassRows; ++pass) {
        const int tr = pass * kPassRows + lane / kRowLanes, c = lane % kRowLanes, f = tr >> 1;
        u32x4 x = *reinterpret_cast<const u32x4*>(buf + tr * (kWaveRows * 2) + ((c ^ (f >> 1)) << 4));
        if (f & 1) x = __builtin_shufflevector(x, x, 2, 3, 0, 1);
        // token nbase + j*32 + tr; tokens past N fall outside the descriptor
        // (the whole offset goes in the lane offset: the scalar offset is not
        // part of the range check)
        __builtin_amdgcn_raw_buffer_store_b128(x, out, voff + (j * 32 + pass * kPassRows) * ld_bytes,
                                               0, 0);
        if constexpr (BIAS) {
          if (cs) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              csum[2 * k] += __builtin_bit_cast(float, x[k] << 16);
              csum[2 * k + 1] += __builtin_bit_cast(float, x[k] & 0xffff0000u);
            }
          }
        }
      }
    }
    if constexpr (BIAS) {
      if (cs) {
        // the kPassRows token rows of a pass sit in lanes l, l + 8, ...: a fixed
        // butterfly over them, then lanes 0..7 hold the wave's sums
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          csum[e] += __shfl_xor(csum[e], 8);
          csum[e] += __shfl_xor(csum[e], 16);
          csum[e] += __shfl_xor(csum[e], 32);
        }
        static_assert(kRowLanes == 8 && kPassRows == 8, "column-sum lanes");
        if (lane < kRowLanes) {
          // one partial row per token tile and wave column: seg = nbase / 128
          const int seg = nbase / (kLogitTileN / LT::kWN);
          const int v = vw + 8 * lane;
          float* dst = a.cs_part + (int64_t)seg * a.ldz + (v - a.c0);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (v + e < a.v) dst[e] = csum[e];
        }
      }
    }
  }
};

template <class LT, bool CAP, bool BIAS>
__global__ void __launch_bounds__(LT::kThr, wgs_per_cu<LT>())
bwd_dz_kernel(const DzArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[LT::kLdsBytes];
  const int groups = (a.chunk_tiles + a.tiles_per_wg - 1) / a.tiles_per_wg;
  const GridPos gp =
      grouped_order(xcd_remap(blockIdx.x, gridDim.x), a.n_tok_tiles, groups, a.win_tt,
                    a.tt_fastest, window_wgs<LT>());
  const int tt = gp.tt, grp = gp.grp;
  const int n0 = tt * kLogitTileN;
  const int n_rows = a.n_dev ? *a.n_dev : a.n;   // rows computed (compacted rows first)
  if (n0 >= n_rows) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % LT::kWM, wn = wave / LT::kWM;
  const int half = lane >> 5;

  float gs[kColumns], nl[kColumns];
  int tgt[kColumns];
#pragma unroll
  for (int j = 0; j < kColumns; ++j) {
    const int n = n0 + wn * (kLogitTileN / LT::kWN) + j * 32 + (lane & 31);
    const bool in = n < n_rows;
    const int row = in ? (a.perm ? a.perm[n] : n) : 0;
    const int64_t t = in ? a.tgt[row] : -1;
    gs[j] = in ? row_grad(a, row, t) * (CAP ? 4.0f : 1.0f) : 0.f;
    nl[j] = in ? -a.lse[row] * kLog2e : 0.f;
    tgt[j] = (t >= 0 && t < a.v) ? (int)t : -(1 << 30);
  }
  const int vt_begin = grp * a.tiles_per_wg;
  const int ntiles = min(a.chunk_tiles, vt_begin + a.tiles_per_wg) - vt_begin;
  const Operand opA{a.w, a.hdim, a.c0 + vt_begin * LT::kBM, a.v, a.hdim};
  const Operand opB{a.h0, a.hdim, n0, n_rows, a.hdim};
  __shared__ __attribute__((aligned(16))) float rows[BIAS ? LT::kRowDmaBytes / 4 : 4];
  RowDma rd{};
  if constexpr (BIAS)
    rd = RowDma{dma_rsrc(a.bias, (int64_t)a.v * 4), lds_addr(reinterpret_cast<char*>(rows)),
                a.c0 + vt_begin * LT::kBM};
  DzEpilogue<LT, CAP, BIAS> epi{a, gs, nl, tgt, rows, vt_begin, wm, half,
                               __builtin_amdgcn_readfirstlane(n0 + wn * (kLogitTileN / LT::kWN))};
  LT T;
  T.template run_stream<BIAS>(lds, opA, opB, a.hdim, ntiles, epi, rd);
}

// ------------------------------------------- contractions over a dz chunk
// Workgroups [0, gh_wgs): grad_hidden (+)= dz[:, chunk] . W[chunk, :], split
// over the chunk's vocabulary into gh_splits partial slots.  The rest:
// grad_weight[chunk, :] = dz[:, chunk]^T . h.

// cache-policy operand of a buffer store: the non-temporal (nt) bit
constexpr int kStoreNonTemporal = 2;

template <class T>
__device__ __forceinline__ void store_tile(const T& tile, float* c, int64_t ldc, int m0, int n0,
                                           int m_bound, int n_bound, bool accumulate,
                                           bool stream = false) {
  // Rows past m_bound fall outside the descriptor (based at row m0; a tile's
  // rows stay within 2^31 bytes of it) and read zero / are dropped; columns
  // past n_bound are sent out of range per lane.  No per-element branch, and
  // the 16 old values of a 32 x 32 block are loaded together, so an
  // accumulating store costs one memory round trip per block.  `stream`
  // marks results that nothing here reads again (grad_weight rows): their
  // stores carry the non-temporal hint, which leaves fewer dirty L2 lines to
  // write back when the kernel ends.
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % T::kWM, wn = wave / T::kWM;
  const __amdgpu_buffer_rsrc_t rs =
      tile_rsrc(c + (int64_t)m0 * ldc, (int64_t)(m_bound - m0) * ldc * 4);
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
      const int n = n0 + wn * (T::kBN / T::kWN) + j * 32 + (lane & 31);
      uint32_t off[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * (T::kBM / T::kWM) + i * 32 + acc_row(r, lane);
        off[r] = n < n_bound ? (uint32_t)(m * ldc + n) * 4 : kOutOfRange;
      }
      float v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = tile.acc[i][j][r];
      if (accumulate) {
        float old[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          old[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off[r], 0, 0));
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] += old[r];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (stream)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v[r]), rs, off[r], 0,
                                                kStoreNonTemporal);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v[r]), rs, off[r], 0, 0);
      }
    }
}

template <class GH, class GW>
__global__ void __launch_bounds__(GH::kThr, wgs_per_cu<GH>())
contract_kernel(const ContractArgs a) {
  static_assert(GH::kBM == GW::kBM && GH::kBN == GW::kBN && GH::kThr == GW::kThr, "tile pair");
  __shared__ __attribute__((aligned(16))) char
      lds[GH::kLdsBytes > GW::kLdsBytes ? GH::kLdsBytes : GW::kLdsBytes];
  const int width8 = (a.width + 7) & ~7;
  // The grid is cut into units, one per grad_hidden split: the split's tiles
  // (which share its dz columns and lm_head rows) followed by a run of
  // grad_weight tile rows (the H tiles of one dz slab adjacent).  Every unit
  // carries about the same work, and the remap keeps consecutive ids on one
  // XCD, so each XCD gets whole units and its L2 serves their shared operands.
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int gh_per_unit = a.gh_m_tiles * a.n_tiles;
  const int unit_size = gh_per_unit + a.gw_rows_per_unit * a.n_tiles;
  const int unit = bid / unit_size, off = bid % unit_size;
  const int n_rows = a.n_dev ? *a.n_dev : a.n;   // dz rows in use (compacted rows first)
  if (off < gh_per_unit) {
    const int z = unit, rem = off;
    const int tm = rem / a.n_tiles, tn = rem % a.n_tiles;
    if (tm * GH::kBM >= n_rows) return;
    const int kb = z * a.gh_kps;
    const int ke = min(a.width, kb + a.gh_kps);
    const Operand opA{a.dz, a.ldz, tm * GH::kBM, n_rows, width8};
    const Operand opB{a.w, a.hdim, tn * GH::kBN, a.hdim, a.width};
    GH T;
    T.zero();
    T.run(lds, opA, opB, kb, ke);
    store_tile(T, a.gh + (int64_t)z * a.n * a.hdim, a.hdim, tm * GH::kBM, tn * GH::kBN, n_rows,
               a.hdim, a.gh_accumulate != 0);
  } else {
    const int b = off - gh_per_unit;
    const int tm = unit * a.gw_rows_per_unit + b / a.n_tiles, tn = b % a.n_tiles;
    if (tm >= a.gw_m_tiles) return;
    const Operand opA{a.dz, a.ldz, tm * GW::kBM, width8, n_rows};
    const Operand opB{a.h, a.hdim, tn * GW::kBN, a.hdim, n_rows};
    GW T;
    T.zero();
    T.run(lds, opA, opB, 0, n_rows);
    store_tile(T, a.gw, a.hdim, tm * GW::kBM, tn * GW::kBN, a.width, a.hdim, false, true);
  }
}

// out[i] = sum_z part[z][i], z in order.  With the row compaction, element i
// of compact row c goes to row perm[c], and rows c >= *n_dev are zero.
__global__ void sum_partials_kernel(const float* __restrict__ part, int nsplit, int64_t stride,
                                    float* __restrict__ out, int64_t count, int64_t hdim,
                                    const int* __restrict__ perm, const int* __restrict__ n_dev) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  int64_t o = i;
  if (perm) {
    const int64_t c = i / hdim;
    o = (int64_t)perm[c] * hdim + (i - c * hdim);
    if (c >= *n_dev) {
      out[o] = 0.f;
      return;
    }
  }
  float s = part[i];
  for (int z = 1; z < nsplit; ++z) s += part[(int64_t)z * stride + i];
  out[o] = s;
}

// grad_bias of a chunk: out[v] = sum over the partial rows written by the dz
// epilogue (one per token tile and wave column, in row order).  Rows of token
// tiles past the computed rows (row compaction) were never written and are
// not read.  More than kColsumGroup rows are summed in two fixed-order
// passes: groups of kColsumGroup rows into tmp, then the groups.
constexpr int kColsumGroup = kColsumGroupRows;
static_assert(WideTile::kWN == kColsumRowsPerTile && NarrowTile::kWN == kColsumRowsPerTile,
              "grad_bias partial rows per token tile");

// s + rows [g0, g1) of column v, added in row order; the loads of 16 rows are
// issued before their additions
__device__ __forceinline__ float add_rows(float s, const float* __restrict__ p, int64_t ld, int v,
                                          int g0, int g1) {
  int g = g0;
  for (; g + 16 <= g1; g += 16) {
    float t[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) t[k] = p[(int64_t)(g + k) * ld + v];
#pragma unroll
    for (int k = 0; k < 16; ++k) s += t[k];
  }
  for (; g < g1; ++g) s += p[(int64_t)g * ld + v];
  return s;
}

__device__ __forceinline__ int colsum_rows(int nseg, int n, const int* n_dev, int per_tile) {
  if (!n_dev) return nseg;
  const int n_rows = min(n, *n_dev);
  return min(nseg, (n_rows + kLogitTileN - 1) / kLogitTileN * per_tile);
}

__global__ void colsum_reduce_kernel(const float* __restrict__ part, int64_t ld, int nseg, int n,
                                     const int* __restrict__ n_dev, int per_tile, int width,
                                     float* __restrict__ tmp, float* __restrict__ out) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= width) return;
  const int rows = colsum_rows(nseg, n, n_dev, per_tile);
  if (!tmp) {
    out[v] = add_rows(0.f, part, ld, v, 0, rows);
    return;
  }
  const int g0 = blockIdx.y * kColsumGroup, g1 = min(rows, g0 + kColsumGroup);
  tmp[(int64_t)blockIdx.y * width + v] = add_rows(0.f, part, ld, v, g0, g1);
}

__global__ void colsum_groups_kernel(const float* __restrict__ tmp, int ngroups, int nseg, int n,
                                     const int* __restrict__ n_dev, int per_tile, int width,
                                     float* __restrict__ out) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= width) return;
  const int groups = (colsum_rows(nseg, n, n_dev, per_tile) + kColsumGroup - 1) / kColsumGroup;
  out[v] = add_rows(0.f, tmp, width, v, 0, min(groups, ngroups));
}

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0.f;
}

// ================================================================ launchers

static inline unsigned grid1(int64_t count, int block) {
  return (unsigned)((count + block - 1) / block);
}

hipError_t launch_round_bf16(const float* x, uint16_t* out, int64_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  if (count % 8 != 0) return hipErrorInvalidValue;   // whole rows of H % 8 == 0 values
  round_bf16_kernel<<<grid1(count / 8, 256), 256, 0, s>>>(x, out, count);
  return hipGetLastError();
}

hipError_t launch_target_logits(const TargetArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  target_logit_kernel<<<grid1(a.n, kTargetRowsPerBlock), 64 * kTargetRowsPerBlock, 0, s>>>(a);
  return hipGetLastError();
}

template <class LT>
static void launch_fwd_shape(const FwdArgs& a, bool cap, bool fixed_ref, unsigned grid,
                             hipStream_t s) {
  const bool bias = a.bias != nullptr;
#define FLCE_FWD(C, F, B) fwd_stats_kernel<LT, C, F, B><<<grid, LT::kThr, 0, s>>>(a)
  if (cap && fixed_ref) {
    if (bias) FLCE_FWD(true, true, true); else FLCE_FWD(true, true, false);
  } else if (cap) {
    if (bias) FLCE_FWD(true, false, true); else FLCE_FWD(true, false, false);
  } else {
    if (bias) FLCE_FWD(false, false, true); else FLCE_FWD(false, false, false);
  }
#undef FLCE_FWD
}

hipError_t launch_fwd_stats(const FwdArgs& a, bool cap, bool fixed_ref, hipStream_t s) {
  const unsigned grid = (unsigned)(a.n_tok_tiles * a.n_splits);
  if (grid == 0) return hipSuccess;
  if (a.tile_v == kWideTileV)
    launch_fwd_shape<WideTile>(a, cap, fixed_ref, grid, s);
  else if (a.tile_v == kNarrowTileV)
    launch_fwd_shape<NarrowTile>(a, cap, fixed_ref, grid, s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_fwd_finalize(const FinalArgs& a, int nblocks, float mean_divisor,
                               float* red_f32, int64_t* red_i64, const int* n_bad_extra,
                               hipStream_t s) {
  if (nblocks > 0) fwd_finalize_kernel<<<nblocks, 256, 0, s>>>(a);
  fwd_reduce_kernel<<<1, kReduceThreads, 0, s>>>(a.block_sums, nblocks, mean_divisor, red_f32,
                                                  red_i64, n_bad_extra);
  return hipGetLastError();
}

template <class LT>
static void launch_dz_shape(const DzArgs& a, bool cap, unsigned grid, hipStream_t s) {
  const bool bias = a.bias != nullptr;
#define FLCE_DZ(C, B) bwd_dz_kernel<LT, C, B><<<grid, LT::kThr, 0, s>>>(a)
  if (cap) {
    if (bias) FLCE_DZ(true, true); else FLCE_DZ(true, false);
  } else {
    if (bias) FLCE_DZ(false, true); else FLCE_DZ(false, false);
  }
#undef FLCE_DZ
}

hipError_t launch_bwd_dz(const DzArgs& a, bool cap, hipStream_t s) {
  const int groups = (a.chunk_tiles + a.tiles_per_wg - 1) / a.tiles_per_wg;
  const unsigned grid = (unsigned)(a.n_tok_tiles * groups);
  if (grid == 0) return hipSuccess;
  if (a.tile_v == kWideTileV)
    launch_dz_shape<WideTile>(a, cap, grid, s);
  else if (a.tile_v == kNarrowTileV)
    launch_dz_shape<NarrowTile>(a, cap, grid, s);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_contract(const ContractArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)(a.gh_splits *
                                   (a.gh_m_tiles * a.n_tiles + a.gw_rows_per_unit * a.n_tiles));
  if (grid == 0) return hipSuccess;
  if (a.tile_n == kGemmTileNWide)
    contract_kernel<GhTileWide, GwTileWide><<<grid, GhTileWide::kThr, 0, s>>>(a);
  else if (a.tile_n == kGemmTileNNarrow)
    contract_kernel<GhTile, GwTile><<<grid, GhTile::kThr, 0, s>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_sum_partials(const float* part, int nsplit, int64_t stride, float* out,
                               int64_t count, int64_t hdim, const int* perm, const int* n_dev,
                               hipStream_t s) {
  if (count == 0) return hipSuccess;
  sum_partials_kernel<<<grid1(count, 256), 256, 0, s>>>(part, nsplit, stride, out, count, hdim,
                                                        perm, n_dev);
  return hipGetLastError();
}

hipError_t launch_colsum(const float* part, int64_t ld, int nseg, int n, const int* n_dev,
                         int per_tile, int width, float* tmp, float* out, hipStream_t s) {
  if (width == 0) return hipSuccess;
  // 64 columns per block: a chunk's few thousand columns reach many CUs
  if (nseg <= kColsumGroup) {
    colsum_reduce_kernel<<<grid1(width, 64), 64, 0, s>>>(part, ld, nseg, n, n_dev, per_tile,
                                                         width, nullptr, out);
    return hipGetLastError();
  }
  const int ngroups = (nseg + kColsumGroup - 1) / kColsumGroup;
  const dim3 grid(grid1(width, 64), (unsigned)ngroups);
  colsum_reduce_kernel<<<grid, 64, 0, s>>>(part, ld, nseg, n, n_dev, per_tile, width, tmp, out);
  colsum_groups_kernel<<<grid1(width, 64), 64, 0, s>>>(tmp, ngroups, nseg, n, n_dev, per_tile,
                                                       width, out);
  return hipGetLastError();
}

hipError_t launch_compact(const int64_t* tgt, int n, int64_t ignore, int v, int* blk, int* cnt,
                          int* perm, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int nblk = (n + kCompactBlock - 1) / kCompactBlock;
  compact_count_kernel<<<nblk, kCompactBlock, 0, s>>>(tgt, n, ignore, v, blk, blk + nblk);
  compact_scan_kernel<<<1, kScanThreads, 0, s>>>(blk, blk + nblk, nblk, cnt);
  compact_scatter_kernel<<<nblk, kCompactBlock, 0, s>>>(tgt, n, ignore, v, blk, cnt, perm);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const uint16_t* h, const int* perm, const int* cnt, int64_t n,
                              int64_t hdim, uint16_t* out, hipStream_t s) {
  const int64_t threads = n * (hdim / 8);
  if (threads == 0) return hipSuccess;
  gather_rows_kernel<<<grid1(threads, 256), 256, 0, s>>>(h, perm, cnt, hdim, out, n);
  return hipGetLastError();
}

hipError_t launch_gather_round(const float* h, const int* perm, const int* cnt, int64_t n,
                               int64_t hdim, uint16_t* out, hipStream_t s) {
  const int64_t threads = n * (hdim / 8);
  if (threads == 0) return hipSuccess;
  gather_round_kernel<<<grid1(threads, 256), 256, 0, s>>>(h, perm, cnt, hdim, out, n);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  fill_zero_kernel<<<grid1(count, 256), 256, 0, s>>>(p, count);
  return hipGetLastError();
}

}  // namespace flce
