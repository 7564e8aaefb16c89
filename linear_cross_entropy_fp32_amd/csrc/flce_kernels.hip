// HIP kernels of the fused linear cross-entropy for gfx950.
//
// The method (TRL pull request "Add loss_type="cce", a fused linear
// cross-entropy loaded from the Hub", sections "What it supports" and the
// review's "Correctness" facts): the logits are the hidden x lm_head product
// accumulated in fp32, plus an fp32 bias, times logit_scale, then softcapped;
// the loss, the entropy (lse - sum p z) and the argmax all come from one pass
// over those logits, which are never stored.
//
// Units: inside the kernels a final logit z is carried as u = z * log2(e), so
// every exponential is one v_exp_f32 (2^x).  The forward keeps, per token, an
// online state (running max m, S = sum 2^(u-m), T = sum 2^(u-m) u, best value,
// best index, target value), all in base-2 units.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flce_internal.h"
#include "tile_gemm.h"

namespace flce {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

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

// Merge two online states.  Sums are rescaled to the larger running max; the
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
// `r` is returned for the backward's softcap slope 1 - tanh^2 = 4 r (1 - r).
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

// --------------------------------------------------- fp32 hidden: hi / lo split
// h = hi + lo with hi = bf16(h), lo = bf16(h - hi); the lm_head is exact in
// bf16, so two bf16 MFMA passes reproduce the fp32 product to ~2^-17.
__global__ void split_hidden_kernel(const float* __restrict__ h, uint16_t* __restrict__ hi,
                                    uint16_t* __restrict__ lo, int64_t count) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 2;
  if (i >= count) return;
  const float a = h[i];
  const float b = (i + 1 < count) ? h[i + 1] : 0.f;
  const uint32_t ph = pack_bf16x2(a, b);
  const float ah = __builtin_bit_cast(float, ph << 16);
  const float bh = __builtin_bit_cast(float, ph & 0xffff0000u);
  const uint32_t pl = pack_bf16x2(a - ah, b - bh);
  hi[i] = (uint16_t)(ph & 0xffffu);
  lo[i] = (uint16_t)(pl & 0xffffu);
  if (i + 1 < count) {
    hi[i + 1] = (uint16_t)(ph >> 16);
    lo[i + 1] = (uint16_t)(pl >> 16);
  }
}

// ------------------------------------------------------------- forward: K1
// One workgroup = one token tile x one contiguous range ("split") of vocab
// tiles.  For each vocab tile the logit tile is computed with MFMA and folded
// into the per-token online state held in registers; at the end of the split
// the states of the two half-waves and of the two waves sharing a token are
// merged and written as one partial state per (split, token).
template <int TM, int TN, bool CAP>
__global__ void __launch_bounds__(kThreads)
fwd_stats_kernel(const FwdArgs a) {
  using T = Tile<TM, TN, true, true>;
  __shared__ __attribute__((aligned(16))) char lds[T::kLdsBytes];
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int tt = bid % a.n_tok_tiles, sp = bid / a.n_tok_tiles;
  const int n0 = tt * T::BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int half = lane >> 5;

  int tgt[TN];
  PartState st[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + wn * (T::BN / 2) + j * 32 + (lane & 31);
    int64_t t = (n < a.n) ? a.tgt[n] : -1;
    tgt[j] = (t >= 0 && t < a.v) ? (int)t : -1;
    st[j] = PartState{kNegInf, 0.f, 0.f, kNegInf, kNegInf, 0x7fffffff};
  }

  const Operand opB0{a.h0, a.hdim, n0, a.n, a.hdim};
  const Operand opB1{a.h1, a.hdim, n0, a.n, a.hdim};
  const int vt_begin = sp * a.tiles_per_split;
  const int vt_end = min(a.n_voc_tiles, vt_begin + a.tiles_per_split);
  T tile;
  for (int vt = vt_begin; vt < vt_end; ++vt) {
    const int v0 = vt * T::BM;
    const Operand opA{a.w, a.hdim, v0, a.v, a.hdim};
    tile.zero();
    tile.run(lds, opA, opB0, opB1, a.h1 != nullptr, 0, a.hdim);

    const int vw = v0 + wm * (T::BM / 2);   // first vocab row of this wave
    const bool tail = (v0 + T::BM > a.v);
    // bias term per accumulator row, shared by the TN token columns
    float bk[TM][16];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = vw + i * 32 + acc_row(r, lane);
        float b = 0.f;
        if (a.bias && v < a.v) b = a.bias[v];
        bk[i][r] = b * a.kx;
      }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      float u[TM * 16];
      float mt = kNegInf;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float rr;
          float x = final_u<CAP>(tile.acc[i][j][r], a.kx, bk[i][r], a.c1, a.c2, rr);
          if (tail && vw + i * 32 + acc_row(r, lane) >= a.v) x = kNegInf;
          u[i * 16 + r] = x;
          mt = fmaxf(mt, x);
        }
      // argmax: the first (lowest-index) position holding the tile maximum
      if (mt > st[j].bu) {
        int idx = 0x7fffffff;
#pragma unroll
        for (int q = TM * 16 - 1; q >= 0; --q)
          if (u[q] == mt) idx = vw + (q >> 4) * 32 + acc_row(q & 15, lane);
        st[j].bu = mt;
        st[j].bi = idx;
      }
      // target logit: only lanes whose target row falls in this wave's rows
      {
        const int rel = tgt[j] - vw;
        if (rel >= 0 && rel < TM * 32 && ((rel >> 2) & 1) == half) {
#pragma unroll
          for (int q = 0; q < TM * 16; ++q)
            if ((q >> 4) * 32 + acc_row(q & 15, lane) == rel) st[j].zt = u[q];
        }
      }
      const float mn = fmaxf(st[j].m, mt);
      if (mn != kNegInf) {
        const float alpha = fast_exp2(st[j].m - mn);
        float s4[4] = {0.f, 0.f, 0.f, 0.f}, t4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < TM * 16; ++q) {
          const float p = fast_exp2(u[q] - mn);
          s4[q & 3] += p;
          if (tail) {
            t4[q & 3] += (u[q] != kNegInf) ? p * u[q] : 0.f;
          } else {
            t4[q & 3] = fmaf(p, u[q], t4[q & 3]);
          }
        }
        st[j].s = fmaf(st[j].s, alpha, (s4[0] + s4[1]) + (s4[2] + s4[3]));
        st[j].t = fmaf(st[j].t, alpha, (t4[0] + t4[1]) + (t4[2] + t4[3]));
        st[j].m = mn;
      }
    }
  }

  // merge the two half-waves (same token, interleaved vocab rows)
#pragma unroll
  for (int j = 0; j < TN; ++j) st[j] = merge_state(st[j], shfl_xor_state(st[j], 32));
  // merge the two waves that share a token column, then write the partial
  PartState* sh = reinterpret_cast<PartState*>(lds);
  if (wm == 1 && half == 0) {
#pragma unroll
    for (int j = 0; j < TN; ++j) sh[(wn * TN + j) * 32 + lane] = st[j];
  }
  __syncthreads();
  if (wm == 0 && half == 0) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const PartState o = merge_state(st[j], sh[(wn * TN + j) * 32 + lane]);
      const int n = n0 + wn * (T::BN / 2) + j * 32 + lane;
      if (n < a.n) a.part[(int64_t)sp * a.n + n] = o;
    }
  }
}

// ------------------------------------------------------- forward: K2 merge
// One thread per token merges the partial states of all splits in split
// order, then derives lse, loss, entropy, argmax and hit; each block writes
// fixed-order partial sums for the reductions.
__global__ void __launch_bounds__(256)
fwd_finalize_kernel(const FinalArgs a) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  double l_sum = 0.0, e_sum = 0.0;
  int nv = 0, nc = 0, nb = 0;
  if (n < a.n) {
    PartState st = a.part[n];
    for (int s = 1; s < a.n_splits; ++s) st = merge_state(st, a.part[(int64_t)s * a.n + n]);
    const float lse2 = st.m + log2f(st.s);
    const float lse = lse2 * kLn2;
    const int64_t t = a.tgt[n];
    const bool ignored = (t == a.ignore_index);
    const bool valid = !ignored && t >= 0 && t < a.v;
    float loss = 0.f, ent = 0.f;
    uint8_t hit = 0;
    if (valid) {
      loss = (lse2 - st.zt) * kLn2;
      ent = (lse2 - st.t / st.s) * kLn2;
      hit = (st.bi == (int)t) ? 1 : 0;
    }
    a.loss[n] = loss;
    a.lse[n] = lse;
    a.entropy[n] = ent;
    a.hit[n] = hit;
    if (a.argmax) a.argmax[n] = st.bi;
    l_sum = loss;
    e_sum = ent;
    nv = valid;
    nc = hit;
    nb = (!ignored && !valid);
  }
  // fixed-shape tree reduction inside the block
  __shared__ double sl[256], se[256];
  __shared__ int sv[256], sc[256], sb[256];
  sl[threadIdx.x] = l_sum;
  se[threadIdx.x] = e_sum;
  sv[threadIdx.x] = nv;
  sc[threadIdx.x] = nc;
  sb[threadIdx.x] = nb;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      sl[threadIdx.x] += sl[threadIdx.x + w];
      se[threadIdx.x] += se[threadIdx.x + w];
      sv[threadIdx.x] += sv[threadIdx.x + w];
      sc[threadIdx.x] += sc[threadIdx.x + w];
      sb[threadIdx.x] += sb[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    BlockSums bs{sl[0], se[0], sv[0], sc[0], sb[0], 0};
    a.block_sums[blockIdx.x] = bs;
  }
}

__global__ void fwd_reduce_kernel(const BlockSums* __restrict__ bs, int nblocks,
                                  float mean_divisor, float* __restrict__ red_f32,
                                  int64_t* __restrict__ red_i64) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  double l = 0.0, e = 0.0;
  int64_t nv = 0, nc = 0, nb = 0;
  for (int i = 0; i < nblocks; ++i) {
    l += bs[i].loss;
    e += bs[i].entropy;
    nv += bs[i].n_valid;
    nc += bs[i].n_correct;
    nb += bs[i].n_bad;
  }
  const double div = mean_divisor > 0.f ? (double)mean_divisor : (double)nv;
  red_f32[0] = (float)l;
  red_f32[1] = div > 0.0 ? (float)(l / div) : 0.f;
  red_f32[2] = (float)e;
  red_i64[0] = nv;
  red_i64[1] = nc;
  red_i64[2] = nb;
}

// --------------------------------------------------- backward: dz recompute
// Recomputes one logit tile and writes the fp32 chain-ruled gradient w.r.t.
// the raw product, rounded to bf16, into a vocab chunk of the workspace:
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

template <int TM, int TN, bool CAP>
__global__ void __launch_bounds__(kThreads)
bwd_dz_kernel(const DzArgs a) {
  using T = Tile<TM, TN, true, true>;
  __shared__ __attribute__((aligned(16))) char lds[T::kLdsBytes];
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int tt = bid % a.n_tok_tiles, vt = bid / a.n_tok_tiles;
  const int n0 = tt * T::BN;
  const int v0 = a.c0 + vt * T::BM;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int half = lane >> 5;

  const Operand opA{a.w, a.hdim, v0, a.v, a.hdim};
  const Operand opB0{a.h0, a.hdim, n0, a.n, a.hdim};
  const Operand opB1{a.h1, a.hdim, n0, a.n, a.hdim};
  T tile;
  tile.zero();
  tile.run(lds, opA, opB0, opB1, a.h1 != nullptr, 0, a.hdim);

  const int vw = v0 + wm * (T::BM / 2);
  const bool tail = (v0 + T::BM > a.v);
  float bk[TM][16];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int v = vw + i * 32 + acc_row(r, lane);
      float b = 0.f;
      if (a.bias && v < a.v) b = a.bias[v];
      bk[i][r] = b * a.kx;
    }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + wn * (T::BN / 2) + j * 32 + (lane & 31);
    const int64_t t = (n < a.n) ? a.tgt[n] : -1;
    const float gs = row_grad(a, n, t);
    const float lse2 = (n < a.n) ? a.lse[n] * kLog2e : 0.f;
    float d[TM * 16];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float rr;
        const float u = final_u<CAP>(tile.acc[i][j][r], a.kx, bk[i][r], a.c1, a.c2, rr);
        float p = fast_exp2(u - lse2);
        if constexpr (CAP) p *= 4.0f * rr * (1.0f - rr);
        d[i * 16 + r] = p;
      }
    // one-hot term, only where the target row is one of this lane's rows
    const int rel = (int)t - vw;
    if (t >= 0 && rel >= 0 && rel < TM * 32 && ((rel >> 2) & 1) == half) {
#pragma unroll
      for (int q = 0; q < TM * 16; ++q)
        if ((q >> 4) * 32 + acc_row(q & 15, lane) == rel) {
          float rr;
          const float u = final_u<CAP>(tile.acc[q >> 4][j][q & 15], a.kx, bk[q >> 4][q & 15],
                                       a.c1, a.c2, rr);
          (void)u;
          d[q] -= CAP ? 4.0f * rr * (1.0f - rr) : 1.0f;
        }
    }
    if (n < a.n) {
      uint16_t* row = a.dz + (int64_t)n * a.ldz;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int vl = vw + i * 32 + g4 * 8 + half * 4;   // first of 4 consecutive rows
          float x0 = d[i * 16 + g4 * 4 + 0] * gs, x1 = d[i * 16 + g4 * 4 + 1] * gs;
          float x2 = d[i * 16 + g4 * 4 + 2] * gs, x3 = d[i * 16 + g4 * 4 + 3] * gs;
          if (tail) {
            if (vl + 0 >= a.v) x0 = 0.f;
            if (vl + 1 >= a.v) x1 = 0.f;
            if (vl + 2 >= a.v) x2 = 0.f;
            if (vl + 3 >= a.v) x3 = 0.f;
          }
          u32x2 pk;
          pk[0] = pack_bf16x2(x0, x1);
          pk[1] = pack_bf16x2(x2, x3);
          *reinterpret_cast<u32x2*>(row + (vl - a.c0)) = pk;
        }
    }
  }
}

// ------------------------------------------- contractions over a dz chunk
// C[m, n] (+)= sum_k A(m, k) B(n, k) for one tile; grid.y splits K, each
// split owning its own slice of C (partials reduced later in fixed order).
template <int TM, int TN, bool A_KMAJ, bool B_KMAJ>
__global__ void __launch_bounds__(kThreads)
gemm_store_kernel(const GemmArgs a) {
  using T = Tile<TM, TN, A_KMAJ, B_KMAJ>;
  __shared__ __attribute__((aligned(16))) char lds[T::kLdsBytes];
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int tn = bid % a.n_tiles, tm = bid / a.n_tiles;
  const int m0 = tm * T::BM, n0 = tn * T::BN;
  const int kb = blockIdx.y * a.k_per_split;
  const int ke = min(a.k_len, kb + a.k_per_split);
  Operand opA{a.a_ptr, a.lda, m0, a.a_row_bound, a.a_k_bound};
  Operand opB{a.b_ptr, a.ldb, n0, a.b_row_bound, a.b_k_bound};
  T tile;
  tile.zero();
  tile.run(lds, opA, opB, opB, false, kb, ke);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  float* c = a.c + (int64_t)blockIdx.y * a.c_split_stride;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * (T::BN / 2) + j * 32 + (lane & 31);
      if (n >= a.n_store) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * (T::BM / 2) + i * 32 + acc_row(r, lane);
        if (m < a.m_store) {
          float* p = c + (int64_t)m * a.ldc + n;
          *p = a.accumulate ? (*p + tile.acc[i][j][r]) : tile.acc[i][j][r];
        }
      }
    }
}

// out[i] = sum_z part[z][i], z in order.
__global__ void sum_partials_kernel(const float* __restrict__ part, int nsplit, int64_t stride,
                                    float* __restrict__ out, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float s = part[i];
  for (int z = 1; z < nsplit; ++z) s += part[(int64_t)z * stride + i];
  out[i] = s;
}

// gb[c0 + v] = sum_n dz[n, v] for one chunk (fp32 accumulation of bf16 dz).
__global__ void colsum_kernel(const uint16_t* __restrict__ dz, int64_t ldz, int n_tok,
                              int width, float* __restrict__ out) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= width) return;
  float s0 = 0.f, s1 = 0.f;
  int n = 0;
  for (; n + 1 < n_tok; n += 2) {
    s0 += __builtin_bit_cast(float, (uint32_t)dz[(int64_t)n * ldz + v] << 16);
    s1 += __builtin_bit_cast(float, (uint32_t)dz[(int64_t)(n + 1) * ldz + v] << 16);
  }
  if (n < n_tok) s0 += __builtin_bit_cast(float, (uint32_t)dz[(int64_t)n * ldz + v] << 16);
  out[v] = s0 + s1;
}

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0.f;
}

// ================================================================ launchers

static inline unsigned grid1(int64_t count, int block) {
  return (unsigned)((count + block - 1) / block);
}

hipError_t launch_split_hidden(const float* h, uint16_t* hi, uint16_t* lo, int64_t count,
                               hipStream_t s) {
  if (count == 0) return hipSuccess;
  split_hidden_kernel<<<grid1((count + 1) / 2, 256), 256, 0, s>>>(h, hi, lo, count);
  return hipGetLastError();
}

hipError_t launch_fwd_stats(const FwdArgs& a, bool cap, hipStream_t s) {
  const unsigned grid = (unsigned)(a.n_tok_tiles * a.n_splits);
  if (grid == 0) return hipSuccess;
  if (cap) {
    fwd_stats_kernel<kTM, kTN, true><<<grid, kThreads, 0, s>>>(a);
  } else {
    fwd_stats_kernel<kTM, kTN, false><<<grid, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_finalize(const FinalArgs& a, int nblocks, float mean_divisor,
                               float* red_f32, int64_t* red_i64, hipStream_t s) {
  if (nblocks > 0) fwd_finalize_kernel<<<nblocks, 256, 0, s>>>(a);
  fwd_reduce_kernel<<<1, 64, 0, s>>>(a.block_sums, nblocks, mean_divisor, red_f32, red_i64);
  return hipGetLastError();
}

hipError_t launch_bwd_dz(const DzArgs& a, int n_voc_tiles_chunk, bool cap, hipStream_t s) {
  const unsigned grid = (unsigned)(a.n_tok_tiles * n_voc_tiles_chunk);
  if (grid == 0) return hipSuccess;
  if (cap) {
    bwd_dz_kernel<kTM, kTN, true><<<grid, kThreads, 0, s>>>(a);
  } else {
    bwd_dz_kernel<kTM, kTN, false><<<grid, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_store(const GemmArgs& a, int m_tiles, int splits, bool a_kmaj,
                             hipStream_t s) {
  dim3 grid((unsigned)(m_tiles * a.n_tiles), (unsigned)splits);
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  if (a_kmaj) {
    gemm_store_kernel<kGM, kGN, true, false><<<grid, kThreads, 0, s>>>(a);
  } else {
    gemm_store_kernel<kGM, kGN, false, false><<<grid, kThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_sum_partials(const float* part, int nsplit, int64_t stride, float* out,
                               int64_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  sum_partials_kernel<<<grid1(count, 256), 256, 0, s>>>(part, nsplit, stride, out, count);
  return hipGetLastError();
}

hipError_t launch_colsum(const uint16_t* dz, int64_t ldz, int n_tok, int width, float* out,
                         hipStream_t s) {
  if (width == 0) return hipSuccess;
  colsum_kernel<<<grid1(width, 256), 256, 0, s>>>(dz, ldz, n_tok, width, out);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  fill_zero_kernel<<<grid1(count, 256), 256, 0, s>>>(p, count);
  return hipGetLastError();
}

}  // namespace flce
