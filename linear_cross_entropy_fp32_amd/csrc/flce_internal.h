// Internal interface between the C-ABI host layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

// Tile shape of the logit-tile kernels (forward stats, backward dz) and of
// the contraction kernels: TM x TN blocks of 32x32 per wave, 2x2 waves.
constexpr int kTM = 2, kTN = 2;     // 128 vocab x 128 tokens
constexpr int kGM = 2, kGN = 2;     // 128 x 128 output tile
constexpr int kLogitTileV = 64 * kTM;
constexpr int kLogitTileN = 64 * kTN;
constexpr int kGemmTileM = 64 * kGM;
constexpr int kGemmTileN = 64 * kGN;

// Online softmax state of one token over a range of vocabulary rows, in base-2
// units (u = z * log2 e): running max m, S = sum 2^(u-m), T = sum 2^(u-m) u,
// best value bu at lowest index bi, target value zt (-inf when not seen).
struct PartState {
  float m, s, t, bu, zt;
  int bi;
};

struct BlockSums {
  double loss, entropy;
  int n_valid, n_correct, n_bad, pad;
};

struct FwdArgs {
  const uint16_t* w;     // [V, H] bf16
  const uint16_t* h0;    // [N, H] bf16 (hidden, or its high part)
  const uint16_t* h1;    // [N, H] bf16 low part of an fp32 hidden, or null
  const float* bias;     // [V] or null
  const int64_t* tgt;    // [N]
  int n, hdim, v;
  float kx, c1, c2;      // see final_u()
  int n_tok_tiles, n_splits, tiles_per_split, n_voc_tiles;
  PartState* part;       // [n_splits, N]
};

struct FinalArgs {
  const PartState* part;
  int n_splits, n, v;
  const int64_t* tgt;
  int64_t ignore_index;
  float* loss;
  float* lse;
  float* entropy;
  uint8_t* hit;
  int32_t* argmax;       // may be null
  BlockSums* block_sums;
};

struct DzArgs {
  const uint16_t* w;
  const uint16_t* h0;
  const uint16_t* h1;
  const float* bias;
  const int64_t* tgt;
  const float* lse;      // [N], natural log units
  const int64_t* red_i64;  // n_valid at [0]
  const float* grad_out;   // [1] or [N]
  int mode;              // 0 mean, 1 sum, 2 per token
  float mean_divisor;
  float scale;           // logit_scale
  int n, hdim, v;
  int64_t ignore_index;
  float kx, c1, c2;
  int c0;                // first vocab row of the chunk
  int n_tok_tiles;
  uint16_t* dz;          // [N, ldz] bf16 chunk buffer
  int64_t ldz;
};

struct GemmArgs {
  const uint16_t* a_ptr;
  int64_t lda;
  int a_row_bound, a_k_bound;
  const uint16_t* b_ptr;
  int64_t ldb;
  int b_row_bound, b_k_bound;
  int n_tiles;
  int k_len, k_per_split;
  float* c;
  int64_t ldc, c_split_stride;
  int m_store, n_store;
  int accumulate;
};

hipError_t launch_split_hidden(const float* h, uint16_t* hi, uint16_t* lo, int64_t count,
                               hipStream_t s);
hipError_t launch_fwd_stats(const FwdArgs& a, bool cap, hipStream_t s);
hipError_t launch_fwd_finalize(const FinalArgs& a, int nblocks, float mean_divisor,
                               float* red_f32, int64_t* red_i64, hipStream_t s);
hipError_t launch_bwd_dz(const DzArgs& a, int n_voc_tiles_chunk, bool cap, hipStream_t s);
hipError_t launch_gemm_store(const GemmArgs& a, int m_tiles, int splits, bool a_kmaj,
                             hipStream_t s);
hipError_t launch_sum_partials(const float* part, int nsplit, int64_t stride, float* out,
                               int64_t count, hipStream_t s);
hipError_t launch_colsum(const uint16_t* dz, int64_t ldz, int n_tok, int width, float* out,
                         hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t count, hipStream_t s);

}  // namespace flce
