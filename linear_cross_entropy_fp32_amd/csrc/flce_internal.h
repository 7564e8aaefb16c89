// Internal interface between the C-ABI host layer and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

// Logit tiles (forward stats, backward dz) are 256 tokens wide, and every
// wave owns 64 vocabulary rows x 128 tokens of one.  Two shapes:
//  * narrow: 128 vocabulary rows, four waves in a 2 x 2 grid, a three-stage
//    ring (72 KB of LDS), two workgroups per CU, so that the epilogue of one
//    overlaps the K loop of the other;
//  * wide: 256 vocabulary rows, eight waves in a 4 x 2 grid, a four-stage
//    ring (128 KB), one workgroup per CU: a third fewer L2-to-LDS bytes per
//    MFMA and three slices in flight instead of two, but the eight waves
//    reach their epilogues together.
// The forward takes the wide shape from kFwdWideMinHidden on, where a tile's
// K loop (H / 32 slices) is long against its epilogue; the dz recompute takes
// it unless one wide tile's column of dz (N x 256 bf16) would not fit the
// 2^31-byte extent of a buffer descriptor (N >= 2^22).
constexpr int kLogitTileN = 256;
constexpr int kNarrowTileV = 128;
constexpr int kWideTileV = 256;
constexpr int kFwdWideMinHidden = 1024;
// Contraction tiles (grad_hidden, grad_weight): 256 output rows and either
// 128 columns (four waves in a 2 x 2 grid, a three-stage ring, two workgroups
// per CU) or 256 columns (eight waves in a 2 x 4 grid, a four-stage ring, one
// workgroup per CU); every wave owns 128 x 64 outputs.  The wide shape is
// taken when H is a multiple of 256 from kContractWideMinHidden on (at
// H = 640 a third of its last column tile would be padding).
constexpr int kGemmTileM = 256;
constexpr int kGemmTileNNarrow = 128;
constexpr int kGemmTileNWide = 256;
constexpr int kContractWideMinHidden = 1024;
constexpr int kSliceK = 32;   // K values per pipeline slice
constexpr int kFinalTokens = 8;   // tokens per block of the forward merge
// grad_bias partial rows per 256-token tile (the dz tiles' wave columns)
constexpr int kColsumRowsPerTile = 2;
constexpr int kColsumGroupRows = 256;   // rows summed per group when there are more

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
  const uint16_t* w;     // [V, H] bf16 (lm_head, or an fp32 one rounded to bf16)
  const uint16_t* h0;    // [N, H] bf16 (hidden, or fp32 hidden rounded to bf16)
  const float* bias;     // [V] or null
  const int64_t* tgt;    // [N]
  int n, hdim, v;
  float kx, c1, c2;      // see final_u()
  int tile_v;            // vocabulary rows per tile: kNarrowTileV or kWideTileV
  int n_tok_tiles, n_splits, tiles_per_split, n_voc_tiles;
  int tt_fastest;        // workgroup order (see grouped_order)
  int win_tt;            // token tiles per workgroup window (see grouped_order)
  PartState* part;       // [n_splits, N]
  // row compaction (both null without it): compact row c is row perm[c] of
  // tgt; only rows c < *n_dev are computed (the hidden rows are compacted)
  const int* perm;
  const int* n_dev;
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
  // the target logits in base-2 units [N] (by original row), computed from the
  // unrounded operands when an fp32 operand was rounded for the products; or
  // null, and the target value of the tile fold is used
  const float* zt_exact;
  // row compaction (both null without it): compact row c is row perm[c]; rows
  // c >= *n_dev get zero outputs (lse 0, argmax -1)
  const int* perm;
  const int* n_dev;
};

struct DzArgs {
  const uint16_t* w;     // [V, H] bf16 (lm_head, or an fp32 one rounded to bf16)
  const uint16_t* h0;    // [N, H] bf16 (hidden, or fp32 hidden rounded to bf16)
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
  int tile_v;            // vocabulary rows per tile: kNarrowTileV or kWideTileV
  int chunk_tiles;       // vocab tiles (tile_v rows) in the chunk
  int tiles_per_wg;      // vocab tiles streamed by one workgroup
  int n_tok_tiles;
  int tt_fastest;        // workgroup order (see grouped_order)
  int win_tt;            // token tiles per workgroup window (see grouped_order)
  uint16_t* dz;          // [N, ldz] bf16 chunk buffer
  int64_t ldz;
  // grad_bias partials (null without grad_bias): row tt * kColsumRowsPerTile + wn
  // holds the column sums of the stored dz over the 128 tokens of wave column
  // wn of token tile tt, at the chunk's vocabulary offsets; stride ldz
  float* cs_part;
  // row compaction (both null without it): dz row c belongs to row perm[c] of
  // tgt, lse and grad_out; only rows c < *n_dev are computed
  const int* perm;
  const int* n_dev;
};

// One launch per vocab chunk computes both contractions of the chunk's dz:
// the grad_hidden split-K partials and the grad_weight rows of the chunk.
struct ContractArgs {
  const uint16_t* dz;    // [N, ldz] bf16
  int64_t ldz;
  const uint16_t* w;     // lm_head rows of the chunk: w + c0 * H
  const uint16_t* h;     // [N, H] bf16 (fp32 hidden rounded to bf16)
  int n, hdim, width;    // tokens, hidden, vocab rows in the chunk
  int tile_n;            // output columns per tile: kGemmTileNNarrow or kGemmTileNWide
  int gh_splits, gh_kps, gh_m_tiles, n_tiles;
  int gw_m_tiles, gw_rows_per_unit;   // unit u: gh split u, then gw tile rows of the unit
  float* gh;             // [gh_splits, N, H] partials, or grad_hidden when gh_splits == 1
  int gh_accumulate;
  float* gw;             // grad_weight + c0 * H
  const int* n_dev;      // row compaction: only dz rows c < *n_dev are used; else null
};

// out = bf16(x) (round to nearest even) for count values (a multiple of 8;
// the pointers 16-byte aligned): fp32 hidden states or an fp32 lm_head.
hipError_t launch_round_bf16(const float* x, uint16_t* out, int64_t count, hipStream_t s);
// The exact target logit of every valid row, in base-2 units (see final_u):
// the dot product of the unrounded hidden row (bf16 or fp32) and the
// unrounded lm_head row of the target (bf16 or fp32), accumulated in double,
// then + bias, * scale, softcap.  One wave per row; rows without a loss get 0.
struct TargetArgs {
  const void* hidden;    // [N, H]
  const void* weight;    // [V, H]
  const float* bias;     // [V] or null
  const int64_t* tgt;    // [N]
  int h_f32, w_f32;
  int64_t n, hdim, v, ignore_index;
  double scale, softcap; // logit_scale; c (<= 0: none)
  float* zt;             // [N] out
};
hipError_t launch_target_logits(const TargetArgs& a, hipStream_t s);
hipError_t launch_fwd_stats(const FwdArgs& a, bool cap, bool fixed_ref, hipStream_t s);
// n_bad_extra: null, or a device count of out-of-range targets that the
// finalize did not see (rows left out by the row compaction)
hipError_t launch_fwd_finalize(const FinalArgs& a, int nblocks, float mean_divisor,
                               float* red_f32, int64_t* red_i64, const int* n_bad_extra,
                               hipStream_t s);
hipError_t launch_bwd_dz(const DzArgs& a, bool cap, hipStream_t s);
hipError_t launch_contract(const ContractArgs& a, hipStream_t s);
// out[perm[c], :] = sum_z part[z][c, :] for rows c < *n_dev and 0 for the
// other rows (perm, n_dev null: out = sum_z part[z]); rows of hdim floats.
hipError_t launch_sum_partials(const float* part, int nsplit, int64_t stride, float* out,
                               int64_t count, int64_t hdim, const int* perm, const int* n_dev,
                               hipStream_t s);
// grad_bias of one chunk from the dz epilogue's partial rows: part holds nseg
// rows (per_tile per token tile, stride ld; with row compaction only the rows
// of the computed token tiles are read); tmp, one row of width floats per
// kColsumGroupRows rows, is used when nseg exceeds kColsumGroupRows.
hipError_t launch_colsum(const float* part, int64_t ld, int nseg, int n, const int* n_dev,
                         int per_tile, int width, float* tmp, float* out, hipStream_t s);
// Row compaction (see compact_scatter_kernel): perm [N], cnt [2] = {rows that
// carry a loss, out-of-range targets}; blk: 2 * cdiv(N, 256) ints of scratch.
// Then the hidden rows of the first cnt[0] compact rows are gathered into
// out (bf16 hidden), or gathered and rounded to bf16 (fp32 hidden).
hipError_t launch_compact(const int64_t* tgt, int n, int64_t ignore, int v, int* blk, int* cnt,
                          int* perm, hipStream_t s);
hipError_t launch_gather_rows(const uint16_t* h, const int* perm, const int* cnt, int64_t n,
                              int64_t hdim, uint16_t* out, hipStream_t s);
hipError_t launch_gather_round(const float* h, const int* perm, const int* cnt, int64_t n,
                               int64_t hdim, uint16_t* out, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t count, hipStream_t s);

}  // namespace flce
