/*
 * flce.h -- C ABI of the MI355X fused linear cross-entropy library (libflce.so).
 *
 * What is computed (TRL pull request "Add loss_type="cce", a fused linear
 * cross-entropy loaded from the Hub": the description, "What it supports" and
 * the review's "Correctness" facts):
 *
 *   z_raw[n, v] = sum_k hidden[n, k] * weight[v, k]   (fp32 accumulation)
 *   z[n, v]     = softcap(logit_scale * (z_raw[n, v] + bias[v]))
 *   softcap(x)  = c * tanh(x / c) when c = softcap > 0, else x
 *   lse[n]      = log sum_v exp z[n, v]
 *   loss[n]     = lse[n] - z[n, t_n]
 *   entropy[n]  = lse[n] - sum_v p[n, v] z[n, v],  p = exp(z - lse)
 *   argmax[n]   = lowest v with z[n, v] = max_v z[n, v];  hit[n] = (argmax == t_n)
 *
 * without ever storing the (tokens x vocab) logits, plus the backward
 * grad_hidden / grad_weight / grad_bias.  By default, rows whose target
 * equals ignore_index are still projected but carry no loss and no gradient,
 * as the review's "Correctness" item 2 describes.  With compact_valid set,
 * they are left out of the work instead: see flce_problem.
 *
 * Conventions for every entry point:
 *   - all tensor pointers are DEVICE pointers, row-major and contiguous;
 *   - `stream` is a hipStream_t (passed as void*); all work is enqueued on it,
 *     nothing is synchronised and no host<->device copy is made;
 *   - the caller owns every buffer, including the workspace; the library
 *     allocates nothing and keeps no state between calls (apart from the
 *     optional per-thread benchmark timing hook below), so calls are
 *     re-entrant and the backward may be called any number of times;
 *   - outputs are overwritten, never accumulated into;
 *   - on error nothing is launched, a negative FLCE_ERR_* code is returned and
 *     flce_last_error() (thread-local) describes it.
 */
#ifndef FLCE_H_
#define FLCE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLCE_OK 0
#define FLCE_ERR_NULL (-1)      /* a required pointer is null */
#define FLCE_ERR_SHAPE (-2)     /* N < 0, H < 8, H % 8 != 0, V < 1, or a size too large:
                                   N < 2^23, N*H < 2^30, V*H < 2^31, H <= 2^20, V <= 2^30 */
#define FLCE_ERR_DTYPE (-3)     /* a dtype code other than FLCE_BF16 / FLCE_F32 */
#define FLCE_ERR_ALIGN (-4)     /* a pointer is not aligned as documented */
#define FLCE_ERR_WORKSPACE (-5) /* workspace smaller than flce_workspace_bytes() */
#define FLCE_ERR_HIP (-6)       /* a kernel launch failed */
#define FLCE_ERR_ARG (-7)       /* a scalar argument is invalid (NaN scale, bad mode, ...) */

#define FLCE_BF16 0
#define FLCE_F32 1

#define FLCE_GRAD_MEAN 0       /* grad_out[0] / divisor for every valid row */
#define FLCE_GRAD_SUM 1        /* grad_out[0] for every valid row */
#define FLCE_GRAD_PER_TOKEN 2  /* grad_out[n] for row n (reduction "none") */

typedef struct flce_problem {
  int64_t n_tokens;      /* N >= 0 rows of hidden / targets                      */
  int64_t hidden;        /* H >= 8, H % 8 == 0                                    */
  int64_t vocab;         /* V >= 1 rows of weight                                 */
  int32_t hidden_dtype;  /* FLCE_BF16 or FLCE_F32 (fp32 hidden states)            */
  int32_t weight_dtype;  /* FLCE_BF16, or FLCE_F32 (an fp32 lm_head, e.g. an fp32
                            master weight).  An fp32 operand (lm_head or hidden)
                            enters the MFMA products rounded to bf16 on the
                            device (2*V*H or 2*N*H workspace bytes), and the
                            target logit, which the loss takes directly, is
                            computed from the unrounded operands, so the
                            per-token loss stays within ~1e-4 of the fp32
                            definition at H = 4096.                            */
  float logit_scale;     /* s, finite; 1 = off                                    */
  float softcap;         /* c, final_logit_softcapping; <= 0 = off                */
  int64_t ignore_index;  /* usually -100                                          */
  float mean_divisor;    /* > 0: the mean divides by it (num_items_in_batch);
                            otherwise by n_valid.  0 valid rows -> mean 0.        */
  int32_t compact_valid; /* 0 or 1.  1 = valid-row compaction: the rows that carry
                            a loss (target in [0, V), not ignore_index) are
                            gathered on the device and only they are projected,
                            forward and backward, with no host sync, so the work
                            scales with n_valid instead of N.  The other rows get
                            loss = entropy = 0, hit = 0, lse = 0, argmax = -1
                            and grad_hidden = 0 (without compaction lse and
                            argmax are computed for every row).  The valid rows'
                            results and the gradients are the same in both
                            modes up to summation order.                        */
  int32_t reuse_prepared; /* 0 or 1, read by flce_backward.  1 = reuse the
                            operands the forward prepared in the same workspace
                            (fp32 operands rounded to bf16, and with compaction
                            the scan and the gathered rows) instead of preparing
                            them again: the workspace must be the one the
                            forward used, unchanged since, with the same
                            inputs.  0 = stateless (prepare again).             */
} flce_problem;

/* Check the problem description only (no HIP call).  0 or FLCE_ERR_*.
 * Defined by: the first TRL page's review, "Correctness" preamble (the fused
 * kernel refuses mismatched operand dtypes) and the Liger-Kernel page,
 * "Summary" (unsupported options are refused up front): an unsupported dtype,
 * shape or scalar is an error code here, before any work is queued.
 * H must be a multiple of 8 (one 16-byte bf16 load covers 8 hidden values and
 * every row starts 16-byte aligned); N*H*2 and V*H*2 bytes stay below 2^31 so
 * that one buffer descriptor addresses each operand.  A larger batch is split
 * by the caller: the loss is a sum over rows (reduction "sum", or "mean" with
 * mean_divisor = the total number of valid rows). */
int flce_validate(const flce_problem* p);

/* Bytes of device workspace one forward or backward call needs (the same
 * buffer serves both).  Returns 0 and sets *bytes (host memory) on success;
 * FLCE_ERR_NULL for a null bytes, else flce_validate's code.  The workspace
 * holds partial states and at most one backward vocabulary chunk of dz, never
 * the (tokens x vocab) logits: the first TRL page's opening description (the
 * loss of hidden @ lm_head.T without materialising the logit matrix). */
int flce_workspace_bytes(const flce_problem* p, size_t* bytes);

/* Forward: per-token loss, lse, entropy, argmax and hit, and the reductions.
 * Defined by the first TRL page ("Add loss_type="cce", a fused linear
 * cross-entropy loaded from the Hub"): "What it supports" (bias, logit_scale,
 * fp32 hidden states, final_logit_softcapping; entropy and token accuracy from
 * the same fused pass; the helper's 4-tuple) and the review's "Correctness"
 * preamble (product in the compute dtype with fp32 accumulation, then + bias
 * in fp32, then * logit_scale, then softcap; entropy = lse - sum p z; argmax
 * on the final logits), with item 2 (ignored rows still projected unless
 * compact_valid is set; validity zeroes their weight) and item 5 (an
 * all-ignored batch gives a zero loss).
 *   hidden   [N, H]  bf16 or fp32 (per p->hidden_dtype), 16-byte aligned
 *   weight   [V, H]  bf16 or fp32 (per p->weight_dtype), 16-byte aligned
 *   bias     [V]     fp32, or NULL for no bias
 *   targets  [N]     int64; ignore_index marks ignored rows; a value outside
 *                    [0, V) that is not ignore_index is treated as ignored and
 *                    counted in reduced_i64[2]
 * Outputs (all required except argmax):
 *   loss, lse, entropy [N] fp32 (loss and entropy are 0 on ignored rows; lse
 *                    is always written), hit [N] uint8, argmax [N] int32 or NULL,
 *   reduced_f32 [3]: loss_sum, loss_mean, entropy_sum (over valid rows)
 *   reduced_i64 [3]: n_valid, n_correct, n_bad_target
 * workspace: 256-byte aligned, at least the forward's part of the plan
 * (flce_plan_info field 9); flce_workspace_bytes() always suffices. */
int flce_forward(const flce_problem* p, const void* hidden, const void* weight,
                 const float* bias, const int64_t* targets, float* loss, float* lse,
                 float* entropy, uint8_t* hit, int32_t* argmax, float* reduced_f32,
                 int64_t* reduced_i64, void* workspace, size_t workspace_bytes, void* stream);

/* flce_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, outputs and errors as
 * flce_forward; the forward's partial states live in a scratch array that the
 * library holds in device memory, 16 MiB per GPU, from the first call on that
 * GPU until the process ends (the device is the one `stream` belongs to).
 * Nothing is allocated: a problem whose forward needs more than 16 MiB of
 * scratch (flce_plan_info field 9: e.g. fp32 hidden states, whose bf16 copy
 * alone is 2*N*H bytes) returns FLCE_ERR_WORKSPACE before anything is
 * launched.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race, so serialise them.
 * The first call on a device also looks the array's address up (no
 * allocation, no kernel). */
int flce_forward_noalloc(const flce_problem* p, const void* hidden, const void* weight,
                         const float* bias, const int64_t* targets, float* loss, float* lse,
                         float* entropy, uint8_t* hit, int32_t* argmax, float* reduced_f32,
                         int64_t* reduced_i64, void* stream);

/* Backward of the reduced loss: grad_hidden, grad_weight, grad_bias.
 * Defined by the first TRL page's review, "Correctness" item 2 (the backward
 * recomputes the softmax gradient d for the rows and contracts it with the
 * lm_head and the hidden states) and item 5 (an all-ignored batch still
 * produces exactly-zero gradients for every parameter), and by the Liger-Kernel
 * page, "Summary" item 2 (the per-row upstream gradient of reduction "none" is
 * one fp32 multiply per row, with no device-to-host sync and no BT x V
 * temporary).  dz is formed in fp32 and rounded to bf16 for the MFMA
 * contractions, one vocabulary chunk at a time (see flce_plan_info).
 * Ownership and errors as for flce_forward.
 *   lse [N] and reduced_i64 [3] are the forward's outputs for the same inputs
 *   (n_valid is read on the device for FLCE_GRAD_MEAN; no host sync).
 *   grad_mode: FLCE_GRAD_MEAN / FLCE_GRAD_SUM read grad_out[0];
 *              FLCE_GRAD_PER_TOKEN reads grad_out[0..N) (reduction "none").
 * Outputs (fp32, overwritten): grad_hidden [N, H], grad_weight [V, H],
 *   grad_bias [V] (may be NULL; must be NULL when bias is NULL).
 * Entropy and accuracy are logged metrics and carry no gradient. */
int flce_backward(const flce_problem* p, const void* hidden, const void* weight,
                  const float* bias, const int64_t* targets, const float* lse,
                  const int64_t* reduced_i64, int grad_mode, const float* grad_out,
                  float* grad_hidden, float* grad_weight, float* grad_bias, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Benchmark instrumentation (support, not part of the loss API; it measures
 * the kernels as the Liger-Kernel page's "Details" times them: events around
 * the launches on the caller's stream).  While set, every
 * launch of `kernel` made by this thread is bracketed by hipEventRecord of
 * events[2i] before and events[2i+1] after it, on the launch stream, for
 * i = 0 .. n_pairs-1; later launches are not recorded.  `events` holds
 * hipEvent_t handles owned by the caller and must stay valid while set.
 * kernel: FLCE_KERNEL_FWD_STATS, FLCE_KERNEL_BWD_DZ or FLCE_KERNEL_CONTRACT.
 * n_pairs = 0 clears it.  Returns the number of pairs recorded under the
 * previous setting (>= 0) or FLCE_ERR_ARG. */
#define FLCE_KERNEL_FWD_STATS 0
#define FLCE_KERNEL_BWD_DZ 1
#define FLCE_KERNEL_CONTRACT 2
int flce_set_timing_events(int kernel, void* const* events, int n_pairs);

/* ------------------------------------------------------------------------
 * Standalone cross-entropy on materialised logits (Liger-Kernel pull request
 * 1574, "Summary" items 1 and 2): for logits that are already in memory, the
 * per-token loss lse_n - z[n, t_n] in fp32, its reductions, and the gradient
 * with respect to the logits written in place of them, which the backward
 * scales row by row in place (one fp32 multiply and one rounding per
 * element: no (rows x vocabulary) temporary, no device-to-host sync).
 * The z_loss the page mentions has no formula on it and is not provided.
 */
typedef struct flce_ce_problem {
  int64_t n_rows;        /* N >= 0 rows of logits / targets                      */
  int64_t vocab;         /* V >= 1 logits per row; V * element size < 2^31       */
  int32_t logits_dtype;  /* FLCE_BF16 or FLCE_F32: logits and the gradient        */
  int32_t reserved;      /* must be 0                                            */
  int64_t ignore_index;  /* usually -100                                         */
  float mean_divisor;    /* > 0: the mean divides by it, else by n_valid          */
  int32_t reserved2;     /* must be 0                                            */
} flce_ce_problem;

/* Forward.  logits [N, V] (dtype per p->logits_dtype, 16-byte aligned) is read;
 * with grad_in_place = 1 each row is then overwritten with
 * softmax(z_n) - onehot(t_n) in the same dtype (a zero row for a row that
 * carries no loss): the gradient of sum_n loss_n, which flce_ce_backward
 * scales.  targets [N] int64 (ignore_index marks ignored rows; other values
 * outside [0, V) are ignored and counted in reduced_i64[1]).
 * Outputs (device, fp32 unless noted): loss [N] (0 on ignored rows), lse [N],
 * reduced_f32 [2]: loss_sum, loss_mean; reduced_i64 [2]: n_valid, n_bad.
 * No workspace.  Errors as for flce_forward (FLCE_ERR_* before any launch). */
int flce_ce_forward(const flce_ce_problem* p, void* logits, const int64_t* targets,
                    float* loss, float* lse, float* reduced_f32, int64_t* reduced_i64,
                    int grad_in_place, void* stream);

/* Backward, in place: grad_logits [N, V] (the forward's in-place output) row n
 * is multiplied by g_n in fp32 and rounded once to the logits dtype, with
 * g_n = grad_out[0] / divisor (FLCE_GRAD_MEAN; divisor = mean_divisor if > 0,
 * else n_valid from reduced_i64, read on the device), grad_out[0]
 * (FLCE_GRAD_SUM) or grad_out[n] (FLCE_GRAD_PER_TOKEN, reduction "none"
 * with any per-row weights); rows that carry no loss are set to 0.  The
 * stored gradient is consumed: a second call scales it again. */
int flce_ce_backward(const flce_ce_problem* p, void* grad_logits, const int64_t* targets,
                     const int64_t* reduced_i64, int grad_mode, const float* grad_out,
                     void* stream);

/* How the library tiles a problem (support; nothing is launched, no HIP
 * call).  Writes min(n_out, FLCE_PLAN_FIELDS) values to out (host memory), in
 * this order, and returns that count, or a negative FLCE_ERR_* code for an
 * invalid problem or a null out:
 *   0 chunk_rows       vocabulary rows per backward chunk (Vc, a multiple of
 *                      dz_tile_rows)
 *   1 n_chunks         backward chunks (contraction launches per backward)
 *   2 fwd_splits       vocabulary splits of the forward statistics
 *   3 fwd_tiles_per_split  vocabulary tiles (fwd_tile_rows each) per forward split
 *   4 dz_tiles_per_wg  vocabulary tiles (dz_tile_rows each) per workgroup of
 *                      the dz recompute
 *   5 gh_splits        grad_hidden split-K slots per chunk
 *   6 gh_rows_per_split  vocabulary rows per slot (a multiple of 32)
 *   7 window_token_tiles  token tiles per window of the logit order (a window
 *                      is what one XCD holds at once: 64 workgroups of the
 *                      128-row tile, 32 of the 256-row one)
 *   8 token_tile_fastest  1: windows take the token tile fastest
 *   9 fwd_workspace_bytes, 10 bwd_workspace_bytes, 11 workspace_bytes
 *  12 dz_chunk_bytes   N * chunk_rows * 2 (the largest (tokens x vocab) buffer)
 *  13 fwd_tile_rows    vocabulary rows per logit tile of the forward (128, or
 *                      256 from H = 1024 on)
 *  14 dz_tile_rows     vocabulary rows per logit tile of the dz recompute (256,
 *                      or 128 from N = 2^22 on)
 *  15 contract_tile_cols  output columns per grad_hidden / grad_weight tile
 *                      (256 when H is a multiple of 256 from 1024 on, else 128)
 * Every logit tile is 256 tokens wide; every contraction tile 256 rows high.
 */
#define FLCE_PLAN_FIELDS 16
int flce_plan_info(const flce_problem* p, int64_t* out, int n_out);

/* Description of the last error on this thread ("" if none). */
const char* flce_last_error(void);

/* Library ABI version (bumped when a signature or struct changes). */
int flce_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H_ */
