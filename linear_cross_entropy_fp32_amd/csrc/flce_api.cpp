// C-ABI host layer: argument validation, workspace planning and kernel
// dispatch.  No allocation, no synchronisation, no state between calls.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "ce_internal.h"
#include "flce.h"
#include "flce_internal.h"

namespace flce {
namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

constexpr int64_t kMaxRows = int64_t(1) << 30;
constexpr int64_t kMaxTokens = (int64_t(1) << 23) - 1;
constexpr int64_t kMaxHidden = int64_t(1) << 20;
constexpr int64_t kMaxElems = int64_t(1) << 31;      // V*H stays int32-indexable per row
// Operands read along K address a whole K extent from one buffer descriptor,
// whose byte size is kept below 2^31 (offsets at 2^31 read zero): a bf16
// hidden copy (N*H*2 bytes), an lm_head chunk (width*H*2) and a dz chunk
// (N*width*2) must each stay below it.
constexpr int64_t kMaxOperandBytes = (int64_t(1) << 31) - 1;
constexpr size_t kAlign = 256;
constexpr int64_t kTargetWgs = 2048;                 // forward workgroups: ~8 per CU
constexpr int64_t kCus = 256;
constexpr int64_t kDzWgs = kCus;                     // dz workgroups per chunk and workgroup per CU:
                                                     // one round
// ... unless that would give a workgroup more vocab tiles than this (at N =
// 16384 with 16384-row chunks: 8 tiles in two rounds measured 1% faster than
// 16 in one)
constexpr int64_t kMaxDzTilesPerWg = 8;
constexpr int64_t kDzOneTileHidden = 4096;
constexpr int64_t kMaxGhSplits = 32;                  // grad_hidden split-K slots
// bf16 dz of one backward vocab chunk.  A 128 MiB chunk stays in the 256 MB
// last-level cache (MALL) between the dz write and the contraction's two
// reads of it; it is used while it leaves the chunk at least kMinChunkWidth
// vocab rows wide, since narrower chunks unbalance the contraction (few long
// grad_weight tiles against many short grad_hidden ones).  Otherwise the
// chunk is 256 MiB.  Either way the chunk is at least N rows wide (measured:
// at N = 16384, 16384-row chunks take 10% off a step at H = 1024 and 5% at
// H = 4096 against 8192-row ones; at N = 8192, 16384 rows are slower).
constexpr int64_t kDzChunkBytes = int64_t(1) << 27;
constexpr int64_t kDzChunkBytesWide = int64_t(1) << 28;
constexpr int64_t kMinChunkWidth = 8192;
// At most this many vocabulary rows per backward chunk.  The kernels form
// buffer offsets in 32 bits: a dz row of the chunk is 2 * Vc bytes, and a
// tile reaches up to 256 rows past its base (phantom token rows past N
// included), so 256 * 2 * Vc must stay well below 2^31 (here 2^30).  Only tiny
// N reaches the cap: otherwise the 2^27..2^28-byte chunk rule is narrower.
constexpr int64_t kMaxChunkRows = int64_t(1) << 21;
constexpr int64_t kL2Bytes = int64_t(4) << 20;        // L2 of one XCD
// logit-tile workgroups one XCD (32 CUs) holds at once: two per CU of the
// narrow tile, one of the wide
constexpr int64_t window_wgs(int tile_v) { return tile_v == kWideTileV ? 32 : 64; }

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t rup(int64_t a, int64_t b) { return cdiv(a, b) * b; }
inline size_t aup(size_t a) { return (a + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int fwd_tile_v;        // vocabulary rows per forward tile (kNarrowTileV or kWideTileV)
  int dz_tile_v;         // vocabulary rows per dz tile (kNarrowTileV or kWideTileV)
  int gemm_tile_n;       // output columns per contraction tile
  int n_tok_tiles, n_voc_tiles, n_splits, tiles_per_split, fin_blocks;
  int64_t vc;            // vocab chunk width of the backward (multiple of dz_tile_v)
  int n_chunks;
  int dz_tiles_per_wg;   // vocab tiles streamed by one dz workgroup
  int gh_splits;         // split-K of the grad_hidden contraction
  int64_t gh_kps;
  int cs_rows;           // grad_bias partial rows (kColsumRowsPerTile per token tile)
  int win_tt;            // token tiles per window of the logit-tile order
  int tt_fastest;        // logit-tile workgroup order: token tile fastest when
                         // the bf16 hidden operand fits in one XCD's L2
  size_t off_hbf16, off_part, off_bsums, off_dz, off_ghpart, off_cspart, off_cstmp;
  // row compaction: perm [N] int32, cnt [2] int32, block scratch, compact
  // bf16 hidden rows [N, H] (fp32 hidden: its bf16 copy holds the compact rows)
  size_t off_perm, off_cnt, off_blk, off_hc;
  size_t off_wbf16;      // fp32 lm_head: rounded to bf16 [V, H]
  size_t off_zt;         // fp32 operand: the exact target logits [N] (forward part)
  size_t fwd_bytes, bwd_bytes, bytes;
};

int validate(const flce_problem* p) {
  if (!p) return fail(FLCE_ERR_NULL, "problem is NULL");
  if (p->compact_valid != 0 && p->compact_valid != 1)
    return fail(FLCE_ERR_ARG, "problem.compact_valid must be 0 or 1");
  if (p->reuse_prepared != 0 && p->reuse_prepared != 1)
    return fail(FLCE_ERR_ARG, "problem.reuse_prepared must be 0 or 1");
  if (p->n_tokens < 0 || p->n_tokens > kMaxTokens)
    return fail(FLCE_ERR_SHAPE, "n_tokens=%lld out of range [0, 2^23)", (long long)p->n_tokens);
  if (p->vocab < 1 || p->vocab > kMaxRows)
    return fail(FLCE_ERR_SHAPE, "vocab=%lld out of range [1, 2^30]", (long long)p->vocab);
  if (p->hidden < 8 || p->hidden > kMaxHidden || p->hidden % 8 != 0)
    return fail(FLCE_ERR_SHAPE, "hidden=%lld must be a multiple of 8 in [8, 2^20]",
                (long long)p->hidden);
  if (p->n_tokens * p->hidden * 2 > kMaxOperandBytes || p->vocab * p->hidden >= kMaxElems)
    return fail(FLCE_ERR_SHAPE, "N*H must stay below 2^30 and V*H below 2^31 elements");
  if (p->hidden_dtype != FLCE_BF16 && p->hidden_dtype != FLCE_F32)
    return fail(FLCE_ERR_DTYPE, "hidden_dtype=%d unsupported (bf16 or fp32)", p->hidden_dtype);
  if (p->weight_dtype != FLCE_BF16 && p->weight_dtype != FLCE_F32)
    return fail(FLCE_ERR_DTYPE, "weight_dtype=%d unsupported (bf16 or fp32)", p->weight_dtype);
  if (!std::isfinite(p->logit_scale))
    return fail(FLCE_ERR_ARG, "logit_scale must be finite");
  if (std::isnan(p->softcap) || std::isinf(p->softcap))
    return fail(FLCE_ERR_ARG, "softcap must be finite (<= 0 disables it)");
  if (std::isnan(p->mean_divisor) || std::isinf(p->mean_divisor))
    return fail(FLCE_ERR_ARG, "mean_divisor must be finite");
  return FLCE_OK;
}

Plan make_plan(const flce_problem* p) {
  Plan pl{};
  const int64_t n = p->n_tokens, h = p->hidden, v = p->vocab;
  pl.n_tok_tiles = (int)cdiv(n, kLogitTileN);
  pl.fwd_tile_v = h >= kFwdWideMinHidden ? kWideTileV : kNarrowTileV;
  pl.gemm_tile_n = h >= kContractWideMinHidden && h % kGemmTileNWide == 0 ? kGemmTileNWide
                                                                         : kGemmTileNNarrow;
  pl.n_voc_tiles = (int)cdiv(v, pl.fwd_tile_v);
  pl.fin_blocks = (int)cdiv(n, kFinalTokens);
  // the products read one bf16 copy of the hidden states (an fp32 one rounded)
  const int64_t hidden_bf16_bytes = n * h * 2;
  pl.tt_fastest = hidden_bf16_bytes <= kL2Bytes ? 1 : 0;
  // token tiles per window of the logit-tile order: 8 when the hidden
  // operand fits in L2 anyway; else as many as keep their hidden rows within
  // a quarter of one XCD's L2 (the rest streams lm_head tiles), so that the
  // workgroups of a window that drift apart still find them there
  const int64_t tile_bytes = hidden_bf16_bytes / std::max<int64_t>(n, 1) * kLogitTileN;
  pl.win_tt = 8;
  if (!pl.tt_fastest) {
    pl.win_tt = 1;
    while (pl.win_tt < 8 && 2 * pl.win_tt * tile_bytes <= kL2Bytes / 4) pl.win_tt *= 2;
  }
  // forward splits: about kTargetWgs workgroups, and with narrow windows at
  // least 64 / win_tt splits, so that one window of win_tt token tiles fills
  // an XCD (fewer splits would put several windows, and their token tiles'
  // hidden rows, on one XCD at once)
  int64_t splits = n > 0 ? cdiv(kTargetWgs, pl.n_tok_tiles) : 1;
  if (!pl.tt_fastest) splits = std::max<int64_t>(splits, window_wgs(pl.fwd_tile_v) / pl.win_tt);
  splits = std::max<int64_t>(1, std::min<int64_t>(splits, pl.n_voc_tiles));
  pl.tiles_per_split = (int)cdiv(pl.n_voc_tiles, splits);
  pl.n_splits = (int)cdiv(pl.n_voc_tiles, pl.tiles_per_split);

  // backward: vocab chunks of about kDzChunkBytes of bf16 dz, or of
  // kDzChunkBytesWide when the former would be narrower than kMinChunkWidth;
  // and at least N rows wide (so a grad_hidden tile's K, the chunk's rows,
  // is never shorter than a grad_weight tile's K, the N tokens), as long as
  // the chunk stays below the 2^31-byte operand limit
  auto chunk_rows = [&](int64_t dt) {
    int64_t vc = n > 0 ? (kDzChunkBytes / (2 * n)) / dt * dt : rup(v, dt);
    if (n > 0 && vc < kMinChunkWidth)
      vc = (kDzChunkBytesWide / (2 * n)) / dt * dt;
    if (n > 0) {
      vc = std::max<int64_t>(vc, rup(n, dt));
      vc = std::min<int64_t>(vc, kMaxOperandBytes / (2 * n) / dt * dt);
    }
    vc = std::min<int64_t>(vc, kMaxOperandBytes / (2 * h) / dt * dt);
    vc = std::min<int64_t>(vc, kMaxChunkRows);
    vc = std::max<int64_t>(vc, dt);
    return std::min<int64_t>(vc, rup(v, dt));
  };
  // dz tiles: 256 rows, unless one 256-row column of dz would pass the 2^31-byte
  // descriptor extent, or a chunk holds fewer 256-row tiles than there are CUs
  // (one workgroup per CU would leave CUs idle; 128-row tiles double the count)
  pl.dz_tile_v = kWideTileV;
  if (n * 2 * kWideTileV > kMaxOperandBytes ||
      pl.n_tok_tiles * cdiv(chunk_rows(kWideTileV), kWideTileV) < kCus)
    pl.dz_tile_v = kNarrowTileV;
  const int64_t dt = pl.dz_tile_v;
  const int64_t vc = chunk_rows(dt);
  pl.vc = vc;
  pl.n_chunks = (int)cdiv(v, vc);
  const int64_t chunk_tiles = vc / dt;
  // with the row compaction only the valid rows' token tiles have work, so
  // the workgroups take half as many tiles each: twice as many workgroups,
  // which keeps the GPU filled when a third of the rows carry a loss
  pl.dz_tiles_per_wg = (int)std::max<int64_t>(
      1, std::min<int64_t>(kMaxDzTilesPerWg,
                           chunk_tiles * pl.n_tok_tiles /
                               (kDzWgs * (pl.dz_tile_v == kWideTileV ? 1 : 2)) /
                               (p->compact_valid ? 2 : 1)));
  // with a large hidden operand, fewer tiles per workgroup (more vocabulary
  // groups per window) until the token tiles an XCD holds at once keep their
  // hidden rows within half of its L2
  if (!pl.tt_fastest)
    while (pl.dz_tiles_per_wg > 1 &&
           cdiv(window_wgs(pl.dz_tile_v), cdiv(chunk_tiles, pl.dz_tiles_per_wg)) * tile_bytes >
               kL2Bytes / 2)
      pl.dz_tiles_per_wg /= 2;
  // from H = 4096 on (128 K slices per tile), one tile per workgroup: at
  // N = 16384, H = 4096 two tiles per workgroup made the step 3% slower
  if (h >= kDzOneTileHidden) pl.dz_tiles_per_wg = 1;
  // grad_hidden split: its workgroups get twice the K depth of the
  // grad_weight ones (N), but at least 1024; the launch interleaves the two
  // kinds so every XCD gets the same mix, and fewer splits mean fewer partial
  // slots to update.  At most kMaxGhSplits (only small N reaches it: at
  // N = 256, V = 32000, 32 splits of K = 1000 take a step from 91 to 83 us
  // against 16; 64 cost more in the final sum over the slots)
  const int64_t width = std::min<int64_t>(vc, v);
  int64_t ghs = n > 0 ? cdiv(width, std::max<int64_t>(2 * n, 1024)) : 1;
  ghs = std::max<int64_t>(1, std::min<int64_t>(ghs, kMaxGhSplits));
  pl.gh_kps = rup(cdiv(width, ghs), kSliceK);
  pl.gh_splits = (int)cdiv(width, pl.gh_kps);

  size_t off = 0;
  pl.off_wbf16 = off;
  if (p->weight_dtype == FLCE_F32) off += aup(size_t(v) * h * 2);
  pl.off_hbf16 = off;
  if (p->hidden_dtype == FLCE_F32) off += aup(size_t(n) * h * 2);
  pl.off_perm = pl.off_cnt = pl.off_blk = pl.off_hc = off;
  if (p->compact_valid && n > 0) {
    pl.off_perm = off;
    off += aup(size_t(n) * 4);
    pl.off_cnt = off;
    off += aup(2 * 4);
    pl.off_blk = off;
    off += aup(size_t(2) * cdiv(n, 256) * 4);
    pl.off_hc = off;
    if (p->hidden_dtype == FLCE_BF16) off += aup(size_t(n) * h * 2);
  }
  const size_t shared_end = off;
  pl.off_zt = off;
  if (p->hidden_dtype == FLCE_F32 || p->weight_dtype == FLCE_F32) off += aup(size_t(n) * 4);
  pl.off_part = off;
  off += aup(size_t(pl.n_splits) * n * sizeof(PartState));
  pl.off_bsums = off;
  off += aup(size_t(std::max(pl.fin_blocks, 1)) * sizeof(BlockSums));
  pl.fwd_bytes = off;
  off = shared_end;
  pl.off_dz = off;
  off += aup(size_t(n) * vc * 2);
  pl.off_ghpart = off;
  // the split-K slots; with the row compaction also for one split, since the
  // final pass scatters the compact rows back
  if (pl.gh_splits > 1 || p->compact_valid) off += aup(size_t(pl.gh_splits) * n * h * 4);
  // grad_bias: partial rows of the dz epilogue, and with more than
  // kColsumGroupRows of them one row per group for the two-pass sum
  pl.cs_rows = (int)(int64_t(pl.n_tok_tiles) * kColsumRowsPerTile);
  pl.off_cspart = off;
  off += aup(size_t(pl.cs_rows) * vc * 4);
  pl.off_cstmp = off;
  if (pl.cs_rows > kColsumGroupRows) off += aup(size_t(cdiv(pl.cs_rows, kColsumGroupRows)) * vc * 4);
  pl.bwd_bytes = off;
  pl.bytes = std::max(pl.fwd_bytes, pl.bwd_bytes);
  return pl;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// final-logit constants (see final_u() in the kernels)
void logit_consts(const flce_problem* p, float& kx, float& c1, float& c2) {
  const double log2e = 1.4426950408889634;
  if (p->softcap > 0) {
    kx = (float)(2.0 * p->logit_scale * log2e / p->softcap);
    c1 = (float)(p->softcap * log2e);
    c2 = (float)(2.0 * p->softcap * log2e);
  } else {
    kx = (float)(p->logit_scale * log2e);
    c1 = c2 = 0.f;
  }
}

// Benchmark instrumentation: events recorded around one kernel's launches.
struct LaunchTimer {
  int kernel = -1;
  hipEvent_t const* events = nullptr;
  int n_pairs = 0, used = 0;
};
thread_local LaunchTimer g_timer;

template <class F>
hipError_t timed(int kernel, hipStream_t s, F&& launch) {
  const bool on = g_timer.kernel == kernel && g_timer.used < g_timer.n_pairs;
  if (on) {
    const hipError_t e = hipEventRecord(g_timer.events[2 * g_timer.used], s);
    if (e != hipSuccess) return e;
  }
  const hipError_t e = launch();
  if (on && e == hipSuccess) {
    const hipError_t e2 = hipEventRecord(g_timer.events[2 * g_timer.used + 1], s);
    ++g_timer.used;
    return e2;
  }
  return e;
}

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FLCE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return FLCE_OK;
}

// The bf16 operands of the products, and the row compaction when asked for:
// perm, the device count of compact rows, and the device count of the
// out-of-range targets it leaves out (all null without compaction).
struct Rows {
  const uint16_t* w0 = nullptr;   // lm_head (bf16), or an fp32 one rounded to bf16
  const uint16_t* h0 = nullptr;   // hidden (bf16), its compact rows, or fp32 rounded to bf16
  const int* perm = nullptr;
  const int* n_dev = nullptr;
  const int* n_bad = nullptr;
};

// Prepares the operands in the workspace head: an fp32 lm_head or fp32
// hidden rounded to bf16, and with compaction the scan and the gathered rows.
// launch = false only sets the pointers, to what an earlier call on the same
// workspace and inputs prepared (flce_problem.reuse_prepared).
int prepare_rows(const flce_problem* p, const Plan& pl, const void* hidden, const void* weight,
                 const int64_t* targets, char* ws, hipStream_t s, bool launch, Rows& r) {
  const int64_t n = p->n_tokens, h = p->hidden;
  int rc;
  r = Rows{};
  r.w0 = static_cast<const uint16_t*>(weight);
  if (p->weight_dtype == FLCE_F32) {
    uint16_t* wb = reinterpret_cast<uint16_t*>(ws + pl.off_wbf16);
    if (launch && (rc = hip_check(launch_round_bf16(static_cast<const float*>(weight), wb,
                                                    p->vocab * h, s),
                                  "round_weight")))
      return rc;
    r.w0 = wb;
  }
  r.h0 = static_cast<const uint16_t*>(hidden);
  if (n == 0) return FLCE_OK;
  uint16_t* hb = reinterpret_cast<uint16_t*>(ws + pl.off_hbf16);
  if (p->compact_valid) {
    int* perm = reinterpret_cast<int*>(ws + pl.off_perm);
    int* cnt = reinterpret_cast<int*>(ws + pl.off_cnt);
    int* blk = reinterpret_cast<int*>(ws + pl.off_blk);
    if (launch && (rc = hip_check(launch_compact(targets, (int)n, p->ignore_index, (int)p->vocab,
                                                 blk, cnt, perm, s),
                                  "compact")))
      return rc;
    r.perm = perm;
    r.n_dev = cnt;
    r.n_bad = cnt + 1;
    if (p->hidden_dtype == FLCE_F32) {
      if (launch && (rc = hip_check(launch_gather_round(static_cast<const float*>(hidden), perm,
                                                        cnt, n, h, hb, s),
                                    "gather_round")))
        return rc;
      r.h0 = hb;
    } else {
      uint16_t* hc = reinterpret_cast<uint16_t*>(ws + pl.off_hc);
      if (launch && (rc = hip_check(launch_gather_rows(static_cast<const uint16_t*>(hidden), perm,
                                                       cnt, n, h, hc, s),
                                    "gather_rows")))
        return rc;
      r.h0 = hc;
    }
    return FLCE_OK;
  }
  if (p->hidden_dtype == FLCE_F32) {
    if (launch && (rc = hip_check(launch_round_bf16(static_cast<const float*>(hidden), hb, n * h,
                                                    s),
                                  "round_hidden")))
      return rc;
    r.h0 = hb;
  }
  return FLCE_OK;
}

// Scratch of the allocation-free forward (flce_forward_noalloc): one copy of
// this array per GPU, held until the process ends.  Host code never uses the
// array's name as an address: the device address of each GPU's copy is looked
// up once per device (hipGetSymbolAddress, with that device current) and kept.
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that `s` belongs to.
int scratch_for_stream(hipStream_t s, void** out) {
  hipDevice_t dev = 0;
  int rc;
  if ((rc = hip_check(hipStreamGetDevice(s, &dev), "hipStreamGetDevice"))) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fail(FLCE_ERR_ARG, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    if ((rc = hip_check(hipGetDevice(&cur), "hipGetDevice"))) return rc;
    if (cur != dev && (rc = hip_check(hipSetDevice(dev), "hipSetDevice"))) return rc;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if ((rc = hip_check(e, "hipGetSymbolAddress(scratch)"))) return rc;
    if ((rc = hip_check(e2, "hipSetDevice (restore)"))) return rc;
    if (!ptr || reinterpret_cast<uintptr_t>(ptr) % kAlign != 0)
      return fail(FLCE_ERR_HIP, "scratch address %p is not 256-byte aligned", ptr);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FLCE_OK;
}

}  // namespace
}  // namespace flce

using namespace flce;

extern "C" {

int flce_abi_version(void) { return 2; }

int flce_set_timing_events(int kernel, void* const* events, int n_pairs) {
  g_err[0] = 0;
  if (kernel < FLCE_KERNEL_FWD_STATS || kernel > FLCE_KERNEL_CONTRACT || n_pairs < 0 ||
      (n_pairs > 0 && !events))
    return fail(FLCE_ERR_ARG, "invalid timing-event request");
  const int recorded = g_timer.used;
  g_timer.kernel = n_pairs > 0 ? kernel : -1;
  g_timer.events = reinterpret_cast<hipEvent_t const*>(events);
  g_timer.n_pairs = n_pairs;
  g_timer.used = 0;
  return recorded;
}

const char* flce_last_error(void) { return g_err; }

static int ce_validate(const flce_ce_problem* p) {
  if (!p) return fail(FLCE_ERR_NULL, "problem is NULL");
  if (p->reserved != 0 || p->reserved2 != 0)
    return fail(FLCE_ERR_ARG, "flce_ce_problem reserved fields must be 0");
  if (p->logits_dtype != FLCE_BF16 && p->logits_dtype != FLCE_F32)
    return fail(FLCE_ERR_DTYPE, "logits_dtype=%d unsupported (bf16 or fp32)", p->logits_dtype);
  const int64_t elem = p->logits_dtype == FLCE_F32 ? 4 : 2;
  if (p->n_rows < 0 || p->n_rows > (int64_t(1) << 31) - 1)
    return fail(FLCE_ERR_SHAPE, "n_rows=%lld out of range [0, 2^31)", (long long)p->n_rows);
  if (p->vocab < 1 || p->vocab * elem > (int64_t(1) << 31) - 1)
    return fail(FLCE_ERR_SHAPE, "vocab=%lld out of range (a row must stay below 2^31 bytes)",
                (long long)p->vocab);
  if (std::isnan(p->mean_divisor) || std::isinf(p->mean_divisor))
    return fail(FLCE_ERR_ARG, "mean_divisor must be finite");
  return FLCE_OK;
}

int flce_ce_forward(const flce_ce_problem* p, void* logits, const int64_t* targets, float* loss,
                    float* lse, float* reduced_f32, int64_t* reduced_i64, int grad_in_place,
                    void* stream) {
  g_err[0] = 0;
  int rc = ce_validate(p);
  if (rc) return rc;
  if (grad_in_place != 0 && grad_in_place != 1)
    return fail(FLCE_ERR_ARG, "grad_in_place must be 0 or 1");
  if (!reduced_f32 || !reduced_i64) return fail(FLCE_ERR_NULL, "reduced outputs are required");
  if (p->n_rows > 0 && (!logits || !targets || !loss || !lse))
    return fail(FLCE_ERR_NULL, "logits, targets, loss and lse are required");
  if ((logits && !aligned(logits, 16)) || (targets && !aligned(targets, 8)) ||
      (loss && !aligned(loss, 4)) || (lse && !aligned(lse, 4)) || !aligned(reduced_f32, 4) ||
      !aligned(reduced_i64, 8))
    return fail(FLCE_ERR_ALIGN, "logits must be 16-byte aligned, the others per dtype");
  CeArgs a{};
  a.logits = logits;
  a.grad = logits;
  a.tgt = targets;
  a.loss = loss;
  a.lse = lse;
  a.n = p->n_rows;
  a.v = p->vocab;
  a.ignore_index = p->ignore_index;
  a.grad_in_place = grad_in_place;
  return hip_check(launch_ce_forward(a, p->logits_dtype == FLCE_F32,
                                     p->mean_divisor > 0 ? p->mean_divisor : 0.f, reduced_f32,
                                     reduced_i64, reinterpret_cast<hipStream_t>(stream)),
                   "ce_forward");
}

int flce_ce_backward(const flce_ce_problem* p, void* grad_logits, const int64_t* targets,
                     const int64_t* reduced_i64, int grad_mode, const float* grad_out,
                     void* stream) {
  g_err[0] = 0;
  int rc = ce_validate(p);
  if (rc) return rc;
  if (grad_mode < FLCE_GRAD_MEAN || grad_mode > FLCE_GRAD_PER_TOKEN)
    return fail(FLCE_ERR_ARG, "grad_mode=%d invalid", grad_mode);
  if (!grad_out || !reduced_i64) return fail(FLCE_ERR_NULL, "grad_out and reduced_i64 are required");
  if (p->n_rows > 0 && (!grad_logits || !targets))
    return fail(FLCE_ERR_NULL, "grad_logits and targets are required");
  if ((grad_logits && !aligned(grad_logits, 16)) || (targets && !aligned(targets, 8)) ||
      !aligned(reduced_i64, 8) || !aligned(grad_out, 4))
    return fail(FLCE_ERR_ALIGN, "grad_logits must be 16-byte aligned, the others per dtype");
  CeBwdArgs a{};
  a.grad = grad_logits;
  a.tgt = targets;
  a.red_i64 = reduced_i64;
  a.grad_out = grad_out;
  a.n = p->n_rows;
  a.v = p->vocab;
  a.ignore_index = p->ignore_index;
  a.mode = grad_mode;
  a.mean_divisor = p->mean_divisor > 0 ? p->mean_divisor : 0.f;
  return hip_check(launch_ce_backward(a, p->logits_dtype == FLCE_F32,
                                      reinterpret_cast<hipStream_t>(stream)),
                   "ce_backward");
}

int flce_plan_info(const flce_problem* p, int64_t* out, int n_out) {
  g_err[0] = 0;
  if (!out) return fail(FLCE_ERR_NULL, "out is NULL");
  if (n_out < 0) return fail(FLCE_ERR_ARG, "n_out must be >= 0");
  const int rc = validate(p);
  if (rc) return rc;
  const Plan pl = make_plan(p);
  const int64_t v[FLCE_PLAN_FIELDS] = {
      pl.vc, pl.n_chunks, pl.n_splits, pl.tiles_per_split, pl.dz_tiles_per_wg, pl.gh_splits,
      pl.gh_kps, pl.win_tt, pl.tt_fastest, (int64_t)pl.fwd_bytes, (int64_t)pl.bwd_bytes,
      (int64_t)pl.bytes, p->n_tokens * pl.vc * 2, pl.fwd_tile_v, pl.dz_tile_v,
      pl.gemm_tile_n};
  const int k = n_out < FLCE_PLAN_FIELDS ? n_out : FLCE_PLAN_FIELDS;
  for (int i = 0; i < k; ++i) out[i] = v[i];
  return k;
}

int flce_validate(const flce_problem* p) {
  g_err[0] = 0;
  return validate(p);
}

int flce_workspace_bytes(const flce_problem* p, size_t* bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(FLCE_ERR_NULL, "bytes is NULL");
  const int rc = validate(p);
  if (rc) return rc;
  *bytes = make_plan(p).bytes;
  return FLCE_OK;
}

int flce_forward(const flce_problem* p, const void* hidden, const void* weight,
                 const float* bias, const int64_t* targets, float* loss, float* lse,
                 float* entropy, uint8_t* hit, int32_t* argmax, float* reduced_f32,
                 int64_t* reduced_i64, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  int rc = validate(p);
  if (rc) return rc;
  const int64_t n = p->n_tokens;
  if (!weight || !reduced_f32 || !reduced_i64 || !workspace)
    return fail(FLCE_ERR_NULL, "weight, reduced outputs and workspace are required");
  if (n > 0 && (!hidden || !targets || !loss || !lse || !entropy || !hit))
    return fail(FLCE_ERR_NULL, "hidden, targets and per-token outputs are required");
  if ((hidden && !aligned(hidden, 16)) || !aligned(weight, 16))
    return fail(FLCE_ERR_ALIGN, "hidden and weight must be 16-byte aligned");
  if ((bias && !aligned(bias, 4)) || (targets && !aligned(targets, 8)) ||
      (loss && !aligned(loss, 4)) || (lse && !aligned(lse, 4)) ||
      (entropy && !aligned(entropy, 4)) || (argmax && !aligned(argmax, 4)) ||
      !aligned(reduced_f32, 4) || !aligned(reduced_i64, 8))
    return fail(FLCE_ERR_ALIGN, "bias/targets/outputs misaligned for their dtype");
  if (!aligned(workspace, kAlign)) return fail(FLCE_ERR_ALIGN, "workspace must be 256-byte aligned");
  const Plan pl = make_plan(p);
  if (workspace_bytes < pl.fwd_bytes)
    return fail(FLCE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes,
                pl.fwd_bytes);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);

  Rows rows;
  if ((rc = prepare_rows(p, pl, hidden, weight, targets, ws, s, true, rows))) return rc;
  PartState* part = reinterpret_cast<PartState*>(ws + pl.off_part);
  // with an fp32 operand rounded for the products, the target logit comes from
  // the unrounded operands
  float* zt_exact = nullptr;
  if (n > 0 && (p->hidden_dtype == FLCE_F32 || p->weight_dtype == FLCE_F32)) {
    zt_exact = reinterpret_cast<float*>(ws + pl.off_zt);
    TargetArgs ta{};
    ta.hidden = hidden;
    ta.weight = weight;
    ta.bias = bias;
    ta.tgt = targets;
    ta.h_f32 = p->hidden_dtype == FLCE_F32;
    ta.w_f32 = p->weight_dtype == FLCE_F32;
    ta.n = n;
    ta.hdim = p->hidden;
    ta.v = p->vocab;
    ta.ignore_index = p->ignore_index;
    ta.scale = p->logit_scale;
    ta.softcap = p->softcap;
    ta.zt = zt_exact;
    if ((rc = hip_check(launch_target_logits(ta, s), "target_logits"))) return rc;
  }
  if (n > 0) {
    FwdArgs a{};
    a.w = rows.w0;
    a.h0 = rows.h0;
    a.bias = bias;
    a.tgt = targets;
    a.perm = rows.perm;
    a.n_dev = rows.n_dev;
    a.n = (int)n;
    a.hdim = (int)p->hidden;
    a.v = (int)p->vocab;
    logit_consts(p, a.kx, a.c1, a.c2);
    a.n_tok_tiles = pl.n_tok_tiles;
    a.n_splits = pl.n_splits;
    a.tt_fastest = pl.tt_fastest;
    a.win_tt = pl.win_tt;
    a.tiles_per_split = pl.tiles_per_split;
    a.n_voc_tiles = pl.n_voc_tiles;
    a.tile_v = pl.fwd_tile_v;
    a.part = part;
    // softcapped logits lie below c: with 2c*log2(e) <= 120 the sums can use
    // the fixed reference c (no running max) without underflowing fp32
    const bool fixed_ref = p->softcap > 0 && 2.0 * p->softcap * 1.4426950408889634 <= 120.0;
    if ((rc = hip_check(timed(FLCE_KERNEL_FWD_STATS, s,
                              [&] { return launch_fwd_stats(a, p->softcap > 0, fixed_ref, s); }),
                        "fwd_stats")))
      return rc;
  }
  FinalArgs f{};
  f.part = part;
  f.n_splits = pl.n_splits;
  f.n = (int)n;
  f.v = (int)p->vocab;
  f.tgt = targets;
  f.ignore_index = p->ignore_index;
  f.loss = loss;
  f.lse = lse;
  f.entropy = entropy;
  f.hit = hit;
  f.argmax = argmax;
  f.block_sums = reinterpret_cast<BlockSums*>(ws + pl.off_bsums);
  f.zt_exact = zt_exact;
  f.perm = rows.perm;
  f.n_dev = rows.n_dev;
  return hip_check(launch_fwd_finalize(f, pl.fin_blocks, p->mean_divisor > 0 ? p->mean_divisor : 0.f,
                                       reduced_f32, reduced_i64, rows.n_bad, s),
                   "fwd_finalize");
}

int flce_forward_noalloc(const flce_problem* p, const void* hidden, const void* weight,
                         const float* bias, const int64_t* targets, float* loss, float* lse,
                         float* entropy, uint8_t* hit, int32_t* argmax, float* reduced_f32,
                         int64_t* reduced_i64, void* stream) {
  g_err[0] = 0;
  const int rc = validate(p);
  if (rc) return rc;
  const size_t need = make_plan(p).fwd_bytes;
  if (need > kScratchBytes)
    return fail(FLCE_ERR_WORKSPACE,
                "flce_forward_noalloc: this problem needs %zu bytes of scratch, more than the "
                "%zu bytes it holds (use flce_forward with a workspace)",
                need, kScratchBytes);
  void* ws = nullptr;
  const int rc2 = scratch_for_stream(reinterpret_cast<hipStream_t>(stream), &ws);
  if (rc2) return rc2;
  return flce_forward(p, hidden, weight, bias, targets, loss, lse, entropy, hit, argmax,
                      reduced_f32, reduced_i64, ws, kScratchBytes, stream);
}

int flce_backward(const flce_problem* p, const void* hidden, const void* weight,
                  const float* bias, const int64_t* targets, const float* lse,
                  const int64_t* reduced_i64, int grad_mode, const float* grad_out,
                  float* grad_hidden, float* grad_weight, float* grad_bias, void* workspace,
                  size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  int rc = validate(p);
  if (rc) return rc;
  const int64_t n = p->n_tokens, h = p->hidden, v = p->vocab;
  if (grad_mode < FLCE_GRAD_MEAN || grad_mode > FLCE_GRAD_PER_TOKEN)
    return fail(FLCE_ERR_ARG, "grad_mode=%d invalid", grad_mode);
  if (!weight || !grad_weight || !workspace || !reduced_i64 || !grad_out)
    return fail(FLCE_ERR_NULL, "weight, grad_weight, reduced_i64, grad_out and workspace are required");
  if (n > 0 && (!hidden || !targets || !lse || !grad_hidden))
    return fail(FLCE_ERR_NULL, "hidden, targets, lse and grad_hidden are required");
  if (grad_bias && !bias) return fail(FLCE_ERR_ARG, "grad_bias given without bias");
  if ((hidden && !aligned(hidden, 16)) || !aligned(weight, 16))
    return fail(FLCE_ERR_ALIGN, "hidden and weight must be 16-byte aligned");
  if ((bias && !aligned(bias, 4)) || (targets && !aligned(targets, 8)) ||
      (lse && !aligned(lse, 4)) || !aligned(reduced_i64, 8) || !aligned(grad_out, 4) ||
      (grad_hidden && !aligned(grad_hidden, 4)) || !aligned(grad_weight, 4) ||
      (grad_bias && !aligned(grad_bias, 4)))
    return fail(FLCE_ERR_ALIGN, "inputs/outputs misaligned for their dtype");
  if (!aligned(workspace, kAlign)) return fail(FLCE_ERR_ALIGN, "workspace must be 256-byte aligned");
  const Plan pl = make_plan(p);
  if (workspace_bytes < pl.bytes)
    return fail(FLCE_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes,
                pl.bytes);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);

  if (n == 0) {
    if ((rc = hip_check(launch_fill_zero(grad_weight, v * h, s), "fill_zero"))) return rc;
    if (grad_bias && (rc = hip_check(launch_fill_zero(grad_bias, v, s), "fill_zero"))) return rc;
    return FLCE_OK;
  }

  Rows rows;
  if ((rc = prepare_rows(p, pl, hidden, weight, targets, ws, s, p->reuse_prepared == 0, rows)))
    return rc;
  const uint16_t* h0 = rows.h0;
  const bool slots = pl.gh_splits > 1 || rows.perm != nullptr;   // grad_hidden via the slots
  uint16_t* dz = reinterpret_cast<uint16_t*>(ws + pl.off_dz);
  float* ghpart = reinterpret_cast<float*>(ws + pl.off_ghpart);

  DzArgs d{};
  d.w = rows.w0;
  d.h0 = h0;
  d.bias = bias;
  d.tgt = targets;
  d.lse = lse;
  d.red_i64 = reduced_i64;
  d.grad_out = grad_out;
  d.mode = grad_mode;
  d.mean_divisor = p->mean_divisor > 0 ? p->mean_divisor : 0.f;
  d.scale = p->logit_scale;
  d.n = (int)n;
  d.hdim = (int)h;
  d.v = (int)v;
  d.ignore_index = p->ignore_index;
  logit_consts(p, d.kx, d.c1, d.c2);
  d.n_tok_tiles = pl.n_tok_tiles;
  d.tt_fastest = pl.tt_fastest;
  d.win_tt = pl.win_tt;
  d.tiles_per_wg = pl.dz_tiles_per_wg;
  d.dz = dz;
  d.ldz = pl.vc;
  d.cs_part = grad_bias ? reinterpret_cast<float*>(ws + pl.off_cspart) : nullptr;
  d.perm = rows.perm;
  d.n_dev = rows.n_dev;

  ContractArgs g{};
  g.dz = dz;
  g.ldz = pl.vc;
  g.h = h0;
  g.n = (int)n;
  g.hdim = (int)h;
  g.gh_splits = pl.gh_splits;
  g.gh_kps = (int)pl.gh_kps;
  g.tile_n = pl.gemm_tile_n;
  g.gh_m_tiles = (int)cdiv(n, kGemmTileM);
  g.n_tiles = (int)cdiv(h, pl.gemm_tile_n);
  g.gh = slots ? ghpart : grad_hidden;
  g.n_dev = rows.n_dev;

  for (int c = 0; c < pl.n_chunks; ++c) {
    const int64_t c0 = int64_t(c) * pl.vc;
    const int64_t width = std::min<int64_t>(pl.vc, v - c0);
    d.c0 = (int)c0;
    d.tile_v = pl.dz_tile_v;
    d.chunk_tiles = (int)cdiv(width, pl.dz_tile_v);
    if ((rc = hip_check(timed(FLCE_KERNEL_BWD_DZ, s,
                              [&] { return launch_bwd_dz(d, p->softcap > 0, s); }),
                        "bwd_dz")))
      return rc;

    g.w = rows.w0 + c0 * h;   // an fp32 lm_head enters grad_hidden rounded to bf16
    g.width = (int)width;
    g.gh_accumulate = c > 0;
    g.gw = grad_weight + c0 * h;
    g.gw_m_tiles = (int)cdiv(width, kGemmTileM);
    g.gw_rows_per_unit = (int)cdiv(g.gw_m_tiles, pl.gh_splits);
    if ((rc = hip_check(timed(FLCE_KERNEL_CONTRACT, s, [&] { return launch_contract(g, s); }),
                        "contract")))
      return rc;

    if (grad_bias &&
        (rc = hip_check(launch_colsum(reinterpret_cast<float*>(ws + pl.off_cspart), pl.vc,
                                      pl.cs_rows, (int)n, rows.n_dev, kColsumRowsPerTile,
                                      (int)width, reinterpret_cast<float*>(ws + pl.off_cstmp),
                                      grad_bias + c0, s),
                        "colsum")))
      return rc;
  }
  if (slots &&
      (rc = hip_check(launch_sum_partials(ghpart, pl.gh_splits, n * h, grad_hidden, n * h, h,
                                          rows.perm, rows.n_dev, s),
                      "sum_partials")))
    return rc;
  return FLCE_OK;
}

}  // extern "C"
