// HIP kernels of the standalone cross-entropy on materialised logits (gfx950).
//
// What is computed (Liger-Kernel pull request 1574, "Summary" items 1 and 2):
// the per-token loss lse_n - z[n, t_n] in fp32 from logits that are already
// in memory (bf16 or fp32), its reductions in a fixed order, and, in place
// of the logits, the gradient softmax(z_n) - onehot(t_n) of every row; the
// backward then scales each stored row by its upstream gradient with one
// fp32 multiply and one rounding per element, in place, with no (rows x
// vocabulary) temporary and no device-to-host synchronisation.
//
// The work is HBM-bound: the forward reads every logit once and writes every
// gradient once, the backward reads and writes every gradient once.  A row
// whose bytes fit (up to 20 x 16 bytes per thread of a 1024-thread
// workgroup, 320 KiB) is held in registers between its read and its write,
// so the forward touches HBM exactly twice per element; other rows take a
// streaming two-pass kernel that reads them twice.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ce_internal.h"

namespace flce {

namespace {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
constexpr float kLog2eCe = 1.4426950408889634f;
constexpr float kLn2Ce = 0.6931471805599453f;
constexpr float kNegInfCe = -__builtin_huge_valf();

template <class E>
struct Elem;
template <>
struct Elem<uint16_t> {   // bf16 stored as its bits
  static constexpr int kPerChunk = 8;
  __device__ static __forceinline__ float get(const u32x4v& c, int e) {
    const uint32_t w = c[e >> 1];
    return __builtin_bit_cast(float, (e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  __device__ static __forceinline__ void put(u32x4v& c, int e, float x) {
    const uint32_t b = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
    c[e >> 1] = (e & 1) ? ((c[e >> 1] & 0xffffu) | (b << 16)) : ((c[e >> 1] & 0xffff0000u) | b);
  }
  __device__ static __forceinline__ float load1(const void* p, int64_t i) {
    return __builtin_bit_cast(float, (uint32_t)static_cast<const uint16_t*>(p)[i] << 16);
  }
  __device__ static __forceinline__ void store1(void* p, int64_t i, float x) {
    static_cast<uint16_t*>(p)[i] = __builtin_bit_cast(uint16_t, (__bf16)x);
  }
};
template <>
struct Elem<float> {
  static constexpr int kPerChunk = 4;
  __device__ static __forceinline__ float get(const u32x4v& c, int e) {
    // copy the element out first: a bit_cast of a vector element lvalue reads
    // the vector's first element here
    const uint32_t w = c[e];
    return __builtin_bit_cast(float, w);
  }
  __device__ static __forceinline__ void put(u32x4v& c, int e, float x) {
    c[e] = __builtin_bit_cast(uint32_t, x);
  }
  __device__ static __forceinline__ float load1(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  __device__ static __forceinline__ void store1(void* p, int64_t i, float x) {
    static_cast<float*>(p)[i] = x;
  }
};

// (max, sum of 2^(u - max)) pairs in base-2 units, merged by rescaling to the
// larger max; an empty pair is (-inf, 0).
struct MS {
  float m, s;
};
__device__ __forceinline__ MS merge_ms(MS a, MS b) {
  const float m = fmaxf(a.m, b.m);
  if (m == kNegInfCe) return MS{m, 0.f};
  return MS{m, a.s * __builtin_amdgcn_exp2f(a.m - m) + b.s * __builtin_amdgcn_exp2f(b.m - m)};
}

// Merge of every thread's pair across the workgroup (xor tree inside each
// wave, then the waves' pairs in order); every thread gets the result.
template <int THREADS>
__device__ __forceinline__ MS block_ms(MS v, MS* sh) {
  for (int k = 32; k >= 1; k >>= 1) {
    MS o{__shfl_xor(v.m, k), __shfl_xor(v.s, k)};
    v = merge_ms(v, o);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[wave] = v;
  __syncthreads();
  MS r = sh[0];
  for (int w = 1; w < THREADS / 64; ++w) r = merge_ms(r, sh[w]);
  return r;
}

__device__ __forceinline__ bool ce_row_valid(int64_t t, int64_t ignore, int64_t v) {
  return t != ignore && t >= 0 && t < v;
}

}  // namespace

// Forward with the row held in registers: R chunks of 16 bytes per thread,
// chunk i of thread x at chunk index x + i * THREADS of the row (consecutive
// threads read consecutive 16-byte pieces).  Requires V * sizeof(E) % 16 == 0
// and V * sizeof(E) <= THREADS * R * 16.
template <class E, int THREADS, int R>
__global__ void __launch_bounds__(THREADS) ce_fwd_reg_kernel(const CeArgs a) {
  constexpr int EPC = Elem<E>::kPerChunk;
  const int64_t row = blockIdx.x;
  const int64_t row_bytes = a.v * (int64_t)sizeof(E);
  const char* src = static_cast<const char*>(a.logits) + row * row_bytes;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src), 0, (int)row_bytes, 0x00020000);
  const int64_t t = a.tgt[row];
  const bool valid = ce_row_valid(t, a.ignore_index, a.v);
  u32x4v c[R];
#pragma unroll
  for (int i = 0; i < R; ++i)
    c[i] = __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(
                                          rs, (uint32_t)(threadIdx.x + i * THREADS) * 16, 0, 0));
  const int nchunks = (int)(a.v / EPC);
  // this thread's (max, sum) in base-2 units over its in-range values
  float m = kNegInfCe;
#pragma unroll
  for (int i = 0; i < R; ++i)
    if ((int)threadIdx.x + i * THREADS < nchunks)
#pragma unroll
      for (int e = 0; e < EPC; ++e) m = fmaxf(m, Elem<E>::get(c[i], e));
  const float mu = m * kLog2eCe;
  float s = 0.f;
  if (m != kNegInfCe) {
#pragma unroll
    for (int i = 0; i < R; ++i)
      if ((int)threadIdx.x + i * THREADS < nchunks)
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          s += __builtin_amdgcn_exp2f(fmaf(Elem<E>::get(c[i], e), kLog2eCe, -mu));
  }
  __shared__ MS sh[THREADS / 64];
  const MS tot = block_ms<THREADS>(MS{mu, s}, sh);
  const float lse2 = tot.m + __builtin_amdgcn_logf(tot.s);   // log2 of sum 2^u
  // the target logit comes from the registers of the thread that read it
  // (the row may be overwritten in place right after this)
  const uint32_t tchunk = valid ? (uint32_t)(t / EPC) : 0xffffffffu;
  const int te = valid ? (int)(t % EPC) : -1;
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (threadIdx.x + i * THREADS == tchunk) {
      float zt = 0.f;
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        if (e == te) zt = Elem<E>::get(c[i], e);
      // (max - z_t) + log2 S in base-2 units: exact 0 when the row has one
      // logit, and no cancellation between a rounded lse and z_t
      a.loss[row] = ((tot.m - zt * kLog2eCe) + __builtin_amdgcn_logf(tot.s)) * kLn2Ce;
    }
  if (threadIdx.x == 0) {
    if (!valid) a.loss[row] = 0.f;
    a.lse[row] = lse2 * kLn2Ce;
  }
  if (!a.grad_in_place) return;
  // gradient softmax - onehot in place (zero rows for rows without a loss);
  // p = 2^((u - max) - log2 S), exactly 1 for a row of one logit
  const float l2s = __builtin_amdgcn_logf(tot.s);
  char* dst = static_cast<char*>(a.grad) + row * row_bytes;
  const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(dst, 0, (int)row_bytes,
                                                                      0x00020000);
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const uint32_t ci = threadIdx.x + i * THREADS;
    if ((int)ci >= nchunks) continue;
    u32x4v o = c[i];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      float g = 0.f;
      if (valid) {
        g = __builtin_amdgcn_exp2f(fmaf(Elem<E>::get(c[i], e), kLog2eCe, -tot.m) - l2s);
        if (ci == tchunk && e == te) g -= 1.0f;
      }
      Elem<E>::put(o, e, g);
    }
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4v, o), ws, ci * 16, 0, 0);
  }
}

// Forward for any row (any alignment or length): one workgroup per row, two
// passes over it (the second re-reads it to write the gradient).
constexpr int kStreamThreads = 256;
template <class E>
__global__ void __launch_bounds__(kStreamThreads) ce_fwd_stream_kernel(const CeArgs a) {
  const int64_t row = blockIdx.x;
  const int64_t base = row * a.v;
  const int64_t t = a.tgt[row];
  const bool valid = ce_row_valid(t, a.ignore_index, a.v);
  MS p{kNegInfCe, 0.f};
  for (int64_t j = threadIdx.x; j < a.v; j += kStreamThreads) {
    const float u = Elem<E>::load1(a.logits, base + j) * kLog2eCe;
    if (u > p.m) {
      p.s = p.s * __builtin_amdgcn_exp2f(p.m - u) + 1.0f;
      p.m = u;
    } else {
      p.s += __builtin_amdgcn_exp2f(u - p.m);
    }
  }
  __shared__ MS sh[kStreamThreads / 64];
  const MS tot = block_ms<kStreamThreads>(p, sh);
  const float lse2 = tot.m + __builtin_amdgcn_logf(tot.s);
  if (threadIdx.x == 0) {
    const float zt = valid ? Elem<E>::load1(a.logits, base + t) : 0.f;
    a.loss[row] = valid ? ((tot.m - zt * kLog2eCe) + __builtin_amdgcn_logf(tot.s)) * kLn2Ce : 0.f;
    a.lse[row] = lse2 * kLn2Ce;
  }
  if (!a.grad_in_place) return;
  __syncthreads();   // the target logit is read before any thread overwrites it
  const float l2s = __builtin_amdgcn_logf(tot.s);
  for (int64_t j = threadIdx.x; j < a.v; j += kStreamThreads) {
    float g = 0.f;
    if (valid) {
      g = __builtin_amdgcn_exp2f(fmaf(Elem<E>::load1(a.logits, base + j), kLog2eCe, -tot.m) -
                                 l2s);
      if (j == t) g -= 1.0f;
    }
    Elem<E>::store1(a.grad, base + j, g);
  }
}

// Reductions over the rows in a fixed order: thread x adds rows x, x + 1024,
// ... in sequence (double), then a fixed tree adds the thread sums.
constexpr int kCeReduceThreads = 1024;
__global__ void __launch_bounds__(kCeReduceThreads)
ce_reduce_kernel(const float* __restrict__ loss, const int64_t* __restrict__ tgt, int64_t n,
                 int64_t v, int64_t ignore, float mean_divisor, float* __restrict__ red_f32,
                 int64_t* __restrict__ red_i64) {
  double l = 0.0;
  int64_t nv = 0, nb = 0;
  for (int64_t i = threadIdx.x; i < n; i += kCeReduceThreads) {
    const int64_t t = tgt[i];
    const bool valid = ce_row_valid(t, ignore, v);
    l += valid ? (double)loss[i] : 0.0;
    nv += valid;
    nb += (t != ignore && !valid);
  }
  __shared__ double sl[kCeReduceThreads];
  __shared__ int64_t sv[kCeReduceThreads], sb[kCeReduceThreads];
  sl[threadIdx.x] = l;
  sv[threadIdx.x] = nv;
  sb[threadIdx.x] = nb;
  __syncthreads();
  for (int w = kCeReduceThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      sl[threadIdx.x] += sl[threadIdx.x + w];
      sv[threadIdx.x] += sv[threadIdx.x + w];
      sb[threadIdx.x] += sb[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
  const double div = mean_divisor > 0.f ? (double)mean_divisor : (double)sv[0];
  red_f32[0] = (float)sl[0];
  red_f32[1] = div > 0.0 ? (float)(sl[0] / div) : 0.f;
  red_i64[0] = sv[0];
  red_i64[1] = sb[0];
}

// Backward: grad[n, :] *= g_n in place, one fp32 multiply and one rounding
// per element; g_n = 0 on rows without a loss.
__device__ __forceinline__ float ce_row_scale(const CeBwdArgs& a, int64_t row) {
  const int64_t t = a.tgt[row];
  if (!ce_row_valid(t, a.ignore_index, a.v)) return 0.f;
  if (a.mode == 2) return a.grad_out[row];
  if (a.mode == 1) return a.grad_out[0];
  const float div = a.mean_divisor > 0.f ? a.mean_divisor : (float)a.red_i64[0];
  return div > 0.f ? a.grad_out[0] / div : 0.f;
}

// Rows of 16-byte-aligned length: one 16-byte chunk per thread per step of a
// grid-stride loop (a chunk never straddles two rows).
template <class E>
__global__ void __launch_bounds__(256) ce_bwd_chunk_kernel(const CeBwdArgs a) {
  constexpr int EPC = Elem<E>::kPerChunk;
  const int64_t chunks = a.n * a.v / EPC, per_row = a.v / EPC;
  u32x4v* g = static_cast<u32x4v*>(a.grad);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < chunks;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float s = ce_row_scale(a, i / per_row);
    u32x4v c = __builtin_nontemporal_load(g + i);
#pragma unroll
    for (int e = 0; e < EPC; ++e) Elem<E>::put(c, e, Elem<E>::get(c, e) * s);
    __builtin_nontemporal_store(c, g + i);
  }
}

template <class E>
__global__ void __launch_bounds__(256) ce_bwd_elem_kernel(const CeBwdArgs a) {
  const int64_t count = a.n * a.v;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    Elem<E>::store1(a.grad, i, Elem<E>::load1(a.grad, i) * ce_row_scale(a, i / a.v));
}

// ================================================================ launchers

namespace {
template <class E, int THREADS, int R>
bool try_reg(const CeArgs& a, hipStream_t s) {
  if (a.v * (int64_t)sizeof(E) > (int64_t)THREADS * R * 16) return false;
  ce_fwd_reg_kernel<E, THREADS, R><<<(unsigned)a.n, THREADS, 0, s>>>(a);
  return true;
}

template <class E>
void launch_fwd_rows(const CeArgs& a, hipStream_t s) {
  const bool aligned16 = (a.v * (int64_t)sizeof(E)) % 16 == 0;
  if (aligned16 && (try_reg<E, 256, 2>(a, s) || try_reg<E, 256, 4>(a, s) ||
                    try_reg<E, 256, 8>(a, s) || try_reg<E, 1024, 4>(a, s) ||
                    try_reg<E, 1024, 8>(a, s) || try_reg<E, 1024, 12>(a, s) ||
                    try_reg<E, 1024, 16>(a, s) || try_reg<E, 1024, 20>(a, s)))
    return;
  ce_fwd_stream_kernel<E><<<(unsigned)a.n, kStreamThreads, 0, s>>>(a);
}
}  // namespace

bool ce_rows_in_registers(int64_t v, int elem_bytes) {
  return (v * elem_bytes) % 16 == 0 && v * elem_bytes <= int64_t(1024) * 20 * 16;
}

hipError_t launch_ce_forward(const CeArgs& a, bool f32, float mean_divisor, float* red_f32,
                             int64_t* red_i64, hipStream_t s) {
  if (a.n > 0) {
    if (f32)
      launch_fwd_rows<float>(a, s);
    else
      launch_fwd_rows<uint16_t>(a, s);
  }
  ce_reduce_kernel<<<1, kCeReduceThreads, 0, s>>>(a.loss, a.tgt, a.n, a.v, a.ignore_index,
                                                  mean_divisor, red_f32, red_i64);
  return hipGetLastError();
}

hipError_t launch_ce_backward(const CeBwdArgs& a, bool f32, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  const int elem = f32 ? 4 : 2;
  const bool aligned16 = (a.v * elem) % 16 == 0;
  const int64_t work = aligned16 ? a.n * a.v * elem / 16 : a.n * a.v;
  const unsigned grid = (unsigned)std::min<int64_t>((work + 255) / 256, 256 * 64);
  if (aligned16) {
    if (f32)
      ce_bwd_chunk_kernel<float><<<grid, 256, 0, s>>>(a);
    else
      ce_bwd_chunk_kernel<uint16_t><<<grid, 256, 0, s>>>(a);
  } else {
    if (f32)
      ce_bwd_elem_kernel<float><<<grid, 256, 0, s>>>(a);
    else
      ce_bwd_elem_kernel<uint16_t><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace flce
