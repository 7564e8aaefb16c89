// Internal interface between the C-ABI host layer and the kernels of the
// standalone cross-entropy on materialised logits.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace flce {

struct CeArgs {
  const void* logits;    // [N, V] bf16 or fp32
  void* grad;            // [N, V] same dtype (may alias logits), written when grad_in_place
  const int64_t* tgt;    // [N]
  float* loss;           // [N]
  float* lse;            // [N]
  int64_t n, v, ignore_index;
  int grad_in_place;
};

struct CeBwdArgs {
  void* grad;            // [N, V], scaled in place
  const int64_t* tgt;    // [N]
  const int64_t* red_i64;  // n_valid at [0] (mean without a divisor)
  const float* grad_out;   // [1] or [N]
  int64_t n, v, ignore_index;
  int mode;              // 0 mean, 1 sum, 2 per row
  float mean_divisor;
};

hipError_t launch_ce_forward(const CeArgs& a, bool f32, float mean_divisor, float* red_f32,
                             int64_t* red_i64, hipStream_t s);
hipError_t launch_ce_backward(const CeBwdArgs& a, bool f32, hipStream_t s);
// true when the forward holds a row in registers (one read per element)
bool ce_rows_in_registers(int64_t v, int elem_bytes);

}  // namespace flce
