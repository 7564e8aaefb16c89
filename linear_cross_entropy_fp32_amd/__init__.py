"""MI355X fused linear cross-entropy: hidden @ lm_head.T (+ bias) * scale ->
softcap -> loss / entropy / argmax accuracy and the backward, computed by HIP
kernels in libflce.so without storing the (tokens x vocab) logits.

The library is loaded on first use; if it has not been built, the first call
raises (there is no fallback path).
"""
from ._binding import (FLCE_BF16, FLCE_F32, FLCE_GRAD_MEAN, FLCE_GRAD_PER_TOKEN,  # noqa: F401
                       FLCE_GRAD_SUM, FLCE_KERNEL_BWD_DZ, FLCE_KERNEL_CONTRACT,
                       FLCE_KERNEL_FWD_STATS, FlceError, FlceProblem, flce_backward, flce_forward,
                       flce_forward_noalloc,
                       flce_last_error, flce_plan_info, flce_set_timing_events, flce_validate,
                       flce_workspace_bytes, lib,
                       linear_cross_entropy, make_problem)
from ._binding import (FlceCeProblem, cross_entropy, flce_ce_backward,  # noqa: F401,E402
                       flce_ce_forward)
