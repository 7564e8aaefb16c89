"""CPU oracle (test infrastructure): see flce_oracle.py (the fused linear
cross-entropy) and ce_oracle.py (the standalone cross-entropy on materialised
logits).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The library under linear_cross_entropy_fp32_amd/ never does.
"""
from .flce_oracle import (IGNORE_INDEX, Problem, backward, final_logits, forward,  # noqa: F401
                          grad_raw_logits, loss_value, row_grad_scale, valid_mask)
from .ce_oracle import ce_backward, ce_forward, ce_row_scale, ce_valid  # noqa: F401,E402
