"""CPU oracle (test infrastructure): see flce_oracle.py.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The library under linear_cross_entropy_fp32_amd/ never does.
"""
from .flce_oracle import (IGNORE_INDEX, Problem, backward, final_logits, forward,  # noqa: F401
                          grad_raw_logits, loss_value, row_grad_scale, valid_mask)
