"""CPU oracle for the standalone cross-entropy on materialised logits (test
infrastructure only: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it; the library never does).

Source: Liger-Kernel pull request 1574 ("Summary" items 1 and 2, "Details").
What it computes, restated:
  * the per-token loss is computed and reduced in fp32 (here: float64, the
    exact reference), loss_n = lse_n - z[n, t_n] for a valid row, 0 for a row
    whose target is the ignore index;
  * the gradient with respect to the logits of row n is (softmax(z_n) -
    onehot(t_n)) scaled by the row's upstream gradient g_n; for reduction
    "none" g_n is grad_output[n] (any 1-D weights: mean, sum, weighted), the
    in-place backward applies it as one multiply per element;
  * "mean" divides by the number of valid rows (or a given divisor), "sum"
    does not.
Readings where the page is silent (listed in the design notes): targets
outside [0, V) that are not the ignore index count as ignored and are
reported in n_bad, as for the fused loss; a mean over zero valid rows is 0
with a zero gradient.  The page's z_loss has no formula on it and is not
computed here (parity unpinned, not built).

Pinned by tests/test_ce_oracle_pins.py against torch's cross_entropy with
float64 autograd, closed forms and invariants.
"""
from __future__ import annotations

import numpy as np

IGNORE_INDEX = -100


def ce_valid(targets: np.ndarray, vocab: int, ignore_index: int = IGNORE_INDEX):
    t = np.asarray(targets, dtype=np.int64)
    ignored = t == ignore_index
    in_range = (t >= 0) & (t < vocab)
    return in_range & ~ignored, ~ignored & ~in_range


def ce_forward(logits: np.ndarray, targets: np.ndarray, ignore_index: int = IGNORE_INDEX,
               mean_divisor: float = 0.0) -> dict:
    """Per-token loss and lse (float64), the reductions, and the unscaled
    gradient softmax(z_n) - onehot(t_n) of every valid row (zero rows for the
    others): the gradient of sum_n loss_n, which the backward scales row by
    row."""
    z = np.asarray(logits, dtype=np.float64)
    n, vocab = z.shape
    t = np.asarray(targets, dtype=np.int64)
    valid, bad = ce_valid(t, vocab, ignore_index)
    m = z.max(axis=1, keepdims=True) if vocab > 0 else np.zeros((n, 1))
    e = np.exp(z - m)
    s = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(s))[:, 0]
    p = e / s
    loss = np.zeros(n)
    rows = np.nonzero(valid)[0]
    loss[rows] = lse[rows] - z[rows, t[rows]]
    grad = np.where(valid[:, None], p, 0.0)
    grad[rows, t[rows]] -= 1.0
    n_valid = int(valid.sum())
    divisor = mean_divisor if mean_divisor > 0 else float(n_valid)
    loss_sum = float(loss.sum())
    return dict(loss=loss, lse=lse, grad=grad, valid=valid, n_valid=n_valid,
                n_bad=int(bad.sum()), loss_sum=loss_sum,
                loss_mean=loss_sum / divisor if divisor > 0 else 0.0)


def ce_row_scale(targets: np.ndarray, vocab: int, mode: str, grad_out,
                 ignore_index: int = IGNORE_INDEX, mean_divisor: float = 0.0) -> np.ndarray:
    """Upstream gradient of each row: grad_out / divisor ("mean"), grad_out
    ("sum") or grad_out[n] ("none"); 0 on rows that carry no loss."""
    valid, _ = ce_valid(targets, vocab, ignore_index)
    g = np.asarray(grad_out, dtype=np.float64)
    if mode == "mean":
        divisor = mean_divisor if mean_divisor > 0 else float(valid.sum())
        gn = np.full(len(valid), float(g.reshape(-1)[0]) / divisor if divisor > 0 else 0.0)
    elif mode == "sum":
        gn = np.full(len(valid), float(g.reshape(-1)[0]))
    elif mode == "none":
        gn = g.reshape(-1).copy()
    else:
        raise ValueError(mode)
    return np.where(valid, gn, 0.0)


def ce_backward(grad: np.ndarray, targets: np.ndarray, mode: str, grad_out,
                ignore_index: int = IGNORE_INDEX, mean_divisor: float = 0.0) -> np.ndarray:
    """The gradient of the reduced loss with respect to the logits: each row of
    the forward's unscaled gradient times that row's upstream gradient."""
    gr = np.asarray(grad, dtype=np.float64)
    gn = ce_row_scale(targets, gr.shape[1], mode, grad_out, ignore_index, mean_divisor)
    return gr * gn[:, None]
