"""CPU oracle for the fused linear cross-entropy (test infrastructure only).

This module is the plain, slow definition the GPU library is checked against.
Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the library itself never does, and the two share
no code.  Everything is computed in float64 with numpy, from the exact values
of the (bf16 / fp32) inputs, and the (tokens x vocab) logits are materialised a
block of rows at a time with a float64 matmul.

Sources (page titles as published):
  [cce]   TRL pull request "Add loss_type="cce", a fused linear cross-entropy
          loaded from the Hub".
  [proj]  TRL pull request "Do the chunked-CE lm_head projection on tensor
          cores instead of in fp32".
  [liger] Liger-Kernel pull request 1574 (standalone cross entropy: fp32
          per-token loss, reduction="none" backward).

Readings taken where the pages are silent (each listed in the design notes):
  * softcapping is c * tanh(x / c) with c = final_logit_softcapping, applied
    after the logit scale; c <= 0 disables it;
  * argmax ties resolve to the lowest vocabulary index;
  * ignored rows (target == ignore_index) report loss, entropy and hit as 0,
    but their lse is still reported;
  * a target outside [0, V) that is not the ignore index is treated as ignored
    and counted in n_bad;
  * the mean divides by ``mean_divisor`` when it is > 0 (the trainer's
    num_items_in_batch), else by the number of valid rows, and is 0 (with all
    gradients exactly 0) when that divisor is 0.

Every function below is pinned by tests/test_oracle_pins.py against closed
forms, a library routine (torch cross_entropy + autograd in float64),
finite differences and invariants.  No function here is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

IGNORE_INDEX = -100


@dataclass
class Problem:
    logit_scale: float = 1.0
    softcap: float = 0.0
    ignore_index: int = IGNORE_INDEX
    mean_divisor: float = 0.0


def final_logits(h: np.ndarray, w: np.ndarray, bias: Optional[np.ndarray],
                 prob: Problem) -> np.ndarray:
    """Final logits z for a block of rows, in the op order of [cce], review
    "Correctness" paragraph of the maintainer's verified facts: the product of
    hidden and lm_head (float64 here, exact for bf16/fp32 inputs), then the
    bias, then the logit scale, then softcapping ([cce] "What it supports"
    names final_logit_softcapping; its form c*tanh(x/c) is the reading taken).
    """
    z = h @ w.T
    if bias is not None:
        z = z + bias[None, :]
    z = z * prob.logit_scale
    if prob.softcap > 0:
        z = prob.softcap * np.tanh(z / prob.softcap)
    return z


def _row_blocks(n: int, vocab: int, max_elems: int = 1 << 24):
    step = max(1, min(n, max_elems // max(1, vocab)))
    for r0 in range(0, n, step):
        yield r0, min(n, r0 + step)


def valid_mask(targets: np.ndarray, vocab: int, prob: Problem):
    """Rows that carry a loss.  The ignore index marks padding / prompt tokens
    ([cce] review "Correctness" item 2: validity only zeroes the row's weight
    after the projection, so ignored rows are still projected)."""
    t = np.asarray(targets, dtype=np.int64)
    ignored = t == prob.ignore_index
    in_range = (t >= 0) & (t < vocab)
    valid = in_range & ~ignored
    bad = ~ignored & ~in_range
    return valid, bad


def forward(hidden: np.ndarray, weight: np.ndarray, bias: Optional[np.ndarray],
            targets: np.ndarray, prob: Problem, rows: Optional[np.ndarray] = None) -> dict:
    """Per-token loss, lse, entropy, argmax and hit, plus the reductions.

    [cce] "What it supports": the fused pass yields the loss and, from the same
    pass, the entropy and the argmax accuracy that the trainer logs.  [cce]
    review "Correctness" (verified facts): entropy is lse - sum_v p_v z_v, and
    the argmax is taken on the final (scaled, softcapped) logits.

    ``rows`` restricts the per-token outputs to those row indices (used to
    sample very large workloads); the reductions are then over those rows only.
    """
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    b = None if bias is None else np.asarray(bias, dtype=np.float64)
    t_all = np.asarray(targets, dtype=np.int64)
    vocab = w.shape[0]
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        h = h[rows]
        t_all = t_all[rows]
    n = h.shape[0]
    valid, bad = valid_mask(t_all, vocab, prob)

    lse = np.zeros(n)
    loss = np.zeros(n)
    entropy = np.zeros(n)
    amax = np.zeros(n, dtype=np.int64)
    hit = np.zeros(n, dtype=np.uint8)
    margin = np.zeros(n)              # top-1 minus top-2 final logit (inf if V == 1)
    for r0, r1 in _row_blocks(n, vocab):
        z = final_logits(h[r0:r1], w, b, prob)
        m = z.max(axis=1)
        e = np.exp(z - m[:, None])
        s = e.sum(axis=1)
        lse_b = m + np.log(s)
        p = e / s[:, None]
        lse[r0:r1] = lse_b
        idx = np.argmax(z, axis=1)                       # first (lowest) index on ties
        amax[r0:r1] = idx
        if vocab > 1:
            top2 = np.partition(z, vocab - 2, axis=1)[:, vocab - 2:]
            margin[r0:r1] = top2[:, 1] - top2[:, 0]
        else:
            margin[r0:r1] = np.inf
        for i in range(r1 - r0):
            n_i = r0 + i
            if not valid[n_i]:
                continue
            tz = z[i, t_all[n_i]]
            loss[n_i] = lse_b[i] - tz
            entropy[n_i] = lse_b[i] - float(np.dot(p[i], z[i]))
            hit[n_i] = 1 if idx[i] == t_all[n_i] else 0

    n_valid = int(valid.sum())
    loss_sum = float(loss.sum())
    divisor = prob.mean_divisor if prob.mean_divisor > 0 else float(n_valid)
    loss_mean = loss_sum / divisor if divisor > 0 else 0.0
    return dict(
        loss=loss, lse=lse, entropy=entropy, argmax=amax, hit=hit, valid=valid,
        margin=margin, loss_sum=loss_sum, loss_mean=loss_mean,
        entropy_sum=float(entropy.sum()), n_valid=n_valid,
        n_correct=int(hit.sum()), n_bad=int(bad.sum()),
    )


def row_grad_scale(targets: np.ndarray, vocab: int, prob: Problem, mode: str,
                   grad_out, n_valid: Optional[int] = None) -> np.ndarray:
    """Upstream gradient per row, g_n.

    "mean": g / divisor (the divisor as in ``forward``; 0 when it is 0, which
    gives the all-ignored batch its exactly-zero gradients, [cce] review
    "Correctness" item 5 and the "Overview": that batch must still produce
    gradients for every parameter); "sum": g; "none": grad_out[n], a per-token
    weight ([liger] "Summary" item 2: the per-row upstream multiply).
    Ignored rows get 0.
    """
    valid, _ = valid_mask(targets, vocab, prob)
    if n_valid is None:
        n_valid = int(valid.sum())
    g = np.asarray(grad_out, dtype=np.float64)
    if mode == "mean":
        divisor = prob.mean_divisor if prob.mean_divisor > 0 else float(n_valid)
        gn = np.full(len(valid), float(g) / divisor if divisor > 0 else 0.0)
    elif mode == "sum":
        gn = np.full(len(valid), float(g))
    elif mode == "none":
        gn = g.reshape(-1).copy()
    else:
        raise ValueError(mode)
    return np.where(valid, gn, 0.0)


def grad_raw_logits(z: np.ndarray, t: np.ndarray, gn: np.ndarray, valid: np.ndarray,
                    prob: Problem) -> np.ndarray:
    """d loss / d (h W^T) for a block of rows, from the final logits z.

    Softmax cross-entropy gives g_n (p - onehot(t)); the chain rule then goes
    back through softcapping (derivative 1 - (z/c)^2 of c*tanh(x/c)), the
    logit scale (factor s) and the bias (factor 1) in the reverse of the
    forward op order.
    """
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    p = e / e.sum(axis=1, keepdims=True)
    d = p.copy()
    rows = np.nonzero(valid)[0]
    d[rows, t[rows]] -= 1.0
    d *= gn[:, None]
    if prob.softcap > 0:
        d *= 1.0 - (z / prob.softcap) ** 2
    d *= prob.logit_scale
    return d


def backward(hidden: np.ndarray, weight: np.ndarray, bias: Optional[np.ndarray],
             targets: np.ndarray, prob: Problem, mode: str, grad_out,
             need_weight: bool = True, rows: Optional[np.ndarray] = None,
             vocab_rows: Optional[np.ndarray] = None, sketch=None) -> dict:
    """grad_hidden, grad_weight and grad_bias of the reduced loss.

    grad_hidden[n] = sum_v d[n, v] W[v]; grad_weight[v] = sum_n d[n, v] h[n];
    grad_bias[v] = sum_n d[n, v], with d from ``grad_raw_logits``.  Entropy and
    accuracy are logged metrics and carry no gradient.

    ``rows`` restricts grad_hidden to those rows (it only needs their own
    logits).  ``vocab_rows`` restricts grad_weight / grad_bias to those vocab
    entries; they still need every row's softmax, so all rows are projected.

    ``sketch = (sigma, rho)``, sign matrices of shapes [K, N] and [K, V], adds
    fixed linear summaries of the whole gradients (test infrastructure, for
    checking outputs too large to store):
      sketch_grad_hidden[k] = sum_n sigma[k, n] grad_hidden[n]
                            = (sum_n sigma[k, n] d[n, :]) @ W,
      sketch_grad_weight[k] = sum_v rho[k, v] grad_weight[v]
                            = sum_n (sum_v rho[k, v] d[n, v]) h[n],
      sketch_grad_bias[k]   = sum_v rho[k, v] grad_bias[v];
    the right-hand sides are the same sums with the order of summation
    exchanged, so no full gradient has to be formed.
    """
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    b = None if bias is None else np.asarray(bias, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64)
    n, vocab = h.shape[0], w.shape[0]
    valid, _ = valid_mask(t, vocab, prob)
    gn = row_grad_scale(t, vocab, prob, mode, grad_out)

    out = {}
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        gh = np.zeros((len(rows), h.shape[1]))
        for r0, r1 in _row_blocks(len(rows), vocab):
            sel = rows[r0:r1]
            z = final_logits(h[sel], w, b, prob)
            d = grad_raw_logits(z, t[sel], gn[sel], valid[sel], prob)
            gh[r0:r1] = d @ w
        out["grad_hidden_rows"] = gh
    else:
        out["grad_hidden"] = np.zeros_like(h)
    if not need_weight and rows is not None:
        return out

    vsel = None if vocab_rows is None else np.asarray(vocab_rows, dtype=np.int64)
    nv = vocab if vsel is None else len(vsel)
    gw = np.zeros((nv, h.shape[1]))
    gb = np.zeros(nv)
    if sketch is not None:
        sigma = np.asarray(sketch[0], dtype=np.float64)
        rho = np.asarray(sketch[1], dtype=np.float64)
        assert sigma.shape[1] == n and rho.shape[1] == vocab and sigma.shape[0] == rho.shape[0]
        sd = np.zeros((sigma.shape[0], vocab))          # sum_n sigma[k, n] d[n, :]
        sk_gw = np.zeros((rho.shape[0], h.shape[1]))
        sk_gb = np.zeros(rho.shape[0])
    for r0, r1 in _row_blocks(n, vocab):
        z = final_logits(h[r0:r1], w, b, prob)
        d = grad_raw_logits(z, t[r0:r1], gn[r0:r1], valid[r0:r1], prob)
        if rows is None:
            out["grad_hidden"][r0:r1] = d @ w
        dv = d if vsel is None else d[:, vsel]
        gw += dv.T @ h[r0:r1]
        gb += dv.sum(axis=0)
        if sketch is not None:
            sd += sigma[:, r0:r1] @ d
            dr = d @ rho.T                               # [rows, K]
            sk_gw += dr.T @ h[r0:r1]
            sk_gb += dr.sum(axis=0)
    if sketch is not None:
        out["sketch_grad_hidden"] = sd @ w
        out["sketch_grad_weight"] = sk_gw
        out["sketch_grad_bias"] = sk_gb
    if vsel is None:
        out["grad_weight"] = gw
        out["grad_bias"] = gb
    else:
        out["grad_weight_rows"] = gw
        out["grad_bias_rows"] = gb
    return out


def loss_value(hidden, weight, bias, targets, prob: Problem, mode: str, grad_out) -> float:
    """The scalar whose gradient ``backward`` returns: sum_n g_n * loss_n.

    For "mean" this is loss_sum / divisor times g, for "sum" g * loss_sum, for
    "none" the grad_out-weighted sum of per-token losses.  Used by the
    finite-difference pin of the backward.
    """
    f = forward(hidden, weight, bias, targets, prob)
    gn = row_grad_scale(targets, np.asarray(weight).shape[0], prob, mode, grad_out)
    return float(np.dot(gn, f["loss"]))

