"""Write the oracle's expected values for the full-size workloads.

Run from the repository root:  python tests/golden/make_fullsize_golden.py [name ...]

For each workload in linear_cross_entropy_fp32_amd.synth.WORKLOADS this draws
the seeded inputs, runs the CPU oracle (float64) over every row, and stores:
  * the input checksum (to detect generator drift);
  * per-token loss, lse, entropy, argmax, hit and top-2 margin for every row;
  * the reductions (loss_sum, loss_mean, entropy_sum, n_valid, n_correct, n_bad);
  * grad_hidden for a fixed sample of rows;
  * grad_weight and grad_bias for a fixed sample of vocabulary entries.
Nothing here reads anything produced by the GPU library.
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from linear_cross_entropy_fp32_amd import synth  # noqa: E402
from oracle import Problem, backward, forward  # noqa: E402

OUT_DIR = os.path.dirname(os.path.abspath(__file__))


def sample_rows(n: int, targets: np.ndarray) -> np.ndarray:
    rng = np.random.default_rng(7)
    pick = {0, 1, n - 1, n // 2}
    pick.update(int(x) for x in rng.choice(n, size=min(n, 12), replace=False))
    return np.array(sorted(pick), dtype=np.int64)


def sample_vocab(v: int, targets: np.ndarray) -> np.ndarray:
    rng = np.random.default_rng(9)
    pick = {0, v - 1}
    valid_t = targets[(targets >= 0) & (targets < v)]
    if len(valid_t):
        # the most frequent targets carry the largest grad_weight rows
        vals, counts = np.unique(valid_t, return_counts=True)
        pick.update(int(x) for x in vals[np.argsort(-counts)[:4]])
    pick.update(int(x) for x in rng.choice(v, size=min(v, 8), replace=False))
    return np.array(sorted(pick), dtype=np.int64)


def golden_path(name: str) -> str:
    return os.path.join(OUT_DIR, f"fullsize_{name}.npz")


def make(name: str) -> None:
    w = synth.WORKLOADS[name]
    t0 = time.time()
    inp = synth.make_inputs(w)
    checksum = synth.input_checksum(inp)
    h = inp.hidden.float().numpy().astype(np.float64)
    wt = inp.weight.float().numpy().astype(np.float64)
    b = None if inp.bias is None else inp.bias.numpy().astype(np.float64)
    t = inp.targets.numpy()
    go = inp.grad_out.numpy()
    prob = Problem(logit_scale=w.logit_scale, softcap=w.softcap)
    f = forward(h, wt, b, t, prob)
    rows = sample_rows(w.n_tokens, t)
    vrows = sample_vocab(w.vocab, t)
    g = backward(h, wt, b, t, prob, w.reduction, go, rows=rows, vocab_rows=vrows)
    np.savez_compressed(
        golden_path(name), checksum=np.array(checksum), name=np.array(name),
        loss=f["loss"], lse=f["lse"], entropy=f["entropy"],
        argmax=f["argmax"].astype(np.int32), hit=f["hit"], margin=f["margin"].astype(np.float32),
        loss_sum=f["loss_sum"], loss_mean=f["loss_mean"], entropy_sum=f["entropy_sum"],
        n_valid=f["n_valid"], n_correct=f["n_correct"], n_bad=f["n_bad"],
        rows=rows, grad_hidden_rows=g["grad_hidden_rows"],
        vocab_rows=vrows, grad_weight_rows=g["grad_weight_rows"],
        grad_bias_rows=g["grad_bias_rows"])
    print(f"{name}: {time.time() - t0:.1f} s, n_valid={f['n_valid']}, "
          f"loss_mean={f['loss_mean']:.6f}", flush=True)


if __name__ == "__main__":
    names = sys.argv[1:] or list(synth.WORKLOADS)
    for nm in names:
        make(nm)
