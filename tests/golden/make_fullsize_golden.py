"""Write the oracle's expected values for the full-size workloads.

Run from the repository root:  python tests/golden/make_fullsize_golden.py [name ...]

For each workload in linear_cross_entropy_fp32_amd.synth.WORKLOADS this draws
the seeded inputs, runs the CPU oracle (float64) over every row, and stores:
  * the input checksum (to detect generator drift);
  * per-token loss, lse, entropy, argmax, hit and top-2 margin for every row;
  * the reductions (loss_sum, loss_mean, entropy_sum, n_valid, n_correct, n_bad);
  * grad_hidden rows: the first and last row of every 256-token tile and one
    drawn row inside it, so every token tile of the kernels is checked;
  * grad_weight / grad_bias rows: in every backward vocabulary chunk its
    first two and last two rows, the two rows on each side of every
    grad_hidden split-K slot edge inside it, and two drawn rows; plus the most
    frequent targets (the largest rows) and the first and last vocabulary row;
  * sketches of the whole gradients: for four seeded sign vectors sigma_k over
    the tokens and rho_k over the vocabulary, sum_n sigma_k[n] grad_hidden[n],
    sum_v rho_k[v] grad_weight[v] and sum_v rho_k[v] grad_bias[v]; a zeroed,
    doubled or misplaced chunk, slot or tile changes them far beyond the
    gradient tolerance.  rho_2 and rho_3 are zero on every vocabulary row that
    is some valid row's target, so those two sketches hold only the softmax
    part of the gradient (sum_n g_n p[n, v] h[n]), which the one-hot rows
    would otherwise outweigh.
Gradient rows and sketches are stored as float32 (the tolerance is 1e-2).

The chunk and slot edges come from the backward's chunk rule restated below
(chunk_plan); the file records the plan it assumed, and the tests check it
against the library's planner (flce_plan_info) so that a changed rule shows up
as a failed check rather than as unsampled chunks.  Nothing here imports or
reads anything of the GPU library.
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
SKETCHES = 4


def _cdiv(a, b):
    return -(-a // b)


def chunk_plan(n: int, h: int, v: int):
    """(chunk_rows, gh_rows_per_split) of the backward for N, H, V: vocabulary
    chunks of 2^27 bytes of bf16 dz (2^28 when that is under 8192 rows), at
    least N rows (rounded up to 128) while under 2^31 bytes, at most 2^21 rows
    and (2^31 - 1) / (2 H) rows, multiples of 128; grad_hidden split-K slots of
    about max(2N, 1024) rows, at most 32 per chunk, multiples of 32."""
    op = (1 << 31) - 1
    vc = ((1 << 27) // (2 * n)) // 128 * 128
    if vc < 8192:
        vc = ((1 << 28) // (2 * n)) // 128 * 128
    vc = max(vc, _cdiv(n, 128) * 128)
    vc = min(vc, op // (2 * n) // 128 * 128)
    vc = min(vc, op // (2 * h) // 128 * 128)
    vc = min(vc, 1 << 21)
    vc = max(vc, 128)
    vc = min(vc, _cdiv(v, 128) * 128)
    width = min(vc, v)
    ghs = max(1, min(_cdiv(width, max(2 * n, 1024)), 32))
    kps = _cdiv(_cdiv(width, ghs), 32) * 32
    return vc, kps


def sample_rows(n: int) -> np.ndarray:
    rng = np.random.default_rng(7)
    pick = set()
    for t0 in range(0, n, 256):
        t1 = min(n, t0 + 256)
        pick.update({t0, t1 - 1, int(rng.integers(t0, t1))})
    return np.array(sorted(pick), dtype=np.int64)


def sample_vocab(v: int, targets: np.ndarray, vc: int, kps: int) -> np.ndarray:
    rng = np.random.default_rng(9)
    pick = {0, v - 1}
    for c0 in range(0, v, vc):
        c1 = min(v, c0 + vc)
        pick.update({c0, c0 + 1, c1 - 2, c1 - 1})
        for e in range(c0 + kps, c1, kps):
            pick.update({e - 2, e - 1, e, e + 1})
        pick.update(int(x) for x in rng.integers(c0, c1, size=2))
    valid_t = targets[(targets >= 0) & (targets < v)]
    if len(valid_t):
        vals, counts = np.unique(valid_t, return_counts=True)
        pick.update(int(x) for x in vals[np.argsort(-counts, kind="stable")[:4]])
    return np.array(sorted(x for x in pick if 0 <= x < v), dtype=np.int64)


def sketch_signs(n: int, v: int, targets: np.ndarray):
    rng = np.random.default_rng(11)
    sigma = rng.choice([-1.0, 1.0], size=(SKETCHES, n))
    rho = rng.choice([-1.0, 1.0], size=(SKETCHES, v))
    t = targets[(targets >= 0) & (targets < v)]
    rho[2:, t] = 0.0
    return sigma, rho


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
    vc, kps = chunk_plan(w.n_tokens, w.hidden, w.vocab)
    rows = sample_rows(w.n_tokens)
    vrows = sample_vocab(w.vocab, t, vc, kps)
    sigma, rho = sketch_signs(w.n_tokens, w.vocab, t)
    g = backward(h, wt, b, t, prob, w.reduction, go, rows=rows, vocab_rows=vrows,
                 sketch=(sigma, rho))
    f32 = lambda x: np.asarray(x, dtype=np.float32)
    np.savez_compressed(
        golden_path(name), checksum=np.array(checksum), name=np.array(name),
        loss=f["loss"], lse=f["lse"], entropy=f["entropy"],
        argmax=f["argmax"].astype(np.int32), hit=f["hit"], margin=f["margin"].astype(np.float32),
        loss_sum=f["loss_sum"], loss_mean=f["loss_mean"], entropy_sum=f["entropy_sum"],
        n_valid=f["n_valid"], n_correct=f["n_correct"], n_bad=f["n_bad"],
        chunk_rows=vc, gh_rows_per_split=kps,
        rows=rows, grad_hidden_rows=f32(g["grad_hidden_rows"]),
        vocab_rows=vrows, grad_weight_rows=f32(g["grad_weight_rows"]),
        grad_bias_rows=f32(g["grad_bias_rows"]),
        sketch_grad_hidden=g["sketch_grad_hidden"], sketch_grad_weight=g["sketch_grad_weight"],
        sketch_grad_bias=g["sketch_grad_bias"])
    print(f"{name}: {time.time() - t0:.1f} s, n_valid={f['n_valid']}, "
          f"loss_mean={f['loss_mean']:.6f}, chunk_rows={vc}, gh_rows_per_split={kps}, "
          f"{len(rows)} grad_hidden rows, {len(vrows)} grad_weight rows", flush=True)


if __name__ == "__main__":
    names = sys.argv[1:] or list(synth.WORKLOADS)
    for nm in names:
        make(nm)
