"""Shared helpers of the GPU parity tests: run the library through the C ABI
on seeded inputs and compare with the CPU oracle at the stated tolerances.

Tolerances (fixed for this method, not tuned): per-token loss, entropy and
lse within 2e-3 absolute; reduced loss and entropy sum within 1e-4 relative;
grad_hidden / grad_weight / grad_bias within 1e-2 relative Frobenius error and
exactly zero where the oracle's gradient is exactly zero; argmax and hit exact
on every row whose oracle top-2 margin is at least 1e-2.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import linear_cross_entropy_fp32_amd as flce
from linear_cross_entropy_fp32_amd import synth
from oracle import Problem

TOL_TOKEN = 2e-3
TOL_REDUCED = 1e-4
TOL_GRAD = 1e-2
MARGIN = 1e-2
MODES = {"mean": flce.FLCE_GRAD_MEAN, "sum": flce.FLCE_GRAD_SUM,
         "none": flce.FLCE_GRAD_PER_TOKEN}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_f64(t):
    return None if t is None else t.detach().float().cpu().numpy().astype(np.float64) \
        if t.dtype != torch.float64 else t.detach().cpu().numpy()


def prob_of(w: synth.Workload, mean_divisor: float = 0.0, ignore_index: int = -100) -> Problem:
    return Problem(logit_scale=w.logit_scale, softcap=w.softcap, mean_divisor=mean_divisor,
                   ignore_index=ignore_index)


def run_gpu(w: synth.Workload, inp: synth.Inputs, mean_divisor: float = 0.0,
            backward: bool = True, dev: str = "cuda:0", compact: bool = False,
            ignore_index: int = -100) -> dict:
    """Forward (+ backward) through the C ABI; returns CPU tensors.  compact:
    with valid-row compaction (flce_problem.compact_valid)."""
    h = inp.hidden.to(dev)
    wt = inp.weight.to(dev)
    b = None if inp.bias is None else inp.bias.to(dev)
    t = inp.targets.to(dev)
    f = flce.flce_forward(h, wt, t, b, w.logit_scale, w.softcap, ignore_index, mean_divisor,
                          compact_valid=compact)
    out = {k: (v.cpu() if v is not None else None) for k, v in f.items()}
    if backward:
        go = inp.grad_out.to(dev).reshape(-1)
        gh, gw, gb = flce.flce_backward(h, wt, t, f["lse"], f["reduced_i64"], MODES[w.reduction],
                                        go, b, w.logit_scale, w.softcap, ignore_index,
                                        mean_divisor, compact_valid=compact)
        out["grad_hidden"] = gh.cpu()
        out["grad_weight"] = gw.cpu()
        out["grad_bias"] = None if gb is None else gb.cpu()
    torch.cuda.synchronize()
    return out


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    nb = float(np.linalg.norm(b))
    if nb == 0.0:
        return 0.0 if float(np.abs(a).max(initial=0.0)) == 0.0 else float("inf")
    return float(np.linalg.norm(a - b)) / nb


def check_tokens(g: dict, o: dict, rows=None, label: str = "") -> None:
    sel = slice(None) if rows is None else rows
    for k in ("loss", "entropy", "lse"):
        d = np.abs(g[k].numpy().astype(np.float64)[sel] - o[k])
        assert d.max(initial=0.0) <= TOL_TOKEN, f"{label} {k}: max |diff| {d.max()}"
    sure = o["margin"] >= MARGIN
    gam = g["argmax"].numpy()[sel]
    assert np.array_equal(gam[sure], o["argmax"][sure]), f"{label} argmax differs on sure rows"
    ghit = g["hit"].numpy()[sel]
    valid = o["valid"] if "valid" in o else None
    if valid is not None:
        assert np.all(ghit[~valid] == 0), f"{label} hit set on an ignored row"
        assert np.all(g["loss"].numpy()[sel][~valid] == 0)
        assert np.all(g["entropy"].numpy()[sel][~valid] == 0)
    assert np.array_equal(ghit[sure], o["hit"][sure]), f"{label} hit differs on sure rows"


def check_compact_tokens(g: dict, o: dict, valid: np.ndarray, label: str = "") -> None:
    """With valid-row compaction: the rows that carry a loss as check_tokens;
    the other rows hold the documented fill (loss, entropy, hit, lse 0,
    argmax -1)."""
    idx = np.nonzero(valid)[0]
    sub = {k: (o[k][idx] if isinstance(o[k], np.ndarray) and o[k].shape[:1] == valid.shape
               else o[k]) for k in ("loss", "entropy", "lse", "argmax", "hit", "margin")}
    sub["valid"] = np.ones(len(idx), dtype=bool)
    check_tokens(g, sub, rows=idx, label=label)
    skip = ~valid
    for k in ("loss", "entropy", "lse"):
        assert np.all(g[k].numpy()[skip] == 0), f"{label} {k} not 0 on a skipped row"
    assert np.all(g["hit"].numpy()[skip] == 0), f"{label} hit set on a skipped row"
    assert np.all(g["argmax"].numpy()[skip] == -1), f"{label} argmax not -1 on a skipped row"


def check_reduced(g: dict, o: dict, label: str = "") -> None:
    rf = g["reduced_f32"].numpy().astype(np.float64)
    ri = g["reduced_i64"].numpy()
    for i, k in enumerate(("loss_sum", "loss_mean", "entropy_sum")):
        ref = o[k]
        if ref == 0.0:
            assert rf[i] == 0.0, f"{label} {k} should be exactly 0, got {rf[i]}"
        else:
            assert abs(rf[i] - ref) <= TOL_REDUCED * abs(ref), f"{label} {k}: {rf[i]} vs {ref}"
    assert int(ri[0]) == o["n_valid"], f"{label} n_valid {ri[0]} vs {o['n_valid']}"
    assert int(ri[2]) == o["n_bad"], f"{label} n_bad {ri[2]} vs {o['n_bad']}"
    assert int(ri[1]) == int(g["hit"].numpy().astype(np.int64).sum()), f"{label} n_correct != sum hit"


def check_vocab_grad_parts(a: np.ndarray, b: np.ndarray, targets: np.ndarray, vocab: int,
                           name: str, label: str = "") -> None:
    """grad_weight / grad_bias rows split in two, each within the tolerance on
    its own: the rows that are some valid row's target (dominated by the
    one-hot term) and the others (the softmax term alone, which the first
    would otherwise outweigh at large vocabularies)."""
    t = np.asarray(targets)
    is_t = np.zeros(vocab, dtype=bool)
    is_t[t[(t >= 0) & (t < vocab)]] = True
    for sel, part in ((is_t, "target rows"), (~is_t, "softmax-only rows")):
        if sel.any():
            check_grad(a[sel], b[sel], f"{name} {part}", label)


def check_grad(a: np.ndarray, b: np.ndarray, name: str, label: str = "") -> None:
    e = rel_fro(a, b)
    assert e <= TOL_GRAD, f"{label} {name}: relative Frobenius error {e}"
    zero_rows = np.all(b == 0, axis=tuple(range(1, b.ndim))) if b.ndim > 1 else (b == 0)
    assert np.all(a[zero_rows] == 0), f"{label} {name}: nonzero where the oracle is exactly 0"


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_oracle(gold, w, inp) -> dict:
    """Per-token and reduced oracle values of a stored full-size golden."""
    o = {k: gold[k] for k in ("loss", "lse", "entropy", "argmax", "hit", "margin")}
    t = inp.targets.numpy()
    o["valid"] = (t >= 0) & (t < w.vocab)
    for k in ("loss_sum", "loss_mean", "entropy_sum"):
        o[k] = float(gold[k])
    for k in ("n_valid", "n_correct", "n_bad"):
        o[k] = int(gold[k])
    return o


def check_fullsize_grads(g: dict, gold, w, inp, name: str) -> None:
    """Gradients of a full-size run against a stored golden: grad_hidden rows
    of every token tile; grad_weight / grad_bias rows around every chunk and
    split-K slot edge, the rows that are some valid row's target and the
    softmax-only rows each checked on their own; and the sign sketches of the
    whole outputs (tests/golden/make_fullsize_golden.py)."""
    t = inp.targets.numpy()
    valid = (t >= 0) & (t < w.vocab)
    if not valid.any():
        for k in ("grad_hidden", "grad_weight"):
            assert torch.count_nonzero(g[k]).item() == 0, k
        if g.get("grad_bias") is not None:
            assert torch.count_nonzero(g["grad_bias"]).item() == 0
        return
    rows, vrows = gold["rows"], gold["vocab_rows"]
    gh, gw = g["grad_hidden"], g["grad_weight"]
    check_grad(gh.numpy()[rows].astype(np.float64), gold["grad_hidden_rows"].astype(np.float64),
               "grad_hidden rows", name)
    is_t = np.isin(vrows, t[valid])
    parts = ((is_t, "target"), (~is_t, "softmax-only"))
    gwr = gw.numpy()[vrows].astype(np.float64)
    ref = gold["grad_weight_rows"].astype(np.float64)
    for sel, part in parts:
        if sel.any():
            check_grad(gwr[sel], ref[sel], f"grad_weight {part} rows", name)
    if inp.bias is not None:
        gbr = g["grad_bias"].numpy()[vrows].astype(np.float64)
        rb = gold["grad_bias_rows"].astype(np.float64)
        for sel, part in parts:
            if sel.any():
                check_grad(gbr[sel], rb[sel], f"grad_bias {part} rows", name)
    if GOLDEN not in sys.path:
        sys.path.insert(0, GOLDEN)
    from make_fullsize_golden import sketch_signs
    sigma, rho = sketch_signs(w.n_tokens, w.vocab, t)
    sk_gh = (torch.from_numpy(sigma) @ gh.double()).numpy()
    sk_gw = sum(torch.from_numpy(rho[:, v0:v0 + 16384]) @ gw[v0:v0 + 16384].double()
                for v0 in range(0, w.vocab, 16384)).numpy()
    check_grad(sk_gh, gold["sketch_grad_hidden"], "grad_hidden sketch", name)
    check_grad(sk_gw[:2], gold["sketch_grad_weight"][:2], "grad_weight sketch", name)
    check_grad(sk_gw[2:], gold["sketch_grad_weight"][2:], "grad_weight softmax-only sketch", name)
    if inp.bias is not None:
        sk_gb = (torch.from_numpy(rho) @ g["grad_bias"].double()).numpy()
        check_grad(sk_gb[:2], gold["sketch_grad_bias"][:2], "grad_bias sketch", name)
        check_grad(sk_gb[2:], gold["sketch_grad_bias"][2:], "grad_bias softmax-only sketch",
                   name)


def check_fullsize(g: dict, gold, w, inp, name: str) -> None:
    o = golden_oracle(gold, w, inp)
    check_tokens(g, o, label=name)
    check_reduced(g, o, label=name)
    check_fullsize_grads(g, gold, w, inp, name)
