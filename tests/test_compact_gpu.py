"""GPU parity with valid-row compaction (flce_problem.compact_valid): only the
rows that carry a loss are projected, forward and backward.  Against the CPU
oracle at the stated tolerances, and against the library's own full path on
the same inputs, which must agree exactly on every per-row result and on
grad_hidden (each row's arithmetic is unchanged by where the row sits in a
tile), and to summation order on grad_weight / grad_bias (sums over rows)."""
import os

import numpy as np
import pytest
import torch

import linear_cross_entropy_fp32_amd as flce
from linear_cross_entropy_fp32_amd import _binding, synth
from oracle import backward, forward
from tests.gpu_cases import (check_compact_tokens, check_fullsize_grads, check_grad,
                             check_reduced, check_vocab_grad_parts, prob_of, rel_fro,
                             run_gpu, say, to_f64)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    flce.lib()


def _valid(inp, vocab):
    t = inp.targets.numpy()
    return (t >= 0) & (t < vocab)


def _oracle(w, inp):
    h, wt, b = to_f64(inp.hidden), to_f64(inp.weight), to_f64(inp.bias)
    t = inp.targets.numpy()
    prob = prob_of(w)
    return forward(h, wt, b, t, prob), backward(h, wt, b, t, prob, w.reduction,
                                                inp.grad_out.numpy())


CASES = [
    synth.small_workload(300, 136, 1000, 31),                            # every 17th ignored
    synth.small_workload(1000, 64, 3001, 32, softcap=30.0, bias=True, ignore_every=0,
                         prompt_frac=0.7, prompt_block=300, reduction="none"),
    synth.small_workload(700, 96, 2500, 33, hidden_dtype="f32", prompt_frac=0.5,
                         prompt_block=128),
    synth.small_workload(4100, 128, 30000, 34, prompt_frac=0.6),         # two vocab chunks
    synth.small_workload(333, 128, 2500, 35, logit_scale=0.0625, targets="zipf",
                         reduction="sum", prompt_frac=0.3, prompt_block=100),
    synth.small_workload(64, 128, 1, 36),                                # V = 1
    synth.small_workload(260, 64, 900, 37, targets="all_ignored", hidden_dtype="f32"),
    synth.small_workload(800, 96, 2000, 42, weight_dtype="f32", hidden_dtype="f32",
                         prompt_frac=0.6, prompt_block=200, softcap=30.0),
    # H = 640: 128-row dz tiles (one chunk of 25), two grad_hidden slots
    synth.small_workload(900, 640, 3100, 45, softcap=30.0, bias=True, prompt_frac=0.6),
    # 256-row forward, dz and 256x256 contraction tiles (H a multiple of 256 from 1024 on)
    synth.small_workload(900, 1024, 3100, 43, softcap=30.0, bias=True, prompt_frac=0.6,
                         prompt_block=300, reduction="none"),
    # 256-row forward and dz tiles with the 256x128 contraction (H = 1152)
    synth.small_workload(700, 1152, 2300, 44, hidden_dtype="f32", prompt_frac=0.5,
                         prompt_block=128),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_compact_parity(w):
    say(f"[compact] {w.name}")
    inp = synth.make_inputs(w)
    g = run_gpu(w, inp, compact=True)
    o, og = _oracle(w, inp)
    valid = _valid(inp, w.vocab)
    check_compact_tokens(g, o, valid, label=w.name)
    check_reduced(g, o, label=w.name)
    check_grad(g["grad_hidden"].numpy(), og["grad_hidden"], "grad_hidden", w.name)
    check_grad(g["grad_weight"].numpy(), og["grad_weight"], "grad_weight", w.name)
    check_vocab_grad_parts(g["grad_weight"].numpy(), og["grad_weight"], inp.targets.numpy(),
                           w.vocab, "grad_weight", w.name)
    if inp.bias is not None:
        check_grad(g["grad_bias"].numpy(), og["grad_bias"], "grad_bias", w.name)
        check_vocab_grad_parts(g["grad_bias"].numpy(), og["grad_bias"], inp.targets.numpy(),
                               w.vocab, "grad_bias", w.name)
    if not valid.any():
        for k in ("grad_hidden", "grad_weight"):
            assert torch.count_nonzero(g[k]).item() == 0, k


def test_compact_bad_targets_counted_and_skipped():
    w = synth.small_workload(500, 64, 700, 39, bias=True)
    inp = synth.make_inputs(w)
    inp.targets[5] = 700
    inp.targets[7] = -3
    inp.targets[300] = 10 ** 9
    say("[compact] bad targets")
    g = run_gpu(w, inp, compact=True)
    o, og = _oracle(w, inp)
    assert o["n_bad"] == 3
    check_compact_tokens(g, o, _valid(inp, w.vocab), label="bad targets")
    check_reduced(g, o, label="bad targets")
    check_grad(g["grad_hidden"].numpy(), og["grad_hidden"], "grad_hidden", "bad targets")
    check_grad(g["grad_weight"].numpy(), og["grad_weight"], "grad_weight", "bad targets")


@pytest.mark.parametrize("hidden_dtype", ["bf16", "f32"])
def test_compact_matches_full_path(hidden_dtype):
    w = synth.small_workload(1500, 128, 5000, 38, softcap=30.0, bias=True, prompt_frac=0.7,
                             prompt_block=256, reduction="none", hidden_dtype=hidden_dtype)
    inp = synth.make_inputs(w)
    say(f"[compact] against the full path, {hidden_dtype} hidden")
    full = run_gpu(w, inp)
    comp = run_gpu(w, inp, compact=True)
    valid = _valid(inp, w.vocab)
    for k in ("loss", "lse", "entropy", "argmax", "hit"):
        assert np.array_equal(full[k].numpy()[valid], comp[k].numpy()[valid]), k
    assert torch.equal(full["grad_hidden"], comp["grad_hidden"])
    for k in ("grad_weight", "grad_bias"):
        assert rel_fro(comp[k].numpy().astype(np.float64),
                       full[k].numpy().astype(np.float64)) <= 1e-5, k
    fi, ci = full["reduced_i64"].numpy(), comp["reduced_i64"].numpy()
    assert np.array_equal(fi, ci)
    ff, cf = full["reduced_f32"].numpy(), comp["reduced_f32"].numpy()
    assert np.allclose(cf, ff, rtol=1e-6, atol=0.0)


def test_compact_repeatable_and_workspace_reuse():
    """Two calls in a row on one workspace, the second with another mask,
    give the same results as fresh calls: no state survives a call."""
    w1 = synth.small_workload(900, 64, 1200, 40, prompt_frac=0.7, prompt_block=90)
    w2 = synth.small_workload(900, 64, 1200, 40, prompt_frac=0.2, prompt_block=90)
    i1, i2 = synth.make_inputs(w1), synth.make_inputs(w2)
    dev = "cuda:0"
    h, wt = i1.hidden.to(dev), i1.weight.to(dev)
    prob = _binding.problem_for(h, wt, compact_valid=True)
    ws = torch.empty(flce.flce_workspace_bytes(prob), dtype=torch.uint8, device=dev)
    outs = []
    for inp in (i1, i2, i1):
        f = flce.flce_forward(h, wt, inp.targets.to(dev), compact_valid=True, workspace=ws)
        gh, gw, _ = flce.flce_backward(h, wt, inp.targets.to(dev), f["lse"], f["reduced_i64"],
                                       flce.FLCE_GRAD_MEAN, torch.ones(1, device=dev),
                                       compact_valid=True, workspace=ws)
        outs.append((f["loss"].cpu(), gh.cpu(), gw.cpu()))
    for a, b in zip(outs[0], outs[2]):
        assert torch.equal(a, b)
    fresh = run_gpu(w2, i2, compact=True)
    assert torch.equal(outs[1][0], fresh["loss"])
    assert torch.equal(outs[1][1], fresh["grad_hidden"])


def test_compact_autograd_wrapper():
    w = synth.small_workload(600, 128, 3000, 41, softcap=30.0, prompt_frac=0.6, prompt_block=200)
    inp = synth.make_inputs(w)
    dev = "cuda:0"
    res = []
    for compact in (False, True):
        h = inp.hidden.to(dev).requires_grad_(True)
        wt = inp.weight.to(dev).requires_grad_(True)
        loss, ent, nc, nv = flce.linear_cross_entropy(h, wt, inp.targets.to(dev), softcap=30.0,
                                                      compact_valid=compact)
        loss.backward()
        res.append((loss.item(), h.grad.cpu(), wt.grad.float().cpu(), int(nv)))
    assert res[0][0] == res[1][0] or abs(res[0][0] - res[1][0]) <= 1e-6 * abs(res[0][0])
    assert res[0][3] == res[1][3]
    assert torch.equal(res[0][1], res[1][1])
    assert rel_fro(res[1][2].numpy().astype(np.float64),
                   res[0][2].numpy().astype(np.float64)) <= 1e-2


@pytest.mark.parametrize("name", ["huge_vocab_sft", "bias_none", "zipf_sum", "fp32_hidden",
                                  "fp32_hidden_all_ignored", "huge_vocab_fp32_lm_head"])
def test_fullsize_compact_against_stored_oracle(name):
    """Full-size workloads, compacted, in the bench's launch configuration,
    against oracle values written by tests/golden/make_fullsize_golden.py
    (huge_vocab_sft: 70% prompt masking; the others ignore every 17th row,
    or every row)."""
    path = os.path.join(GOLDEN, f"fullsize_{name}.npz")
    gold = np.load(path, allow_pickle=False)
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w)
    assert synth.input_checksum(inp) == str(gold["checksum"]), "input generator drifted"
    say(f"[compact] full size {name}")
    g = run_gpu(w, inp, compact=True)
    o = {k: gold[k] for k in ("loss", "lse", "entropy", "argmax", "hit", "margin")}
    for k in ("loss_sum", "loss_mean", "entropy_sum"):
        o[k] = float(gold[k])
    for k in ("n_valid", "n_correct", "n_bad"):
        o[k] = int(gold[k])
    check_compact_tokens(g, o, _valid(inp, w.vocab), label=name)
    check_reduced(g, o, label=name)
    check_fullsize_grads(g, gold, w, inp, name)
