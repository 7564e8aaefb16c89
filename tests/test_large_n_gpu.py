"""A batch past 2^22 tokens.  There one 256-row logit tile's column of bf16
dz (N x 256 x 2 bytes) would pass the 2^31-byte extent of a buffer
descriptor, so the dz recompute takes 128-row vocabulary tiles and the
backward's chunks are 128 rows wide (the planner's rule, checked below on
the plan).  Most rows are ignored, so that the oracle needs only the valid
rows for the reductions and the gradients: the library still computes every
row, and the ignored rows' gradients must come out exactly zero.  The valid
rows are spread over the whole batch, the last one included, so that the
highest buffer offsets of the dz chunk and of the hidden operand are used."""
import numpy as np
import pytest
import torch

import linear_cross_entropy_fp32_amd as flce
from linear_cross_entropy_fp32_amd import synth
from oracle import backward, forward
from tests.gpu_cases import (TOL_TOKEN, check_grad, check_reduced, check_tokens,
                             check_vocab_grad_parts, prob_of, run_gpu, say, to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    flce.lib()


def test_batch_past_2_pow_22_tokens():
    n, h, v = (1 << 22) + 77, 16, 300
    w = synth.small_workload(n, h, v, 71, softcap=30.0, bias=True)
    pl = flce.flce_plan_info(flce.make_problem(n, h, v))
    assert pl["dz_tile_rows"] == 128 and pl["chunk_rows"] == 128 and pl["n_chunks"] == 3
    assert pl["fwd_tile_rows"] == 128
    inp = synth.make_inputs(w)
    gen = np.random.default_rng(7101)
    valid = np.zeros(n, dtype=bool)
    valid[::4099] = True
    valid[-1] = True
    t = np.full(n, -100, dtype=np.int64)
    t[valid] = gen.integers(0, v, size=int(valid.sum()))
    inp.targets = torch.from_numpy(t)
    say(f"[large N] {w.name}: {int(valid.sum())} valid rows")
    g = run_gpu(w, inp)

    idx = np.nonzero(valid)[0]
    hid = to_f64(inp.hidden)
    wt, b = to_f64(inp.weight), to_f64(inp.bias)
    prob = prob_of(w)
    o = forward(hid[idx], wt, b, t[idx], prob)
    og = backward(hid[idx], wt, b, t[idx], prob, w.reduction, inp.grad_out.numpy())
    sub = {k: g[k][torch.from_numpy(idx)] for k in ("loss", "entropy", "lse", "argmax", "hit")}
    check_tokens(sub, o, label=w.name)
    check_reduced(g, o, label=w.name)
    # lse of ignored rows near both ends and in the middle of the batch
    skip = np.nonzero(~valid)[0]
    probe = np.concatenate([skip[:64], skip[len(skip) // 2:len(skip) // 2 + 64], skip[-64:]])
    op = forward(hid[probe], wt, b, t[probe], prob)
    d = np.abs(g["lse"].numpy().astype(np.float64)[probe] - op["lse"])
    assert d.max() <= TOL_TOKEN, f"lse of ignored rows: max |diff| {d.max()}"
    assert np.all(g["loss"].numpy()[~valid] == 0)

    gh = g["grad_hidden"].numpy()
    assert np.all(gh[~valid] == 0), "grad_hidden nonzero on an ignored row"
    check_grad(gh[idx], og["grad_hidden"], "grad_hidden", w.name)
    check_grad(g["grad_weight"].numpy(), og["grad_weight"], "grad_weight", w.name)
    check_vocab_grad_parts(g["grad_weight"].numpy(), og["grad_weight"], t[idx], v,
                           "grad_weight", w.name)
    check_grad(g["grad_bias"].numpy(), og["grad_bias"], "grad_bias", w.name)
