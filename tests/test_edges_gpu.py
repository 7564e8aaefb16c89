"""GPU parity at the edges of the problem description, against the CPU oracle,
with and without valid-row compaction: an ignore_index that is a valid
vocabulary id (so -100 becomes an out-of-range target), the smallest hidden
size, a single token, and negative or large logit scales."""
import numpy as np
import pytest
import torch

import linear_cross_entropy_fp32_amd as flce
from linear_cross_entropy_fp32_amd import synth
from oracle import backward, forward
from tests.gpu_cases import (check_compact_tokens, check_grad, check_reduced, check_tokens,
                             prob_of, run_gpu, say, to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    flce.lib()


def _check(w, inp, compact, ignore_index=-100, mean_divisor=0.0):
    label = f"{w.name} compact={compact} ignore={ignore_index}"
    say(f"[edges] {label}")
    g = run_gpu(w, inp, mean_divisor=mean_divisor, compact=compact, ignore_index=ignore_index)
    prob = prob_of(w, mean_divisor, ignore_index)
    h, wt, b = to_f64(inp.hidden), to_f64(inp.weight), to_f64(inp.bias)
    t = inp.targets.numpy()
    o = forward(h, wt, b, t, prob)
    og = backward(h, wt, b, t, prob, w.reduction, inp.grad_out.numpy())
    valid = (t != ignore_index) & (t >= 0) & (t < w.vocab)
    if compact:
        check_compact_tokens(g, o, valid, label=label)
    else:
        check_tokens(g, o, label=label)
    check_reduced(g, o, label=label)
    check_grad(g["grad_hidden"].numpy(), og["grad_hidden"], "grad_hidden", label)
    check_grad(g["grad_weight"].numpy(), og["grad_weight"], "grad_weight", label)
    if inp.bias is not None:
        check_grad(g["grad_bias"].numpy(), og["grad_bias"], "grad_bias", label)
    return o


@pytest.mark.parametrize("compact", [False, True])
def test_ignore_index_is_a_vocabulary_id(compact):
    """ignore_index = 5: rows whose target is 5 carry no loss, and the rows the
    generator marked -100 are now out-of-range targets, counted as bad."""
    w = synth.small_workload(400, 64, 900, 51, bias=True, softcap=30.0)
    inp = synth.make_inputs(w)
    inp.targets[10:30] = 5
    o = _check(w, inp, compact, ignore_index=5)
    assert o["n_bad"] == int((inp.targets == -100).sum())
    assert o["n_valid"] == int(((inp.targets != 5) & (inp.targets >= 0)).sum())


@pytest.mark.parametrize("compact", [False, True])
def test_smallest_hidden(compact):
    w = synth.small_workload(37, 8, 1000, 52, reduction="none")
    _check(w, synth.make_inputs(w), compact)


@pytest.mark.parametrize("compact", [False, True])
def test_single_token(compact):
    w = synth.small_workload(1, 64, 3000, 53, bias=True, ignore_every=0)
    _check(w, synth.make_inputs(w), compact)


@pytest.mark.parametrize("compact", [False, True])
def test_negative_logit_scale(compact):
    w = synth.small_workload(300, 72, 1500, 54, logit_scale=-0.5, softcap=20.0, bias=True)
    _check(w, synth.make_inputs(w), compact)


def test_large_scale_saturates_softcap():
    """logit_scale 40 with softcap 5: most logits sit at the cap, where the
    softcap slope is tiny; argmax is only checked on rows with a clear margin."""
    w = synth.small_workload(200, 64, 1200, 55, logit_scale=40.0, softcap=5.0)
    _check(w, synth.make_inputs(w), False)


def test_num_items_with_compaction():
    w = synth.small_workload(500, 64, 800, 56, prompt_frac=0.5, prompt_block=100)
    _check(w, synth.make_inputs(w), True, mean_divisor=321.0)
