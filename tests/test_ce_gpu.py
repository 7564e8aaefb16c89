"""GPU parity of the standalone cross-entropy on materialised logits (the C ABI
flce_ce_forward / flce_ce_backward) against the CPU oracle (oracle/ce_oracle.py).

Tolerances, from the arithmetic: the per-token loss is an fp32 log-sum-exp
whose sums run over at most ~10^3 terms per thread and a tree of partial
pairs (relative error of the sum ~1e-5, so |loss - oracle| <= 1e-4); the
reductions are summed in double from those losses (relative 1e-5); the
stored gradient is one fp32 exp rounded once to the logits dtype
(|g - oracle| <= 2^-8 |oracle| for bf16, 1e-4 |oracle| for fp32, plus 2^-22 for
the fp32 rounding of p next to 1 in a target's p - 1),
and the backward adds one more rounding of one fp32 multiply, which is also
checked bit for bit against that multiply done on the CPU."""
import numpy as np
import pytest
import torch

import linear_cross_entropy_fp32_amd as flce
from linear_cross_entropy_fp32_amd import synth
from oracle import ce_backward, ce_forward
from tests.gpu_cases import say

pytestmark = pytest.mark.gpu
MODES = {"mean": flce.FLCE_GRAD_MEAN, "sum": flce.FLCE_GRAD_SUM, "none": flce.FLCE_GRAD_PER_TOKEN}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    flce.lib()


def _grad_tol(dtype):
    # relative: one rounding to the dtype plus the fp32 exp; absolute: the
    # fp32 rounding of p next to 1 in the target's p - 1
    return (2.0 ** -8, 2.0 ** -22) if dtype == "bf16" else (1e-4, 2.0 ** -22)


def _check_grad(gpu, ref, dtype, label, rounds=1):
    rel, absf = _grad_tol(dtype)
    d = np.abs(gpu - ref)
    lim = rounds * rel * np.abs(ref) + absf
    bad = d > lim
    assert not bad.any(), f"{label}: {int(bad.sum())} elements off, worst {d[bad].max()}"


def _run(logits_cpu, targets, mode, grad_out, dtype, mean_divisor=0.0):
    dev = "cuda:0"
    x = logits_cpu.to(dev)
    t = targets.to(dev)
    f = flce.flce_ce_forward(x, t, mean_divisor=mean_divisor)
    stored = x.clone()
    go = grad_out.to(dev).reshape(-1)
    flce.flce_ce_backward(x, t, f["reduced_i64"], MODES[mode], go, mean_divisor=mean_divisor)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in f.items()}, stored.cpu(), x.cpu()


CASES = [  # (N, V, dtype, mode): register rows, streamed rows, ragged rows, tiny vocabularies
    (300, 1000, "bf16", "none"), (257, 1001, "bf16", "mean"), (130, 1000, "f32", "sum"),
    (200, 777, "f32", "none"), (64, 32000, "bf16", "none"), (40, 151936, "bf16", "mean"),
    (24, 151936, "f32", "none"), (33, 130000, "f32", "sum"), (50, 1, "bf16", "mean"),
    (70, 2, "f32", "none"), (90, 8, "bf16", "sum"),
]


@pytest.mark.parametrize("n,v,dtype,mode", CASES)
def test_ce_parity(n, v, dtype, mode):
    say(f"[ce] N={n} V={v} {dtype} {mode}")
    logits, targets, weights = synth.ce_inputs(n, v, 100 + v % 97, dtype)
    grad_out = weights if mode == "none" else torch.tensor([1.7])
    f, stored, scaled = _run(logits, targets, mode, grad_out, dtype)
    z = logits.double().numpy()
    t = targets.numpy()
    o = ce_forward(z, t)
    assert np.abs(f["loss"].double().numpy() - o["loss"]).max() <= 1e-4
    assert np.abs(f["lse"].double().numpy() - o["lse"]).max() <= 1e-4
    assert np.all(f["loss"].numpy()[~o["valid"]] == 0)
    rf, ri = f["reduced_f32"].double().numpy(), f["reduced_i64"].numpy()
    assert int(ri[0]) == o["n_valid"] and int(ri[1]) == o["n_bad"]
    # the per-token bound (1e-4) summed over the valid rows, or averaged
    for got, ref, floor in ((rf[0], o["loss_sum"], 1e-4 * o["n_valid"]),
                            (rf[1], o["loss_mean"], 1e-4)):
        assert abs(got - ref) <= 1e-5 * abs(ref) + floor, (got, ref)
    _check_grad(stored.double().numpy(), o["grad"], dtype, "forward gradient")
    ref_b = ce_backward(o["grad"], t, mode, grad_out.double().numpy())
    _check_grad(scaled.double().numpy(), ref_b, dtype, "backward gradient", rounds=2)
    # the backward is one fp32 multiply and one rounding per element
    gn = torch.from_numpy(np.where(o["valid"], (grad_out.numpy() if mode == "none" else
                                                np.full(n, float(grad_out[0]) /
                                                        (o["n_valid"] if mode == "mean" else 1))),
                                   0.0)).float()
    expect = (stored.float() * gn[:, None]).to(stored.dtype)
    if mode == "mean":   # the divisor is applied on the device in fp32: g / n_valid
        gn32 = torch.where(torch.from_numpy(o["valid"]),
                           torch.tensor(1.7, dtype=torch.float32) /
                           torch.tensor(float(o["n_valid"]), dtype=torch.float32),
                           torch.tensor(0.0))
        expect = (stored.float() * gn32[:, None]).to(stored.dtype)
    assert torch.equal(scaled, expect)


def test_ce_all_ignored_and_bad_targets():
    logits, targets, _ = synth.ce_inputs(100, 500, 7, "bf16")
    targets[:] = -100
    f, stored, scaled = _run(logits, targets, "mean", torch.tensor([1.0]), "bf16")
    assert f["reduced_f32"].tolist() == [0.0, 0.0] and f["reduced_i64"].tolist() == [0, 0]
    assert torch.count_nonzero(stored).item() == 0 and torch.count_nonzero(scaled).item() == 0
    logits, targets, _ = synth.ce_inputs(100, 500, 8, "bf16")
    targets[3], targets[4] = 500, -5
    f, stored, _ = _run(logits, targets, "sum", torch.tensor([1.0]), "bf16")
    assert int(f["reduced_i64"][1]) == 2 - int((targets[3:5] == -100).sum())
    assert torch.count_nonzero(stored[3:5]).item() == 0


def test_ce_empty_batch():
    dev = "cuda:0"
    x = torch.zeros(0, 64, dtype=torch.bfloat16, device=dev)
    t = torch.zeros(0, dtype=torch.int64, device=dev)
    f = flce.flce_ce_forward(x, t)
    torch.cuda.synchronize()
    assert f["reduced_f32"].cpu().tolist() == [0.0, 0.0]
    assert f["reduced_i64"].cpu().tolist() == [0, 0]


def test_ce_autograd_wrapper():
    """cross_entropy(...).backward() through the in-place autograd function
    equals the oracle's gradient for reduction none with weights, and mean."""
    dev = "cuda:0"
    logits, targets, weights = synth.ce_inputs(128, 5000, 21, "bf16")
    o = ce_forward(logits.double().numpy(), targets.numpy())
    x = logits.to(dev).requires_grad_(True)
    loss, nv = flce.cross_entropy(x, targets.to(dev), reduction="none")
    (loss * weights.to(dev)).sum().backward()
    torch.cuda.synchronize()
    ref = ce_backward(o["grad"], targets.numpy(), "none", weights.double().numpy())
    _check_grad(x.grad.double().cpu().numpy(), ref, "bf16", "autograd none", rounds=2)
    assert np.abs(loss.detach().double().cpu().numpy() - o["loss"]).max() <= 1e-4
    x2 = logits.to(dev).requires_grad_(True)
    lm, _ = flce.cross_entropy(x2, targets.to(dev), reduction="mean")
    lm.backward()
    torch.cuda.synchronize()
    assert abs(lm.item() - o["loss_mean"]) <= 1e-5 * abs(o["loss_mean"])
    ref_m = ce_backward(o["grad"], targets.numpy(), "mean", 1.0)
    _check_grad(x2.grad.double().cpu().numpy(), ref_m, "bf16", "autograd mean", rounds=2)


@pytest.mark.parametrize("name", list(synth.CE_WORKLOADS))
def test_ce_fullsize_sampled_rows(name):
    """The benchmark shapes (8192 rows, bf16 logits drawn on the GPU), none with
    per-row weights: sampled rows against the oracle computed from the same
    logits, every row's reductions against the per-token losses, and the
    backward's single rounding checked on every element of the sampled rows."""
    n, v = synth.CE_WORKLOADS[name]
    dev = "cuda:0"
    logits, targets, weights = synth.ce_inputs(n, v, 4242, "bf16", device=dev)
    rows = np.array(sorted({0, 1, 16, 17, 18, 4095, 4096, n - 2, n - 1} |
                           set(np.random.default_rng(5).integers(0, n, 8).tolist())))
    z = logits[rows].double().cpu().numpy()
    say(f"[ce] full size {name}")
    t = targets.to(dev)
    f = flce.flce_ce_forward(logits, t)
    stored = logits[rows].clone()
    flce.flce_ce_backward(logits, t, f["reduced_i64"], flce.FLCE_GRAD_PER_TOKEN,
                          weights.to(dev))
    torch.cuda.synchronize()
    tr = targets.numpy()[rows]
    o = ce_forward(z, tr)
    loss = f["loss"].cpu().double().numpy()
    assert np.abs(loss[rows] - o["loss"]).max() <= 1e-4
    _check_grad(stored.double().cpu().numpy(), o["grad"], "bf16", "forward gradient")
    ref_b = ce_backward(o["grad"], tr, "none", weights.double().numpy()[rows])
    scaled = logits[rows].cpu()
    _check_grad(scaled.double().numpy(), ref_b, "bf16", "backward gradient", rounds=2)
    wv = torch.where(torch.from_numpy((tr >= 0)), weights[rows], torch.tensor(0.0))
    assert torch.equal(scaled, (stored.cpu().float() * wv[:, None]).to(torch.bfloat16))
    valid = (targets.numpy() >= 0)
    assert int(f["reduced_i64"][0]) == int(valid.sum())
    assert abs(float(f["reduced_f32"][0]) - loss[valid].sum()) <= 1e-5 * loss[valid].sum()
