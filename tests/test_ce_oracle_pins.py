"""Pins of the standalone cross-entropy oracle (oracle/ce_oracle.py) against
things other than itself (CPU only): torch's cross_entropy with float64
autograd (a library routine on an independent code path), closed forms
(equal logits give ln V and a gradient 1/V - onehot; V = 1; V = 2 gives
softplus), and invariants (each valid row's gradient sums to 0, adding a
constant to a row changes nothing)."""
import math

import numpy as np
import pytest
import torch

from oracle import ce_backward, ce_forward

IGN = -100


def _case(n, v, seed, ignore_every=4, scale=4.0):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((n, v)) * scale
    t = rng.integers(0, v, n)
    if ignore_every:
        t[::ignore_every] = IGN
    return z, t


def _torch_ref(z, t, reduction, grad_out):
    zt = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(zt, torch.tensor(t), ignore_index=IGN,
                                             reduction=reduction)
    if reduction == "none":
        obj = (loss * torch.tensor(grad_out, dtype=torch.float64)).sum()
    else:
        obj = loss * float(grad_out)
    obj.backward()
    return loss.detach().numpy(), zt.grad.numpy()


@pytest.mark.parametrize("reduction", ["none", "mean", "sum"])
def test_against_torch(reduction):
    z, t = _case(37, 53, 5)
    rng = np.random.default_rng(6)
    grad_out = rng.uniform(0, 2, 37) if reduction == "none" else 1.7
    ref_loss, ref_grad = _torch_ref(z, t, reduction, grad_out)
    f = ce_forward(z, t)
    if reduction == "none":
        assert np.allclose(f["loss"], ref_loss, atol=1e-12)
    elif reduction == "mean":
        assert math.isclose(f["loss_mean"], float(ref_loss), rel_tol=1e-12)
    else:
        assert math.isclose(f["loss_sum"], float(ref_loss), rel_tol=1e-12)
    g = ce_backward(f["grad"], t, reduction, grad_out)
    assert np.allclose(g, ref_grad, atol=1e-12)
    lse = torch.logsumexp(torch.tensor(z), dim=1).numpy()
    assert np.allclose(f["lse"], lse, atol=1e-12)


def test_closed_forms():
    n, v = 6, 11
    z = np.full((n, v), 2.5)
    t = np.array([0, 3, IGN, 10, 5, 5])
    f = ce_forward(z, t)
    valid = t != IGN
    assert np.allclose(f["loss"][valid], math.log(v), atol=1e-14)
    assert np.all(f["loss"][~valid] == 0)
    expect = np.where(valid[:, None], np.full((n, v), 1.0 / v), 0.0)
    expect[np.nonzero(valid)[0], t[valid]] -= 1.0
    assert np.allclose(f["grad"], expect, atol=1e-15)
    # V = 1: loss 0, gradient 0
    f1 = ce_forward(np.array([[3.0], [-1.0]]), np.array([0, 0]))
    assert np.all(f1["loss"] == 0) and np.all(f1["grad"] == 0)
    # V = 2: loss = softplus(z_other - z_target)
    z2 = np.array([[0.3, -1.2], [2.0, 0.5]])
    f2 = ce_forward(z2, np.array([1, 0]))
    sp = lambda x: math.log1p(math.exp(x))
    assert math.isclose(f2["loss"][0], sp(0.3 + 1.2), rel_tol=1e-14)
    assert math.isclose(f2["loss"][1], sp(0.5 - 2.0), rel_tol=1e-14)


def test_invariants_and_reductions():
    z, t = _case(20, 30, 9)
    f = ce_forward(z, t)
    valid = f["valid"]
    assert np.allclose(f["grad"][valid].sum(axis=1), 0.0, atol=1e-14)
    assert np.all(f["grad"][~valid] == 0)
    f_shift = ce_forward(z + np.arange(20)[:, None] * 3.0, t)
    assert np.allclose(f_shift["loss"], f["loss"], atol=1e-12)
    assert math.isclose(f["loss_mean"] * f["n_valid"], f["loss_sum"], rel_tol=1e-14)
    gm = ce_backward(f["grad"], t, "mean", 1.0)
    gs = ce_backward(f["grad"], t, "sum", 1.0)
    assert np.allclose(gm * f["n_valid"], gs, atol=1e-14)
    w = np.linspace(0, 2, 20)
    gw = ce_backward(f["grad"], t, "none", w)
    assert np.allclose(gw, f["grad"] * w[:, None], atol=1e-15)
    # bad targets: ignored and counted
    t2 = t.copy()
    t2[1], t2[2] = 30, -7
    f2 = ce_forward(z, t2)
    assert f2["n_bad"] == 2
    assert f2["loss"][1] == 0 and f2["loss"][2] == 0 and np.all(f2["grad"][1:3] == 0)
    # all ignored: zero mean and zero gradient
    f3 = ce_forward(z, np.full(20, IGN))
    assert f3["loss_mean"] == 0.0 and np.all(ce_backward(f3["grad"], np.full(20, IGN), "mean",
                                                          1.0) == 0)
