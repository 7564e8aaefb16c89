"""Pins of the CPU oracle against things other than itself (CPU only).

Each test states what it pins.  Together they are chosen so that a plausible
mistake in the oracle (a dropped bias or scale, a wrong sign, a transposed
operand, a wrong softcap derivative, a wrong tie-break, a wrong divisor)
fails at least one of them:
  * closed forms (lm_head = 0 gives loss = entropy = ln V; V = 1; V = 2;
    hand-derived logits with known lse);
  * a library routine on an independent code path: torch's cross_entropy,
    Categorical entropy, argmax and float64 autograd;
  * brute-force central finite differences of the oracle's own loss;
  * invariants (softmax sums to 1, entropy = -sum p ln p, shift / permutation
    invariance, gradient identities).
"""
import math

import numpy as np
import pytest
import torch

from oracle import IGNORE_INDEX, Problem, backward, final_logits, forward, loss_value


def _rand_problem(n, h, v, seed, bias=True, ignore_every=3):
    rng = np.random.default_rng(seed)
    hid = rng.standard_normal((n, h))
    w = rng.standard_normal((v, h)) * 0.5
    b = rng.standard_normal(v) * 0.3 if bias else None
    t = rng.integers(0, v, n)
    if ignore_every:
        t[::ignore_every] = IGNORE_INDEX
    return hid, w, b, t


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("scale,cap", [(1.0, 0.0), (0.3, 0.0), (2.0, 5.0)])
def test_zero_weight_closed_form(scale, cap):
    """lm_head = 0 (no bias): every logit is 0, so loss = entropy = ln V,
    argmax = 0 (lowest index wins the all-way tie), grad_hidden = 0 and
    grad_weight[v] = sum_n g_n (1/V - [t_n = v]) s h_n (softcap slope 1 at 0)."""
    n, h, v = 7, 5, 11
    rng = np.random.default_rng(3)
    hid = rng.standard_normal((n, h))
    w = np.zeros((v, h))
    t = np.array([0, 4, IGNORE_INDEX, 10, 0, 3, 7])
    prob = Problem(logit_scale=scale, softcap=cap)
    f = forward(hid, w, None, t, prob)
    valid = t != IGNORE_INDEX
    assert np.allclose(f["loss"][valid], math.log(v), atol=1e-14)
    assert np.allclose(f["entropy"][valid], math.log(v), atol=1e-14)
    assert np.all(f["loss"][~valid] == 0) and np.all(f["entropy"][~valid] == 0)
    assert np.allclose(f["lse"], math.log(v), atol=1e-14)
    assert np.all(f["argmax"] == 0)
    assert list(f["hit"]) == [1, 0, 0, 0, 1, 0, 0]
    assert f["n_valid"] == 6 and f["n_correct"] == 2
    assert math.isclose(f["loss_mean"], math.log(v), rel_tol=1e-14)

    g = backward(hid, w, None, t, prob, "sum", 1.0)
    assert np.all(g["grad_hidden"] == 0)
    expect = np.zeros((v, h))
    for i in range(n):
        if t[i] == IGNORE_INDEX:
            continue
        for j in range(v):
            expect[j] += (1.0 / v - (1.0 if j == t[i] else 0.0)) * scale * hid[i]
    assert np.allclose(g["grad_weight"], expect, atol=1e-14)


def test_hand_derived_logits():
    """h = I, W picks logits [1, 0, 0] and [0, 1, 0]: lse = ln(e + 2) for both
    rows; row 0 (target 0) has loss ln(e + 2) - 1 and hit 1; row 1 (target 2)
    has loss ln(e + 2), argmax 1 and hit 0; entropy = lse - e/(e + 2)."""
    hid = np.eye(2)
    w = np.array([[1.0, 0.0], [0.0, 1.0], [0.0, 0.0]])
    t = np.array([0, 2])
    f = forward(hid, w, None, t, Problem())
    lse = math.log(math.e + 2)
    assert np.allclose(f["lse"], [lse, lse], atol=1e-15)
    assert np.allclose(f["loss"], [lse - 1, lse], atol=1e-15)
    assert np.allclose(f["entropy"], lse - math.e / (math.e + 2), atol=1e-15)
    assert list(f["argmax"]) == [0, 1] and list(f["hit"]) == [1, 0]
    # bias shifts the logits before the scale: z = 2 * ([1,0,0] + [0, 0, 1])
    f2 = forward(hid[:1], w, np.array([0.0, 0.0, 1.0]), t[:1], Problem(logit_scale=2.0))
    lse2 = math.log(2 * math.exp(2) + 1)
    assert math.isclose(f2["loss"][0], lse2 - 2, rel_tol=1e-14)
    assert f2["argmax"][0] == 0          # tie between index 0 and 2 -> lowest


def test_vocab_one_and_two():
    """V = 1: loss 0, entropy 0, hit 1.  V = 2: loss = softplus(z_other - z_t)."""
    rng = np.random.default_rng(5)
    hid = rng.standard_normal((4, 3))
    w1 = rng.standard_normal((1, 3))
    f = forward(hid, w1, None, np.zeros(4, dtype=np.int64), Problem())
    assert np.allclose(f["loss"], 0, atol=1e-15) and np.allclose(f["entropy"], 0, atol=1e-15)
    assert np.all(f["hit"] == 1)
    w2 = rng.standard_normal((2, 3))
    t = np.array([0, 1, 1, 0])
    f = forward(hid, w2, None, t, Problem())
    z = hid @ w2.T
    for i in range(4):
        other = z[i, 1 - t[i]] - z[i, t[i]]
        assert math.isclose(f["loss"][i], math.log1p(math.exp(other)), rel_tol=1e-13)


def test_all_ignored_batch_is_zero():
    """Every target = -100: loss, mean, entropy, accuracy and every gradient
    are exactly 0 (the all-ignored branch of the cce pull request)."""
    hid, w, b, _ = _rand_problem(9, 6, 13, 1)
    t = np.full(9, IGNORE_INDEX)
    prob = Problem(logit_scale=0.5, softcap=3.0)
    f = forward(hid, w, b, t, prob)
    assert f["n_valid"] == 0 and f["loss_sum"] == 0 and f["loss_mean"] == 0
    assert np.all(f["loss"] == 0) and np.all(f["entropy"] == 0) and np.all(f["hit"] == 0)
    for mode in ("mean", "sum"):
        g = backward(hid, w, b, t, prob, mode, 1.0)
        for k in ("grad_hidden", "grad_weight", "grad_bias"):
            assert np.all(g[k] == 0), k


# ---------------------------------------------------------- library routines

def _torch_reference(hid, w, b, t, prob, reduction, grad_out):
    """torch float64: logits + F.cross_entropy + autograd (independent path)."""
    h_t = torch.tensor(hid, dtype=torch.float64, requires_grad=True)
    w_t = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    b_t = None if b is None else torch.tensor(b, dtype=torch.float64, requires_grad=True)
    logits = torch.nn.functional.linear(h_t, w_t, b_t) * prob.logit_scale
    if prob.softcap > 0:
        logits = torch.tanh(logits / prob.softcap) * prob.softcap
    tt = torch.tensor(t)
    loss = torch.nn.functional.cross_entropy(logits, tt, ignore_index=IGNORE_INDEX,
                                             reduction=reduction)
    if reduction == "none":
        obj = (loss * torch.tensor(grad_out, dtype=torch.float64)).sum()
    else:
        obj = loss * float(grad_out)
    obj.backward()
    ent = torch.distributions.Categorical(logits=logits.detach()).entropy()
    return dict(loss=loss.detach().numpy(), entropy=ent.numpy(),
                argmax=torch.argmax(logits.detach(), dim=1).numpy(),
                gh=h_t.grad.numpy(), gw=w_t.grad.numpy(),
                gb=None if b_t is None else b_t.grad.numpy())


@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
@pytest.mark.parametrize("scale,cap,bias", [(1.0, 0.0, False), (0.0625, 0.0, True),
                                            (1.3, 4.0, True), (1.0, 30.0, False)])
def test_against_torch_cross_entropy(reduction, scale, cap, bias):
    """Per-token loss, entropy, argmax, reductions and all gradients equal
    torch's cross_entropy / Categorical / autograd in float64."""
    n, h, v = 23, 9, 37
    hid, w, b, t = _rand_problem(n, h, v, 11, bias=bias)
    prob = Problem(logit_scale=scale, softcap=cap)
    rng = np.random.default_rng(2)
    grad_out = rng.uniform(0, 2, n) if reduction == "none" else 1.7
    ref = _torch_reference(hid, w, b, t, prob, reduction, grad_out)
    f = forward(hid, w, b, t, prob)
    valid = t != IGNORE_INDEX
    if reduction == "none":
        assert np.allclose(f["loss"], ref["loss"], atol=1e-12)
    elif reduction == "mean":
        assert math.isclose(f["loss_mean"], float(ref["loss"]), rel_tol=1e-12)
    else:
        assert math.isclose(f["loss_sum"], float(ref["loss"]), rel_tol=1e-12)
    assert np.allclose(f["entropy"][valid], ref["entropy"][valid], atol=1e-12)
    assert np.array_equal(f["argmax"], ref["argmax"])
    g = backward(hid, w, b, t, prob, reduction, grad_out)
    assert np.allclose(g["grad_hidden"], ref["gh"], atol=1e-12)
    assert np.allclose(g["grad_weight"], ref["gw"], atol=1e-12)
    if bias:
        assert np.allclose(g["grad_bias"], ref["gb"], atol=1e-12)


def test_num_items_divisor():
    """mean_divisor > 0 replaces the valid-row count in the mean (the trainer's
    num_items_in_batch): loss_mean * divisor = loss_sum, and the gradient is
    the sum gradient divided by it."""
    hid, w, b, t = _rand_problem(12, 4, 9, 4)
    prob = Problem(mean_divisor=40.0)
    f = forward(hid, w, b, t, prob)
    assert math.isclose(f["loss_mean"] * 40.0, f["loss_sum"], rel_tol=1e-14)
    gm = backward(hid, w, b, t, prob, "mean", 1.0)
    gs = backward(hid, w, b, t, prob, "sum", 1.0)
    assert np.allclose(gm["grad_weight"] * 40.0, gs["grad_weight"], atol=1e-13)


# ---------------------------------------------------- finite differences

@pytest.mark.parametrize("mode", ["mean", "sum", "none"])
def test_finite_differences(mode):
    """Brute-force central differences of the oracle's loss match its backward
    for every entry of hidden, weight and bias (bias, scale and a softcap that
    is far from linear are all on)."""
    n, h, v = 3, 4, 7
    hid, w, b, t = _rand_problem(n, h, v, 21, ignore_every=0)
    t[1] = IGNORE_INDEX
    hid *= 2.0
    prob = Problem(logit_scale=0.7, softcap=1.5)
    rng = np.random.default_rng(8)
    go = rng.uniform(0.2, 2.0, n) if mode == "none" else 1.3
    g = backward(hid, w, b, t, prob, mode, go)
    eps = 1e-6

    def fd(arr, setter):
        out = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = setter()
            arr[idx] = old - eps
            lm = setter()
            arr[idx] = old
            out[idx] = (lp - lm) / (2 * eps)
        return out

    def loss():
        return loss_value(hid, w, b, t, prob, mode, go)

    assert np.allclose(fd(hid, loss), g["grad_hidden"], atol=1e-8)
    assert np.allclose(fd(w, loss), g["grad_weight"], atol=1e-8)
    assert np.allclose(fd(b, loss), g["grad_bias"], atol=1e-8)
    assert np.all(g["grad_hidden"][1] == 0)      # ignored row


# ------------------------------------------------------------- invariants

def test_softmax_and_entropy_identities():
    """sum_v exp(z - lse) = 1 per row, and lse - sum p z equals the direct
    -sum p ln p."""
    hid, w, b, t = _rand_problem(16, 8, 50, 31)
    prob = Problem(logit_scale=1.7, softcap=2.0)
    f = forward(hid, w, b, t, prob)
    z = final_logits(hid, w, b, prob)
    p = np.exp(z - f["lse"][:, None])
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)
    direct = -(p * np.log(p)).sum(axis=1)
    valid = t != IGNORE_INDEX
    assert np.allclose(f["entropy"][valid], direct[valid], atol=1e-10)


def test_shift_and_permutation_invariance():
    """Without softcap, a constant added to every bias leaves every output
    unchanged; permuting the vocabulary (rows of W and bias, targets
    remapped) permutes grad_weight the same way and leaves the rest unchanged."""
    hid, w, b, t = _rand_problem(10, 5, 17, 41)
    prob = Problem(logit_scale=0.9)
    f0 = forward(hid, w, b, t, prob)
    f1 = forward(hid, w, b + 3.25, t, prob)
    assert np.allclose(f0["loss"], f1["loss"], atol=1e-12)
    assert np.allclose(f0["entropy"], f1["entropy"], atol=1e-12)

    perm = np.random.default_rng(0).permutation(17)
    inv = np.argsort(perm)
    tp = np.where(t == IGNORE_INDEX, t, inv[np.maximum(t, 0)])
    fp = forward(hid, w[perm], b[perm], tp, prob)
    assert np.allclose(f0["loss"], fp["loss"], atol=1e-12)
    assert np.allclose(f0["lse"], fp["lse"], atol=1e-12)
    assert np.array_equal(f0["hit"], fp["hit"])
    g0 = backward(hid, w, b, t, prob, "sum", 1.0)
    gp = backward(hid, w[perm], b[perm], tp, prob, "sum", 1.0)
    assert np.allclose(g0["grad_weight"][perm], gp["grad_weight"], atol=1e-12)
    assert np.allclose(g0["grad_hidden"], gp["grad_hidden"], atol=1e-12)


def test_gradient_identities():
    """(a) with scale 1 and no softcap every valid row's gradient w.r.t. the
    logits sums to 0, so grad_bias sums to 0; (b) mean = sum / n_valid;
    (c) "none" with unit weights = "sum"; (d) sum_v <gw_v, W_v> equals
    sum_n <gh_n, h_n> (both are sum_{n,v} d[n,v] (h W^T)[n,v])."""
    hid, w, b, t = _rand_problem(14, 6, 21, 51)
    prob = Problem()
    gs = backward(hid, w, b, t, prob, "sum", 1.0)
    assert abs(gs["grad_bias"].sum()) < 1e-12
    gm = backward(hid, w, b, t, prob, "mean", 1.0)
    nv = int((t != IGNORE_INDEX).sum())
    assert np.allclose(gm["grad_weight"] * nv, gs["grad_weight"], atol=1e-12)
    gn = backward(hid, w, b, t, prob, "none", np.ones(14))
    assert np.allclose(gn["grad_hidden"], gs["grad_hidden"], atol=1e-14)
    prob2 = Problem(logit_scale=0.4, softcap=2.0)
    g2 = backward(hid, w, b, t, prob2, "sum", 1.0)
    lhs = float((g2["grad_weight"] * w).sum())
    rhs = float((g2["grad_hidden"] * hid).sum())
    assert math.isclose(lhs, rhs, rel_tol=1e-10)


def test_scale_folding_and_large_cap():
    """With no bias or softcap, logit_scale s equals scaling W by s; a softcap
    of 1e6 is the identity to 1e-9."""
    hid, w, _, t = _rand_problem(8, 5, 19, 61, bias=False)
    a = forward(hid, w, None, t, Problem(logit_scale=0.25))
    c = forward(hid, w * 0.25, None, t, Problem())
    assert np.allclose(a["loss"], c["loss"], atol=1e-13)
    d = forward(hid, w, None, t, Problem(softcap=1e6))
    e = forward(hid, w, None, t, Problem())
    assert np.allclose(d["loss"], e["loss"], atol=1e-9)


def test_rows_and_vocab_sampling_agree_with_full():
    """The sampled forms used at full workload size (``rows`` for per-token
    outputs and grad_hidden, ``vocab_rows`` for grad_weight / grad_bias)
    return the same numbers as the full computation."""
    hid, w, b, t = _rand_problem(20, 7, 30, 71)
    prob = Problem(logit_scale=1.1, softcap=3.0)
    full_f = forward(hid, w, b, t, prob)
    rows = np.array([0, 3, 19, 7])
    sf = forward(hid, w, b, t, prob, rows=rows)
    for k in ("loss", "lse", "entropy", "argmax", "hit", "margin"):
        assert np.allclose(sf[k], full_f[k][rows]), k
    full_g = backward(hid, w, b, t, prob, "mean", 1.0)
    vr = np.array([29, 0, 5])
    sg = backward(hid, w, b, t, prob, "mean", 1.0, rows=rows, vocab_rows=vr)
    assert np.allclose(sg["grad_hidden_rows"], full_g["grad_hidden"][rows], atol=1e-14)
    assert np.allclose(sg["grad_weight_rows"], full_g["grad_weight"][vr], atol=1e-14)
    assert np.allclose(sg["grad_bias_rows"], full_g["grad_bias"][vr], atol=1e-14)


def test_argmax_targets_give_exact_accuracy():
    """Targets set to the argmax of the final logits give accuracy exactly 1
    on rows whose top-2 margin is at least 1e-2 (the cce pull request's
    "Correctness" experiment, at small size)."""
    hid, w, b, _ = _rand_problem(64, 16, 300, 81, ignore_every=0)
    prob = Problem(softcap=30.0)
    z = final_logits(hid, w, b, prob)
    t = np.argmax(z, axis=1)
    f = forward(hid, w, b, t, prob)
    assert np.all(f["hit"][f["margin"] >= 1e-2] == 1)
    assert f["n_correct"] == 64


def test_bad_targets_are_counted_and_ignored():
    """A target outside [0, V) that is not -100 contributes nothing and is
    counted in n_bad."""
    hid, w, b, t = _rand_problem(6, 3, 5, 91, ignore_every=0)
    t[2] = 5
    t[4] = -7
    f = forward(hid, w, b, t, Problem())
    assert f["n_bad"] == 2 and f["n_valid"] == 4
    assert f["loss"][2] == 0 and f["loss"][4] == 0


# ------------------------------------------------------------- top-2 margin

def _torch_final_logits(hid, w, b, prob):
    """Final logits through torch float64 (an independent code path)."""
    h_t = torch.tensor(hid, dtype=torch.float64)
    w_t = torch.tensor(w, dtype=torch.float64)
    b_t = None if b is None else torch.tensor(b, dtype=torch.float64)
    z = torch.nn.functional.linear(h_t, w_t, b_t) * prob.logit_scale
    if prob.softcap > 0:
        z = torch.tanh(z / prob.softcap) * prob.softcap
    return z


def _topk_margin(z):
    if z.shape[1] == 1:
        return np.full(z.shape[0], np.inf)
    top = torch.topk(z, 2, dim=1).values
    return (top[:, 0] - top[:, 1]).numpy()


def test_margin_against_topk():
    """The top-2 margin that decides which rows get argmax / hit parity is
    top-1 minus top-2 of the final logits (argmax is taken on the final
    logits: cce pull request, review "Correctness"), checked against
    torch.topk in float64: random rows, exact ties (two identical lm_head
    rows, so the margin is exactly 0 on every row where they lead, and the
    argmax is the lower of the two), V = 2 (|z0 - z1|) and V = 1 (inf)."""
    hid, w, b, t = _rand_problem(40, 6, 29, 101)
    prob = Problem(logit_scale=0.8, softcap=4.0)
    f = forward(hid, w, b, t, prob)
    z = _torch_final_logits(hid, w, b, prob)
    assert np.allclose(f["margin"], _topk_margin(z), atol=1e-13)
    assert np.all(f["margin"] > 0)

    # ties: rows 3 and 17 of W and of the bias are equal, and the bias makes
    # them lead on every row
    w2 = w.copy()
    w2[17] = w2[3]
    b2 = b.copy()
    b2[17] = b2[3] = 50.0
    f2 = forward(hid, w2, b2, t, Problem())
    z2 = _torch_final_logits(hid, w2, b2, Problem())
    lead = torch.argmax(z2, dim=1).numpy()
    assert np.all(lead == 3) and np.all(f2["argmax"] == 3)
    assert np.all(f2["margin"] == 0.0)
    assert np.array_equal(f2["margin"], _topk_margin(z2))

    w3 = w[:2]
    f3 = forward(hid, w3, None, np.zeros(40, dtype=np.int64), Problem())
    z3 = hid @ w3.T
    assert np.allclose(f3["margin"], np.abs(z3[:, 0] - z3[:, 1]), atol=1e-13)

    f4 = forward(hid, w[:1], None, np.zeros(40, dtype=np.int64), Problem())
    assert np.all(np.isinf(f4["margin"]))


def test_many_row_blocks_against_torch():
    """N * V > 3 * 2^24, so the oracle materialises its logits in four row
    blocks (the path every full-size workload takes): per-token loss, lse,
    entropy, argmax and margin against torch float64 (linear + cross_entropy
    + logsumexp + Categorical entropy + topk) on every row, ragged V."""
    n, h, v = 600, 8, 100003
    rng = np.random.default_rng(111)
    hid = rng.standard_normal((n, h))
    w = rng.standard_normal((v, h)) * 0.3
    b = rng.standard_normal(v) * 0.1
    t = rng.integers(0, v, n)
    t[::17] = IGNORE_INDEX
    prob = Problem(logit_scale=1.5)
    f = forward(hid, w, b, t, prob)
    z = _torch_final_logits(hid, w, b, prob)
    tt = torch.tensor(t)
    loss = torch.nn.functional.cross_entropy(z, tt, ignore_index=IGNORE_INDEX,
                                             reduction="none").numpy()
    valid = t != IGNORE_INDEX
    assert np.allclose(f["loss"], loss, atol=1e-11)
    assert np.allclose(f["lse"], torch.logsumexp(z, dim=1).numpy(), atol=1e-11)
    ent = torch.distributions.Categorical(logits=z).entropy().numpy()
    assert np.allclose(f["entropy"][valid], ent[valid], atol=1e-10)
    assert np.array_equal(f["argmax"], torch.argmax(z, dim=1).numpy())
    assert np.allclose(f["margin"], _topk_margin(z), atol=1e-12)
    assert math.isclose(f["loss_mean"], float(loss[valid].mean()), rel_tol=1e-12)


def test_gradient_sketches_against_torch():
    """The oracle's gradient sketches (fixed sign projections of the whole
    gradients, used to check full-size outputs) equal the same projections of
    torch's float64 autograd gradients, with and without bias and softcap, on
    a shape cut into several row blocks.  Without a bias, torch's gradient
    with respect to an all-zero bias stands in for grad_bias."""
    import oracle.flce_oracle as orc
    for bias, cap, red in ((True, 4.0, "none"), (False, 0.0, "mean"), (False, 2.0, "sum")):
        n, h, v = 40, 6, 50
        hid, w, b, t = _rand_problem(n, h, v, 77, bias=bias)
        prob = Problem(logit_scale=0.8, softcap=cap)
        rng = np.random.default_rng(3)
        grad_out = rng.uniform(0, 2, n) if red == "none" else 1.3
        sigma = rng.choice([-1.0, 1.0], size=(3, n))
        rho = rng.choice([-1.0, 1.0], size=(3, v))
        ref = _torch_reference(hid, w, b if bias else np.zeros(v), t, prob, red, grad_out)
        real = orc._row_blocks
        orc._row_blocks = lambda nn, vv, max_elems=1 << 24: real(nn, vv, max_elems=7 * vv)
        try:
            g = orc.backward(hid, w, b, t, prob, red, grad_out, rows=np.arange(0, n, 5),
                             vocab_rows=np.array([0, v - 1]), sketch=(sigma, rho))
        finally:
            orc._row_blocks = real
        assert np.allclose(g["sketch_grad_hidden"], sigma @ ref["gh"], atol=1e-12)
        assert np.allclose(g["sketch_grad_weight"], rho @ ref["gw"], atol=1e-12)
        assert np.allclose(g["sketch_grad_bias"], rho @ ref["gb"], atol=1e-12)
        assert np.abs(g["sketch_grad_weight"]).max() > 1e-3
