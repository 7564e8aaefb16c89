"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
in test_oracle_pins.py catch every one of them."""
import numpy as np
import pytest

import oracle.flce_oracle as orc
import tests.test_oracle_pins as pins

PIN_TESTS = [
    (pins.test_zero_weight_closed_form, dict(scale=2.0, cap=5.0)),
    (pins.test_zero_weight_closed_form, dict(scale=1.0, cap=0.0)),
    (pins.test_hand_derived_logits, {}),
    (pins.test_vocab_one_and_two, {}),
    (pins.test_all_ignored_batch_is_zero, {}),
    (pins.test_against_torch_cross_entropy, dict(reduction="mean", scale=1.3, cap=4.0, bias=True)),
    (pins.test_against_torch_cross_entropy, dict(reduction="none", scale=0.0625, cap=0.0,
                                                 bias=True)),
    (pins.test_finite_differences, dict(mode="sum")),
    (pins.test_softmax_and_entropy_identities, {}),
    (pins.test_gradient_identities, {}),
    (pins.test_num_items_divisor, {}),
    (pins.test_bad_targets_are_counted_and_ignored, {}),
    (pins.test_margin_against_topk, {}),
    (pins.test_gradient_sketches_against_torch, {}),
]


def _logits_bias_after_scale(h, w, bias, prob):
    z = (h @ w.T) * prob.logit_scale
    if bias is not None:
        z = z + bias[None, :]
    if prob.softcap > 0:
        z = prob.softcap * np.tanh(z / prob.softcap)
    return z


def _logits_cap_before_scale(h, w, bias, prob):
    z = h @ w.T
    if bias is not None:
        z = z + bias[None, :]
    if prob.softcap > 0:
        z = prob.softcap * np.tanh(z / prob.softcap)
    return z * prob.logit_scale


def _logits_transposed(h, w, bias, prob):
    return orc_final_logits_orig(h[:, ::-1], w, bias, prob)


def _grad_wrong_cap_derivative(z, t, gn, valid, prob):
    d = orc_grad_orig(z, t, gn, valid, Problem_nocap(prob))
    if prob.softcap > 0:
        d *= 1.0 + (z / prob.softcap) ** 2
    return d


def _grad_no_scale(z, t, gn, valid, prob):
    return orc_grad_orig(z, t, gn, valid, prob) / (prob.logit_scale or 1.0)


def _grad_wrong_sign(z, t, gn, valid, prob):
    return -orc_grad_orig(z, t, gn, valid, prob)


def _row_scale_divide_by_n(targets, vocab, prob, mode, grad_out, n_valid=None):
    out = orc_row_scale_orig(targets, vocab, prob, mode, grad_out, n_valid)
    if mode == "mean" and prob.mean_divisor <= 0:
        nv = int(orc.valid_mask(targets, vocab, prob)[0].sum())
        if nv:
            out = out * nv / len(targets)
    return out


def _valid_counts_bad_targets(targets, vocab, prob):
    t = np.asarray(targets, dtype=np.int64)
    valid = t != prob.ignore_index
    return valid & (t < vocab) & (t >= 0), np.zeros_like(valid)


orc_final_logits_orig = orc.final_logits
orc_grad_orig = orc.grad_raw_logits
orc_row_scale_orig = orc.row_grad_scale


def Problem_nocap(prob):
    return orc.Problem(prob.logit_scale, 0.0, prob.ignore_index, prob.mean_divisor)


def _forward_entropy_sign(*a, **k):
    f = orc_forward_orig(*a, **k)
    f["entropy"] = np.where(f["valid"], 2 * f["lse"] - f["entropy"], 0.0)
    return f


def _forward_last_argmax(hidden, weight, bias, targets, prob, rows=None):
    f = orc_forward_orig(hidden, weight, bias, targets, prob, rows)
    h = np.asarray(hidden, dtype=np.float64)
    if rows is not None:
        h = h[rows]
    z = orc.final_logits(h, np.asarray(weight, dtype=np.float64), bias, prob)
    v = z.shape[1]
    f["argmax"] = v - 1 - np.argmax(z[:, ::-1], axis=1)
    return f


def _forward_margin_zero(*a, **k):
    f = orc_forward_orig(*a, **k)
    f["margin"] = np.zeros_like(f["margin"])
    return f


def _forward_margin_top1_minus_top3(hidden, weight, bias, targets, prob, rows=None):
    f = orc_forward_orig(hidden, weight, bias, targets, prob, rows)
    h = np.asarray(hidden, dtype=np.float64)
    if rows is not None:
        h = h[rows]
    z = orc.final_logits(h, np.asarray(weight, dtype=np.float64), bias, prob)
    v = z.shape[1]
    if v >= 3:
        top = np.sort(z, axis=1)
        f["margin"] = top[:, -1] - top[:, -3]
    return f


orc_forward_orig = orc.forward

MUTATIONS = {
    "bias_after_scale": ("final_logits", _logits_bias_after_scale),
    "softcap_before_scale": ("final_logits", _logits_cap_before_scale),
    "transposed_hidden": ("final_logits", _logits_transposed),
    "softcap_derivative_sign": ("grad_raw_logits", _grad_wrong_cap_derivative),
    "missing_scale_in_grad": ("grad_raw_logits", _grad_no_scale),
    "grad_sign": ("grad_raw_logits", _grad_wrong_sign),
    "mean_over_all_rows": ("row_grad_scale", _row_scale_divide_by_n),
    "bad_targets_not_counted": ("valid_mask", _valid_counts_bad_targets),
    "entropy_sign": ("forward", _forward_entropy_sign),
    "argmax_highest_index": ("forward", _forward_last_argmax),
    "margin_zero": ("forward", _forward_margin_zero),
    "margin_top1_minus_top3": ("forward", _forward_margin_top1_minus_top3),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(orc, attr, fn)
    # the pin module imported some names directly; route them to the mutant too
    for mod_name in ("forward", "backward", "final_logits", "loss_value"):
        monkeypatch.setattr(pins, mod_name, getattr(orc, mod_name))
    caught = 0
    for test, kw in PIN_TESTS:
        try:
            test(**kw)
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught > 0, f"mutation {name} passed every pin"


# ------------------------------------------- standalone cross-entropy oracle
import oracle.ce_oracle as ceo  # noqa: E402
import tests.test_ce_oracle_pins as cepins  # noqa: E402

CE_PINS = [(cepins.test_against_torch, dict(reduction=r)) for r in ("none", "mean", "sum")] + [
    (cepins.test_closed_forms, {}), (cepins.test_invariants_and_reductions, {})]
_ce_forward_orig = ceo.ce_forward
_ce_scale_orig = ceo.ce_row_scale


def _ce_no_onehot(logits, targets, ignore_index=-100, mean_divisor=0.0):
    f = _ce_forward_orig(logits, targets, ignore_index, mean_divisor)
    f["grad"] = np.where(f["valid"][:, None], np.exp(np.asarray(logits) - f["lse"][:, None]), 0.0)
    return f


def _ce_ignored_rows_keep_grad(logits, targets, ignore_index=-100, mean_divisor=0.0):
    f = _ce_forward_orig(logits, targets, ignore_index, mean_divisor)
    f["grad"] = f["grad"] + np.where(f["valid"][:, None], 0.0,
                                     np.exp(np.asarray(logits) - f["lse"][:, None]))
    return f


def _ce_mean_over_all_rows(targets, vocab, mode, grad_out, ignore_index=-100, mean_divisor=0.0):
    out = _ce_scale_orig(targets, vocab, mode, grad_out, ignore_index, mean_divisor)
    if mode == "mean":
        nv = int(ceo.ce_valid(targets, vocab, ignore_index)[0].sum())
        out = out * nv / len(targets)
    return out


def _ce_loss_sign(logits, targets, ignore_index=-100, mean_divisor=0.0):
    f = _ce_forward_orig(logits, targets, ignore_index, mean_divisor)
    f["loss"] = -f["loss"]
    f["loss_sum"] = -f["loss_sum"]
    f["loss_mean"] = -f["loss_mean"]
    return f


CE_MUTATIONS = {
    "ce_no_onehot": ("ce_forward", _ce_no_onehot),
    "ce_ignored_rows_keep_grad": ("ce_forward", _ce_ignored_rows_keep_grad),
    "ce_mean_over_all_rows": ("ce_row_scale", _ce_mean_over_all_rows),
    "ce_loss_sign": ("ce_forward", _ce_loss_sign),
}


@pytest.mark.parametrize("name", sorted(CE_MUTATIONS))
def test_ce_mutation_is_caught(name, monkeypatch):
    attr, fn = CE_MUTATIONS[name]
    monkeypatch.setattr(ceo, attr, fn)
    for mod_name in ("ce_forward", "ce_backward"):
        monkeypatch.setattr(cepins, mod_name, getattr(ceo, mod_name))
    caught = 0
    for test, kw in CE_PINS:
        try:
            test(**kw)
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught > 0, f"mutation {name} passed every pin"
