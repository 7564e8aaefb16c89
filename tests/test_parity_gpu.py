"""GPU parity: the HIP path through the C ABI against the CPU oracle."""
import os

import numpy as np
import pytest
import torch

import linear_cross_entropy_fp32_amd as flce
from linear_cross_entropy_fp32_amd import synth
from oracle import Problem, backward, final_logits, forward
from tests.gpu_cases import (check_fullsize, check_grad, check_reduced, check_tokens,
                             check_vocab_grad_parts, prob_of, rel_fro, run_gpu,
                             say, to_f64)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    flce.lib()


def _oracle_all(w, inp, mean_divisor=0.0):
    h, wt, b = to_f64(inp.hidden), to_f64(inp.weight), to_f64(inp.bias)
    t = inp.targets.numpy()
    prob = prob_of(w, mean_divisor)
    o = forward(h, wt, b, t, prob)
    g = backward(h, wt, b, t, prob, w.reduction, inp.grad_out.numpy())
    return o, g


# Small shapes that span several tiles and leave ragged tails in N (tokens),
# H (the K loop, in steps of 8) and V (vocabulary), one per feature combination.
SMALL = [
    synth.small_workload(300, 136, 1000, 11),
    synth.small_workload(257, 64, 4099, 12, softcap=30.0, bias=True, logit_scale=0.5,
                         reduction="sum"),
    synth.small_workload(130, 264, 777, 13, hidden_dtype="f32", bias=True, reduction="none"),
    synth.small_workload(333, 128, 2500, 14, logit_scale=0.0625, targets="zipf",
                         reduction="sum"),
    synth.small_workload(200, 256, 3001, 15, softcap=5.0, reduction="none", bias=True),
    synth.small_workload(4100, 128, 40000, 16, reduction="mean"),       # three vocab chunks, the last ragged
    synth.small_workload(96, 512, 1500, 17, hidden_dtype="f32", softcap=30.0),
    synth.small_workload(64, 128, 1, 18),                                # V = 1
    synth.small_workload(70, 64, 2, 19, bias=True),                      # V = 2
    # softcap above 120 / (2 log2 e): the forward keeps a running reference
    synth.small_workload(180, 96, 2100, 24, softcap=50.0, logit_scale=20.0, bias=True),
    synth.small_workload(300, 64, 1700, 25, softcap=60.0, logit_scale=8.0, reduction="none"),
    # fp32 lm_head (split into bf16 high + low parts on the device)
    synth.small_workload(290, 72, 2300, 27, weight_dtype="f32", softcap=30.0, bias=True),
    synth.small_workload(260, 136, 1900, 28, weight_dtype="f32", hidden_dtype="f32",
                         reduction="none"),
    synth.small_workload(4100, 64, 30000, 29, weight_dtype="f32", logit_scale=2.0),
    # hidden operands past one XCD's L2 (4 MB as bf16): windows of one token
    # tile, at least 64 forward splits, and (fp32) one dz tile per workgroup
    synth.small_workload(600, 4096, 9000, 41, softcap=30.0, bias=True),
    synth.small_workload(2000, 4096, 16500, 42, hidden_dtype="f32", reduction="none"),
    # H = 1024, where the forward takes 256-row tiles; running-max softcap path
    synth.small_workload(700, 1024, 5000, 43, softcap=50.0, logit_scale=2.0, bias=True,
                         reduction="none"),
    # H = 1152: 256-row forward and dz tiles with the 256x128 contraction; ragged N and V
    synth.small_workload(520, 1152, 4100, 44, softcap=30.0, bias=True, reduction="none"),
    # H = 2048 with both operands fp32: the 256x256 contraction on the rounded copies
    synth.small_workload(300, 2048, 2600, 45, hidden_dtype="f32", weight_dtype="f32",
                         targets="zipf", reduction="sum"),
    # H = 640 (the 256 x 128 contraction, five column tiles): ragged N and V, three
    # grad_hidden slots
    synth.small_workload(300, 640, 2100, 46, softcap=30.0, bias=True),
    synth.small_workload(2200, 640, 9000, 47, hidden_dtype="f32", reduction="none"),
    # H = 640 over two vocabulary chunks, the last ragged
    synth.small_workload(4100, 640, 20000, 48, softcap=30.0),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_parity(w):
    say(f"[parity] {w.name}")
    inp = synth.make_inputs(w)
    g = run_gpu(w, inp)
    o, og = _oracle_all(w, inp)
    check_tokens(g, o, label=w.name)
    check_reduced(g, o, label=w.name)
    check_grad(g["grad_hidden"].numpy(), og["grad_hidden"], "grad_hidden", w.name)
    check_grad(g["grad_weight"].numpy(), og["grad_weight"], "grad_weight", w.name)
    check_vocab_grad_parts(g["grad_weight"].numpy(), og["grad_weight"], inp.targets.numpy(),
                           w.vocab, "grad_weight", w.name)
    if inp.bias is not None:
        check_grad(g["grad_bias"].numpy(), og["grad_bias"], "grad_bias", w.name)
        check_vocab_grad_parts(g["grad_bias"].numpy(), og["grad_bias"], inp.targets.numpy(),
                               w.vocab, "grad_bias", w.name)


def test_lm_head_over_2gib():
    """An lm_head of more than 2 GiB (262272 x 4096 bf16) with few tokens: the
    backward's vocabulary chunk is capped so that the lm_head chunk, read along
    the vocabulary from one buffer descriptor, stays under 2^31 bytes (262016
    rows, then a 256-row chunk).  Every token against the oracle, grad_hidden
    whole, grad_weight rows on both sides of the chunk edge and a stride
    through the first chunk."""
    w = synth.small_workload(16, 4096, 262272, 1010)
    say("[parity] lm_head over 2 GiB: drawing inputs")
    inp = synth.make_inputs(w)
    say("[parity] lm_head over 2 GiB: running")
    g = run_gpu(w, inp)
    h, wt = to_f64(inp.hidden), to_f64(inp.weight)
    t = inp.targets.numpy()
    prob = prob_of(w)
    o = forward(h, wt, None, t, prob)
    vrows = np.concatenate([np.arange(262016 - 64, 262272), np.arange(0, 262016, 4099)])
    og = backward(h, wt, None, t, prob, w.reduction, inp.grad_out.numpy(), vocab_rows=vrows)
    check_tokens(g, o, label=w.name)
    check_reduced(g, o, label=w.name)
    check_grad(g["grad_hidden"].numpy(), og["grad_hidden"], "grad_hidden", w.name)
    check_grad(g["grad_weight"].numpy()[vrows], og["grad_weight_rows"], "grad_weight rows",
               w.name)


def test_num_items_divisor():
    w = synth.small_workload(150, 64, 900, 21)
    say("[parity] num_items divisor")
    inp = synth.make_inputs(w)
    g = run_gpu(w, inp, mean_divisor=400.0)
    o, og = _oracle_all(w, inp, mean_divisor=400.0)
    check_reduced(g, o, "num_items")
    check_grad(g["grad_weight"].numpy(), og["grad_weight"], "grad_weight", "num_items")


def test_all_ignored_small_is_exactly_zero():
    w = synth.small_workload(150, 128, 600, 22, targets="all_ignored", hidden_dtype="f32",
                             bias=True, softcap=10.0)
    say("[parity] all ignored (small)")
    inp = synth.make_inputs(w)
    g = run_gpu(w, inp)
    assert np.all(g["loss"].numpy() == 0) and np.all(g["entropy"].numpy() == 0)
    assert np.all(g["hit"].numpy() == 0)
    assert g["reduced_f32"].numpy().tolist() == [0.0, 0.0, 0.0]
    assert g["reduced_i64"].numpy().tolist() == [0, 0, 0]
    for k in ("grad_hidden", "grad_weight", "grad_bias"):
        assert torch.count_nonzero(g[k]).item() == 0, k


@pytest.mark.parametrize("softcap", [0.0, 30.0, 50.0])
def test_zero_lm_head_ties(softcap):
    """lm_head = 0 and no bias: every logit is 0, so the loss and the entropy
    are ln V exactly, the argmax is the lowest index (0) on every row across
    all vocabulary splits, grad_hidden is 0 and grad_weight[v] = sum_n g_n
    (1/V - [t_n = v]) h_n (oracle)."""
    w = synth.small_workload(260, 64, 5003, 26, softcap=softcap)
    inp = synth.make_inputs(w)
    inp.weight.zero_()
    say(f"[parity] zero lm_head, softcap {softcap}")
    g = run_gpu(w, inp)
    valid = inp.targets.numpy() != -100
    ln_v = float(np.log(5003.0))
    assert np.abs(g["loss"].numpy()[valid] - ln_v).max() <= 2e-3
    assert np.abs(g["entropy"].numpy()[valid] - ln_v).max() <= 2e-3
    assert np.all(g["argmax"].numpy() == 0)
    assert np.array_equal(g["hit"].numpy().astype(bool), valid & (inp.targets.numpy() == 0))
    assert torch.count_nonzero(g["grad_hidden"]).item() == 0
    o, og = _oracle_all(w, inp)
    check_grad(g["grad_weight"].numpy(), og["grad_weight"], "grad_weight", "zero lm_head")


def test_timing_hook_records_each_launch():
    """flce_set_timing_events brackets every launch of the chosen kernel: a
    backward over 30000 vocabulary rows with 4100 tokens runs two vocabulary
    chunks (the planning rule gives chunks of 16256 rows: 2^27 bytes of bf16 dz
    per chunk, rounded down to 128-row tiles), hence two contraction launches,
    each with a positive duration."""
    import ctypes
    w = synth.small_workload(4100, 128, 30000, 16)
    inp = synth.make_inputs(w)
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = (ctypes.c_void_p * 8)()
    for i in range(8):
        assert hip.hipEventCreate(ctypes.byref(evs, i * ctypes.sizeof(ctypes.c_void_p))) == 0
    say("[parity] timing hook")
    try:
        flce.flce_set_timing_events(flce.FLCE_KERNEL_CONTRACT, evs, 4)
        run_gpu(w, inp)
        recorded = flce.flce_set_timing_events(flce.FLCE_KERNEL_CONTRACT, None, 0)
        assert recorded == 2, recorded
        for i in range(recorded):
            ms = ctypes.c_float(0.0)
            assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(evs[2 * i]),
                                           ctypes.c_void_p(evs[2 * i + 1])) == 0
            assert ms.value > 0.0
    finally:
        flce.flce_set_timing_events(flce.FLCE_KERNEL_CONTRACT, None, 0)
        for i in range(8):
            hip.hipEventDestroy(ctypes.c_void_p(evs[i]))


def test_bad_targets_counted():
    w = synth.small_workload(200, 64, 500, 23)
    inp = synth.make_inputs(w)
    inp.targets[5] = 500
    inp.targets[7] = -3
    inp.targets[9] = 10 ** 9
    say("[parity] bad targets")
    g = run_gpu(w, inp)
    o, og = _oracle_all(w, inp)
    assert o["n_bad"] == 3
    check_tokens(g, o, label="bad")
    check_reduced(g, o, label="bad")
    check_grad(g["grad_hidden"].numpy(), og["grad_hidden"], "grad_hidden", "bad")


def test_empty_batch():
    say("[parity] N = 0")
    dev = "cuda:0"
    h = torch.zeros(0, 64, dtype=torch.bfloat16, device=dev)
    w = torch.randn(300, 64, device=dev).to(torch.bfloat16)
    t = torch.zeros(0, dtype=torch.int64, device=dev)
    b = torch.randn(300, device=dev)
    f = flce.flce_forward(h, w, t, b)
    gh, gw, gb = flce.flce_backward(h, w, t, f["lse"], f["reduced_i64"], flce.FLCE_GRAD_MEAN,
                                    torch.ones(1, device=dev), b)
    torch.cuda.synchronize()
    assert f["reduced_f32"].cpu().tolist() == [0.0, 0.0, 0.0]
    assert f["reduced_i64"].cpu().tolist() == [0, 0, 0]
    assert gh.numel() == 0 and torch.count_nonzero(gw).item() == 0
    assert torch.count_nonzero(gb).item() == 0


def test_deterministic_and_repeatable():
    """Same inputs twice -> bitwise-identical outputs; the backward can be
    called again (it keeps no state)."""
    w = synth.small_workload(500, 192, 5000, 24, softcap=30.0, bias=True)
    inp = synth.make_inputs(w)
    say("[parity] determinism")
    a = run_gpu(w, inp)
    b = run_gpu(w, inp)
    for k in ("loss", "lse", "entropy", "hit", "argmax", "reduced_f32", "reduced_i64",
              "grad_hidden", "grad_weight", "grad_bias"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("vocab", [32000, 150000, 200000])
def test_argmax_targets_give_exact_accuracy(vocab):
    """Targets set to the oracle's argmax of the final logits: every row whose
    top-2 margin is at least 1e-2 must be a hit (the cce pull request's
    accuracy check at V = 200000, 32000 and 150000)."""
    w = synth.Workload(f"argmax_{vocab}", 256, 256, vocab, softcap=30.0, seed=31,
                       ignore_every=0)
    inp = synth.make_inputs(w)
    z = final_logits(to_f64(inp.hidden), to_f64(inp.weight), None, prob_of(w))
    inp.targets = torch.from_numpy(np.argmax(z, axis=1).astype(np.int64))
    top2 = np.partition(z, vocab - 2, axis=1)[:, vocab - 2:]
    sure = (top2[:, 1] - top2[:, 0]) >= 1e-2
    say(f"[parity] argmax targets V={vocab}")
    g = run_gpu(w, inp, backward=False)
    assert np.all(g["hit"].numpy()[sure] == 1)
    assert int(g["reduced_i64"][1]) == int(g["hit"].numpy().astype(np.int64).sum())


def test_autograd_wrapper_matches_c_abi():
    w = synth.small_workload(260, 128, 3000, 25, softcap=30.0, bias=True)
    inp = synth.make_inputs(w)
    dev = "cuda:0"
    say("[parity] autograd wrapper")
    ref = run_gpu(w, inp)
    h = inp.hidden.to(dev).requires_grad_(True)
    wt = inp.weight.to(dev).requires_grad_(True)
    b = inp.bias.to(dev).requires_grad_(True)
    t = inp.targets.to(dev)
    loss, ent_sum, n_correct, n_valid = flce.linear_cross_entropy(h, wt, t, b, softcap=30.0)
    loss.backward()
    torch.cuda.synchronize()
    assert loss.item() == ref["reduced_f32"][1].item()
    assert ent_sum.item() == ref["reduced_f32"][2].item()
    assert n_correct.item() == ref["reduced_i64"][1].item()
    assert n_valid.item() == ref["reduced_i64"][0].item()
    assert torch.equal(b.grad.cpu(), ref["grad_bias"])
    assert torch.equal(h.grad.cpu(), ref["grad_hidden"].to(torch.bfloat16))
    assert torch.equal(wt.grad.cpu(), ref["grad_weight"].to(torch.bfloat16))
    # per-token reduction with weights: grad of sum(g * loss)
    h.grad = None
    lt, *_ = flce.linear_cross_entropy(h, wt, t, b, softcap=30.0, reduction="none")
    gw8 = torch.rand(lt.shape, device=dev)
    (lt * gw8).sum().backward()
    o = forward(to_f64(inp.hidden), to_f64(inp.weight), to_f64(inp.bias), inp.targets.numpy(),
                Problem(softcap=30.0))
    assert np.abs(lt.detach().cpu().numpy() - o["loss"]).max() <= 2e-3
    og = backward(to_f64(inp.hidden), to_f64(inp.weight), to_f64(inp.bias), inp.targets.numpy(),
                  Problem(softcap=30.0), "none", gw8.cpu().numpy().astype(np.float64))
    assert rel_fro(h.grad.float().cpu().numpy(), og["grad_hidden"]) <= 1e-2


# ------------------------------------------------------- full-size workloads

FULL = ["tiny", "huge_vocab", "bias_none", "zipf_sum", "fp32_hidden", "fp32_hidden_all_ignored",
        "huge_vocab_sft", "huge_vocab_fp32_lm_head"]


@pytest.mark.parametrize("name", FULL)
def test_fullsize_against_stored_oracle(name):
    """The full workloads, in the launch configuration the bench times,
    against oracle values written by tests/golden/make_fullsize_golden.py:
    every row's loss / entropy / lse / argmax / hit, the reductions,
    grad_hidden rows of every token tile, grad_weight / grad_bias rows on
    both sides of every chunk and split-K slot edge (the target-heavy rows and
    the softmax-only rows each within the tolerance on their own), and sign
    sketches of the whole gradients."""
    path = os.path.join(GOLDEN, f"fullsize_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    gold = np.load(path, allow_pickle=False)
    w = synth.WORKLOADS[name]
    say(f"[parity] full size {name}: drawing inputs")
    inp = synth.make_inputs(w)
    assert synth.input_checksum(inp) == str(gold["checksum"]), "input generator drifted"
    plan = flce.flce_plan_info(flce.make_problem(
        w.n_tokens, w.hidden, w.vocab, hidden_dtype=1 if w.hidden_dtype == "f32" else 0,
        weight_dtype=1 if w.weight_dtype == "f32" else 0))
    assert plan["chunk_rows"] == int(gold["chunk_rows"]), "golden sampled another chunk plan"
    assert plan["gh_rows_per_split"] == int(gold["gh_rows_per_split"])
    say(f"[parity] full size {name}: running")
    g = run_gpu(w, inp)
    check_fullsize(g, gold, w, inp, name)


@pytest.mark.parametrize("name", ["zipf_sum", "huge_vocab", "bias_none"])
def test_fullsize_argmax_targets_give_exact_accuracy(name):
    """The pages' accuracy experiment at full size: every target set to the
    oracle's argmax of the final logits (stored in the golden), forward only;
    each row whose top-2 margin is at least 1e-2 must be a hit, and the
    argmax must agree there.  At logit scale 1/16 (zipf_sum) the final logits
    have a spread of ~0.04, so most rows sit under the margin and this is
    where the near-tie handling is exercised; the sure rows still number in
    the thousands."""
    path = os.path.join(GOLDEN, f"fullsize_{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    gold = np.load(path, allow_pickle=False)
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w)
    assert synth.input_checksum(inp) == str(gold["checksum"]), "input generator drifted"
    inp.targets = torch.from_numpy(gold["argmax"].astype(np.int64))
    sure = gold["margin"] >= 1e-2
    say(f"[parity] full size {name}, argmax targets: {int(sure.sum())} sure rows")
    g = run_gpu(w, inp, backward=False)
    hit = g["hit"].numpy()
    assert np.all(hit[sure] == 1), int((hit[sure] == 0).sum())
    assert np.array_equal(g["argmax"].numpy()[sure], gold["argmax"][sure])
    assert int(g["reduced_i64"][1]) == int(hit.astype(np.int64).sum())
    assert int(g["reduced_i64"][0]) == w.n_tokens
    assert sure.sum() >= 1000


def test_argmax_targets_zipf_shape_class():
    """The same experiment on a fresh draw of the zipf_sum shape class (H =
    1024, V = 151936, logit scale 1/16, no softcap) with the oracle computed
    here: 1024 tokens."""
    w = synth.Workload("argmax_zipf_class", 1024, 1024, 151936, logit_scale=0.0625,
                       targets="zipf", ignore_every=0, reduction="sum", seed=4321)
    inp = synth.make_inputs(w)
    z = final_logits(to_f64(inp.hidden), to_f64(inp.weight), None, prob_of(w))
    am = np.argmax(z, axis=1)
    top2 = np.partition(z, w.vocab - 2, axis=1)[:, w.vocab - 2:]
    sure = (top2[:, 1] - top2[:, 0]) >= 1e-2
    inp.targets = torch.from_numpy(am.astype(np.int64))
    say(f"[parity] argmax targets, zipf shape class: {int(sure.sum())} sure rows")
    g = run_gpu(w, inp, backward=False)
    assert np.all(g["hit"].numpy()[sure] == 1)
    assert np.array_equal(g["argmax"].numpy()[sure], am[sure])
    assert sure.sum() >= 100


@pytest.mark.parametrize("hd,wd,compact", [("f32", "bf16", False), ("bf16", "f32", False),
                                           ("f32", "f32", True), ("bf16", "bf16", True)])
def test_backward_reuses_prepared_operands(hd, wd, compact):
    """flce_problem.reuse_prepared: the backward reads the bf16-rounded fp32
    operands (and with compaction the scan and gathered rows) that the
    forward left in the same workspace; the gradients are bitwise those of a
    backward that prepares them again."""
    w = synth.small_workload(700, 136, 3000, 51, hidden_dtype=hd, weight_dtype=wd, softcap=30.0,
                             bias=True, prompt_frac=0.5 if compact else 0.0, prompt_block=128,
                             reduction="none")
    inp = synth.make_inputs(w)
    dev = "cuda:0"
    h, wt, b, t = (inp.hidden.to(dev), inp.weight.to(dev), inp.bias.to(dev),
                   inp.targets.to(dev))
    go = inp.grad_out.to(dev)
    prob = flce._binding.problem_for(h, wt, w.logit_scale, w.softcap, compact_valid=compact)
    ws = torch.empty(flce.flce_workspace_bytes(prob), dtype=torch.uint8, device=dev)
    say(f"[parity] reuse_prepared {hd}/{wd} compact={compact}")
    f = flce.flce_forward(h, wt, t, b, w.logit_scale, w.softcap, workspace=ws,
                          compact_valid=compact)
    reused = flce.flce_backward(h, wt, t, f["lse"], f["reduced_i64"], flce.FLCE_GRAD_PER_TOKEN,
                                go, b, w.logit_scale, w.softcap, workspace=ws,
                                compact_valid=compact, reuse_prepared=True)
    fresh = flce.flce_backward(h, wt, t, f["lse"], f["reduced_i64"], flce.FLCE_GRAD_PER_TOKEN,
                               go, b, w.logit_scale, w.softcap, compact_valid=compact)
    torch.cuda.synchronize()
    for a, c in zip(reused, fresh):
        assert torch.equal(a, c)
    o, og = _oracle_all(w, inp)
    check_grad(reused[1].cpu().numpy(), og["grad_weight"], "grad_weight", w.name)
