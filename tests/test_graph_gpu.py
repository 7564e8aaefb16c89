"""The library under HIP graph capture: forward + backward captured once with
torch.cuda.graph (the library allocates nothing and issues no memset, so every
call is a plain kernel launch on the capturing stream) and replayed several
times, with eager work of the library on other inputs between the replays;
every replay must equal the eager results bit for bit."""
import pytest
import torch

import linear_cross_entropy_fp32_amd as flce
from linear_cross_entropy_fp32_amd import synth
from tests.gpu_cases import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    flce.lib()


def _step(h, wt, t, b, go, w, ws):
    f = flce.flce_forward(h, wt, t, b, w.logit_scale, w.softcap, workspace=ws)
    gh, gw, gb = flce.flce_backward(h, wt, t, f["lse"], f["reduced_i64"], flce.FLCE_GRAD_PER_TOKEN,
                                    go, b, w.logit_scale, w.softcap, workspace=ws)
    return [f["loss"], f["lse"], f["entropy"], f["hit"], f["argmax"], f["reduced_f32"],
            f["reduced_i64"], gh, gw, gb]


@pytest.mark.parametrize("w", [synth.small_workload(500, 192, 5000, 61, softcap=30.0, bias=True,
                                                    reduction="none"),
                               synth.small_workload(256, 256, 32000, 62, reduction="none"),
                               synth.small_workload(600, 1024, 3000, 63, bias=True,
                                                    reduction="none")],
                         ids=lambda w: w.name)
def test_graph_replays_match_eager(w):
    dev = "cuda:0"
    inp = synth.make_inputs(w)
    h, wt, t = inp.hidden.to(dev), inp.weight.to(dev), inp.targets.to(dev)
    b = None if inp.bias is None else inp.bias.to(dev)
    go = inp.grad_out.to(dev).reshape(-1)
    prob = flce._binding.problem_for(h, wt, w.logit_scale, w.softcap)
    ws = torch.empty(flce.flce_workspace_bytes(prob), dtype=torch.uint8, device=dev)
    say(f"[graph] {w.name}")
    eager = [x.clone() for x in _step(h, wt, t, b, go, w, ws) if x is not None]
    other = synth.make_inputs(synth.small_workload(w.n_tokens, w.hidden, w.vocab, 99,
                                                   softcap=w.softcap, bias=w.bias,
                                                   reduction="none"))
    oh, ot = other.hidden.to(dev), other.targets.to(dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(h, wt, t, b, go, w, ws)          # warm the allocator on the side stream
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        static = _step(h, wt, t, b, go, w, ws)
    for rep in range(3):
        # eager work of the library on other inputs and the same workspace
        _step(oh, wt, ot, b, go, w, ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [x for x in static if x is not None]
        for i, (a, e) in enumerate(zip(got, eager)):
            assert torch.equal(a, e), (rep, i)
