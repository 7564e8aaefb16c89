"""flce_forward_noalloc (the forward with the library's per-GPU scratch in
place of a workspace) against flce_forward through the C ABI: two calls in a
row, the second on a smaller problem, each bitwise equal to the workspace
entry point on the same inputs (the same kernels run, with the same plan)."""
import numpy as np
import pytest
import torch

import linear_cross_entropy_fp32_amd as flce
from linear_cross_entropy_fp32_amd import synth

pytestmark = pytest.mark.gpu

KEYS = ("loss", "lse", "entropy", "hit", "argmax", "reduced_f32", "reduced_i64")


def _on_gpu(inp, dev="cuda:0"):
    return (inp.hidden.to(dev), inp.weight.to(dev),
            None if inp.bias is None else inp.bias.to(dev), inp.targets.to(dev))


def test_noalloc_forward_matches_workspace_forward():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    cases = [synth.WORKLOADS["huge_vocab"],
             synth.small_workload(300, 136, 3001, 7, softcap=30.0, bias=True)]
    for w in cases:
        print(f"[no-alloc] {w.name}", flush=True)
        inp = synth.make_inputs(w)
        h, wt, b, t = _on_gpu(inp)
        ref = flce.flce_forward(h, wt, t, b, w.logit_scale, w.softcap)
        got = flce.flce_forward_noalloc(h, wt, t, b, w.logit_scale, w.softcap)
        torch.cuda.synchronize()
        for k in KEYS:
            assert torch.equal(ref[k].cpu(), got[k].cpu()), (w.name, k)
        assert int(got["reduced_i64"][0]) == int((inp.targets >= 0).sum())
        assert np.isfinite(got["loss"].cpu().numpy()).all()
