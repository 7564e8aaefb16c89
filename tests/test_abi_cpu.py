"""C-ABI checks that need no GPU: the library loads, exports every function
include/flce.h declares, its struct layout matches the binding, and argument
errors are reported before anything is launched."""
import ctypes
import os
import re
import subprocess

import pytest

import linear_cross_entropy_fp32_amd as flce
from linear_cross_entropy_fp32_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flce.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flce_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = flce.lib()
    declared = _declared_functions()
    assert set(declared) == set(_binding.EXPORTED), declared
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", _binding.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    for name in declared:
        assert re.search(rf"\bT {name}$", out, flags=re.M), f"{name} missing from dynamic symbols"


@pytest.mark.parametrize("struct,cname", [(_binding.FlceProblem, "flce_problem"),
                                          (_binding.FlceCeProblem, "flce_ce_problem")])
def test_struct_layout_matches_header(tmp_path, struct, cname):
    src = tmp_path / "layout.c"
    fields = [f for f, _ in struct._fields_]
    fmt = " ".join(["%zu"] * (len(fields) + 1))
    offs = "".join(f", offsetof({cname}, {f})" for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "flce.h"\n'
                   f'int main(void) {{ printf("{fmt}\\n", sizeof({cname}){offs}); '
                   'return 0; }\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    expect = [ctypes.sizeof(struct)] + [getattr(struct, f).offset for f, _ in struct._fields_]
    assert vals == expect


@pytest.mark.parametrize("kw,code", [
    (dict(n_tokens=-1, hidden=64, vocab=10), -2),
    (dict(n_tokens=4, hidden=12, vocab=10), -2),
    (dict(n_tokens=4, hidden=0, vocab=10), -2),
    (dict(n_tokens=4, hidden=64, vocab=0), -2),
    (dict(n_tokens=1 << 20, hidden=1 << 12, vocab=10), -2),
    (dict(n_tokens=1 << 23, hidden=8, vocab=10), -2),
    (dict(n_tokens=(1 << 23) - 1, hidden=8, vocab=10), 0),
    (dict(n_tokens=1 << 18, hidden=1 << 12, vocab=10), -2),
    (dict(n_tokens=(1 << 18) - 1, hidden=1 << 12, vocab=10), 0),
    (dict(n_tokens=4, hidden=1 << 12, vocab=1 << 19), -2),
    (dict(n_tokens=4, hidden=1 << 12, vocab=(1 << 19) - 1), 0),
    (dict(n_tokens=4, hidden=64, vocab=10, weight_dtype=2), -3),
    (dict(n_tokens=4, hidden=64, vocab=10, weight_dtype=1), 0),
    (dict(n_tokens=4, hidden=64, vocab=10, hidden_dtype=7), -3),
    (dict(n_tokens=4, hidden=64, vocab=10, logit_scale=float("nan")), -7),
    (dict(n_tokens=4, hidden=64, vocab=10, softcap=float("inf")), -7),
    (dict(n_tokens=0, hidden=64, vocab=1), 0),
    (dict(n_tokens=16384, hidden=4096, vocab=151936, hidden_dtype=1), 0),
])
def test_validate(kw, code):
    p = flce.make_problem(**kw)
    assert flce.flce_validate(p) == code
    if code:
        assert flce.flce_last_error()
        with pytest.raises(flce.FlceError):
            flce.flce_workspace_bytes(p)
    else:
        assert flce.flce_workspace_bytes(p) > 0


def test_compact_flag_is_zero_or_one():
    p = flce.make_problem(4, 64, 10)
    for value, rc in ((0, 0), (1, 0), (2, -7), (-1, -7)):
        p.compact_valid = value
        assert flce.flce_validate(p) == rc, value


def test_compact_workspace_adds_rows_only():
    """Row compaction adds per-row state (perm, counts, compact bf16 hidden
    rows) and the grad_hidden slot; nothing that grows with N x V."""
    for n, h, v, dt in ((2048, 640, 262144, flce.FLCE_BF16), (16384, 4096, 151936, flce.FLCE_F32),
                        (5, 8, 3, flce.FLCE_BF16)):
        base = flce.flce_workspace_bytes(flce.make_problem(n, h, v, hidden_dtype=dt))
        comp = flce.flce_workspace_bytes(flce.make_problem(n, h, v, hidden_dtype=dt,
                                                           compact_valid=True))
        extra = comp - base
        assert 0 <= extra <= n * 4 + 8 + 2 * (n // 256 + 1) * 4 + n * h * 2 + n * h * 4 + 4 * 256


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_entry_points_reject_before_launch():
    """Null pointers, misalignment, a short workspace and bad modes return an
    error code without touching the (fake, never dereferenced) pointers."""
    lib = flce.lib()
    p = flce.make_problem(8, 64, 100)
    A = 0x100000
    ok = [_fake(A)] * 2
    args = lambda **o: dict(dict(h=_fake(A), w=_fake(A), b=None, t=_fake(A), loss=_fake(A),
                                 lse=_fake(A), ent=_fake(A), hit=_fake(A), am=None,
                                 rf=_fake(A), ri=_fake(A), ws=_fake(A), wsb=1 << 20,
                                 s=None), **o)

    def fwd(**o):
        a = args(**o)
        return lib.flce_forward(ctypes.byref(p), a["h"], a["w"], a["b"], a["t"], a["loss"],
                                a["lse"], a["ent"], a["hit"], a["am"], a["rf"], a["ri"], a["ws"],
                                a["wsb"], a["s"])

    assert fwd(w=None) == -1
    assert fwd(t=None) == -1
    assert fwd(h=_fake(A + 8)) == -4
    assert fwd(t=_fake(A + 4)) == -4
    assert fwd(ws=_fake(A + 128)) == -4
    assert fwd(wsb=16) == -5
    assert "workspace" in flce.flce_last_error()

    def bwd(mode=0, **o):
        a = args(**o)
        return lib.flce_backward(ctypes.byref(p), a["h"], a["w"], a["b"], a["t"], a["lse"],
                                 a["ri"], mode, a["rf"], a["loss"], a["ent"], a.get("gb"),
                                 a["ws"], a["wsb"], a["s"])

    assert bwd(mode=3) == -7
    assert bwd(mode=-1) == -7
    assert bwd(w=None) == -1
    assert bwd(wsb=16) == -5
    # grad_bias without bias
    a = args()
    assert lib.flce_backward(ctypes.byref(p), a["h"], a["w"], None, a["t"], a["lse"], a["ri"],
                             0, a["rf"], a["loss"], a["ent"], _fake(A), a["ws"], a["wsb"],
                             None) == -7
    del ok


def test_binding_requires_targets_and_reduction():
    import torch
    h = torch.zeros(4, 64, dtype=torch.bfloat16)
    w = torch.zeros(10, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        flce.linear_cross_entropy(h, w, None)
    with pytest.raises(ValueError):
        flce.linear_cross_entropy(h, w, torch.zeros(4, dtype=torch.int64), reduction="avg")


def test_timing_hook_arguments():
    """The benchmark timing hook rejects bad requests and reports how many
    launches it recorded under the previous setting (none here: no launch
    happens without a GPU)."""
    lib = flce.lib()
    events = (ctypes.c_void_p * 2)()
    assert lib.flce_set_timing_events(7, events, 1) == -7
    assert lib.flce_set_timing_events(-1, events, 1) == -7
    assert lib.flce_set_timing_events(flce.FLCE_KERNEL_CONTRACT, events, -1) == -7
    assert lib.flce_set_timing_events(flce.FLCE_KERNEL_CONTRACT, None, 1) == -7
    assert lib.flce_set_timing_events(flce.FLCE_KERNEL_CONTRACT, events, 1) == 0
    assert lib.flce_set_timing_events(flce.FLCE_KERNEL_CONTRACT, None, 0) == 0



def test_noalloc_forward_rejects_oversized_problem():
    """flce_forward_noalloc holds 16 MiB of scratch per GPU: a forward that
    needs more (fp32 hidden states at 16384 x 4096, whose bf16 split alone is
    268 MB) is refused with FLCE_ERR_WORKSPACE before any HIP call."""
    lib = flce.lib()
    p = flce.make_problem(16384, 4096, 151936, hidden_dtype=flce.FLCE_F32)
    assert flce.flce_plan_info(p)["fwd_workspace_bytes"] > 16 << 20
    A = _fake(0x100000)
    rc = lib.flce_forward_noalloc(ctypes.byref(p), A, A, None, A, A, A, A, A, None, A, A, None)
    assert rc == -5
    assert "16777216" in flce.flce_last_error()
    assert flce.flce_plan_info(flce.make_problem(2048, 640, 262144))["fwd_workspace_bytes"] \
        <= 16 << 20


def test_lds_dma_hazard_scan():
    """The build's scan of the kernel assembly flags an LDS-DMA load whose
    descriptor an SGPR reload (v_readlane) wrote fewer than five wait states
    before, and passes one with enough wait states or a scalar-written
    descriptor."""
    from linear_cross_entropy_fp32_amd.build import lds_dma_hazards
    bad = ("_Zk:\n\tv_readlane_b32 s11, v251, 16\n\ts_nop 0\n"
           "\tbuffer_load_dword v1, s[8:11], 0 offen lds\n")
    ok1 = ("_Zk:\n\tv_readlane_b32 s11, v251, 16\n\ts_nop 4\n"
           "\tbuffer_load_dword v1, s[8:11], 0 offen lds\n")
    ok2 = ("_Zk:\n\ts_mov_b32 s11, 0x20000\n\ts_nop 0\n"
           "\tbuffer_load_dwordx4 v1, s[8:11], 0 offen lds\n")
    m0 = "_Zk:\n\ts_mov_b32 m0, s4\n\tbuffer_load_dwordx4 v1, s[8:11], 0 offen lds\n"
    assert len(lds_dma_hazards(bad)) == 1
    assert lds_dma_hazards(ok1) == [] and lds_dma_hazards(ok2) == []
    assert len(lds_dma_hazards(m0)) == 1


def test_ce_entry_points_reject_before_launch():
    """The cross-entropy entry points check the problem and the pointers
    before anything is launched (fake pointers, never dereferenced)."""
    lib = flce.lib()
    A = _fake(0x100000)
    P = lambda **kw: ctypes.byref(_binding.FlceCeProblem(**dict(
        dict(n_rows=8, vocab=100, logits_dtype=0, reserved=0, ignore_index=-100,
             mean_divisor=0.0, reserved2=0), **kw)))
    fwd = lambda p, logits=A, inplace=1: lib.flce_ce_forward(p, logits, A, A, A, A, A, inplace,
                                                              None)
    assert fwd(P(vocab=0)) == -2
    assert fwd(P(n_rows=-1)) == -2
    assert fwd(P(vocab=1 << 30, logits_dtype=1)) == -2      # a row of 4 GiB
    assert fwd(P(logits_dtype=5)) == -3
    assert fwd(P(reserved=1)) == -7
    assert fwd(P(mean_divisor=float("nan"))) == -7
    assert fwd(P(), inplace=2) == -7
    assert fwd(P(), logits=None) == -1
    assert fwd(P(), logits=_fake(0x100008)) == -4
    bwd = lambda p, mode=0: lib.flce_ce_backward(p, A, A, A, mode, A, None)
    assert bwd(P(), mode=3) == -7
    assert bwd(P(vocab=0)) == -2
    assert lib.flce_ce_backward(P(), A, A, A, 0, None, None) == -1
