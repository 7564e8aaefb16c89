"""Seeded synthetic inputs for the fused linear cross-entropy.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the loss arithmetic, so both the HIP path (tests, bench) and
the CPU oracle can take their inputs from it without sharing any of the
method's code.

Workloads.  The pages measure on released models and an unnamed dataset; none
of that is available here, so seeded synthetic tensors with the same shapes
stand in for them.  The shapes follow the pages' own synthetic cross-entropy
benchmark (Liger-Kernel pull request 1574, "Details": 8192 tokens, every 17th
target ignored, vocabularies 32000 / 128256 / 151936) and the model sizes of
the TRL "cce" pull request's "Benchmark" table (gemma-3-270m: 262k vocabulary,
hidden 640, sequence 2048; Qwen3-0.6B: 152k vocabulary; Qwen3-8B-sized hidden
4096 with float32 hidden states, listed under "What it supports").

Drawing rules (fixed so that every machine with this torch build regenerates
bit-identical tensors):
  * one CPU ``torch.Generator`` per workload, seeded with ``seed``;
  * draw order: hidden, weight, bias, targets, grad_out;
  * hidden ~ N(0, 1), weight ~ N(0, 0.02), bias ~ N(0, 0.1), drawn in float32
    and rounded to bfloat16 (round-to-nearest-even) where the dtype is bf16
    (hidden and weight each have their own dtype);
  * targets uniform in [0, V) or bounded Zipf(a): P(k) proportional to
    (k+1)^-a for k in [0, V), sampled by inverse CDF from float64 uniforms;
  * every 17th position (n % 17 == 0) is set to the ignore index -100;
  * with prompt masking (the SFT-style workload), the first
    round(prompt_frac * prompt_block) positions of every block of prompt_block
    positions are set to -100 as well, as a completion-only loss masks the
    prompt;
  * per-token grad_out ~ U[0, 2) for reduction "none".
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

IGNORE_INDEX = -100


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_tokens: int
    hidden: int
    vocab: int
    hidden_dtype: str = "bf16"        # "bf16" or "f32"
    weight_dtype: str = "bf16"        # "bf16" or "f32" (an fp32 lm_head, not rounded)
    bias: bool = False
    logit_scale: float = 1.0
    softcap: float = 0.0              # <= 0: no softcapping
    targets: str = "uniform"          # "uniform", "zipf", "all_ignored", "argmax" (set later)
    zipf_a: float = 1.1
    ignore_every: int = 17            # 0: nothing ignored
    prompt_frac: float = 0.0          # share of each prompt_block masked at its start
    prompt_block: int = 512
    reduction: str = "mean"           # "mean", "sum", "none"
    seed: int = 0

    @property
    def flops(self) -> int:
        """Credited floating-point work of one forward+backward: 8*N*H*V."""
        return 8 * self.n_tokens * self.hidden * self.vocab


# The five workloads.  Seeds are 1000 + the workload's position (1-based).
WORKLOADS = {
    "tiny": Workload("tiny", 256, 256, 32000, seed=1001),
    "huge_vocab": Workload("huge_vocab", 2048, 640, 262144, softcap=30.0, seed=1002),
    "bias_none": Workload("bias_none", 8192, 2048, 128256, bias=True, reduction="none",
                          seed=1003),
    "zipf_sum": Workload("zipf_sum", 16384, 1024, 151936, logit_scale=0.0625,
                         targets="zipf", reduction="sum", seed=1004),
    "fp32_hidden": Workload("fp32_hidden", 16384, 4096, 151936, hidden_dtype="f32",
                            seed=1005),
    "fp32_hidden_all_ignored": Workload("fp32_hidden_all_ignored", 16384, 4096, 151936,
                                        hidden_dtype="f32", targets="all_ignored",
                                        seed=1006),
    # huge_vocab with 70% of every 512-token block masked as prompt (30% of
    # the positions carry a loss): the case that valid-row compaction is for
    "huge_vocab_sft": Workload("huge_vocab_sft", 2048, 640, 262144, softcap=30.0,
                               ignore_every=0, prompt_frac=0.7, seed=1007),
    # huge_vocab with an fp32 lm_head (an fp32 master weight, as under FSDP2
    # mixed precision)
    "huge_vocab_fp32_lm_head": Workload("huge_vocab_fp32_lm_head", 2048, 640, 262144,
                                        softcap=30.0, weight_dtype="f32", seed=1008),
}


@dataclasses.dataclass
class Inputs:
    hidden: torch.Tensor              # [N, H] bf16 or f32 (CPU)
    weight: torch.Tensor              # [V, H] bf16 (CPU)
    bias: Optional[torch.Tensor]      # [V] f32 or None
    targets: torch.Tensor             # [N] int64
    grad_out: torch.Tensor            # [] f32 for mean/sum, [N] f32 for none


def _zipf_targets(gen: torch.Generator, n: int, vocab: int, a: float) -> torch.Tensor:
    ranks = np.arange(1, vocab + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-a))
    u = torch.rand(n, generator=gen, dtype=torch.float64).numpy() * cdf[-1]
    idx = np.searchsorted(cdf, u, side="right")
    return torch.from_numpy(np.minimum(idx, vocab - 1).astype(np.int64))


def make_inputs(w: Workload, n_tokens: Optional[int] = None) -> Inputs:
    """Draw the workload's tensors on the CPU.  ``n_tokens`` overrides N."""
    n = w.n_tokens if n_tokens is None else n_tokens
    gen = torch.Generator().manual_seed(w.seed)
    hidden = torch.randn(n, w.hidden, generator=gen, dtype=torch.float32)
    if w.hidden_dtype == "bf16":
        hidden = hidden.to(torch.bfloat16)
    elif w.hidden_dtype != "f32":
        raise ValueError(f"unknown hidden dtype {w.hidden_dtype}")
    weight = torch.randn(w.vocab, w.hidden, generator=gen, dtype=torch.float32) * 0.02
    if w.weight_dtype == "bf16":
        weight = weight.to(torch.bfloat16)
    elif w.weight_dtype != "f32":
        raise ValueError(f"unknown weight dtype {w.weight_dtype}")
    bias = None
    if w.bias:
        bias = torch.randn(w.vocab, generator=gen, dtype=torch.float32) * 0.1
    if w.targets in ("uniform", "all_ignored", "argmax"):
        targets = torch.randint(0, w.vocab, (n,), generator=gen, dtype=torch.int64)
    elif w.targets == "zipf":
        targets = _zipf_targets(gen, n, w.vocab, w.zipf_a)
    else:
        raise ValueError(f"unknown target distribution {w.targets}")
    if w.ignore_every > 0:
        targets[:: w.ignore_every] = IGNORE_INDEX
    if w.prompt_frac > 0:
        masked = int(round(w.prompt_frac * w.prompt_block))
        pos = torch.arange(n) % w.prompt_block
        targets[pos < masked] = IGNORE_INDEX
    if w.targets == "all_ignored":
        targets[:] = IGNORE_INDEX
    if w.reduction == "none":
        grad_out = torch.rand(n, generator=gen, dtype=torch.float32) * 2.0
    else:
        grad_out = torch.ones((), dtype=torch.float32)
    return Inputs(hidden, weight, bias, targets, grad_out)


def small_workload(n: int, h: int, v: int, seed: int, **kw) -> Workload:
    """A parity-sized workload with arbitrary (ragged) shapes."""
    return Workload(f"small_{n}x{h}x{v}_{seed}", n, h, v, seed=seed, **kw)


def input_checksum(inp: Inputs) -> str:
    """A short digest of the tensors, used to detect generator drift."""
    import hashlib
    hsh = hashlib.sha256()
    for t in (inp.hidden, inp.weight, inp.bias, inp.targets, inp.grad_out):
        if t is None:
            hsh.update(b"none")
            continue
        t = t.contiguous()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        hsh.update(t.numpy().tobytes())
    return hsh.hexdigest()[:32]


# ------------------------------------------- materialised-logit workloads
# The Liger-Kernel pull request's benchmark ("Details"): 8192 rows, random
# logits, targets uniform with every 17th ignored, vocabularies 32000, 128256
# and 151936; here logits ~ N(0, 1) in bf16 (the page's "random logits"), and
# per-row weights ~ U[0, 2) for its "none+weighted" usage.
CE_WORKLOADS = {f"ce_{v}": (8192, v) for v in (32000, 128256, 151936)}


def ce_inputs(n: int, v: int, seed: int, dtype: str = "bf16", device: str = "cpu",
              ignore_every: int = 17):
    """(logits [n, v], targets [n] int64, weights [n] f32) drawn from one
    generator on `device` (logits) and one CPU generator (targets, weights),
    both seeded with `seed`."""
    g = torch.Generator(device=device).manual_seed(seed)
    logits = torch.randn(n, v, generator=g, dtype=torch.float32, device=device)
    if dtype == "bf16":
        logits = logits.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(dtype)
    gc = torch.Generator().manual_seed(seed + 1)
    targets = torch.randint(0, v, (n,), generator=gc, dtype=torch.int64)
    if ignore_every > 0:
        targets[::ignore_every] = IGNORE_INDEX
    weights = torch.rand(n, generator=gc, dtype=torch.float32) * 2.0
    return logits, targets, weights
