"""ctypes binding of libflce.so: argument marshalling only.

Every step of the loss runs in the library's HIP kernels; PyTorch supplies the
device memory (its caching allocator) and the current stream.  Nothing here
computes any part of the loss, and there is no fallback: if the library is not
built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libflce.so")

FLCE_BF16, FLCE_F32 = 0, 1
FLCE_GRAD_MEAN, FLCE_GRAD_SUM, FLCE_GRAD_PER_TOKEN = 0, 1, 2
ERROR_NAMES = {-1: "FLCE_ERR_NULL", -2: "FLCE_ERR_SHAPE", -3: "FLCE_ERR_DTYPE",
               -4: "FLCE_ERR_ALIGN", -5: "FLCE_ERR_WORKSPACE", -6: "FLCE_ERR_HIP",
               -7: "FLCE_ERR_ARG"}
EXPORTED = ("flce_validate", "flce_workspace_bytes", "flce_forward", "flce_backward",
            "flce_last_error", "flce_abi_version", "flce_set_timing_events", "flce_plan_info",
            "flce_forward_noalloc", "flce_ce_forward", "flce_ce_backward")
PLAN_FIELDS = ("chunk_rows", "n_chunks", "fwd_splits", "fwd_tiles_per_split",
               "dz_tiles_per_wg", "gh_splits", "gh_rows_per_split", "window_token_tiles",
               "token_tile_fastest", "fwd_workspace_bytes", "bwd_workspace_bytes",
               "workspace_bytes", "dz_chunk_bytes", "fwd_tile_rows", "dz_tile_rows",
               "contract_tile_cols")
FLCE_KERNEL_FWD_STATS, FLCE_KERNEL_BWD_DZ, FLCE_KERNEL_CONTRACT = 0, 1, 2


class FlceProblem(ctypes.Structure):
    """Mirror of ``flce_problem`` in include/flce.h."""
    _fields_ = [("n_tokens", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("vocab", ctypes.c_int64), ("hidden_dtype", ctypes.c_int32),
                ("weight_dtype", ctypes.c_int32), ("logit_scale", ctypes.c_float),
                ("softcap", ctypes.c_float), ("ignore_index", ctypes.c_int64),
                ("mean_divisor", ctypes.c_float), ("compact_valid", ctypes.c_int32),
                ("reuse_prepared", ctypes.c_int32)]


class FlceCeProblem(ctypes.Structure):
    """Mirror of ``flce_ce_problem`` in include/flce.h."""
    _fields_ = [("n_rows", ctypes.c_int64), ("vocab", ctypes.c_int64),
                ("logits_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("ignore_index", ctypes.c_int64), ("mean_divisor", ctypes.c_float),
                ("reserved2", ctypes.c_int32)]


class FlceError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load libflce.so (built in-tree by ``python -m linear_cross_entropy_fp32_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run "
                               "`python -m linear_cross_entropy_fp32_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64p, f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        pp = ctypes.POINTER(FlceProblem)
        L.flce_validate.argtypes = [pp]
        L.flce_validate.restype = ctypes.c_int
        L.flce_workspace_bytes.argtypes = [pp, ctypes.POINTER(ctypes.c_size_t)]
        L.flce_workspace_bytes.restype = ctypes.c_int
        L.flce_forward.argtypes = [pp, vp, vp, f32p, i64p, f32p, f32p, f32p, vp, vp, f32p, i64p,
                                   vp, ctypes.c_size_t, vp]
        L.flce_forward.restype = ctypes.c_int
        L.flce_forward_noalloc.argtypes = [pp, vp, vp, f32p, i64p, f32p, f32p, f32p, vp, vp,
                                           f32p, i64p, vp]
        L.flce_forward_noalloc.restype = ctypes.c_int
        L.flce_backward.argtypes = [pp, vp, vp, f32p, i64p, f32p, i64p, ctypes.c_int, f32p,
                                    f32p, f32p, f32p, vp, ctypes.c_size_t, vp]
        L.flce_backward.restype = ctypes.c_int
        L.flce_last_error.argtypes = []
        L.flce_last_error.restype = ctypes.c_char_p
        L.flce_abi_version.argtypes = []
        L.flce_abi_version.restype = ctypes.c_int
        L.flce_set_timing_events.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        L.flce_set_timing_events.restype = ctypes.c_int
        cp = ctypes.POINTER(FlceCeProblem)
        L.flce_ce_forward.argtypes = [cp, vp, i64p, f32p, f32p, f32p, i64p, ctypes.c_int, vp]
        L.flce_ce_forward.restype = ctypes.c_int
        L.flce_ce_backward.argtypes = [cp, vp, i64p, i64p, ctypes.c_int, f32p, vp]
        L.flce_ce_backward.restype = ctypes.c_int
        L.flce_plan_info.argtypes = [pp, ctypes.POINTER(ctypes.c_int64), ctypes.c_int]
        L.flce_plan_info.restype = ctypes.c_int
        if L.flce_abi_version() != 2:
            raise RuntimeError("libflce.so ABI version mismatch: rebuild it")
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != 0:
        raise FlceError(rc, lib().flce_last_error().decode())


def make_problem(n_tokens: int, hidden: int, vocab: int, hidden_dtype: int = FLCE_BF16,
                 weight_dtype: int = FLCE_BF16, logit_scale: float = 1.0, softcap: float = 0.0,
                 ignore_index: int = -100, mean_divisor: float = 0.0,
                 compact_valid: bool = False, reuse_prepared: bool = False) -> FlceProblem:
    return FlceProblem(n_tokens, hidden, vocab, hidden_dtype, weight_dtype, logit_scale,
                       softcap if softcap else 0.0, ignore_index, mean_divisor,
                       1 if compact_valid else 0, 1 if reuse_prepared else 0)


def flce_validate(prob: FlceProblem) -> int:
    return lib().flce_validate(ctypes.byref(prob))


def flce_workspace_bytes(prob: FlceProblem) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().flce_workspace_bytes(ctypes.byref(prob), ctypes.byref(out)))
    return out.value


def flce_plan_info(prob: FlceProblem) -> dict:
    """``flce_plan_info``: how the library tiles the problem (host only)."""
    out = (ctypes.c_int64 * len(PLAN_FIELDS))()
    rc = lib().flce_plan_info(ctypes.byref(prob), out, len(PLAN_FIELDS))
    if rc < 0:
        raise FlceError(rc, flce_last_error())
    return dict(zip(PLAN_FIELDS, (int(x) for x in out[:rc])))


def flce_last_error() -> str:
    return lib().flce_last_error().decode()


def flce_set_timing_events(kernel: int, events, n_pairs: int) -> int:
    """Instrumentation: bracket `kernel`'s launches on this thread with the
    given HIP events (a ctypes array of 2*n_pairs hipEvent_t); 0 clears."""
    rc = lib().flce_set_timing_events(int(kernel), events, int(n_pairs))
    if rc < 0:
        raise FlceError(rc, flce_last_error())
    return rc


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FLCE_BF16
    if t.dtype == torch.float32:
        return FLCE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def problem_for(hidden: torch.Tensor, weight: torch.Tensor, logit_scale: float = 1.0,
                softcap: Optional[float] = None, ignore_index: int = -100,
                mean_divisor: float = 0.0, compact_valid: bool = False,
                reuse_prepared: bool = False) -> FlceProblem:
    if hidden.dim() != 2 or weight.dim() != 2 or hidden.shape[1] != weight.shape[1]:
        raise ValueError(f"hidden {tuple(hidden.shape)} and weight {tuple(weight.shape)} "
                         "must be [N, H] and [V, H]")
    return make_problem(hidden.shape[0], hidden.shape[1], weight.shape[0], _dtype_code(hidden),
                        _dtype_code(weight), float(logit_scale), float(softcap or 0.0),
                        int(ignore_index), float(mean_divisor), compact_valid, reuse_prepared)


def _require(t: torch.Tensor, name: str, device: torch.device) -> None:
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def flce_forward(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
                 bias: Optional[torch.Tensor] = None, logit_scale: float = 1.0,
                 softcap: Optional[float] = None, ignore_index: int = -100,
                 mean_divisor: float = 0.0, want_argmax: bool = True,
                 workspace: Optional[torch.Tensor] = None,
                 compact_valid: bool = False) -> dict:
    """Run ``flce_forward`` on the current stream.  Returns device tensors:
    loss, lse, entropy [N] f32, hit [N] u8, argmax [N] i32 (or None),
    reduced_f32 [3] (loss_sum, loss_mean, entropy_sum) and reduced_i64 [3]
    (n_valid, n_correct, n_bad_target).  compact_valid: project only the rows
    that carry a loss (the others get lse 0 and argmax -1)."""
    if targets is None:
        raise ValueError("targets are required")
    dev = weight.device
    for t, nm in ((hidden, "hidden"), (weight, "weight"), (targets, "targets")):
        _require(t, nm, dev)
    if targets.dtype != torch.int64 or targets.shape != (hidden.shape[0],):
        raise ValueError("targets must be int64 [N]")
    if bias is not None:
        _require(bias, "bias", dev)
        if bias.dtype != torch.float32 or bias.shape != (weight.shape[0],):
            raise ValueError("bias must be float32 [V]")
    prob = problem_for(hidden, weight, logit_scale, softcap, ignore_index, mean_divisor,
                       compact_valid)
    n = hidden.shape[0]
    ws_bytes = flce_workspace_bytes(prob)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(loss=torch.empty(n, **f32), lse=torch.empty(n, **f32),
               entropy=torch.empty(n, **f32),
               hit=torch.empty(n, dtype=torch.uint8, device=dev),
               argmax=torch.empty(n, dtype=torch.int32, device=dev) if want_argmax else None,
               reduced_f32=torch.empty(3, **f32),
               reduced_i64=torch.empty(3, dtype=torch.int64, device=dev))
    _check(lib().flce_forward(
        ctypes.byref(prob), _ptr(hidden), _ptr(weight), _ptr(bias), _ptr(targets),
        _ptr(out["loss"]), _ptr(out["lse"]), _ptr(out["entropy"]), _ptr(out["hit"]),
        _ptr(out["argmax"]), _ptr(out["reduced_f32"]), _ptr(out["reduced_i64"]),
        _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


def flce_forward_noalloc(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
                         bias: Optional[torch.Tensor] = None, logit_scale: float = 1.0,
                         softcap: Optional[float] = None, ignore_index: int = -100,
                         mean_divisor: float = 0.0, out: Optional[dict] = None) -> dict:
    """Run ``flce_forward_noalloc`` (no workspace: the library's per-GPU
    scratch) on the current stream, into ``out`` (the same keys as
    ``flce_forward`` returns) or into new tensors."""
    if targets is None:
        raise ValueError("targets are required")
    dev = weight.device
    for t, nm in ((hidden, "hidden"), (weight, "weight"), (targets, "targets")):
        _require(t, nm, dev)
    prob = problem_for(hidden, weight, logit_scale, softcap, ignore_index, mean_divisor)
    n = hidden.shape[0]
    if out is None:
        f32 = dict(dtype=torch.float32, device=dev)
        out = dict(loss=torch.empty(n, **f32), lse=torch.empty(n, **f32),
                   entropy=torch.empty(n, **f32),
                   hit=torch.empty(n, dtype=torch.uint8, device=dev),
                   argmax=torch.empty(n, dtype=torch.int32, device=dev),
                   reduced_f32=torch.empty(3, **f32),
                   reduced_i64=torch.empty(3, dtype=torch.int64, device=dev))
    _check(lib().flce_forward_noalloc(
        ctypes.byref(prob), _ptr(hidden), _ptr(weight), _ptr(bias), _ptr(targets),
        _ptr(out["loss"]), _ptr(out["lse"]), _ptr(out["entropy"]), _ptr(out["hit"]),
        _ptr(out["argmax"]), _ptr(out["reduced_f32"]), _ptr(out["reduced_i64"]), _stream(dev)))
    return out


def flce_backward(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
                  lse: torch.Tensor, reduced_i64: torch.Tensor, grad_mode: int,
                  grad_out: torch.Tensor, bias: Optional[torch.Tensor] = None,
                  logit_scale: float = 1.0, softcap: Optional[float] = None,
                  ignore_index: int = -100, mean_divisor: float = 0.0,
                  need_bias_grad: Optional[bool] = None,
                  workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None,
                  compact_valid: bool = False, reuse_prepared: bool = False):
    """Run ``flce_backward`` on the current stream.  Returns fp32
    (grad_hidden [N, H], grad_weight [V, H], grad_bias [V] or None).
    reuse_prepared: reuse the operands the forward prepared in ``workspace``
    (which must then be the forward's, unchanged)."""
    dev = weight.device
    for t, nm in ((hidden, "hidden"), (weight, "weight"), (targets, "targets"), (lse, "lse"),
                  (reduced_i64, "reduced_i64"), (grad_out, "grad_out")):
        _require(t, nm, dev)
    if grad_out.dtype != torch.float32:
        raise ValueError("grad_out must be float32")
    n = hidden.shape[0]
    if grad_mode == FLCE_GRAD_PER_TOKEN and grad_out.numel() != n:
        raise ValueError("per-token grad_out must have N elements")
    if grad_mode != FLCE_GRAD_PER_TOKEN and grad_out.numel() != 1:
        raise ValueError("mean/sum grad_out must have one element")
    if reuse_prepared and workspace is None:
        raise ValueError("reuse_prepared needs the forward's workspace")
    prob = problem_for(hidden, weight, logit_scale, softcap, ignore_index, mean_divisor,
                       compact_valid, reuse_prepared)
    ws_bytes = flce_workspace_bytes(prob)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    if need_bias_grad is None:
        need_bias_grad = bias is not None
    if out is None:
        gh = torch.empty(hidden.shape, dtype=torch.float32, device=dev)
        gw = torch.empty(weight.shape, dtype=torch.float32, device=dev)
        gb = torch.empty(weight.shape[0], dtype=torch.float32, device=dev) if need_bias_grad else None
    else:
        gh, gw, gb = out["grad_hidden"], out["grad_weight"], out.get("grad_bias")
    _check(lib().flce_backward(
        ctypes.byref(prob), _ptr(hidden), _ptr(weight), _ptr(bias), _ptr(targets), _ptr(lse),
        _ptr(reduced_i64), int(grad_mode), _ptr(grad_out), _ptr(gh), _ptr(gw), _ptr(gb),
        _ptr(workspace), workspace.numel(), _stream(dev)))
    return gh, gw, gb


_MODES = {"mean": FLCE_GRAD_MEAN, "sum": FLCE_GRAD_SUM, "none": FLCE_GRAD_PER_TOKEN}


class _LinearCrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, hidden, weight, bias, targets, logit_scale, softcap, reduction,
                num_items, ignore_index, compact_valid):
        mean_div = float(num_items) if num_items else 0.0
        out = flce_forward(hidden, weight, targets, bias, logit_scale, softcap, ignore_index,
                           mean_div, want_argmax=False, compact_valid=compact_valid)
        ctx.save_for_backward(hidden, weight, bias, targets, out["lse"], out["reduced_i64"])
        ctx.cfg = (logit_scale, softcap, reduction, mean_div, ignore_index, compact_valid)
        if reduction == "none":
            loss = out["loss"]
        elif reduction == "sum":
            loss = out["reduced_f32"][0]
        else:
            loss = out["reduced_f32"][1]
        ctx.mark_non_differentiable(out["reduced_f32"], out["reduced_i64"])
        return loss, out["reduced_f32"][2], out["reduced_i64"][1], out["reduced_i64"][0]

    @staticmethod
    def backward(ctx, g_loss, _g_ent, _g_nc, _g_nv):
        hidden, weight, bias, targets, lse, red_i64 = ctx.saved_tensors
        logit_scale, softcap, reduction, mean_div, ignore_index, compact_valid = ctx.cfg
        g = g_loss.to(torch.float32).contiguous().reshape(-1)
        gh, gw, gb = flce_backward(hidden, weight, targets, lse, red_i64, _MODES[reduction], g,
                                   bias, logit_scale, softcap, ignore_index, mean_div,
                                   need_bias_grad=bias is not None and ctx.needs_input_grad[2],
                                   compact_valid=compact_valid)
        gh = gh.to(hidden.dtype) if ctx.needs_input_grad[0] else None
        gw = gw.to(weight.dtype) if ctx.needs_input_grad[1] else None
        return gh, gw, gb, None, None, None, None, None, None, None


def linear_cross_entropy(hidden: torch.Tensor, weight: torch.Tensor, targets: torch.Tensor,
                         bias: Optional[torch.Tensor] = None, logit_scale: float = 1.0,
                         softcap: Optional[float] = None, reduction: str = "mean",
                         num_items: Optional[float] = None, ignore_index: int = -100,
                         compact_valid: bool = False):
    """Fused linear cross-entropy with autograd.

    Returns (loss, entropy_sum, n_correct, n_valid): loss is the mean / sum
    scalar or the per-token vector (reduction "none"), entropy_sum is fp32 and
    the two counts are int64 device scalars (no host synchronisation).
    compact_valid: only the rows that carry a loss are projected (device-side
    compaction), so the work scales with the number of valid rows.
    """
    if targets is None:
        raise ValueError("targets must be provided")
    if reduction not in _MODES:
        raise ValueError(f"reduction must be one of {sorted(_MODES)}")
    return _LinearCrossEntropy.apply(hidden, weight, bias, targets, logit_scale, softcap,
                                     reduction, num_items, ignore_index, bool(compact_valid))


# ------------------------------------- cross-entropy on materialised logits

def ce_problem_for(logits: torch.Tensor, ignore_index: int = -100,
                   mean_divisor: float = 0.0) -> FlceCeProblem:
    if logits.dim() != 2:
        raise ValueError(f"logits must be [N, V], got {tuple(logits.shape)}")
    return FlceCeProblem(logits.shape[0], logits.shape[1], _dtype_code(logits), 0,
                         int(ignore_index), float(mean_divisor), 0)


def flce_ce_forward(logits: torch.Tensor, targets: torch.Tensor, ignore_index: int = -100,
                    mean_divisor: float = 0.0, grad_in_place: bool = True) -> dict:
    """Run ``flce_ce_forward`` on the current stream.  With grad_in_place the
    logits tensor is overwritten with softmax - onehot per row.  Returns
    device tensors loss, lse [N] f32, reduced_f32 [2] (loss_sum, loss_mean),
    reduced_i64 [2] (n_valid, n_bad)."""
    if targets is None:
        raise ValueError("targets are required")
    dev = logits.device
    for t, nm in ((logits, "logits"), (targets, "targets")):
        _require(t, nm, dev)
    if targets.dtype != torch.int64 or targets.shape != (logits.shape[0],):
        raise ValueError("targets must be int64 [N]")
    prob = ce_problem_for(logits, ignore_index, mean_divisor)
    n = logits.shape[0]
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(loss=torch.empty(n, **f32), lse=torch.empty(n, **f32),
               reduced_f32=torch.empty(2, **f32),
               reduced_i64=torch.empty(2, dtype=torch.int64, device=dev))
    _check(lib().flce_ce_forward(ctypes.byref(prob), _ptr(logits), _ptr(targets),
                                 _ptr(out["loss"]), _ptr(out["lse"]), _ptr(out["reduced_f32"]),
                                 _ptr(out["reduced_i64"]), 1 if grad_in_place else 0,
                                 _stream(dev)))
    return out


def flce_ce_backward(grad_logits: torch.Tensor, targets: torch.Tensor,
                     reduced_i64: torch.Tensor, grad_mode: int, grad_out: torch.Tensor,
                     ignore_index: int = -100, mean_divisor: float = 0.0) -> torch.Tensor:
    """Run ``flce_ce_backward``: scales grad_logits (the forward's in-place
    output) row by row in place and returns it."""
    dev = grad_logits.device
    for t, nm in ((grad_logits, "grad_logits"), (targets, "targets"),
                  (reduced_i64, "reduced_i64"), (grad_out, "grad_out")):
        _require(t, nm, dev)
    if grad_out.dtype != torch.float32:
        raise ValueError("grad_out must be float32")
    prob = ce_problem_for(grad_logits, ignore_index, mean_divisor)
    _check(lib().flce_ce_backward(ctypes.byref(prob), _ptr(grad_logits), _ptr(targets),
                                  _ptr(reduced_i64), int(grad_mode), _ptr(grad_out),
                                  _stream(dev)))
    return grad_logits


class _CrossEntropyInPlace(torch.autograd.Function):
    """Cross-entropy on materialised logits whose forward writes the gradient
    in place of the logits and whose backward scales it in place: the graph
    can be backpropagated once."""

    @staticmethod
    def forward(ctx, logits, targets, reduction, num_items, ignore_index):
        mean_div = float(num_items) if num_items else 0.0
        out = flce_ce_forward(logits, targets, ignore_index, mean_div, grad_in_place=True)
        ctx.save_for_backward(logits, targets, out["reduced_i64"])
        ctx.cfg = (reduction, mean_div, ignore_index)
        ctx.mark_non_differentiable(out["reduced_i64"])
        if reduction == "none":
            loss = out["loss"]
        elif reduction == "sum":
            loss = out["reduced_f32"][0]
        else:
            loss = out["reduced_f32"][1]
        return loss, out["reduced_i64"][0]

    @staticmethod
    def backward(ctx, g_loss, _g_nv):
        logits, targets, red_i64 = ctx.saved_tensors
        reduction, mean_div, ignore_index = ctx.cfg
        g = g_loss.to(torch.float32).contiguous().reshape(-1)
        flce_ce_backward(logits, targets, red_i64, _MODES[reduction], g, ignore_index, mean_div)
        return logits, None, None, None, None


def cross_entropy(logits: torch.Tensor, targets: torch.Tensor, reduction: str = "mean",
                  num_items: Optional[float] = None, ignore_index: int = -100):
    """Cross-entropy on [N, V] logits (bf16 or fp32) with fp32 per-token
    losses; the gradient is written in place of the logits (which must be a
    leaf tensor the caller does not need afterwards).  Returns
    (loss, n_valid)."""
    if targets is None:
        raise ValueError("targets must be provided")
    if reduction not in _MODES:
        raise ValueError(f"reduction must be one of {sorted(_MODES)}")
    return _CrossEntropyInPlace.apply(logits, targets, reduction, num_items, ignore_index)
