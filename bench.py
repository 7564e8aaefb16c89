"""Throughput of the fused linear cross-entropy forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload huge_vocab]

One step = flce_forward + flce_backward (the whole hot path) over one batch of
seeded synthetic inputs already resident in HBM.  The default workload is the
262144-vocabulary / hidden-640 / 2048-token batch with softcap 30 (the
configuration the metric is quoted on).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused linear-CE fwd+bwd tokens/s on 1 MI355X; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="after the timed steps, this many steps each preceded (outside their "
                         "event bracket) by a 512 MiB write that evicts L2 and MALL; 0 = none")
    ap.add_argument("--workload", default="huge_vocab")
    ap.add_argument("--compact", action="store_true",
                    help="valid-row compaction (flce_problem.compact_valid): only the rows that "
                         "carry a loss are projected; tokens/s still counts every position, and "
                         "the flop figures count the valid rows")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (HBM counter scale)")
    ap.add_argument("--traffic-record", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR",
                                                          "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="only write profiles/traffic_<kernel>_<workload>.json from rocprofv3 "
                         "--pmc FETCH_SIZE / WRITE_SIZE output directories of a bench run and of "
                         "a --copy-calibration-mib run (no GPU needed)")
    ap.add_argument("--traffic-kernel", default="contract_kernel")
    ap.add_argument("--library-gemm", action="store_true",
                    help="only time the vendor GEMM library (torch.mm, hipBLASLt) on the plain "
                         "products of the workload's step, as a reference for what a bf16 GEMM "
                         "of these shapes reaches on this GPU")
    return ap.parse_args()


def library_gemm(args) -> int:
    """Plain bf16 products of one step of the workload through torch.mm
    (hipBLASLt): the logits (bf16 out), one backward chunk's grad_hidden and
    grad_weight products, and a square 8192^3 pair for scale.  Each is timed
    with events over repeated calls after a warmup; nothing here is part of
    the loss path."""
    import torch

    from linear_cross_entropy_fp32_amd import synth
    w = synth.WORKLOADS[args.workload]
    n, hd, v = w.n_tokens, w.hidden, w.vocab
    vc = max(128, ((1 << 27) // (2 * n)) // 128 * 128)     # the backward's chunk width
    vc = min(vc, v)
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(0)

    def rnd(*shape):
        return torch.randn(*shape, generator=g).to(dev).bfloat16()

    wt, h, dz = rnd(v, hd), rnd(n, hd), rnd(n, vc)
    wc = wt[:vc].contiguous()
    a8, b8 = rnd(8192, 8192), rnd(8192, 8192)
    cases = [
        ("logits lm_head.hidden^T", lambda: torch.mm(wt, h.t()), 2 * v * n * hd),
        ("logits hidden.lm_head^T", lambda: torch.mm(h, wt.t()), 2 * v * n * hd),
        ("grad_hidden chunk dz.lm_head", lambda: torch.mm(dz, wc), 2 * n * vc * hd),
        ("grad_weight chunk dz^T.hidden", lambda: torch.mm(dz.t(), h), 2 * n * vc * hd),
        ("square 8192 NN", lambda: torch.mm(a8, b8), 2 * 8192 ** 3),
        ("square 8192 NT", lambda: torch.mm(a8, b8.t()), 2 * 8192 ** 3),
    ]
    out = {"workload": w.name, "n_tokens": n, "hidden": hd, "vocab": v, "chunk_rows": vc,
           "peak_tflops": PEAK_BF16_TFLOPS, "cases": []}
    for name, fn, flops in cases:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        tf = flops / (ms * 1e-3) / 1e12
        out["cases"].append({"product": name, "us": round(ms * 1e3, 1), "tflops": round(tf, 1),
                             "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 1)})
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline(w, inp, budget_s: float) -> dict:
    """The CPU oracle (float64 numpy, as written) on a bounded sample of the
    workload: consecutive 128-token blocks, each run as a batch of its own
    (forward + backward incl. grad_weight), until the time budget is spent."""
    import numpy as np
    from oracle import Problem, backward, forward
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()
                     if d.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    wt = inp.weight.float().numpy().astype(np.float64)
    bias = None if inp.bias is None else inp.bias.numpy().astype(np.float64)
    prob = Problem(logit_scale=w.logit_scale, softcap=w.softcap)
    rows, blk = 0, 128
    t0 = time.perf_counter()
    while rows < w.n_tokens and time.perf_counter() - t0 < budget_s:
        sl = slice(rows, min(w.n_tokens, rows + blk))
        h = inp.hidden[sl].float().numpy().astype(np.float64)
        t = inp.targets[sl].numpy()
        go = inp.grad_out[sl].numpy() if w.reduction == "none" else inp.grad_out.numpy()
        forward(h, wt, bias, t, prob)
        backward(h, wt, bias, t, prob, w.reduction, go)
        rows = sl.stop
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {rows} of {w.n_tokens} tokens in 128-token batches, fwd+bwd "
                      f"(float64 numpy), {dt:.1f} s"}


# Timing-only events: no system-scope fence (cache writeback and invalidate)
# when an event is recorded, so that recording one between two kernels does
# not open a gap between them (HIP's hipEventDisableSystemFence).
_EVENT_TIMING_ONLY = 0x20000000


def _hip_runtime():
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.c_void_p]
    hip.hipEventCreateWithFlags.argtypes = [ctypes.c_void_p, ctypes.c_uint]
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


def _hip_ok(rc: int) -> None:
    if rc != 0:
        raise RuntimeError(f"HIP runtime call failed with code {rc}")


def _chunks_per_backward(prob) -> int:
    """Upper bound on contraction launches per backward: one per vocab chunk,
    and no chunk is narrower than 2^27 bytes of bf16 dz per token row allows,
    nor than the 2^31-byte limit on one lm_head chunk allows (128-row units)."""
    n = max(1, prob.n_tokens)
    rows = ((1 << 27) // (2 * n)) // 128 * 128
    rows = min(rows, ((1 << 31) - 1) // (2 * max(1, prob.hidden)) // 128 * 128)
    rows = max(128, rows)
    return max(1, -(-prob.vocab // rows))


def _source_digest() -> str:
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "linear_cross_entropy_fp32_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + fh.read())
    return h.hexdigest()[:16]


def _committed_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (rocprofv3 FETCH_SIZE and WRITE_SIZE, copy-calibrated), or None when the
    kernels have changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except OSError:
        return None
    if rec.get("source_digest") != _source_digest():
        return None
    return rec.get("bytes_per_launch")


def _counter_rows(directory: str, counter: str):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            rows += [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
    if not rows:
        raise SystemExit(f"bench.py: no {counter} rows under {directory}")
    return rows


def _per_dispatch_kib(directory: str, counter: str, kernel: str) -> float:
    vals = [float(r["Counter_Value"]) for r in _counter_rows(directory, counter)
            if kernel in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"bench.py: no {kernel} dispatch in {directory}")
    return sum(vals) / len(vals)


def _copy_scale(directory: str, counter: str, copy_bytes: int) -> float:
    """Bytes moved per counter KiB: the copy kernel moves copy_bytes each way."""
    vals = [float(r["Counter_Value"]) for r in _counter_rows(directory, counter)
            if "copyBuffer" in r["Kernel_Name"] or "elementwise" in r["Kernel_Name"].lower()
            or "copy" in r["Kernel_Name"].lower()]
    if not vals:
        raise SystemExit(f"bench.py: no copy kernel in {directory}")
    scale = copy_bytes / (max(vals) * 1024.0)
    if not 0.25 <= scale <= 8.0:
        raise SystemExit(f"bench.py: implausible {counter} scale {scale:.3g} from {directory} "
                         f"(is it a --copy-calibration-mib {copy_bytes >> 20} run?)")
    return scale


def write_traffic_record(args) -> int:
    fetch_dir, write_dir, copy_fetch_dir, copy_write_dir = args.traffic_record
    copy_bytes = (args.copy_calibration_mib or 1024) << 20
    fetch_kib = _per_dispatch_kib(fetch_dir, "FETCH_SIZE", args.traffic_kernel)
    write_kib = _per_dispatch_kib(write_dir, "WRITE_SIZE", args.traffic_kernel)
    fscale = _copy_scale(copy_fetch_dir, "FETCH_SIZE", copy_bytes)
    wscale = _copy_scale(copy_write_dir, "WRITE_SIZE", copy_bytes)
    rec = {
        "workload": args.workload, "kernel": args.traffic_kernel,
        "source_digest": _source_digest(),
        "fetch_kib_per_launch": fetch_kib, "write_kib_per_launch": write_kib,
        "fetch_scale": round(fscale, 3), "write_scale": round(wscale, 3),
        "bytes_per_launch": fetch_kib * 1024 * fscale + write_kib * 1024 * wscale,
        "method": "rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE, on bench.py --steps 2 "
                  "--warmup 1 --no-cpu-baseline; KiB per dispatch averaged over launches, each "
                  "scaled by the same counter's reading for a plain device copy of "
                  f"{copy_bytes >> 20} MiB (bench.py --copy-calibration-mib)",
    }
    path = os.path.join(ROOT, "profiles", f"traffic_{args.traffic_kernel}_{args.workload}.json")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec))
    return 0


def main() -> int:
    args = parse()
    if args.traffic_record:
        return write_traffic_record(args)
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (got --gpus {args.gpus}); "
              "the path's sharding is described in DESIGN.md", file=sys.stderr)
        return 2
    import torch

    if args.library_gemm:
        return library_gemm(args)
    if args.copy_calibration_mib:
        # a plain copy of known size: rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE on
        # this run gives the counters' scale for algorithmic byte counts
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": max(1, args.steps)}), flush=True)
        return 0

    import linear_cross_entropy_fp32_amd as flce
    from linear_cross_entropy_fp32_amd import _binding, synth

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    inp = synth.make_inputs(w)
    h = inp.hidden.to(dev)
    wt = inp.weight.to(dev)
    b = None if inp.bias is None else inp.bias.to(dev)
    t = inp.targets.to(dev)
    go = inp.grad_out.to(dev).reshape(-1)
    n, hd, v = w.n_tokens, w.hidden, w.vocab
    prob = _binding.problem_for(h, wt, w.logit_scale, w.softcap, compact_valid=args.compact)
    ws_bytes = flce.flce_workspace_bytes(prob)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    loss, lse, ent = (torch.empty(n, **f32) for _ in range(3))
    hit = torch.empty(n, dtype=torch.uint8, device=dev)
    red_f = torch.empty(3, **f32)
    red_i = torch.empty(3, dtype=torch.int64, device=dev)
    gh = torch.empty(n, hd, **f32)
    gw = torch.empty(v, hd, **f32)
    gb = torch.empty(v, **f32) if b is not None else None
    mode = {"mean": 0, "sum": 1, "none": 2}[w.reduction]
    L = flce.lib()
    P = _binding._ptr
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def fwd():
        rc = L.flce_forward(ctypes.byref(prob), P(h), P(wt), P(b), P(t), P(loss), P(lse), P(ent),
                            P(hit), None, P(red_f), P(red_i), P(ws), ws_bytes, sp)
        if rc:
            raise flce.FlceError(rc, flce.flce_last_error())

    def bwd():
        rc = L.flce_backward(ctypes.byref(prob), P(h), P(wt), P(b), P(t), P(lse), P(red_i), mode,
                             P(go), P(gh), P(gw), P(gb), P(ws), ws_bytes, sp)
        if rc:
            raise flce.FlceError(rc, flce.flce_last_error())

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()

    # HIP events for the dominant kernel's launches, recorded by the library on
    # the launch stream (flce_set_timing_events) over the whole timed region,
    # and for the forward / backward split of every step; all timing-only
    hip = _hip_runtime()
    n_chunks = _chunks_per_backward(prob)
    n_pairs = args.steps * n_chunks + 1      # one spare pair: a full pool means overflow
    n_step_ev = 3 * args.steps
    evs = (ctypes.c_void_p * (2 * n_pairs + n_step_ev))()
    for i in range(2 * n_pairs + n_step_ev):
        _hip_ok(hip.hipEventCreateWithFlags(ctypes.byref(evs, i * ctypes.sizeof(ctypes.c_void_p)),
                                            _EVENT_TIMING_ONLY))
    step_ev = [evs[2 * n_pairs + i] for i in range(n_step_ev)]

    def elapsed(a, b):
        ms_i = ctypes.c_float(0.0)
        _hip_ok(hip.hipEventElapsedTime(ctypes.byref(ms_i), ctypes.c_void_p(a), ctypes.c_void_p(b)))
        return ms_i.value

    def mark(e):
        _hip_ok(hip.hipEventRecord(ctypes.c_void_p(e), sp))

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    flce.flce_set_timing_events(_binding.FLCE_KERNEL_CONTRACT, evs, n_pairs)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        mark(step_ev[3 * i])
        fwd()
        mark(step_ev[3 * i + 1])
        bwd()
        mark(step_ev[3 * i + 2])
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    recorded = flce.flce_set_timing_events(_binding.FLCE_KERNEL_CONTRACT, None, 0)
    if recorded >= n_pairs:
        raise RuntimeError("more contraction launches than timing events: the per-step "
                           "kernel time would be incomplete")
    kern_ms = [elapsed(evs[2 * i], evs[2 * i + 1]) for i in range(recorded)]
    step_ms = [elapsed(step_ev[3 * i], step_ev[3 * i + 2]) for i in range(args.steps)]
    fwd_ms = sum(elapsed(step_ev[3 * i], step_ev[3 * i + 1]) for i in range(args.steps)) / args.steps
    bwd_ms = sum(elapsed(step_ev[3 * i + 1], step_ev[3 * i + 2])
                 for i in range(args.steps)) / args.steps
    for i in range(2 * n_pairs + n_step_ev):
        hip.hipEventDestroy(ctypes.c_void_p(evs[i]))
    total_ms = start.elapsed_time(stop)
    ms = total_ms / args.steps

    # cold steps: every step starts with L2 and MALL (256 MB) holding none of
    # its operands, after a 512 MiB write outside the step's event bracket
    cold_ms = []
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cev = (ctypes.c_void_p * (2 * args.cold_steps))()
        for i in range(2 * args.cold_steps):
            _hip_ok(hip.hipEventCreateWithFlags(
                ctypes.byref(cev, i * ctypes.sizeof(ctypes.c_void_p)), _EVENT_TIMING_ONLY))
        for i in range(args.cold_steps):
            flush.fill_(i & 255)
            mark(cev[2 * i])
            fwd()
            bwd()
            mark(cev[2 * i + 1])
        torch.cuda.synchronize()
        cold_ms = [elapsed(cev[2 * i], cev[2 * i + 1]) for i in range(args.cold_steps)]
        for i in range(2 * args.cold_steps):
            hip.hipEventDestroy(ctypes.c_void_p(cev[i]))
        del flush
    # with compaction the algorithmic work is that of the rows carrying a loss
    n_work = int(red_i[0].item()) if args.compact else n
    flops = 8.0 * n_work * hd * v
    tflops = flops / (ms * 1e-3) / 1e12
    # dominant kernel: the backward contraction (grad_hidden and grad_weight of
    # one vocabulary chunk per launch); over a step its launches do 4*N*H*V
    # flops of algorithmic work
    launches = max(1, len(kern_ms))
    kern_avg = sum(kern_ms) / launches if kern_ms else float("nan")
    per_step_ms = kern_avg * launches / args.steps
    kern_tflops = 4.0 * n_work * hd * v / (per_step_ms * 1e-3) / 1e12
    traffic = _committed_traffic(w.name, "contract_kernel")
    out = {
        "metric": METRIC, "value": n / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "n_tokens": n, "hidden": hd, "vocab": v,
                   "hidden_dtype": w.hidden_dtype, "bias": w.bias, "logit_scale": w.logit_scale,
                   "softcap": w.softcap, "reduction": w.reduction,
                   "compact_valid": bool(args.compact), "n_valid": int(red_i[0].item())},
        "tflops": tflops, "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "fwd_ms": fwd_ms, "bwd_ms": bwd_ms, "wall_s": wall,
        "step_ms_p20_p50_p80": [float(np.percentile(step_ms, q)) for q in (20, 50, 80)],
        "cold_step_ms_p20_p50_p80": ([float(np.percentile(cold_ms, q)) for q in (20, 50, 80)]
                                     if cold_ms else None),
        "roofline": {"bound": "mfma", "kernel": "contract_kernel", "achieved": kern_tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": kern_tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "launch_ms": kern_avg, "launches_per_step": launches / args.steps},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
