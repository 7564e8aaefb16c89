"""Throughput of the fused linear cross-entropy forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload huge_vocab]

One step = flce_forward + flce_backward (the whole hot path) over one batch of
seeded synthetic inputs already resident in HBM.  The default workload is the
262144-vocabulary / hidden-640 / 2048-token batch with softcap 30 (the
configuration the metric is quoted on).  Prints one JSON line.

Timing protocol (after the Liger-Kernel page's "Details", a do_bench-style
loop): one discarded call, warmup of at least W steps and 25 ms, then K timed
steps, each preceded by a 512 MiB write that evicts L2 and the 256 MB MALL
(outside the step's own event bracket); `value` and `ms_per_step` are the
median of those flushed steps.  The same K steps back to back (caches warm)
are reported beside them.  `per_config` repeats the measurement, with fewer
steps, on the other workloads of the metric.
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
    ap.add_argument("--per-config-steps", type=int, default=5,
                    help="timed steps per workload of the per_config record; 0 = no per_config")
    ap.add_argument("--workload", default="huge_vocab")
    ap.add_argument("--compact", action="store_true",
                    help="valid-row compaction (flce_problem.compact_valid): only the rows that "
                         "carry a loss are projected; tokens/s still counts every position, and "
                         "the flop figures count the valid rows")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--per-config-cpu-seconds", type=float, default=3.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (HBM counter scale)")
    ap.add_argument("--traffic-record", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR",
                                                          "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="only write profiles/traffic_<kernel>_<workload>.json from rocprofv3 "
                         "--pmc FETCH_SIZE / WRITE_SIZE output directories of a bench run and of "
                         "a --copy-calibration-mib run (no GPU needed)")
    ap.add_argument("--traffic-kernel", default="contract_kernel")
    ap.add_argument("--ce-only", action="store_true",
                    help="only measure the standalone cross-entropy on materialised logits "
                         "(the materialised_ce record) and print it")
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

    from linear_cross_entropy_fp32_amd import _binding, synth
    w = synth.WORKLOADS[args.workload]
    n, hd, v = w.n_tokens, w.hidden, w.vocab
    prob = _binding.make_problem(n, hd, v, hidden_dtype=1 if w.hidden_dtype == "f32" else 0,
                                 weight_dtype=1 if w.weight_dtype == "f32" else 0)
    vc = min(int(_binding.flce_plan_info(prob)["chunk_rows"]), v)   # the backward's chunk width
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
            "cpu_model": _cpu_model(), "nproc": len(os.sched_getaffinity(0)),
            "sample": f"first {rows} of {w.n_tokens} tokens in 128-token batches, fwd+bwd "
                      f"(float64 numpy), {dt:.1f} s"}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
    """Contraction launches per backward: one per vocab chunk of the plan."""
    from linear_cross_entropy_fp32_amd import _binding
    return max(1, int(_binding.flce_plan_info(prob)["n_chunks"]))


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


PER_CONFIG = ("tiny", "huge_vocab", "bias_none", "zipf_sum", "fp32_hidden",
              "fp32_hidden_all_ignored")
# workloads also timed as a graph-replayed step: tiny is launch-bound, and
# huge_vocab shows what a graph saves on the headline step
GRAPH_CONFIGS = ("tiny", "huge_vocab")
WARMUP_MS = 25.0
FLUSH_BYTES = 512 << 20


class Runner:
    """One workload's inputs, outputs and workspace resident on the GPU, and
    the two calls of a step through the C ABI on the current stream."""

    def __init__(self, w, compact: bool):
        import torch

        import linear_cross_entropy_fp32_amd as flce
        from linear_cross_entropy_fp32_amd import _binding, synth
        self.w = w
        dev = torch.device("cuda:0")
        self.inp = inp = synth.make_inputs(w)
        self.h = inp.hidden.to(dev)
        self.wt = inp.weight.to(dev)
        self.b = None if inp.bias is None else inp.bias.to(dev)
        self.t = inp.targets.to(dev)
        self.go = inp.grad_out.to(dev).reshape(-1)
        n, hd, v = w.n_tokens, w.hidden, w.vocab
        # the backward reuses what the forward prepared in the same workspace
        self.prob = _binding.problem_for(self.h, self.wt, w.logit_scale, w.softcap,
                                         compact_valid=compact, reuse_prepared=True)
        self.ws_bytes = flce.flce_workspace_bytes(self.prob)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.loss, self.lse, self.ent = (torch.empty(n, **f32) for _ in range(3))
        self.hit = torch.empty(n, dtype=torch.uint8, device=dev)
        self.red_f = torch.empty(3, **f32)
        self.red_i = torch.empty(3, dtype=torch.int64, device=dev)
        self.gh = torch.empty(n, hd, **f32)
        self.gw = torch.empty(v, hd, **f32)
        self.gb = torch.empty(v, **f32) if self.b is not None else None
        self.mode = {"mean": 0, "sum": 1, "none": 2}[w.reduction]
        self.L = flce.lib()
        self.P = _binding._ptr
        self.flce = flce
        self.stream = torch.cuda.current_stream(dev)
        self.sp = ctypes.c_void_p(self.stream.cuda_stream)

    def fwd(self):
        P = self.P
        rc = self.L.flce_forward(ctypes.byref(self.prob), P(self.h), P(self.wt), P(self.b),
                                 P(self.t), P(self.loss), P(self.lse), P(self.ent), P(self.hit),
                                 None, P(self.red_f), P(self.red_i), P(self.ws), self.ws_bytes,
                                 self.sp)
        if rc:
            raise self.flce.FlceError(rc, self.flce.flce_last_error())

    def bwd(self):
        P = self.P
        rc = self.L.flce_backward(ctypes.byref(self.prob), P(self.h), P(self.wt), P(self.b),
                                  P(self.t), P(self.lse), P(self.red_i), self.mode, P(self.go),
                                  P(self.gh), P(self.gw), P(self.gb), P(self.ws), self.ws_bytes,
                                  self.sp)
        if rc:
            raise self.flce.FlceError(rc, self.flce.flce_last_error())


class Events:
    """Timing-only HIP events (no system-scope fence when recorded)."""

    def __init__(self, hip, count: int):
        self.hip = hip
        self.arr = (ctypes.c_void_p * max(1, count))()
        for i in range(count):
            _hip_ok(hip.hipEventCreateWithFlags(
                ctypes.byref(self.arr, i * ctypes.sizeof(ctypes.c_void_p)), _EVENT_TIMING_ONLY))
        self.count = count

    def __getitem__(self, i):
        return self.arr[i]

    def ms(self, a, b) -> float:
        out = ctypes.c_float(0.0)
        _hip_ok(self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(self.arr[a]),
                                             ctypes.c_void_p(self.arr[b])))
        return out.value

    def close(self):
        for i in range(self.count):
            self.hip.hipEventDestroy(ctypes.c_void_p(self.arr[i]))


def measure(r: Runner, steps: int, warmup: int, hip, kernel_events: bool) -> dict:
    """Warm up, then time `steps` flushed steps and `steps` back-to-back ones.
    Returns per-step times, the forward / backward split of the flushed
    steps and, with kernel_events, the contraction launches' durations in
    the flushed steps (recorded by the library on the launch stream)."""
    import torch

    from linear_cross_entropy_fp32_amd import _binding
    sp = r.sp

    def mark(e):
        _hip_ok(hip.hipEventRecord(ctypes.c_void_p(e), sp))

    # one discarded call, then at least `warmup` steps and WARMUP_MS
    r.fwd()
    r.bwd()
    torch.cuda.synchronize()
    t0, done = time.perf_counter(), 0
    while done < warmup or (time.perf_counter() - t0) * 1e3 < WARMUP_MS:
        r.fwd()
        r.bwd()
        done += 1
        if done % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warm_ms_total = (time.perf_counter() - t0) * 1e3

    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda:0")
    ev = Events(hip, 3 * steps + 2 * steps)
    n_pairs = steps * _chunks_per_backward(r.prob) + 1 if kernel_events else 0
    kev = Events(hip, 2 * n_pairs) if kernel_events else None
    if kernel_events:
        r.flce.flce_set_timing_events(_binding.FLCE_KERNEL_CONTRACT, kev.arr, n_pairs)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(steps):
        flush.fill_(i & 255)
        mark(ev[3 * i])
        r.fwd()
        mark(ev[3 * i + 1])
        r.bwd()
        mark(ev[3 * i + 2])
    torch.cuda.synchronize()
    wall_cold = time.perf_counter() - t_wall
    kern_ms = []
    if kernel_events:
        recorded = r.flce.flce_set_timing_events(_binding.FLCE_KERNEL_CONTRACT, None, 0)
        if recorded >= n_pairs:
            raise RuntimeError("more contraction launches than timing events")
        kern_ms = [kev.ms(2 * i, 2 * i + 1) for i in range(recorded)]
        kev.close()
    # the same steps back to back, caches warm
    base = 3 * steps
    for i in range(steps):
        mark(ev[base + 2 * i])
        r.fwd()
        r.bwd()
        mark(ev[base + 2 * i + 1])
    torch.cuda.synchronize()
    cold = [ev.ms(3 * i, 3 * i + 2) for i in range(steps)]
    fwd = [ev.ms(3 * i, 3 * i + 1) for i in range(steps)]
    bwd = [ev.ms(3 * i + 1, 3 * i + 2) for i in range(steps)]
    warm = [ev.ms(base + 2 * i, base + 2 * i + 1) for i in range(steps)]
    ev.close()
    del flush
    return {"cold": cold, "fwd": fwd, "bwd": bwd, "warm": warm, "kern_ms": kern_ms,
            "warmup_steps": done + 1, "warmup_ms": warm_ms_total, "wall_s": wall_cold}


def pct(xs, q):
    return float(np.percentile(xs, q))


def graph_steps(r: Runner, hip, steps: int) -> list:
    """The same step captured once in a HIP graph (the library allocates
    nothing and issues no memset, so both calls capture as plain launches)
    and replayed: per-step times with the flushed protocol, in ms.  For a
    launch-bound workload the difference to the eager step is the launch
    cost."""
    import torch
    cs = torch.cuda.Stream()
    old = r.sp
    r.sp = ctypes.c_void_p(cs.cuda_stream)
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        r.fwd()
        r.bwd()
    cs.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        r.fwd()
        r.bwd()
    r.sp = old
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda:0")
    ev = Events(hip, 2 * steps)
    for i in range(steps + 2):            # two untimed replays
        flush.fill_(i & 255)
        k = i - 2
        if k >= 0:
            _hip_ok(hip.hipEventRecord(ctypes.c_void_p(ev[2 * k]), sp))
        g.replay()
        if k >= 0:
            _hip_ok(hip.hipEventRecord(ctypes.c_void_p(ev[2 * k + 1]), sp))
    torch.cuda.synchronize()
    out = [ev.ms(2 * k, 2 * k + 1) for k in range(steps)]
    ev.close()
    del g, flush
    return out


def per_config(args, hip) -> dict:
    """Every workload of the metric, fewer steps each: ms/step (median of the
    flushed steps), tokens/s, TFLOP/s and % of the bf16 peak (8NHV), the
    forward / backward split, and the oracle's tokens/s on a bounded sample."""
    import gc

    import torch

    from linear_cross_entropy_fp32_amd import synth
    out = {}
    for name in PER_CONFIG:
        w = synth.WORKLOADS[name]
        r = Runner(w, compact=False)
        m = measure(r, args.per_config_steps, 3, hip, kernel_events=False)
        ms = pct(m["cold"], 50)
        flops = 8.0 * w.n_tokens * w.hidden * w.vocab
        rec = {"n_tokens": w.n_tokens, "hidden": w.hidden, "vocab": w.vocab,
               "hidden_dtype": w.hidden_dtype, "bias": w.bias, "logit_scale": w.logit_scale,
               "softcap": w.softcap, "targets": w.targets, "reduction": w.reduction,
               "ms_per_step": ms, "ms_p20_p80": [pct(m["cold"], 20), pct(m["cold"], 80)],
               "warm_ms_per_step": pct(m["warm"], 50),
               "tokens_per_s": w.n_tokens / (ms * 1e-3),
               "tflops": flops / (ms * 1e-3) / 1e12,
               "pct_bf16_peak": 100.0 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
               "fwd_ms": pct(m["fwd"], 50), "bwd_ms": pct(m["bwd"], 50),
               "n_valid": int(r.red_i[0].item())}
        if name in GRAPH_CONFIGS:
            gm = pct(graph_steps(r, hip, max(3, args.per_config_steps)), 50)
            rec["graph_ms_per_step"] = gm
            rec["graph_tokens_per_s"] = w.n_tokens / (gm * 1e-3)
        if not args.no_cpu_baseline and w.targets != "all_ignored":
            cb = cpu_baseline(w, r.inp, args.per_config_cpu_seconds)
            rec["cpu_oracle_tokens_per_s"] = cb["value"]
            rec["gpu_speedup_vs_cpu_oracle"] = rec["tokens_per_s"] / cb["value"]
        out[name] = rec
        print(f"bench.py: per_config {name}: {ms:.3f} ms/step", file=sys.stderr, flush=True)
        del r
        gc.collect()
        torch.cuda.empty_cache()
    return out


# The Liger-Kernel page's in-place "none+weighted" fwd+bwd figures (ms, 8192
# rows, bf16): context for the materialised-logit cross-entropy, not a target.
PAGES_CE_MS = {32000: {"H100": 1.298, "B300": 0.65}, 128256: {"H100": 4.803, "B300": 2.25},
               151936: {"H100": 5.807, "B300": 2.70}}


def materialised_ce(args, hip) -> dict:
    """The standalone cross-entropy on materialised logits (flce_ce_forward with
    the gradient written in place, then flce_ce_backward scaling it by
    per-row weights), 8192 bf16 rows per vocabulary of the Liger-Kernel
    page's benchmark.  Each step restores the logits and evicts L2 and MALL
    outside its events.  HBM bytes per step (algorithmic): the forward reads
    and writes every element once, the backward reads and writes it once:
    4 * N * V * 2 bytes."""
    import torch

    import linear_cross_entropy_fp32_amd as flce
    from linear_cross_entropy_fp32_amd import synth
    out = {}
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    for name, (n, v) in synth.CE_WORKLOADS.items():
        pristine, targets, weights = synth.ce_inputs(n, v, 4242, "bf16", device="cuda:0")
        x = torch.empty_like(pristine)
        t, w = targets.to(dev), weights.to(dev)
        steps = max(3, args.per_config_steps)
        ev = Events(hip, 3 * steps)
        for i in range(steps + 2):        # two untimed warmup steps
            x.copy_(pristine)
            flush.fill_(i & 255)
            k = i - 2
            if k >= 0:
                _hip_ok(hip.hipEventRecord(ctypes.c_void_p(ev[3 * k]), sp))
            f = flce.flce_ce_forward(x, t)
            if k >= 0:
                _hip_ok(hip.hipEventRecord(ctypes.c_void_p(ev[3 * k + 1]), sp))
            flce.flce_ce_backward(x, t, f["reduced_i64"], flce.FLCE_GRAD_PER_TOKEN, w)
            if k >= 0:
                _hip_ok(hip.hipEventRecord(ctypes.c_void_p(ev[3 * k + 2]), sp))
        torch.cuda.synchronize()
        fwd = [ev.ms(3 * k, 3 * k + 1) for k in range(steps)]
        bwd = [ev.ms(3 * k + 1, 3 * k + 2) for k in range(steps)]
        ev.close()
        fm, bm = pct(fwd, 50), pct(bwd, 50)
        nbytes = n * v * 2
        out[name] = {"n_rows": n, "vocab": v, "dtype": "bf16", "usage": "none+weighted, in place",
                     "fwd_ms": fm, "bwd_ms": bm, "ms": fm + bm,
                     "fwd_gbs": 2 * nbytes / (fm * 1e-3) / 1e9,
                     "bwd_gbs": 2 * nbytes / (bm * 1e-3) / 1e9,
                     "hbm_frac": 4 * nbytes / ((fm + bm) * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "row_held_in_registers": (v * 2) % 16 == 0 and v * 2 <= 1024 * 20 * 16,
                     "pages_ms": PAGES_CE_MS.get(v)}
        print(f"bench.py: materialised_ce {name}: fwd {fm:.3f} ms, bwd {bm:.3f} ms",
              file=sys.stderr, flush=True)
        del pristine, x
        torch.cuda.empty_cache()
    del flush
    return out


def chunked_baseline(args, hip, w, chunk: int = 256) -> dict:
    """The pages' default loss path, timed on this GPU for comparison: the
    chunked loss with the projection fix of the TRL pull request "Do the
    chunked-CE lm_head projection on tensor cores instead of in fp32"
    (description and "Numbers").  The rows that carry a loss are packed to the
    front (a stable sort on validity, n_valid read on the host), and each
    chunk of `chunk` of them computes logits = (h @ W^T).float() with the bf16
    product on the vendor GEMM library, then + bias, * logit_scale and the
    softcap in fp32, then the cross-entropy, entropy and accuracy from fp32
    logits; the backward recomputes every chunk under autograd, as a
    checkpointed chunk does, and accumulates grad_weight (bf16, the
    parameter's dtype) and grad_bias across chunks.  The pages give no chunk
    size; 256 tokens is the chunk of their one-chunk benchmark.  Measurement
    context only: nothing of the library runs here."""
    import torch
    import torch.nn.functional as F

    from linear_cross_entropy_fp32_amd import synth
    dev = torch.device("cuda:0")
    inp = synth.make_inputs(w)
    h, wt, t = inp.hidden.to(dev), inp.weight.to(dev), inp.targets.to(dev)
    b = None if inp.bias is None else inp.bias.to(dev)
    scale, cap = w.logit_scale, w.softcap
    if w.reduction != "mean":
        raise ValueError("the chunked baseline is timed on mean-reduced workloads")

    def logits_of(hc, wg, bg):
        z = (hc @ wg.t()).float()
        if bg is not None:
            z = z + bg
        if scale != 1.0:
            z = z * scale
        if cap > 0:
            z = cap * torch.tanh(z / cap)
        return z

    state = {}

    def fwd():
        valid = (t >= 0) & (t < w.vocab)
        order = torch.argsort((~valid).to(torch.int8), stable=True)
        n_valid = int(valid.sum().item())
        loss = torch.zeros((), dtype=torch.float32, device=dev)
        ent = torch.zeros((), dtype=torch.float32, device=dev)
        correct = torch.zeros((), dtype=torch.int64, device=dev)
        with torch.no_grad():
            for c0 in range(0, n_valid, chunk):
                idx = order[c0:min(n_valid, c0 + chunk)]
                z = logits_of(h[idx], wt, b)
                tc = t[idx]
                lse = torch.logsumexp(z, dim=-1)
                loss += (lse - z.gather(1, tc[:, None])[:, 0]).sum()
                ent += (lse - (torch.softmax(z, dim=-1) * z).sum(-1)).sum()
                correct += (z.argmax(-1) == tc).sum()
        state.update(order=order, n_valid=n_valid)
        return loss / max(n_valid, 1), ent, correct

    def bwd():
        order, n_valid = state["order"], state["n_valid"]
        g = 1.0 / max(n_valid, 1)
        grad_h = torch.zeros_like(h)
        grad_w = torch.zeros_like(wt)
        grad_b = None if b is None else torch.zeros_like(b)
        wg = wt.detach().requires_grad_(True)
        bg = None if b is None else b.detach().requires_grad_(True)
        for c0 in range(0, n_valid, chunk):
            idx = order[c0:min(n_valid, c0 + chunk)]
            hc = h[idx].detach().requires_grad_(True)
            lc = F.cross_entropy(logits_of(hc, wg, bg), t[idx], reduction="sum") * g
            grads = torch.autograd.grad(lc, (hc, wg) + ((bg,) if bg is not None else ()))
            grad_h[idx] = grads[0]
            grad_w += grads[1]
            if bg is not None:
                grad_b += grads[2]
        return grad_h, grad_w, grad_b

    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    steps = max(3, args.per_config_steps)
    ev = Events(hip, 3 * steps)
    loss = None
    for i in range(steps + 2):            # two untimed warmup steps
        flush.fill_(i & 255)
        k = i - 2
        if k >= 0:
            _hip_ok(hip.hipEventRecord(ctypes.c_void_p(ev[3 * k]), sp))
        loss, _, _ = fwd()
        if k >= 0:
            _hip_ok(hip.hipEventRecord(ctypes.c_void_p(ev[3 * k + 1]), sp))
        bwd()
        if k >= 0:
            _hip_ok(hip.hipEventRecord(ctypes.c_void_p(ev[3 * k + 2]), sp))
    torch.cuda.synchronize()
    fwd_ms = [ev.ms(3 * k, 3 * k + 1) for k in range(steps)]
    bwd_ms = [ev.ms(3 * k + 1, 3 * k + 2) for k in range(steps)]
    tot = [a + c for a, c in zip(fwd_ms, bwd_ms)]
    ev.close()
    ms = pct(tot, 50)
    out = {"workload": w.name, "chunk_tokens": chunk, "ms": ms, "fwd_ms": pct(fwd_ms, 50),
           "bwd_ms": pct(bwd_ms, 50), "tokens_per_s": w.n_tokens / (ms * 1e-3),
           "loss_mean": float(loss.item()),
           "timing": "median of K steps after two untimed ones, each after a 512 MiB L2+MALL "
                     "eviction; the host reads n_valid in the forward, as the chunked path does"}
    del flush, h, wt, t, b
    torch.cuda.empty_cache()
    return out


def main() -> int:
    args = parse()
    if args.traffic_record:
        return write_traffic_record(args)
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (got --gpus {args.gpus}); "
              "a multi-GPU split of the vocabulary or the tokens is not built", file=sys.stderr)
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

    from linear_cross_entropy_fp32_amd import synth
    hip = _hip_runtime()
    if args.ce_only:
        print(json.dumps({"materialised_ce": materialised_ce(args, hip)}), flush=True)
        return 0
    w = synth.WORKLOADS[args.workload]
    r = Runner(w, args.compact)
    m = measure(r, args.steps, args.warmup, hip, kernel_events=True)
    n, hd, v = w.n_tokens, w.hidden, w.vocab
    ms = pct(m["cold"], 50)
    # with compaction the algorithmic work is that of the rows carrying a loss
    n_valid = int(r.red_i[0].item())
    n_work = n_valid if args.compact else n
    flops = 8.0 * n_work * hd * v
    tflops = flops / (ms * 1e-3) / 1e12
    # dominant kernel: the backward contraction (grad_hidden and grad_weight of
    # one vocabulary chunk per launch); over a step its launches do 4*N*H*V
    # flops of algorithmic work
    kern_ms = m["kern_ms"]
    launches = max(1, len(kern_ms))
    kern_avg = sum(kern_ms) / launches if kern_ms else float("nan")
    per_step_ms = kern_avg * launches / args.steps
    kern_tflops = 4.0 * n_work * hd * v / (per_step_ms * 1e-3) / 1e12
    traffic = _committed_traffic(w.name, "contract_kernel")
    warm_ms = pct(m["warm"], 50)
    out = {
        "metric": METRIC, "value": n / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": m["warmup_steps"], "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "n_tokens": n, "hidden": hd, "vocab": v,
                   "hidden_dtype": w.hidden_dtype, "bias": w.bias, "logit_scale": w.logit_scale,
                   "softcap": w.softcap, "reduction": w.reduction,
                   "compact_valid": bool(args.compact), "n_valid": n_valid},
        "timing": "median of K steps, each after a 512 MiB L2+MALL eviction outside its "
                  "events; warmup >= 25 ms after one discarded call",
        "tflops": tflops, "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "fwd_ms": pct(m["fwd"], 50), "bwd_ms": pct(m["bwd"], 50), "wall_s": m["wall_s"],
        "warmup_ms": m["warmup_ms"],
        "step_ms_p20_p50_p80": [pct(m["cold"], q) for q in (20, 50, 80)],
        "warm_ms_per_step": warm_ms,
        "warm_step_ms_p20_p50_p80": [pct(m["warm"], q) for q in (20, 50, 80)],
        "warm_tokens_per_s": n / (warm_ms * 1e-3),
        "roofline": {"bound": "mfma", "kernel": "contract_kernel", "achieved": kern_tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": kern_tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "launch_ms": kern_avg, "launches_per_step": launches / args.steps},
    }
    fused_loss = float(r.red_f[1].item())
    del r
    torch.cuda.empty_cache()
    if args.per_config_steps > 0 and not args.compact and w.reduction == "mean":
        cb = chunked_baseline(args, hip, w)
        cb["fused_ms"] = ms
        cb["fused_speedup"] = cb["ms"] / ms
        cb["loss_rel_diff"] = abs(cb["loss_mean"] - fused_loss) / max(abs(fused_loss), 1e-30)
        cb["pages_context"] = ("the pages measure cce at 1.65x the fixed chunked path on a whole "
                               "training step of gemma-3-270m (vocab 262k, hidden 640, seq 2048) "
                               "on one H100; this ratio is the loss alone")
        out["chunked_baseline"] = cb
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, synth.make_inputs(w), args.cpu_seconds)
    if args.per_config_steps > 0 and not args.compact:
        out["per_config"] = per_config(args, hip)
        out["materialised_ce"] = materialised_ce(args, hip)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
