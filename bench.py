"""Benchmark: one training step of the packed varlen width-4 depthwise causal
conv1d + SiLU (forward kernel, then the backward main + reduce kernels) on
the headline workload (S = 65536 tokens, C = 4096 channels, 22 lognormal
documents, FP32 weight and bias, "bf16" SiLU' policy), inputs resident in
HBM.

Prints one JSON line.  `value` is the step's algorithmic HBM traffic
(forward 4 B + backward 6 B per token-channel, plus parameters) divided by
the step time: the wall clock of the timed steps, which run back to back
with no instrumentation between them, bracketed by device synchronizations
(`ms_per_step_events` is the same region timed by one pair of HIP events).
Per-direction GB/s, Mtokens/s and fractions of the 8 TB/s MI355X HBM peak
are alongside.  `roofline` prices one conv1d_bwd call (the main kernel and
the small fixed-order reduce it enqueues) and `roofline_fwd` the forward
kernel: algorithmic bytes over the mean launch duration, timed with one
pair of HIP events on the launch stream around as many back-to-back calls
as there are timed steps, and, when profiles/headline_counters.md was taken
on these same kernel sources, the HBM traffic the rocprofv3 counters saw
per launch at the same duration.  `cpu_baseline` times the FP64 CPU oracle on a
bounded sample of the same workload on this host, on one thread and
(`all_cores`) over channel blocks on every core of this process.

`--warmup` is a minimum: warm-up steps continue until launch times settle
(the GPU's clocks ramp over its first ~100 launches), and the JSON records
how many ran.  `workloads` adds per-call forward and backward GB/s of the
other full-size workloads (Long, Stress under both policies, Uniform over
rotated buffer sets) and of the headline under the "fp32" policy.

`--workload long` or `--workload stress` times another full-size workload
in the same way (the headline is the default and the benchmark's line; the
counted traffic is recorded for the headline only).  `--copy-calibration`
instead times a plain device copy of one [S, C] BF16 tensor: the reference
kernel of known size that scales the byte counters.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd/bwd HBM GB/s + Mtokens/s, S=64K C=4096 packed; % of HBM roofline"
HBM_PEAK_GBS = 8000.0
WORKLOAD = "headline"
# Workloads --workload accepts, with their document recipe.  Uniform is left
# out: its 201 MB backward working set fits the 256 MB last-level cache, so
# back-to-back steps on one buffer set would not measure HBM.
DOCS = {"headline": "packed documents (lognormal lengths)",
        "long": "one document",
        "stress": "packed documents (lengths U{0..25}, empty ones included; 1% of x at +-60)"}
CPU_SAMPLE_CHANNELS = 4096
# HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE and
# WRITE_SIZE, scaled by a plain copy's reading) for the kernels as built from
# the sources whose digest the file records; ignored once the sources differ.
COUNTERS_FILE = os.path.join(ROOT, "profiles", "headline_counters.md")
CSRC = os.path.join(ROOT, "varlen_depthwise_causal_amd", "csrc")
KERNEL_SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                        if f.endswith((".hip", ".h", ".cpp")))


def algorithmic_bytes(wl, direction):
    """Minimum HBM bytes of one call: activations plus parameters and cu_seqlens."""
    S, C = wl.S, wl.C
    pw = C * 4 * (4 if wl.w_dtype == "f32" else 2)
    pb = 0 if wl.b is None else C * (4 if wl.b_dtype == "f32" else 2)
    cu = 4 * wl.cu.size
    if direction == "fwd":
        return 4 * S * C + pw + pb + cu            # read x, write y
    # read x and dy, write dx; write dweight and dbias (FP32 here)
    return 6 * S * C + pw + pb + cu + C * 4 * 4 + (0 if wl.b is None else C * 4)


def sources_digest():
    """Digest of the kernel sources' code: comments and layout are left out,
    so a comment edit keeps the recorded counters valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def counted_traffic(policy):
    """{kernel: bytes per launch} from the committed counter summary, or None
    when it is missing, was taken on other sources, or for another policy."""
    try:
        with open(COUNTERS_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    for line in lines:
        if line.startswith("traffic-json: "):
            rec = json.loads(line[len("traffic-json: "):])
            if rec.get("sources") == sources_digest() and rec.get("policy") == policy:
                return rec
    return None


def copy_calibration(steps, warmup):
    """Time a plain device copy of one [S, C] BF16 tensor (the reference for
    scaling the HBM byte counters and a practical bandwidth ceiling)."""
    import torch
    from varlen_depthwise_causal_amd import workloads as W
    spec = W.SPECS[WORKLOAD]
    dev = torch.device("cuda:0")
    x = torch.empty((spec.S, spec.C), dtype=torch.bfloat16, device=dev).fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(warmup):
        y.copy_(x)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        y.copy_(x)
        e[1].record()
    torch.cuda.synchronize()
    ms = statistics.mean(e[0].elapsed_time(e[1]) for e in ev)
    nbytes = 2 * x.numel() * x.element_size()
    print(json.dumps({"copy_calibration": {"S": spec.S, "C": spec.C, "bytes_read": nbytes // 2,
                                           "bytes_written": nbytes // 2, "ms": round(ms, 4),
                                           "GB_s": round(nbytes / (ms * 1e-3) / 1e9, 2),
                                           "steps": steps}}), flush=True)


# Warm-up floor.  The first ~100 launches after the GPU wakes run up to 40%
# slower while its clocks settle, so --warmup is a minimum: warm-up steps
# continue, in blocks of SETTLE_BLOCK, until at least SETTLE_MIN_STEPS steps
# and SETTLE_MIN_S seconds have passed and the last three blocks' mean step
# times agree within SETTLE_TOL, or until SETTLE_MAX_S seconds.
SETTLE_BLOCK = 10
SETTLE_MIN_STEPS = 100
SETTLE_MIN_S = 0.1
SETTLE_TOL = 0.01
SETTLE_MAX_S = 2.0


def settle(step, min_steps):
    """Run warm-up steps until launch times settle (see SETTLE_*); returns
    the steps run, their wall time and the last blocks' step times."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n, blocks = 0, []
    while True:
        e0.record()
        for _ in range(SETTLE_BLOCK):
            step()
        e1.record()
        torch.cuda.synchronize()
        n += SETTLE_BLOCK
        blocks.append(e0.elapsed_time(e1) / SETTLE_BLOCK)
        el = time.perf_counter() - t0
        last = blocks[-3:]
        steady = len(last) == 3 and max(last) - min(last) <= SETTLE_TOL * min(last)
        if (n >= max(min_steps, SETTLE_MIN_STEPS) and el >= SETTLE_MIN_S and steady) \
                or el >= SETTLE_MAX_S:
            return {"steps_run": n, "ms": round(el * 1e3, 1), "settled": steady,
                    "last_block_ms_per_step": [round(b, 4) for b in last]}


def gpu_leg(wl, policy, steps, warmup):
    import torch
    import varlen_depthwise_causal_amd as vdc

    dev = torch.device("cuda:0")

    def bf16(a):
        import numpy as np
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    x, dy = bf16(wl.x), bf16(wl.dy)
    w = torch.from_numpy(wl.w).to(dev) if wl.w_dtype == "f32" else bf16(wl.w)
    b = None
    if wl.b is not None:
        b = torch.from_numpy(wl.b).to(dev) if wl.b_dtype == "f32" else bf16(wl.b)
    cu = torch.from_numpy(wl.cu).to(dev)
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    dw = torch.empty((wl.C, 4), dtype=torch.float32, device=dev)
    db = torch.empty((wl.C,), dtype=torch.float32, device=dev) if b is not None else None
    ws = torch.empty(max(vdc.workspace_bytes("bwd", wl.S, wl.C), 1), dtype=torch.uint8, device=dev)

    def fwd():
        vdc.conv1d_fwd(x, w, cu, bias=b, out=y)

    def bwd():
        vdc.conv1d_bwd(x, w, cu, dy, bias=b, silu_grad_preactivation=policy, workspace=ws,
                       dx=dx, dweight=dw, dbias=db)

    warm = settle(lambda: (fwd(), bwd()), warmup)
    # The timed steps carry no instrumentation between launches: an event
    # recorded between two launches holds the next one back by several
    # microseconds.  One event pair brackets the whole region.
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s0.record()
    for _ in range(steps):
        fwd()
        bwd()
    s1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    steps_event_ms = s0.elapsed_time(s1)

    def per_launch_ms(call):
        """Mean duration of one call over `steps` back-to-back calls, from
        one pair of HIP events on the launch stream."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    return {"wall_s": wall, "steps_event_ms": steps_event_ms, "warm": warm,
            "fwd_ms": per_launch_ms(fwd), "bwd_ms": per_launch_ms(bwd),
            "plan_fwd": vdc.conv1d_plan("fwd", wl.S, wl.C, policy),
            "plan_bwd": vdc.conv1d_plan("bwd", wl.S, wl.C, policy)}


# Workloads timed beside the headline step (`workloads` key): (workload,
# policy, rotated buffer sets).  Uniform's tensors fit the 256 MB last-level
# cache, so its calls rotate over four sets of x, dy, y and dx (800 MB).
EXTRA = (("headline", "fp32", 1), ("long", "fp32", 1), ("stress", "bf16", 1),
         ("stress", "fp32", 1), ("uniform", "bf16", 4))
EXTRA_CALLS = 50


def launch_ms(wl, policies, calls, sets):
    """Per-call duration (ms) of conv1d_fwd and of conv1d_bwd under each
    policy: one pair of HIP events around `calls` back-to-back calls on the
    launch stream, rotating over `sets` buffer sets, after a settling
    warm-up."""
    import numpy as np
    import torch
    import varlen_depthwise_causal_amd as vdc
    dev = torch.device("cuda:0")

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    w = torch.from_numpy(wl.w).to(dev) if wl.w_dtype == "f32" else bf16(wl.w)
    b = None
    if wl.b is not None:
        b = torch.from_numpy(wl.b).to(dev) if wl.b_dtype == "f32" else bf16(wl.b)
    cu = torch.from_numpy(wl.cu).to(dev)
    x0, dy0 = bf16(wl.x), bf16(wl.dy)
    bufs = []
    for i in range(sets):
        x = x0 if i == 0 else x0.clone()
        dy = dy0 if i == 0 else dy0.clone()
        bufs.append((x, dy, torch.empty_like(x), torch.empty_like(x)))
    dw = torch.empty((wl.C, 4), dtype=torch.float32, device=dev)
    db = torch.empty((wl.C,), dtype=torch.float32, device=dev) if b is not None else None
    ws = torch.empty(max(vdc.workspace_bytes("bwd", wl.S, wl.C), 1), dtype=torch.uint8,
                     device=dev)

    def fwd(i):
        x, _, y, _ = bufs[i % sets]
        vdc.conv1d_fwd(x, w, cu, bias=b, out=y)

    def bwd(i, policy):
        x, dy, _, dx = bufs[i % sets]
        vdc.conv1d_bwd(x, w, cu, dy, bias=b, silu_grad_preactivation=policy, workspace=ws,
                       dx=dx, dweight=dw, dbias=db)

    def timed(call):
        ctr = [0]

        def step():
            call(ctr[0])
            ctr[0] += 1
        settle(step, 0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(calls):
            call(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / calls

    out = {"fwd": timed(fwd)}
    for policy in policies:
        out["bwd_" + policy] = timed(lambda i, p=policy: bwd(i, p))
    del bufs, ws
    torch.cuda.empty_cache()
    return out


def workloads_leg():
    """Forward and backward GB/s of the other full-size workloads (and of the
    headline under the "fp32" policy), each call timed on its own."""
    from varlen_depthwise_causal_amd import workloads as W
    by_wl = {}
    for name, policy, sets in EXTRA:
        by_wl.setdefault((name, sets), []).append(policy)
    res = {}
    for (name, sets), policies in by_wl.items():
        wl = W.make(name, workers=16)
        t = launch_ms(wl, policies, EXTRA_CALLS, sets)
        fb, bb = algorithmic_bytes(wl, "fwd"), algorithmic_bytes(wl, "bwd")

        def rate(nbytes, ms):
            gbs = nbytes / (ms * 1e-3) / 1e9
            return {"ms": round(ms, 4), "GB_s": round(gbs, 1),
                    "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                    "mtokens_per_s": round(wl.S / (ms * 1e-3) / 1e6, 2)}
        for policy in policies:
            key = "%s/%s" % (name, policy)
            res[key] = {"S": wl.S, "C": wl.C, "docs": wl.num_docs,
                        "buffer_sets": sets, "calls": EXTRA_CALLS,
                        "fwd": rate(fb, t["fwd"]), "bwd": rate(bb, t["bwd_" + policy])}
            print("workload %s: fwd %.4f ms, bwd %.4f ms" % (key, t["fwd"], t["bwd_" + policy]),
                  file=sys.stderr, flush=True)
        del wl
    return res


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# Host threads of the all-core oracle leg, at most: the host cores a
# one-GPU job is given, which os.cpu_count() may overstate on a shared host.
CPU_THREADS_MAX = 16


def cpu_leg(wl, policy):
    """The FP64 oracle on every token of a channel sample: one thread (the
    baseline), then the same oracle code over channel blocks on all of this
    process's cores (channels are independent)."""
    import numpy as np
    import oracle
    from concurrent.futures import ThreadPoolExecutor

    cols = np.arange(min(CPU_SAMPLE_CHANNELS, wl.C))
    x = oracle.decode_bf16(wl.x[:, cols])
    dy = oracle.decode_bf16(wl.dy[:, cols])
    w = oracle.decode_param(wl.w, wl.w_dtype)[cols]
    b = oracle.decode_param(wl.b, wl.b_dtype)[cols] if wl.b is not None else None

    def run(xs, dys, ws, bs):
        oracle.forward(xs, ws, bs, wl.cu, want=("y",))
        oracle.backward(xs, ws, bs, wl.cu, dys, policy, want=("dx", "dw", "db"))

    t0 = time.perf_counter()
    run(x, dy, w, b)
    dt = time.perf_counter() - t0
    elems = wl.S * len(cols)
    res = {"value": round(10 * elems / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "host_cpu": host_cpu_model(), "host_cpus": os.cpu_count(),
           "sample": "all %d tokens x %d of %d channels (channels are independent), "
                     "forward + backward, FP64 C oracle, one thread, %.1f s"
                     % (wl.S, len(cols), wl.C, dt),
           "mtokens_per_s_full_width": round(elems / wl.C / dt / 1e6, 5)}
    # All cores: the unchanged oracle on contiguous channel blocks, one per
    # thread (its C code runs with the interpreter lock released).
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    n = max(1, min(n, CPU_THREADS_MAX))
    parts = np.array_split(np.arange(len(cols)), n)
    blocks = [(np.ascontiguousarray(x[:, p]), np.ascontiguousarray(dy[:, p]),
               np.ascontiguousarray(w[p]), None if b is None else np.ascontiguousarray(b[p]))
              for p in parts]
    del x, dy
    with ThreadPoolExecutor(n) as pool:
        t0 = time.perf_counter()
        list(pool.map(lambda blk: run(*blk), blocks))
        dt_all = time.perf_counter() - t0
    res["all_cores"] = {"value": round(10 * elems / dt_all / 1e9, 4), "unit": "GB/s",
                        "cores": n, "kind": "oracle",
                        "sample": "the same sample in %d channel blocks, one thread each, "
                                  "%.2f s" % (n, dt_all),
                        "mtokens_per_s_full_width": round(elems / wl.C / dt_all / 1e6, 5)}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # --warmup is a minimum: warm-up continues until launch times settle
    # (settle()), so a small value still times the steady state.
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=WORKLOAD, choices=sorted(DOCS))
    ap.add_argument("--policy", default=None, choices=["bf16", "fp32"],
                    help="SiLU' policy (default: the workload's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other workloads' per-call timings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain copy of one [S, C] BF16 tensor instead")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path runs on one GPU only (no multi-GPU sharding is built); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.steps, args.warmup)
        return

    from varlen_depthwise_causal_amd import workloads as W
    if args.policy is None:
        args.policy = W.SPECS[args.workload].policies[0]
    wl = W.make(args.workload, workers=16)
    g = gpu_leg(wl, args.policy, args.steps, args.warmup)

    traffic = counted_traffic(args.policy) if args.workload == WORKLOAD else None

    def roofline(kernel, alg_bytes, ms, counted, names):
        achieved = alg_bytes / (ms * 1e-3) / 1e9
        out = {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 2),
               "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
               "traffic": None, "algorithmic_bytes": alg_bytes, "launch_ms": round(ms, 4)}
        if counted is not None:
            nbytes = sum(counted["bytes_per_launch"][n] for n in names)
            out["traffic"] = round(nbytes / (ms * 1e-3) / 1e9, 2)
            out["traffic_bytes"] = nbytes
            out["traffic_over_algorithmic"] = round(nbytes / alg_bytes, 4)
        return out

    fwd_ms = g["fwd_ms"]
    bwd_ms = g["bwd_ms"]
    step_ms = g["wall_s"] * 1e3 / args.steps
    fb, bb = algorithmic_bytes(wl, "fwd"), algorithmic_bytes(wl, "bwd")
    fwd_gbs = fb / (fwd_ms * 1e-3) / 1e9
    bwd_gbs = bb / (bwd_ms * 1e-3) / 1e9
    step_gbs = (fb + bb) / (step_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC if args.workload == WORKLOAD else METRIC.replace(
            "S=64K C=4096", "S=%dK C=%d" % (wl.S // 1024, wl.C)),
        "value": round(step_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "ms_per_step_events": round(g["steps_event_ms"] / args.steps, 4),
        "warmup_steps_run": g["warm"]["steps_run"],
        "warmup_ms": g["warm"]["ms"],
        "warmup_settled": g["warm"]["settled"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: S=%d C=%d, %d %s, weight %s, bias %s, "
                               "silu_grad_preactivation=%s"
                               % (args.workload, wl.S, wl.C, wl.num_docs, DOCS[args.workload],
                                  wl.w_dtype, wl.b_dtype, args.policy),
                   "S": wl.S, "C": wl.C, "docs": wl.num_docs, "policy": args.policy},
        "step_frac_of_hbm_peak": round(step_gbs / HBM_PEAK_GBS, 4),
        "step_mtokens_per_s": round(wl.S / (step_ms * 1e-3) / 1e6, 3),
        "fwd": {"ms": round(fwd_ms, 4),
                "GB_s": round(fwd_gbs, 2), "frac_of_peak": round(fwd_gbs / HBM_PEAK_GBS, 4),
                "mtokens_per_s": round(wl.S / (fwd_ms * 1e-3) / 1e6, 3),
                "algorithmic_bytes": fb, "plan": g["plan_fwd"]},
        "bwd": {"ms": round(bwd_ms, 4),
                "GB_s": round(bwd_gbs, 2), "frac_of_peak": round(bwd_gbs / HBM_PEAK_GBS, 4),
                "mtokens_per_s": round(wl.S / (bwd_ms * 1e-3) / 1e6, 3),
                "algorithmic_bytes": bb, "plan": g["plan_bwd"],
                "partial_bytes": 2 * g["plan_bwd"]["prows"] * 5 * wl.C * g["plan_bwd"]["acc_bytes"]},
        "roofline": roofline("conv1d_bwd (bwd_main_kernel then bwd_reduce_kernel, one call)",
                             bb, bwd_ms, traffic, ("bwd_main_kernel", "bwd_reduce_kernel")),
        "roofline_fwd": roofline("fwd_kernel", fb, fwd_ms, traffic, ("fwd_kernel",)),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_leg(wl, args.policy)
    if not args.no_workloads and args.workload == WORKLOAD:
        del wl
        res["workloads"] = workloads_leg()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
