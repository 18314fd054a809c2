"""Benchmark of the CfC K-loop hot path on one MI355X.

One step = forward + backward (overwrite mode, so the scratch clear is part of
the step) + reduce_axis0 over one batch of the training-scale workload (B=256,
K=64, n_in=n_hid=128, dt=0.5), inputs resident in HBM.  By default the
forward and backward are one cfc_forward_backward call (one kernel at this
shape; at widths above 128 with K <= 20 two launches that pass the
pre-activations through the scratch); --path separate times cfc_forward +
cfc_backward instead.  Both paths are timed in every run; the other one is
reported in "other_path".

Prints ONE JSON line.  `value` is batch-steps/s = B*K / seconds per step.
Before any timed pass the measured step runs back to back, untimed, for
--gpu-warmup-ms (default 300 ms), so that the GPU's clocks have left their
idle state (recorded in "gpu_warmup").  Each path is run twice: a breakdown pass with HIP events around every launch
("kernels_ms"), then the timed pass that gives `value`, with events only
around the step's dominant kernel and only on every --event-stride-th step
(each event record costs the stream about 2.5 us).  The roofline object
describes that kernel, with its average duration from the events of the
timed pass, recorded on the stream the kernel runs on.  The cpu_baseline object times the float64 oracle on the
host on a bounded sample of the same workload (all cores, and one thread).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CfC fwd+BPTT batch-steps/s (B=256,K=64,H=128); reduce_axis0 HBM GB/s"
PEAK_F64_TFLOPS = 78.6        # MI355X FP64 vector: 256 CU * 2.4 GHz * 64 FMA/clk * 2
PEAK_HBM_GBPS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "cfc_recurrent_cell_amd", "csrc", "cfc.hip")
PROFILES = os.path.join(ROOT, "profiles")


def algorithmic_work(B, K, n_in, H):
    """FLOPs and bytes per launch that the method itself needs (not what a
    particular kernel happens to move).  FLOPs count multiply-adds of the
    contractions as 2; the O(H) elementwise work is not counted.  The separate
    backward must recompute the pre-activations from h_seq (its inputs hold no
    a_k); the one-call path has them from its own forward."""
    N = H * (n_in + H + 2)
    rows = B * K
    fwd_flops = rows * 2 * H * (n_in + H)
    # bwd: W_rec^T da, dW_in and dW_rec contractions (+ recomputing a)
    grad_flops = rows * (2 * H * H + 2 * H * (n_in + H))
    bwd_flops = rows * 2 * H * (n_in + H) + grad_flops
    f = 4
    fwd_bytes = f * (B * K * n_in + B * H + B * K * H + H * (n_in + H + 2))
    bwd_bytes = f * (B * K * n_in + B * H + B * K * H + B * H + B * N + B + H * (n_in + H + 2))
    fb_bytes = f * (B * K * n_in + B * H + B * K * H + B * H + B * N + B + H * (n_in + H + 2))
    red_bytes = f * (B * N + N)
    return dict(fwd_flops=fwd_flops, bwd_flops=bwd_flops, fb_flops=fwd_flops + grad_flops,
                fwd_bytes=fwd_bytes, bwd_bytes=bwd_bytes, fb_bytes=fb_bytes, reduce_bytes=red_bytes)


def source_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary of this
    workload, only if it was taken on the current kernel source."""
    try:
        with open(os.path.join(PROFILES, f"traffic_{workload}.json")) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256_16") != source_hash():
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def cpu_baseline(inp, budget_s=10.0):
    """The float64 oracle on the host, as it stands: one thread over 32 of the
    rows, then all available cores (up to 16 threads, rows split between them)
    over all rows; each leg repeats whole forward+backward+reduce passes for
    about half the budget.  The all-cores leg is the headline object."""
    from oracle import oracle as O
    B, K = inp.x.shape[0], inp.x.shape[1]
    O.load_oracle()

    def leg(rows, threads, budget):
        sub = type(inp)(inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x[:rows], inp.h0[:rows], inp.y[:rows],
                        inp.dt, inp.cell)
        n, t0 = 0, time.perf_counter()
        while True:
            O.cfc_step(sub, threads=threads)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget:
                break
        return rows * K * n / el, n, el

    try:
        ncores = len(os.sched_getaffinity(0))
    except AttributeError:
        ncores = os.cpu_count() or 1
    threads = max(1, min(16, ncores))
    rows1 = max(1, min(B, 32))
    v1, n1, e1 = leg(rows1, 1, budget_s / 2)
    vn, nn, en = leg(B, threads, budget_s / 2)
    return {"value": vn, "unit": "batch-steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{nn} x (forward+backward+reduce over all {B} rows of the same workload, K={K}), "
                      f"float64, rows split over {threads} threads, {en:.1f} s",
            "single_thread": {"value": v1, "cores": 1,
                              "sample": f"{n1} x ({rows1} of the {B} rows), one thread, {e1:.1f} s"},
            "host_cores_available": ncores}


def profiled_kernel_us(profile, kernel, grid=None):
    """Average duration (us) of `kernel` in the committed rocprofv3 kernel-trace
    summary profiles/<profile>.txt, only if it was taken on the current kernel
    source; `grid` selects the row of that grid size where the summary splits a
    kernel by grid."""
    try:
        with open(os.path.join(PROFILES, profile + ".txt")) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    if not any(l.startswith("kernel source sha256[:16]: " + source_hash()) for l in lines):
        return None
    for l in lines:
        parts = l.split()
        if not parts or parts[0] != kernel:
            continue
        if grid is not None and not any(p == "grid=%d" % grid for p in parts):
            continue
        try:
            return float(parts[parts.index("avg_us") + 1]) if "avg_us" in parts else float(parts[-4])
        except (ValueError, IndexError):
            return None
    return None


def reduce_kernel(B, N):
    """The reduce_axis0 kernel instance the library launches for a 16-byte
    aligned [B, N] input with N % 4 == 0, and its grid (threads): 64 columns
    per workgroup, 128 above 256 MB of input."""
    if B * N > 64 * 1024 * 1024:
        return "reduce_axis0_kernel<4,32>", ((N + 127) // 128) * 256
    return "reduce_axis0_kernel<4,16>", ((N + 63) // 64) * 256


def reduce_standalone(torch, C, W, dev, reps=20):
    """reduce_axis0 alone on the reduce workload [32, 40960] and on the
    large-batch workload's scratch shape [8192, 131584] (4.31 GB), each launch
    preceded by an overwrite of a 512 MiB buffer so that neither the L2 nor the
    256 MB MALL holds its input: HBM-resident numbers.  Each launch is
    bracketed by HIP events on the launch stream (which include the launch gap,
    about 6 us); the rocprofv3 kernel duration of the same launches, from the
    committed summary, is reported beside it."""
    flush = torch.empty(128 * 1024 * 1024, device=dev)
    out = []
    large_N = W.scratch_row_len(W.LARGE.n_in, W.LARGE.n_hid)
    for name, B, N in ((W.REDUCE.name, W.REDUCE.B, W.REDUCE.N),
                       ("scratch_B8192_N131584", W.LARGE.B, large_N)):
        a = torch.randn(B, N, device=dev)
        o = torch.empty(N, device=dev)
        stream = torch.cuda.current_stream(dev)
        C.reduce_axis0(a, out=o)
        times = []
        for _ in range(reps):
            flush.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            C.reduce_axis0(a, out=o)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        med = times[len(times) // 2]
        nbytes = (B * N + N) * 4
        gbps = nbytes / (med * 1e-3) / 1e9
        rec = {"workload": name, "B": B, "N": N, "bytes": nbytes, "flushed": True,
               "kernel_ms_events_median": med, "GB_per_s": gbps, "frac_hbm": gbps / PEAK_HBM_GBPS,
               "hbm_floor_us": nbytes / (PEAK_HBM_GBPS * 1e9) * 1e6}
        us = profiled_kernel_us("kernels_reduce_axis0_standalone", *reduce_kernel(B, N))
        if us is not None:
            rec["kernel_us_rocprof"] = us
            rec["GB_per_s_rocprof"] = nbytes / (us * 1e-6) / 1e9
            rec["frac_hbm_rocprof"] = rec["GB_per_s_rocprof"] / PEAK_HBM_GBPS
        # a launch that cannot approach its HBM floor is bound by launch and
        # memory latency, not by bandwidth
        kernel_us = rec.get("kernel_us_rocprof", med * 1e3)
        rec["bound"] = "hbm" if kernel_us < 4 * rec["hbm_floor_us"] else "launch and memory latency"
        out.append(rec)
        del a, o
    del flush
    return out


def reduce_sweep(torch, C, W, dev, reps=20):
    """reduce_axis0 alone at several [B, N], timed with HIP events per launch,
    with a 512 MiB buffer overwritten between launches so that neither the L2
    nor the 256 MB MALL holds the input (HBM-resident numbers).  Narrow shapes
    (N <= 256 over many rows) are timed with both the one-pass reduce_axis0
    and the two-phase reduce_axis0_split (its two launches together)."""
    flush = torch.empty(128 * 1024 * 1024, device=dev)
    shapes = [(W.REDUCE.B, W.REDUCE.N, False), (256, 33024, False), (1024, 131584, False), (8192, 131584, False),
              (524288, 3, False), (524288, 3, True), (262144, 64, False), (262144, 64, True),
              (65536, 256, False), (65536, 256, True)]
    out = []
    for B, N, split in shapes:
        a = torch.randn(B, N, device=dev)
        o = torch.empty(N, device=dev)
        ws = None
        if split:
            ws = torch.empty((C.reduce_axis0_split_workspace(B, N),), dtype=torch.uint8, device=dev)
        run = lambda: C.reduce_axis0(a, out=o, split=split, workspace=ws)
        run()
        times = []
        for _ in range(reps):
            flush.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        med = times[len(times) // 2]
        gbps = (B * N + N) * 4 / (med * 1e-3) / 1e9
        out.append({"B": B, "N": N, "entry": "reduce_axis0_split" if split else "reduce_axis0",
                    "bytes": (B * N + N) * 4, "median_ms": med, "GB_per_s": gbps, "frac_hbm": gbps / PEAK_HBM_GBPS})
        del a, o, ws
    del flush
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gpu-warmup-ms", type=float, default=300.0,
                    help="before any timed pass, run the measured step back to back for this long (untimed), "
                         "so that the GPU's clocks have left their idle state")
    ap.add_argument("--event-stride", type=int, default=10,
                    help="timed pass: HIP events around the dominant kernel on every Nth step")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (to scale PMC byte counters)")
    ap.add_argument("--workload", default="train",
                    choices=["train", "smoke", "tiny", "large", "long", "tau_train", "tau_tiny"],
                    help="which seeded workload one step runs (the metric is quoted on 'train')")
    ap.add_argument("--no-reduce", action="store_true",
                    help="skip the standalone, cache-flushed reduce_axis0 measurement")
    ap.add_argument("--reduce-sweep", action="store_true",
                    help="also time reduce_axis0 alone, cache-flushed, over a range of sizes")
    ap.add_argument("--main-only", action="store_true",
                    help="time only the selected path in overwrite mode (no other-path or accumulate-mode "
                         "timing): for profiler runs whose per-kernel averages must match one variant")
    ap.add_argument("--input-grads", action="store_true",
                    help="the timed step also writes grad_x [B,K,n_in] and grad_h0 [B,H]")
    ap.add_argument("--window", type=int, default=64,
                    help="steps per window of the windows path")
    ap.add_argument("--path", default=None, choices=["fused", "separate", "windows"],
                    help="fused: one cfc_forward_backward call; separate: cfc_forward + cfc_backward "
                         "(default: fused where that call is one kernel, i.e. n_in, n_hid <= 128 and K <= 64)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the CfC path has no cross-GPU step in this "
              "library (rows shard over GPUs with one [N]-float exchange, not built here). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import cfc_recurrent_cell_amd as C
    from cfc_recurrent_cell_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    C.load_library()
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        n = 64 * 1024 * 1024
        a = torch.ones(n, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4}))
        return

    cfg = {"train": W.TRAIN, "smoke": W.SMOKE, "tiny": W.TINY, "large": W.LARGE, "long": W.LONG,
           "tau_train": W.TAU_TRAIN, "tau_tiny": W.TAU_TINY}[args.workload]
    cell = cfg.cell
    inp = W.make_cfc_inputs(cfg)
    t = lambda a: torch.from_numpy(a).to(dev)
    w_in, w_rec, b, w_tau, x, h0, y = map(t, (inp.w_in, inp.w_rec, inp.b, inp.w_tau, inp.x, inp.h0, inp.y))
    dt = float(inp.dt)
    B, K, n_in, H = cfg.B, cfg.K, cfg.n_in, cfg.n_hid
    N = W.scratch_row_len(n_in, H)
    h_seq = torch.empty((B, K, H), device=dev)
    scratch = torch.empty((B, N), device=dev)
    loss = torch.empty((B,), device=dev)
    out = torch.empty((N,), device=dev)

    one_call_bwd_ok = K * (12 * H + 4 * n_in) + 40 * H + 2048 <= 160 * 1024
    if args.path == "windows" and args.input_grads:
        print("--input-grads is not timed on the windows path", file=sys.stderr)
        sys.exit(2)
    if args.path is None:
        # the one-call entry where it is one kernel, or the two 16-row
        # launches that skip the recomputation; otherwise separate calls
        wide_parked = (n_in > 128 or H > 128) and K <= 20 and (H * (n_in + H + 2)) % 2 == 0
        args.path = "fused" if (n_in <= 128 and H <= 128 and K <= 64) or wide_parked else \
            "separate" if one_call_bwd_ok else "windows"

    grad_x = torch.empty((B, K, n_in), device=dev)
    grad_h0 = torch.empty((B, H), device=dev)
    delta_carry = torch.empty((B, H), device=dev)

    def fwd():
        C.cfc_forward(w_in, w_rec, b, w_tau, x, h0, dt, h_seq=h_seq, cell=cell)

    # accumulate mode at widths above 128 (K <= 20): the 16-row backward parks
    # dL/da in a caller workspace instead of the scratch tail; the one-call
    # entry's size also holds its float64 weight copy at 256 x 256 (the
    # backward alone uses the leading part)
    acc_ws_bytes = C.cfc_forward_backward_workspace(B, K, n_in, H, accumulate=True)
    acc_ws = torch.empty((acc_ws_bytes,), dtype=torch.uint8, device=dev) if acc_ws_bytes > 0 else None

    def bwd(ig=False, accumulate=False):
        C.cfc_backward(w_in, w_rec, b, w_tau, x, h0, h_seq, y, dt, scratch=scratch, loss=loss,
                       grad_x=grad_x if ig else None, grad_h0=grad_h0 if ig else None, accumulate=accumulate,
                       cell=cell, workspace=acc_ws if accumulate else None)

    def fb(ig=False, accumulate=False):
        C.cfc_forward_backward(w_in, w_rec, b, w_tau, x, h0, y, dt, h_seq=h_seq, scratch=scratch, loss=loss,
                               grad_x=grad_x if ig else None, grad_h0=grad_h0 if ig else None,
                               accumulate=accumulate, cell=cell, workspace=acc_ws if accumulate else None)

    def windows():
        # the backward as windows of --window steps (dL/dh carried in place)
        C.cfc_backward_windows(w_in, w_rec, b, w_tau, x, h0, h_seq, y, dt, args.window, scratch=scratch, loss=loss,
                               grad_h0=delta_carry, cell=cell)

    def red():
        C.reduce_axis0(scratch, out=out)

    # each step is a list of (kernel name, launch); the names key kernels_ms
    # and the roofline's kernel
    STEPS = {
        "fused": [("cfc_fb_kernel", fb), ("reduce_axis0_kernel", red)],
        "fused_ig": [("cfc_fb_kernel", lambda: fb(ig=True)), ("reduce_axis0_kernel", red)],
        "separate": [("cfc_fwd_kernel", fwd), ("cfc_bwd_kernel", bwd), ("reduce_axis0_kernel", red)],
        "separate_ig": [("cfc_fwd_kernel", fwd), ("cfc_bwd_kernel", lambda: bwd(ig=True)),
                        ("reduce_axis0_kernel", red)],
        "windows": [("cfc_fwd_kernel", fwd), ("cfc_bwd_kernel", windows), ("reduce_axis0_kernel", red)],
        # the pages' clear-then-accumulate form: explicit zero fill, then += gradient
        "accumulate": [("zero_fill", scratch.zero_), ("cfc_fb_kernel", lambda: fb(accumulate=True)),
                       ("reduce_axis0_kernel", red)],
    }
    acc_step = ("scratch zero fill + cfc_forward_backward(CFC_ACCUMULATE) + reduce_axis0" if acc_ws is None else
                "scratch zero fill + cfc_forward_backward_ws(CFC_ACCUMULATE, %d-byte workspace) + reduce_axis0"
                % acc_ws_bytes)

    def run_pass(path, bracket):
        """W warm-up steps, then K steps bracketed by a sync on both sides.
        bracket=None records a HIP event pair around every launch of every
        step (the per-kernel breakdown).  bracket=name records only the pair
        around that kernel's launch, and only on the last step of every
        --event-stride steps (not the first step, which follows the idle
        sync): each event record costs the stream about 2.5 us, which on a
        0.1 ms step would be counted as step time.  The kernel's average
        duration is taken over the steps that carry the pair; the step-time
        percentiles over the windows between the marks, per step."""
        launches = STEPS[path]
        for _ in range(args.warmup):
            for _, f in launches:
                f()
        torch.cuda.synchronize()
        names = [n for n, _ in launches if bracket is None or n == bracket]
        stride = 1 if bracket is None else max(1, args.event_stride)
        marked = [i for i in range(args.steps) if i % stride == stride - 1] or [args.steps - 1]
        evs = {i: {n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
               for i in marked}
        t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start.record()
        for i in range(args.steps):
            step_evs = evs.get(i, {})
            for n, f in launches:
                e = step_evs.get(n)
                if e is not None:
                    e[0].record()
                f()
                if e is not None:
                    e[1].record()
        t_end.record()
        torch.cuda.synchronize()
        ms = t_start.elapsed_time(t_end) / args.steps
        km = {n: sum(evs[i][n][0].elapsed_time(evs[i][n][1]) for i in marked) / len(marked) for n in names}
        # per-step times: windows from the start to the first marked step's
        # first event, between marked steps, and from the last to the end,
        # each divided by the steps it holds
        first = names[0]
        bounds = [t_start] + [evs[i][first][0] for i in marked] + [t_end]
        idx = [0] + marked + [args.steps]
        steps_ms = sorted(bounds[j].elapsed_time(bounds[j + 1]) / (idx[j + 1] - idx[j])
                          for j in range(len(bounds) - 1) if idx[j + 1] > idx[j])
        q = lambda f: steps_ms[min(len(steps_ms) - 1, int(f * len(steps_ms)))]
        return ms, km, {"p10": q(0.1), "p50": q(0.5), "p90": q(0.9)}

    def timed(path):
        """A breakdown pass (events around every launch), then the timed pass:
        events only around the step's dominant kernel, whose average duration
        there is the roofline's.  Returns (ms per step of the timed pass, the
        breakdown's kernel ms, the dominant kernel, its ms in the timed pass,
        step-time percentiles of the timed pass)."""
        _, k_all, _ = run_pass(path, None)
        dom = max((n for n in k_all if n != "zero_fill"), key=k_all.get)
        ms, k_dom, pct = run_pass(path, dom)
        return ms, k_all, dom, k_dom[dom], pct

    def gpu_warmup(path):
        """The step back to back for --gpu-warmup-ms, untimed.  After an idle
        period the GPU's clocks take tens of milliseconds of load to settle:
        measured on MI355X at the training-scale workload, 20-step passes
        separated by 10 ms of idle ran at 102 us per step, back-to-back steps
        at 96 us for the first 200 and 93 us from then on."""
        launches = STEPS[path]
        t0 = time.perf_counter()
        n = 0
        while True:
            for _ in range(10):
                for _, f in launches:
                    f()
            n += 10
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= args.gpu_warmup_ms:
                return n

    main_path = args.path + ("_ig" if args.input_grads else "")
    warm_steps = gpu_warmup(main_path) if args.gpu_warmup_ms > 0 else 0
    other = "separate" if args.path == "fused" else "fused"
    if args.path == "windows":
        args.main_only = True   # the other one-call paths refuse this K
    if not args.main_only:
        ms_other, k_other, _, _, _ = timed(other)
        ms_acc, k_acc, _, _, pct_acc = timed("accumulate")
        ms_ig, k_ig, _, _, pct_ig = timed(args.path + "_ig")
    ms_per_step, k_ms, dom, dom_ms, pct = timed(main_path)
    work = algorithmic_work(B, K, n_in, H)
    flops = {"cfc_fwd_kernel": work["fwd_flops"], "cfc_bwd_kernel": work["bwd_flops"],
             "cfc_fb_kernel": work["fb_flops"], "reduce_axis0_kernel": 0}
    nbytes = {"cfc_fwd_kernel": work["fwd_bytes"], "cfc_bwd_kernel": work["bwd_bytes"],
              "cfc_fb_kernel": work["fb_bytes"], "reduce_axis0_kernel": work["reduce_bytes"]}
    if args.input_grads:   # W_in^T dL/da per row-step, one more W_rec^T step per row; grad_x, grad_h0 out
        for kname in ("cfc_bwd_kernel", "cfc_fb_kernel"):
            flops[kname] += B * K * 2 * H * n_in + B * 2 * H * H
            nbytes[kname] += 4 * (B * K * n_in + B * H)
    # the bound is the roofline the kernel's algorithmic intensity falls under:
    # below the f64 ridge (78.6 TFLOP/s / 8 TB/s = 9.8 FLOP/B) it is HBM
    ridge = PEAK_F64_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    if flops[dom] / nbytes[dom] < ridge:
        ach = nbytes[dom] / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBPS}
    else:
        ach = flops[dom] / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "alu", "achieved": ach, "peak": PEAK_F64_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_F64_TFLOPS}
    roof["kernel"] = dom
    roof["kernel_ms"] = dom_ms
    roof["algorithmic_flops_per_launch"] = flops[dom]
    roof["algorithmic_bytes_per_launch"] = nbytes[dom]
    roof["traffic"] = measured_traffic(cfg.name + ("_input_grads" if args.input_grads else ""), dom)
    # the same kernel's average duration under rocprofv3 (committed summary of
    # this workload's bench step, current kernel source only)
    launched = {"cfc_fb_kernel": "cfc_fb_small_kernel<true>" if args.path == "fused" else None}.get(dom)
    prof_name = "kernels_" + cfg.name + ("_input_grads" if args.input_grads else "")
    prof_us = profiled_kernel_us(prof_name, launched) if launched else None
    if prof_us is not None:
        roof["kernel_ms_rocprof"] = prof_us * 1e-3
        roof["frac_rocprof"] = (flops[dom] / (prof_us * 1e-6) / 1e12 / PEAK_F64_TFLOPS if roof["bound"] == "alu"
                                else nbytes[dom] / (prof_us * 1e-6) / 1e9 / PEAK_HBM_GBPS)
    red_gbps = work["reduce_bytes"] / (k_ms["reduce_axis0_kernel"] * 1e-3) / 1e9
    # floors of the whole step: algorithmic bytes at 8 TB/s, algorithmic f64
    # flops at 78.6 TFLOP/s; frac = the larger floor / measured time
    step_flops = work["fb_flops"] if args.path == "fused" else work["fwd_flops"] + work["bwd_flops"]
    step_bytes = (work["fb_bytes"] if args.path == "fused" else work["fwd_bytes"] + work["bwd_bytes"]) + \
        work["reduce_bytes"]
    if args.input_grads:
        step_flops += B * K * 2 * H * n_in + B * 2 * H * H
        step_bytes += 4 * (B * K * n_in + B * H)
    hbm_floor_ms = step_bytes / (PEAK_HBM_GBPS * 1e9) * 1e3
    f64_floor_ms = step_flops / (PEAK_F64_TFLOPS * 1e12) * 1e3
    floors = {"algorithmic_bytes": step_bytes, "algorithmic_f64_flops": step_flops,
              "hbm_floor_ms": hbm_floor_ms, "f64_floor_ms": f64_floor_ms,
              "frac_hbm": hbm_floor_ms / ms_per_step, "frac_f64": f64_floor_ms / ms_per_step,
              "frac_of_max_floor": max(hbm_floor_ms, f64_floor_ms) / ms_per_step}

    value = B * K / (ms_per_step * 1e-3)
    rec = {
        "metric": METRIC, "value": value, "unit": "batch-steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": cfg.name, "cell": cell, "B": B, "K": K, "n_in": n_in, "n_hid": H, "dt": dt,
                   "scratch_N": N, "io_dtype": "f32", "seed": cfg.seed},
        "roofline": roof,
        "path": args.path,
        "input_grads": args.input_grads,
        "fused_call_is_one_kernel": n_in <= 128 and H <= 128 and K <= 64,
        "step_ms_percentiles": pct,
        "timed_pass_event_stride": args.event_stride,
        "gpu_warmup": {"ms": args.gpu_warmup_ms, "steps": warm_steps},
        "step_floors": floors,
        "kernels_ms": k_ms,
        "with_input_grads": None if args.main_only else {
            "ms_per_step": ms_ig, "value": B * K / (ms_ig * 1e-3), "step_ms_percentiles": pct_ig,
            "kernels_ms": k_ig,
            "extra_algorithmic_flops": B * K * 2 * H * n_in + B * 2 * H * H,
            "step": f"{args.path} path with grad_x [B,K,n_in] and grad_h0 [B,H] also written"},
        "accumulate_mode": None if args.main_only else {
            "ms_per_step": ms_acc, "value": B * K / (ms_acc * 1e-3), "step_ms_percentiles": pct_acc,
            "kernels_ms": k_acc, "step": acc_step},
        "other_path": None if args.main_only else {
            "path": other, "value": B * K / (ms_other * 1e-3), "ms_per_step": ms_other, "kernels_ms": k_other},
        "reduce_axis0": {
            "standalone": None if args.no_reduce else reduce_standalone(torch, C, W, dev),
            "in_step": {"GB_per_s": red_gbps, "frac_hbm": red_gbps / PEAK_HBM_GBPS, "bytes": work["reduce_bytes"],
                        "note": "HIP events around the launch inside the step, breakdown pass (an empty launch "
                                "measures about 6 us this way); the step's scratch (%.1f MB) was just written, so "
                                "part of it may be served from the MALL" % (work["reduce_bytes"] / 1e6)}},
        "kernel_source_sha256_16": source_hash(),
    }
    if args.reduce_sweep:
        rec["reduce_axis0_sweep"] = reduce_sweep(torch, C, W, dev)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
