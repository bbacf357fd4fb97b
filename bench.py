"""Throughput of the fused, clipped, mixed-precision AdamW step on one GPU.

A step is one pass of the whole path over one shard, on one stream, inputs
resident in HBM.  By default it is one adamw_clipped_step call: a norm launch
(per-block partial sums of g^2), then the update launch, which finishes the
sum, forms the clip coefficient and updates (+ optional bf16 copy + step
counter).  --launches separate times grad_norm_sq (sum and clip coefficient
in one launch) followed by adamw_multi_tensor_step instead.  Prints ONE JSON
line: params updated per second (value), the step's algorithmic GB/s, and for
the dominant kernel (the update) its roofline against MI355X's 8 TB/s HBM
peak, timed live with events on the launch stream; plus the CPU oracle timed
on a bounded sample on the host (one thread, then all threads).

    python bench.py [--steps K] [--warmup W] [--config 3] [--rotate R] [--state8]

The default workload is the largest one that fits one GPU: the full
Llama-3.1-8B as a 291-tensor list (8,030,261,248 parameters, 128.5 GB of
state).  The line also carries, measured in the same process: a practical
ceiling for the update (a plain kernel with the update's exact streams and
trivial arithmetic, bench_ceiling.hip; a 2 GiB device copy beside it) and
the two-launch latency floor (the same call on a list whose one tensor is
empty: the two launches with no bytes to move).

Without --warmup the warm-up lasts at least 10 steps and 0.25 s: the GPU's
clock needs some tens of milliseconds of work to settle (an 8-bit step on
the 8B shard starts ~10 % slower than it runs after ~150 steps).  --state8
times the same workload with 8-bit moments: m and v are the workload's,
encoded once before the timed region.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBPS = 8000.0
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "mixed_precision_sharded_amd", "csrc")
# The sources each timed kernel is built from (its counter record is valid
# only for these exact sources).
KERNEL_SOURCES = {
    "adamw_step_kernel": ("kernels.hip", "device.h", "layout.h"),
    "adamw_clipped_kernel": ("kernels.hip", "device.h", "layout.h"),
    "adamw8_step_kernel": ("kernels_q8.hip", "device.h", "layout.h"),
    "adamw8_clipped_kernel": ("kernels_q8.hip", "device.h", "layout.h"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed warm-up steps (default: at least 10 and at least "
                        "--warmup-seconds of steps)")
    p.add_argument("--warmup-seconds", type=float, default=0.25,
                   help="with the default --warmup, warm up for at least this long: the "
                        "GPU's clock takes some tens of milliseconds of work to settle")
    p.add_argument("--config", type=int, default=3,
                   help="workload 1..5 (default 3: the full Llama-3.1-8B as a 291-tensor list, "
                        "the largest that fits one GPU)")
    p.add_argument("--ceiling-mib", type=int, default=2048,
                   help="size of the same-run copy's buffers, reported beside the same-stream "
                        "ceiling (0 = skip both ceilings)")
    p.add_argument("--rotate", type=int, default=1,
                   help="cycle over this many independent buffer sets (cache-cold small shards)")
    p.add_argument("--trials", type=int, default=5,
                   help="time the K steps this many times (the first is the reported value; "
                        "all give the p10 / median / p90 of ms per step)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="host time budget of each oracle baseline: one thread, then all "
                        "threads (0 = skip)")
    p.add_argument("--cpu-threads", type=int, default=0,
                   help="threads of the all-cores oracle baseline (default: the CPUs this "
                        "process may use, at most 16)")
    p.add_argument("--no-kernel-events", action="store_true")
    p.add_argument("--launches", choices=("separate", "clipped", "fused"), default="clipped",
                   help="separate: grad_norm_sq with the clip output, then "
                        "adamw_multi_tensor_step; clipped: adamw_clipped_step (the norm's "
                        "partials finished inside the update); fused: adamw_fused_step "
                        "(one cooperative launch)")
    p.add_argument("--fused", action="store_true", help="same as --launches fused")
    p.add_argument("--state8", action="store_true",
                   help="8-bit moment state (m: E4M3, v: E5M2, a scale byte per 32 elements)")
    p.add_argument("--no-placement-warmup", dest="placement_warmup", action="store_false",
                   help="time the inputs' first allocation only (by default it is timed, "
                        "released, the allocator cycled through 1.1 times the footprint, and "
                        "the inputs allocated again for the reported run)")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="after the measurement, run 5 plain device copies of this many MiB "
                        "(known bytes, to scale rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = p.parse_args()
    if args.fused:
        args.launches = "fused"
    return args


def kernel_source_digest(kernel):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(kernel, workload_name):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources; else None."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    rec = table.get(f"{kernel} {workload_name}")
    if not rec or rec.get("kernel_source_sha256") != kernel_source_digest(kernel):
        return None
    return rec.get("traffic_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py times one GPU's shard only: over several GPUs each rank runs the same "
              "step on its own shard, with one all-reduce of the 8-byte sum of squares "
              "between the norm and the clip, which the caller performs", file=sys.stderr)
        sys.exit(2)

    import torch

    from mixed_precision_sharded_amd import binding, synth
    from mixed_precision_sharded_amd.configs import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.lib()  # fails loudly if the HIP library is missing

    w = WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.state8 and args.launches == "fused":
        print("--state8 has no single-launch form", file=sys.stderr)
        sys.exit(2)
    log(f"workload {w.cfg} {w.name}: {w.numel:,} params in {w.n_tensors} tensors, "
        f"{'bf16' if w.grad_bf16 else 'fp32'} grads, copy={w.copy_bf16}, rotate={args.rotate}, "
        f"moments={'8-bit' if args.state8 else 'fp32'}")

    def make_sets():
        sets = []
        for r in range(args.rotate):
            cols = synth.workload_inputs(w, dev, cfg_key=w.cfg * 1000 + r if r else None)
            if args.state8:
                states = []
                for m, v in zip(cols["exp_avg"], cols["exp_avg_sq"]):
                    st = binding.zeros_q8_state(m.numel(), dev)
                    if m.numel():
                        binding.adamw8_quantize(m, binding.MPS_Q8_E4M3, st[0], st[1])
                        binding.adamw8_quantize(v, binding.MPS_Q8_E5M2, st[2], st[3])
                    states.append(st)
                torch.cuda.synchronize()
                cols["exp_avg"] = cols["exp_avg_sq"] = None  # only the 8-bit state stays resident
                cols["q8_state"] = states
                tl = binding.TensorList8(cols["master"], states, cols["grad"], cols["param_bf16"])
            else:
                tl = binding.TensorList(cols["master"], cols["exp_avg"], cols["exp_avg_sq"],
                                        cols["grad"], cols["param_bf16"])
            sets.append((cols, tl))
        torch.cuda.synchronize()
        return sets

    sets = make_sets()
    sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
    coef = torch.zeros(1, dtype=torch.float32, device=dev)
    step = torch.tensor([w.step - 1], dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    def one_step(tl, ev=None):
        if ev is not None:
            ev[0].record()
        if args.launches == "fused":
            binding.adamw_fused_step(tl, step, w.lr, w.beta1, w.beta2, w.eps, w.weight_decay,
                                     w.max_norm, sumsq_out=sumsq, coef_out=coef)
            if ev is not None:
                ev[1].record()
                ev[2].record()
            return
        if args.launches == "clipped":
            # Two launches inside one call; the library records ev[1] between them.
            fn = binding.adamw8_clipped_step if args.state8 else binding.adamw_clipped_step
            fn(tl, step, w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, w.max_norm,
               sumsq_out=sumsq, coef_out=coef, mid_event=None if ev is None else ev[1])
            if ev is not None:
                ev[2].record()
            return
        if args.state8:
            binding.adamw8_grad_norm_sq(tl, sumsq, w.max_norm, coef)
            if ev is not None:
                ev[1].record()
            binding.adamw8_multi_tensor_step(tl, coef, step, w.lr, w.beta1, w.beta2, w.eps,
                                             w.weight_decay)
            if ev is not None:
                ev[2].record()
            return
        binding.grad_norm_sq(tl, sumsq, w.max_norm, coef)  # norm + clip coefficient
        if ev is not None:
            ev[1].record()
        binding.adamw_multi_tensor_step(tl, coef, step, w.lr, w.beta1, w.beta2, w.eps,
                                        w.weight_decay)
        if ev is not None:
            ev[2].record()

    # The workload's first allocation in this process, timed, then released:
    # on a freshly started GPU the first allocation of a large footprint
    # streams several per cent slower than any later one (measured on the
    # 8B-parameter list: 5.49 TB/s for the update, steady for a minute, against
    # 5.94-6.04 TB/s once the allocator has been cycled), so the run below
    # first cycles the allocator through 1.1 times the footprint and then
    # allocates the inputs again.
    first_allocation = None
    if args.placement_warmup:
        first_allocation = time_first_allocation(args, w, sets, one_step, step, dev)
        footprint = torch.cuda.memory_allocated()
        for cols, tl in sets:
            tl.release()
        del sets, cols, tl
        torch.cuda.empty_cache()
        try:
            cycle = torch.empty(int(1.1 * footprint), dtype=torch.uint8, device=dev)
            cycle.fill_(1)
            torch.cuda.synchronize()
            del cycle
            log(f"allocator cycled through {1.1 * footprint / 2**30:.1f} GiB")
        except torch.cuda.OutOfMemoryError:
            log("no room to cycle the allocator through 1.1 times the footprint; skipped")
        torch.cuda.empty_cache()
        sets = make_sets()
        step.fill_(w.step - 1)
        torch.cuda.synchronize()
        log("inputs allocated again")

    # Warm-up: exactly --warmup steps if given, else at least 10 steps and at
    # least --warmup-seconds of them.
    warmup = 0
    t_warm = time.perf_counter()
    while True:
        if args.warmup is not None:
            if warmup >= args.warmup:
                break
        elif warmup >= 10 and warmup % 10 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t_warm >= args.warmup_seconds:
                break
        one_step(sets[warmup % len(sets)][1])
        warmup += 1
    torch.cuda.synchronize()

    # Timed region: K whole steps back to back.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        one_step(sets[i % len(sets)][1])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / args.steps

    # The same K steps timed again, for the spread between trials.
    trial_ms = [ms_per_step]
    for _ in range(args.trials - 1):
        torch.cuda.synchronize()
        start.record()
        for i in range(args.steps):
            one_step(sets[i % len(sets)][1])
        end.record()
        torch.cuda.synchronize()
        trial_ms.append(start.elapsed_time(end) / args.steps)
    trials = {"n": len(trial_ms), "ms_per_step": [round(x, 5) for x in trial_ms],
              **{k: round(v, 5) for k, v in zip(("p10", "median", "p90"),
                                                _quantiles(trial_ms, (10, 50, 90)))}}
    log("trials (us/step): " + ", ".join(f"{x * 1e3:.1f}" for x in trial_ms))

    # With rotating buffer sets, also the warm figure: K steps on one set.
    warm = None
    if len(sets) > 1:
        for _ in range(10):
            one_step(sets[0][1])
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            one_step(sets[0][1])
        end.record()
        torch.cuda.synchronize()
        warm_ms = start.elapsed_time(end) / args.steps
        warm = {"ms_per_step": round(warm_ms, 5),
                "params_per_s": w.numel / (warm_ms * 1e-3),
                "what": "the same K steps on one buffer set (its data stays in the caches)"}
        log(f"warm, one buffer set: {warm_ms * 1e3:.1f} us/step")

    # Per-kernel durations: the same K steps again with events between the
    # launches, on the stream the kernels run on.
    kern_us = None
    spread = None
    if not args.no_kernel_events:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for e in evs:
            e[1].record()  # creates the event the library records between its launches
        torch.cuda.synchronize()
        for i in range(args.steps):
            one_step(sets[i % len(sets)][1], evs[i])
        torch.cuda.synchronize()
        norm_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
        upd_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
        per_step = sorted(e[0].elapsed_time(e[2]) * 1e3 for e in evs)
        spread = {f"p{q}": round(per_step[min(len(per_step) - 1, int(q / 100 * len(per_step)))], 2)
                  for q in (10, 50, 90)}
        if args.launches == "fused":
            kern_us = {"adamw_fused_step": norm_ms * 1e3}
        elif args.launches == "clipped":
            kern_us = {"grad_norm partials": norm_ms * 1e3, "clipped update": upd_ms * 1e3}
        elif args.state8:
            kern_us = {"adamw8_grad_norm_sq+clip": norm_ms * 1e3,
                       "adamw8_multi_tensor_step": upd_ms * 1e3}
        else:
            kern_us = {"grad_norm_sq+clip": norm_ms * 1e3, "adamw_multi_tensor_step": upd_ms * 1e3}

    n = w.numel
    bytes_per_param = w.algorithmic8_bytes_per_param() if args.state8 else w.algorithmic_bytes_per_param()
    step_bytes = bytes_per_param * n
    params_per_s = n / (ms_per_step * 1e-3)
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    log(f"{ms_per_step * 1e3:.1f} us/step, {params_per_s:.3e} params/s, {step_gbps:.0f} GB/s "
        f"algorithmic ({step_gbps / HBM_PEAK_GBPS:.1%} of 8 TB/s); host wall {wall:.3f} s")

    roofline = None
    if kern_us is not None:
        if args.launches == "fused":  # one kernel does the whole step
            name, launch_bytes, us = "adamw_fused_kernel", step_bytes, kern_us["adamw_fused_step"]
        elif args.launches == "clipped" and args.state8:
            name, launch_bytes = "adamw8_clipped_kernel", w.update8_bytes_per_param() * n
            us = kern_us["clipped update"]
        elif args.launches == "clipped":
            name, launch_bytes = "adamw_clipped_kernel", w.update_bytes_per_param() * n
            us = kern_us["clipped update"]
        elif args.state8:
            name, launch_bytes = "adamw8_step_kernel", w.update8_bytes_per_param() * n
            us = kern_us["adamw8_multi_tensor_step"]
        else:
            name, launch_bytes = "adamw_step_kernel", w.update_bytes_per_param() * n
            us = kern_us["adamw_multi_tensor_step"]
        achieved = launch_bytes / (us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "kernel": name,
                    "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": (stored_traffic(name, w.name) if name in KERNEL_SOURCES
                                else None),
                    "algorithmic_bytes_per_launch": launch_bytes,
                    "avg_launch_us": round(us, 2)}
        log(f"kernels (us): " + ", ".join(f"{k} {v:.1f}" for k, v in kern_us.items()))

    floor = None if args.no_kernel_events else latency_floor(args, dev)
    if roofline is not None and args.ceiling_mib > 0:
        ceiling = same_stream_ceiling8(w, dev) if args.state8 else same_stream_ceiling(w, dev)
        ceiling["copy"] = copy_ceiling(args.ceiling_mib, dev)
        roofline["ceiling"] = ceiling
        roofline["frac_of_ceiling"] = round(roofline["achieved"] / ceiling["achieved"], 4)

    if args.copy_calibration_mib > 0:
        n_f32 = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n_f32, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 5 copies of {args.copy_calibration_mib} MiB")
        del src, dst

    cpu = None
    if args.cpu_seconds > 0:
        threads = args.cpu_threads or min(16, len(os.sched_getaffinity(0)))
        cpu = (cpu_baseline8(w, sets[0][0], args.cpu_seconds, threads) if args.state8
               else cpu_baseline(w, sets[0][0], args.cpu_seconds, threads))

    out = {
        "metric": "params updated/sec and achieved HBM GB/s (fraction of peak) per AdamW step",
        "value": params_per_s,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "params": n, "tensors": w.n_tensors,
                   "grad_dtype": "bf16" if w.grad_bf16 else "f32", "bf16_copy": w.copy_bf16,
                   "step": w.step, "algorithmic_bytes_per_param": bytes_per_param,
                   "moments": "8-bit (m E4M3, v E5M2, scale byte per 32)" if args.state8 else "f32",
                   "buffer_sets": args.rotate, "launches": args.launches,
                   "parallelism": "one GPU's shard"},
        "step_gbps": round(step_gbps, 1),
        "step_frac_of_peak": round(step_gbps / HBM_PEAK_GBPS, 4),
        "kernel_us": kern_us,
        "step_us_spread": spread,
        "trials": trials,
        "warm_same_buffers": warm,
        "roofline": roofline,
        "latency_floor": floor,
        "first_allocation": first_allocation,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


CEILING_LIB = os.path.join(ROOT, "bench_ceiling.so")
CEILING_ELEMS = 1 << 28


def time_first_allocation(args, w, sets, one_step, step, dev):
    """The workload's K steps on the inputs' first allocation in this process
    (after its own warm-up of W steps), with the update's event time."""
    import torch

    for i in range(args.warmup if args.warmup is not None else 10):
        one_step(sets[i % len(sets)][1])
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in evs:
        e[1].record()
    torch.cuda.synchronize()
    for i in range(args.steps):
        one_step(sets[i % len(sets)][1], evs[i])
    torch.cuda.synchronize()
    ms = sum(e[0].elapsed_time(e[2]) for e in evs) / args.steps
    upd_us = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps * 1e3
    log(f"first allocation: {ms * 1e3:.1f} us/step, update {upd_us:.1f} us")
    return {"ms_per_step": round(ms, 5), "params_per_s": w.numel / (ms * 1e-3),
            "update_us": round(upd_us, 2),
            "what": "the same K steps on the inputs' first allocation in this process, before "
                    "the allocator was cycled (a fresh GPU's first large allocation streams "
                    "slower); value is the run after it"}


def same_stream_ceiling(w, dev, n=CEILING_ELEMS):
    """The update's streams without its arithmetic (bench_ceiling.hip): a
    plain grid-stride kernel reading and writing fp32 master, m and v,
    reading the workload's gradient type and writing the bf16 copy where the
    workload has one, over fresh buffers of n elements (2^28: 4 to 4.3 GB,
    far beyond the caches), timed on the same GPU in the same process.  The
    best of four launch shapes; the GB/s count the same bytes per element as
    the update's roofline."""
    import ctypes

    import torch

    if not os.path.exists(CEILING_LIB):
        raise RuntimeError(f"{CEILING_LIB} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(CEILING_LIB)
    fn = lib.stream_ceiling_us
    fn.restype = ctypes.c_double
    P = ctypes.c_void_p
    fn.argtypes = [ctypes.c_int, P, P, P, P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                   ctypes.c_int, P]
    bufs = [torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(3)]
    g = torch.zeros(n, dtype=torch.bfloat16 if w.grad_bf16 else torch.float32, device=dev)
    p = torch.zeros(n, dtype=torch.bfloat16, device=dev) if w.copy_bf16 else None
    stream = torch.cuda.current_stream().cuda_stream
    bytes_per_elem = w.update_bytes_per_param()
    shapes = {}
    for grid, unroll in ((256, 1), (256, 2), (1280, 1), (1024, 2)):
        us = fn(1 if w.grad_bf16 else 0, *(b.data_ptr() for b in bufs), g.data_ptr(),
                None if p is None else p.data_ptr(), n, grid, unroll, 10, stream)
        if us <= 0:
            raise RuntimeError(f"stream_ceiling_us failed ({us})")
        shapes[f"{grid} blocks x {unroll} group(s) of 4"] = round(bytes_per_elem * n / us / 1e3, 1)
    del bufs, g, p
    torch.cuda.empty_cache()
    best = max(shapes, key=shapes.get)
    log(f"same-stream ceiling: {shapes[best]:.0f} GB/s ({best}); all: {shapes}")
    return {"achieved": shapes[best], "unit": "GB/s", "frac": round(shapes[best] / HBM_PEAK_GBPS, 4),
            "what": f"plain kernel with the update's streams ({bytes_per_elem} B per element, "
                    f"{'bf16' if w.grad_bf16 else 'fp32'} gradient{', bf16 copy' if w.copy_bf16 else ''}), "
                    f"trivial arithmetic, {n:,} elements, best launch shape of 4, same process",
            "shapes": shapes}


def same_stream_ceiling8(w, dev, n=CEILING_ELEMS):
    """The 8-bit-moment update's streams without its arithmetic
    (bench_ceiling.hip's stream_ceiling8_us): fp32 master, m and v codes
    read and written, one scale byte per 32 elements read (cached) and
    written per chunk, the workload's gradient read and its bf16 copy
    written, over fresh buffers of n elements; the best of four grids, GB/s
    by the update's own bytes per element."""
    import ctypes

    import torch

    if not os.path.exists(CEILING_LIB):
        raise RuntimeError(f"{CEILING_LIB} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(CEILING_LIB)
    fn = lib.stream_ceiling8_us
    fn.restype = ctypes.c_double
    P = ctypes.c_void_p
    fn.argtypes = [ctypes.c_int, P, P, P, P, P, P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, P]
    master = torch.zeros(n, dtype=torch.float32, device=dev)
    g = torch.zeros(n, dtype=torch.bfloat16 if w.grad_bf16 else torch.float32, device=dev)
    p = torch.zeros(n, dtype=torch.bfloat16, device=dev) if w.copy_bf16 else None
    codes = [torch.zeros(n, dtype=torch.uint8, device=dev) for _ in range(2)]
    scales = [torch.zeros(n // 32, dtype=torch.uint8, device=dev) for _ in range(2)]
    stream = torch.cuda.current_stream().cuda_stream
    bytes_per_elem = w.update8_bytes_per_param()
    shapes = {}
    for grid in (256, 768, 1280, 2048):
        us = fn(1 if w.grad_bf16 else 0, master.data_ptr(), g.data_ptr(),
                None if p is None else p.data_ptr(), codes[0].data_ptr(), scales[0].data_ptr(),
                codes[1].data_ptr(), scales[1].data_ptr(), n, grid, 10, stream)
        if us <= 0:
            raise RuntimeError(f"stream_ceiling8_us failed ({us})")
        shapes[f"{grid} blocks"] = round(bytes_per_elem * n / us / 1e3, 1)
    del master, g, p, codes, scales
    torch.cuda.empty_cache()
    best = max(shapes, key=shapes.get)
    log(f"same-stream ceiling (8-bit moments): {shapes[best]:.0f} GB/s ({best}); all: {shapes}")
    return {"achieved": shapes[best], "unit": "GB/s", "frac": round(shapes[best] / HBM_PEAK_GBPS, 4),
            "what": f"plain kernel with the 8-bit update's streams ({bytes_per_elem} B per element, "
                    f"{'bf16' if w.grad_bf16 else 'fp32'} gradient{', bf16 copy' if w.copy_bf16 else ''}, "
                    f"m and v codes and scale bytes), trivial arithmetic, {n:,} elements, best grid of "
                    f"4, same process",
            "shapes": shapes}


def copy_ceiling(mib, dev, reps=10):
    """A plain device-to-device copy of `mib` MiB (torch's copy kernel), timed
    with events on the current stream after two warm-ups: read + write bytes
    over the average time.  The practical bound of a stream that reads and
    writes the same number of bytes, measured beside the step on the same GPU
    in the same process."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    gbps = 2 * n * 4 / (us * 1e-6) / 1e9
    log(f"copy ceiling: {mib} MiB in {us:.1f} us, {gbps:.0f} GB/s")
    return {"achieved": round(gbps, 1), "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "what": f"device copy of {mib} MiB (torch), read + write bytes / time, mean of {reps}"}


def latency_floor(args, dev, steps=200):
    """The same call as a step, on a list whose one tensor is empty: the two
    launches (or one, or three calls) and their dependencies with no bytes to
    move.  No step on any list can take less."""
    import torch

    from mixed_precision_sharded_amd import binding

    e = torch.empty(0, dtype=torch.float32, device=dev)
    g = torch.empty(0, dtype=torch.bfloat16, device=dev)
    sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
    coef = torch.zeros(1, dtype=torch.float32, device=dev)
    step = torch.zeros(1, dtype=torch.int32, device=dev)
    if args.state8:
        z = torch.empty(0, dtype=torch.uint8, device=dev)
        tl = binding.TensorList8([e], [(z, z, z, z)], [g])
    else:
        tl = binding.TensorList([e], [e], [e], [g])

    def one():
        if args.launches == "fused" and not args.state8:
            binding.adamw_fused_step(tl, step, 3e-4, 0.9, 0.95, 1e-8, 0.1, 1.0, sumsq_out=sumsq,
                                     coef_out=coef)
        elif args.launches == "clipped":
            fn = binding.adamw8_clipped_step if args.state8 else binding.adamw_clipped_step
            fn(tl, step, 3e-4, 0.9, 0.95, 1e-8, 0.1, 1.0, sumsq_out=sumsq, coef_out=coef)
        elif args.state8:
            binding.adamw8_grad_norm_sq(tl, sumsq, 1.0, coef)
            binding.adamw8_multi_tensor_step(tl, coef, step, 3e-4, 0.9, 0.95, 1e-8, 0.1)
        else:
            binding.grad_norm_sq(tl, sumsq, 1.0, coef)
            binding.adamw_multi_tensor_step(tl, coef, step, 3e-4, 0.9, 0.95, 1e-8, 0.1)

    for _ in range(20):
        one()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        one()
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / steps
    tl.release()
    log(f"latency floor: {us:.1f} us per step on an empty list")
    return {"us_per_step": round(us, 2),
            "what": f"the same call on a list of one empty tensor, {steps} steps back to back "
                    "(launches and their dependencies, no bytes)"}


CPU_SAMPLE_MAX_ELEMS = 64 << 20


def _quantiles(xs, qs):
    xs = sorted(xs)
    return [xs[min(len(xs) - 1, int(q / 100 * len(xs)))] for q in qs]


def _slices(n, parts, align=1):
    """Bounds of `parts` contiguous slices of n elements, each starting at a
    multiple of `align` (empty slices dropped)."""
    cuts = [min(n, (n * k // parts) // align * align) for k in range(parts)] + [n]
    return [(a, b) for a, b in zip(cuts, cuts[1:]) if b > a]


def _time_steps(step, budget_s):
    """Calls step(i) for i = 0, 1, ... until budget_s has passed."""
    steps = 0
    t0 = time.perf_counter()
    while True:
        step(steps)
        steps += 1
        if time.perf_counter() - t0 >= budget_s:
            return steps, time.perf_counter() - t0


def _threads_timing(parts, norm_part, update_part, clip, budget_s):
    """Whole steps with the sample cut into parts, one per thread: the norm
    of each part, the sum of the partial sums, the clip, the update of each
    part.  The oracle's C functions run outside the interpreter lock."""
    from concurrent.futures import ThreadPoolExecutor

    with ThreadPoolExecutor(max_workers=len(parts)) as pool:
        def step(i):
            S = sum(pool.map(norm_part, parts))
            c = clip(S)
            list(pool.map(lambda part: update_part(part, c, i), parts))
        return _time_steps(step, budget_s)


def cpu_baseline(w, cols, budget_s, threads):
    """The oracle, untuned, on the host: whole steps (norm, clip, update) over
    a bounded sample of the workload — its first tensors, at most
    CPU_SAMPLE_MAX_ELEMS elements (the whole shard when it is smaller) —
    repeated until the time budget is spent, on one thread; then the same
    sample on `threads` threads, each running the same oracle functions on
    its own slice of every tensor.  Scaled to params/s."""
    import oracle
    from mixed_precision_sharded_amd.synth import to_numpy

    o = oracle.default()
    host = {k: [] for k in cols}
    taken = 0
    for i in range(w.n_tensors):
        n = min(w.tensors[i][1], CPU_SAMPLE_MAX_ELEMS - taken)
        if n <= 0:
            break
        for k in cols:
            t = cols[k][i]
            host[k].append(None if t is None else to_numpy(t[:n]).copy())
        taken += n
    n_tensors = len(host["master"])

    def update(i, lo, hi, c, t):
        p = host["param_bf16"][i]
        o.adamw_step(host["master"][i][lo:hi], host["exp_avg"][i][lo:hi],
                     host["exp_avg_sq"][i][lo:hi], host["grad"][i][lo:hi],
                     None if p is None else p[lo:hi], c, t, w.lr, w.beta1, w.beta2, w.eps,
                     w.weight_decay)

    def one_thread(k):
        S = o.grad_norm_sq(host["grad"])
        c = o.clip_coef(S, w.max_norm)
        for i in range(n_tensors):
            update(i, 0, host["master"][i].size, c, w.step + k)

    steps, dt = _time_steps(one_thread, budget_s)
    t_next = w.step + steps
    what = _sample_name(w, n_tensors, taken)
    log(f"cpu oracle: {steps} steps of {taken:,} params in {dt:.2f} s, 1 thread")

    # Thread k takes slice k of every tensor.
    parts = [[] for _ in range(threads)]
    for i in range(n_tensors):
        for k, (lo, hi) in enumerate(_slices(host["master"][i].size, threads)):
            parts[k].append((i, lo, hi))
    parts = [p for p in parts if p]
    steps_t, dt_t = _threads_timing(
        parts, lambda part: o.grad_norm_sq([host["grad"][i][lo:hi] for i, lo, hi in part]),
        lambda part, c, k: [update(i, lo, hi, c, t_next + k) for i, lo, hi in part],
        lambda S: o.clip_coef(S, w.max_norm), budget_s)
    log(f"cpu oracle: {steps_t} steps of {taken:,} params in {dt_t:.2f} s, {len(parts)} threads")
    return {"value": taken * steps / dt, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"{what}: norm + clip + update, {steps} consecutive "
                      f"steps, 1 thread, {dt:.1f} s",
            "all_cores": {"value": taken * steps_t / dt_t, "unit": "params/s",
                          "cores": len(parts),
                          "sample": f"the same sample, {steps_t} consecutive steps, each "
                                    f"tensor cut into {len(parts)} slices, one thread per "
                                    f"slice, partial sums added, {dt_t:.1f} s"},
            "host_cpu": _cpu_model(), "host_nproc": os.cpu_count()}


CPU_SAMPLE_MAX_ELEMS_Q8 = 2 << 20


def cpu_baseline8(w, cols, budget_s, threads):
    """The oracle's 8-bit-moment step, as cpu_baseline, on the first tensors
    of the workload up to CPU_SAMPLE_MAX_ELEMS_Q8 elements (its nearest-code
    search is much slower per element than the fp32 update); the threaded
    run cuts every tensor at multiples of the 32-element scale runs."""
    import oracle
    from mixed_precision_sharded_amd.synth import to_numpy

    o = oracle.default()
    host = []
    taken = 0
    for i in range(w.n_tensors):
        n = min(w.tensors[i][1], CPU_SAMPLE_MAX_ELEMS_Q8 - taken)
        if n <= 0:
            break
        nb = (n + 31) // 32
        mc, ms, vc, vs = cols["q8_state"][i]
        p = cols["param_bf16"][i]
        host.append(dict(w=to_numpy(cols["master"][i][:n]).copy(), g=to_numpy(cols["grad"][i][:n]).copy(),
                         mc=mc[:n].cpu().numpy().copy(), ms=ms[:nb].cpu().numpy().copy(),
                         vc=vc[:n].cpu().numpy().copy(), vs=vs[:nb].cpu().numpy().copy(),
                         p=None if p is None else to_numpy(p[:n]).copy()))
        taken += n

    def update(h, lo, hi, c, t):
        r0, r1 = lo // 32, (hi + 31) // 32
        o.adamw8_step(h["w"][lo:hi], h["mc"][lo:hi], h["ms"][r0:r1], h["vc"][lo:hi],
                      h["vs"][r0:r1], h["g"][lo:hi], None if h["p"] is None else h["p"][lo:hi],
                      c, t, w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)

    def one_thread(k):
        S = o.grad_norm_sq([h["g"] for h in host])
        c = o.clip_coef(S, w.max_norm)
        for h in host:
            update(h, 0, h["w"].size, c, w.step + k)

    steps, dt = _time_steps(one_thread, budget_s)
    t_next = w.step + steps
    what = _sample_name(w, len(host), taken)
    log(f"cpu oracle (8-bit moments): {steps} steps of {taken:,} params in {dt:.2f} s, 1 thread")

    parts = [[] for _ in range(threads)]
    for h in host:
        for k, (lo, hi) in enumerate(_slices(h["w"].size, threads, align=32)):
            parts[k].append((h, lo, hi))
    parts = [p for p in parts if p]
    steps_t, dt_t = _threads_timing(
        parts, lambda part: o.grad_norm_sq([h["g"][lo:hi] for h, lo, hi in part]),
        lambda part, c, k: [update(h, lo, hi, c, t_next + k) for h, lo, hi in part],
        lambda S: o.clip_coef(S, w.max_norm), budget_s)
    log(f"cpu oracle (8-bit moments): {steps_t} steps of {taken:,} params in {dt_t:.2f} s, "
        f"{len(parts)} threads")
    return {"value": taken * steps / dt, "unit": "params/s", "cores": 1, "kind": "oracle",
            "sample": f"{what}: norm + clip + 8-bit-moment update, "
                      f"{steps} consecutive steps, 1 thread, {dt:.1f} s",
            "all_cores": {"value": taken * steps_t / dt_t, "unit": "params/s",
                          "cores": len(parts),
                          "sample": f"the same sample, {steps_t} consecutive steps, each "
                                    f"tensor cut at 32-element runs into {len(parts)} slices, "
                                    f"one thread per slice, partial sums added, {dt_t:.1f} s"},
            "host_cpu": _cpu_model(), "host_nproc": os.cpu_count()}


def _sample_name(w, n_tensors, taken):
    """What a CPU sample of `taken` leading parameters (over `n_tensors`
    tensors in list order) covers."""
    if taken == w.numel:
        return f"the whole {w.name} shard ({taken:,} params)"
    cut = sum(n for _, n in w.tensors[:n_tensors]) > taken
    last = (f"; tensor {n_tensors - 1} ({w.tensors[n_tensors - 1][0]}) cut after "
            f"{taken - sum(n for _, n in w.tensors[:n_tensors - 1]):,} of its "
            f"{w.tensors[n_tensors - 1][1]:,}") if cut else ""
    return (f"the first {taken:,} of {w.numel:,} params of {w.name} in list order "
            f"({n_tensors} tensor{'s' if n_tensors > 1 else ''}{last})")


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
