#!/usr/bin/env python3
"""Benchmark of the fused optimizer step on one MI355X.

Headline: AdamW over a Llama-7B-shaped list (290 tensors, 6,738,411,520
elements) with fp32 master weights, bf16 gradients and fp32 m/v -- one kernel
launch per step.  The other hot-path rows (8-bit blockwise AdamW on 2^30
elements, AdEMAMix on 2^28, AdamW with the max_unorm pre-pass on 2^28, BF16
nearest and stochastic rounding on 2^30) are measured the same way and listed
under "rows".  Inputs are synthetic (seeded), resident in HBM before timing.

Prints one JSON line.  `value` is optimizer-step throughput in Gelem/s; the
roofline object reports the achieved algorithmic HBM bandwidth of the step
kernel against the 8 TB/s peak, timed with HIP events on the launch stream.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0
METRIC = "optimizer-step Gelem/s and achieved HBM GB/s (% of MI355X peak), 1 GPU"
COUNTERS = os.path.join(ROOT, "profiles", "step_counters.json")
KERNEL_SOURCES = ["opt_kernels_ew.hip", "opt_elem.h", "opt_device.h", "opt_plan.h"]   # the headline kernel's


def kernel_hash():
    """Hash of the headline kernel's sources with comments and blank space
    taken out, so that the committed counters stay valid across edits to
    comments alone."""
    import re
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "optimizer_step_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def counter_traffic(workload, launches_elems):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_hash():
        return None
    w = c.get("workloads", {}).get(workload)
    if not w:
        return None
    return w.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# workloads on the device

def carve(torch, arrays, device):
    """One device allocation holding every per-element array of a workload
    (p, g, states, absmax), each starting on a 256-byte boundary; returns
    views.  Flat buffers like this are how training frameworks hold a bucket
    of parameters and optimizer states.  (Measured on MI355X: the step's
    bandwidth depends on where an allocation lands physically.  Eighteen
    14 GB arenas allocated in a row in one process ran the same 2^30-element
    step at 5.4 to 6.5 TB/s, each arena at its own steady rate, and the same
    virtual addresses in another process at other rates; DRAM-credit stall
    counters moved with the rate, translation misses did not.)"""
    sizes = {}
    off = 0
    for name, dtype, n in arrays:
        nbytes = n * torch.tensor([], dtype=dtype).element_size()
        sizes[name] = (off, dtype, n, nbytes)
        off += (nbytes + 255) // 256 * 256
    arena = torch.empty(max(off, 256), dtype=torch.uint8, device=device)
    return {name: arena[o:o + nb].view(dt) for name, (o, dt, n, nb) in sizes.items()}, arena


def build_workload(name, torch, osa, synth, share=None):
    """Allocate and fill one workload; returns (tensor list, fmt, opt, hp kwargs,
    elements, bytes per element, what to keep alive).  share: the tensor list
    of an already built workload over the same list (the gradient-norm and
    clipping rows step the headline's own buffers)."""
    w = synth.WORKLOADS[name]
    sizes = w["sizes"]
    total = sum(sizes)
    dev = torch.device("cuda")
    fmt = w["fmt"]
    opt = w["opt"]
    qs, qu = synth.codebook_signed(), synth.codebook_unsigned()
    p16 = w.get("p_dtype") == "bf16"
    bpe = synth.bytes_per_element(opt, fmt, w["grad_bf16"], p_bytes=2 if p16 else 4)
    if w.get("norm_only"):
        bpe = 2 if w["grad_bf16"] else 4
    elif w.get("clip"):
        bpe += 2 if w["grad_bf16"] else 4       # the norm reads g once more
    hp = dict(w["hp"])
    if share is not None:
        return share[0], fmt, opt, hp, total, bpe, share[1]
    nst = 3 if opt == "ademamix" else (2 if opt == "adamw" else 1)
    nb = (total + 255) // 256
    arrays = [("p", torch.bfloat16 if p16 else torch.float32, total),
              ("g", torch.bfloat16 if w["grad_bf16"] else torch.float32, total)]
    for i in range(1, nst + 1):
        if fmt == "f32":
            arrays.append((f"s{i}", torch.float32, total))
        elif fmt.startswith("bf16"):
            arrays.append((f"s{i}", torch.bfloat16, total))
        else:
            arrays.append((f"s{i}", torch.uint8, (total + 1) // 2 if fmt.startswith("fp4") else total))
            arrays.append((f"absmax{i}", torch.float32, nb))
    views, arena = carve(torch, arrays, dev)
    P, G = views["p"], views["g"]
    synth.device_normal_(P, synth.PARAM_SEED, w["p_std"])
    g_std = w["g_std"] if w["g_std"] != "decay" else 1e-2
    G.copy_(synth.device_grads(total, dev, g_std, 1, bf16=w["grad_bf16"], mask_scale=w.get("mask_scale")))
    torch.cuda.empty_cache()
    # fresh states: zeros; 8-bit codes at the code of 0 in each codebook
    fresh = osa.state_buffers(fmt, 1, opt, device=dev, qmap_signed=qs, qmap_unsigned=qu)
    states = {}
    for key in fresh:
        if key.startswith("absmax"):
            views[key].zero_()
        else:
            views[key].copy_(fresh[key][:1].expand(views[key].numel()))
        states[key] = views[key]
    tensors = []
    off = 0
    for n in sizes:
        d = {"p": P[off:off + n], "g": G[off:off + n]}
        for key, buf in states.items():
            if key.startswith("absmax"):
                continue
            d[key] = buf[off // 2:(off + n + 1) // 2] if fmt.startswith("fp4") else buf[off:off + n]
        if fmt in ("q8", "fp8_rn", "fp8_sr", "fp4_rn", "fp4_sr"):
            assert off % 256 == 0
            for key, buf in states.items():
                if key.startswith("absmax"):
                    d[key] = buf[off // 256:(off + n + 255) // 256]
        tensors.append(d)
        off += n
    keep = (arena, None, states, qs, qu)
    return tensors, fmt, opt, hp, total, bpe, keep


def _quantile(per, f):
    per = sorted(per)
    return per[min(len(per) - 1, int(f * (len(per) - 1) + 0.5))]


class Row:
    """One bench row resident on the device: its buffers, and one step of the
    row (gradient norm, update-norm pre-pass and step, as the row has them)
    enqueued on the current stream.  run() times steps with HIP events on
    that stream; the step count t keeps increasing across runs."""

    def __init__(self, name, torch, osa, synth, share=None):
        self.name, self.torch = name, torch
        w = synth.WORKLOADS[name]
        self.w = w
        self.t = 0
        self.stream = torch.cuda.current_stream()
        if w["opt"] == "cast":
            n = w["sizes"][0]
            self.x = torch.empty(n, dtype=torch.float32, device="cuda")
            synth.device_normal_(self.x, synth.PARAM_SEED, w["p_std"])
            self.out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
            sr = w["fmt"].endswith("sr")
            self.elements, self.tensors, self.bpe = n, 1, 6
            self.fmt, self.opt = ("bf16_sr" if sr else "bf16_rn"), "cast"
            self.one = lambda t: osa.opt_round_cast(self.x, self.out, sr, synth.SR_SEED, t, stream=self.stream)
            self.keep = None
            return
        tensors, fmt, opt, hp, total, bpe, keep = build_workload(name, torch, osa, synth, share)
        self.share = (tensors, keep)
        self.keep, self.fmt, self.opt, self.elements, self.tensors = keep, fmt, opt, total, len(tensors)
        qs, qu = keep[3], keep[4]
        tl = osa.TensorList(tensors)
        if opt in osa.ONE_STATE:
            step_fn = lambda tl_, fmt_, h_, un_, stream=None: osa.opt_step_1state(opt, tl_, fmt_, h_, stream=stream)
        else:
            step_fn = osa.opt_step_adamw if opt == "adamw" else osa.opt_step_ademamix
        unorm = None
        if hp.get("max_unorm", 0) > 0:
            unorm = torch.empty(2 * len(tensors), dtype=torch.float64, device="cuda")
        self.bpe = bpe + (16 if unorm is not None else 0)      # the pre-pass reads p, g, m, v once more
        clip = w.get("clip")
        grads = osa.GradList([d["g"] for d in tensors])
        gnorm = torch.empty(2 + 2 * len(tensors), dtype=torch.float64, device="cuda")
        coef = torch.empty(1, dtype=torch.float32, device="cuda")
        p_round = 1 if w.get("p_sr") else 0

        def one(t):
            if clip:
                osa.opt_grad_norm(grads, gnorm, clip[0], clip[1], coef, stream=self.stream)
                if w.get("norm_only"):
                    return
            h = osa.hparams(step=t, seed=synth.SR_SEED, qmap_signed=qs, qmap_unsigned=qu,
                            grad_scale=coef if clip else None, p_rounding=p_round, **hp)
            if unorm is not None:
                osa.opt_precondition_unorm(opt, tl, fmt, h, unorm, stream=self.stream)
            step_fn(tl, fmt, h, unorm, stream=self.stream)
        self.one = one
        self._hold = (tl, grads, gnorm, coef, unorm)

    def run(self, warmup, steps):
        torch = self.torch
        for _ in range(warmup):
            self.t += 1
            self.one(self.t)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        start_all = torch.cuda.Event(enable_timing=True)
        end_all = torch.cuda.Event(enable_timing=True)
        t_wall = time.perf_counter()
        start_all.record(self.stream)
        host = []
        for i in range(steps):
            self.t += 1
            ev[i][0].record(self.stream)
            h0 = time.perf_counter()
            self.one(self.t)
            host.append(time.perf_counter() - h0)
            ev[i][1].record(self.stream)
        end_all.record(self.stream)
        torch.cuda.synchronize()
        return {"samples_ms": [a.elapsed_time(b) for a, b in ev], "total_ms": start_all.elapsed_time(end_all),
                "wall_s": time.perf_counter() - t_wall, "host_s": host}

    def summary(self, runs):
        """Row record from one or more runs: every per-step sample, their mean
        (the launch time the roofline uses), median and p10/p90."""
        per = [x for r in runs for x in r["samples_ms"]]
        steps = len(per)
        launch_ms = sum(per) / steps
        ms = sum(r["total_ms"] for r in runs) / steps
        gbytes = self.bpe * self.elements / 1e9
        host = sorted(h for r in runs for h in r["host_s"])
        return {"workload": self.name, "format": "-" if self.w.get("norm_only") else self.fmt,
                "optimizer": "grad-norm" if self.w.get("norm_only") else
                             self.opt + ("+clip" if self.w.get("clip") else ""),
                "p_dtype": self.w.get("p_dtype", "f32") + ("-sr" if self.w.get("p_sr") else ""),
                "elements": self.elements, "tensors": self.tensors, "bytes_per_element": self.bpe,
                "steps": steps, "ms_per_step": ms, "ms_median": _quantile(per, 0.5),
                "ms_p10": _quantile(per, 0.1), "ms_p90": _quantile(per, 0.9),
                "gelem_per_s": self.elements / (ms * 1e-3) / 1e9,
                "achieved_GBps": gbytes / (launch_ms * 1e-3),
                "frac_of_peak": gbytes / (launch_ms * 1e-3) / PEAK_GBPS,
                "launch_ms": launch_ms,
                # host time to enqueue one step (binding + planning + launch),
                # which overlaps the previous step's kernels
                "host_us_median": host[len(host) // 2] * 1e6,
                "samples_ms": [round(x, 4) for x in per]}


def time_workload(name, steps, warmup, torch, osa, synth):
    """One row on its own: build, W warmup and K timed steps, free."""
    row = Row(name, torch, osa, synth)
    rec = row.summary([row.run(warmup, steps)])
    del row
    torch.cuda.empty_cache()
    return rec


def interleaved_rounds(rows, rounds, torch):
    """The measurement protocol of the issue 'Investigate SM103 bias-correction
    broadcast in 32-bit optimizers' (Benchmark): every row timed in each of
    `rounds` rounds, the rows interleaved within a round, all resident; per
    row every sample, the median and p10/p90 over all samples, and the median
    of each round."""
    per_row = {r.name: [] for r in rows}
    # untimed: every row once, then about 2 s of the first row, so that the
    # rounds start with the device at its working clocks (building the rows
    # leaves it idle for a while)
    for r in rows:
        r.run(1, 0)
    warm = rows[0].run(0, 3)
    k = max(1, int(2000.0 / max(1e-3, sum(warm["samples_ms"]) / 3)))
    rows[0].run(k, 0)
    for _ in range(rounds):
        for r in rows:
            big = r.elements * r.bpe > 50e9
            per_row[r.name].append(r.run(1 if big else 3, 4 if big else 10))
    out = []
    for r in rows:
        rec = r.summary(per_row[r.name])
        rec["round_medians_ms"] = [round(_quantile(x["samples_ms"], 0.5), 4) for x in per_row[r.name]]
        rec["rounds"] = rounds
        out.append(rec)
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the headline workload

_start_barrier = None


def _set_barrier(b):
    global _start_barrier
    _start_barrier = b
    import torch
    torch.set_num_threads(1)      # the inputs' BF16 cast, one thread per worker


def _oracle_steps(k, budget_s, n=1 << 24):
    """AdamW steps of the C oracle (fp32 p/m/v, bf16 g) over n elements of
    tensor k's synthetic inputs for about budget_s seconds: (steps, elements
    stepped, seconds).  Workers of a pool start timing together."""
    import oracle
    import synth
    p = synth.params(n, k)
    g = synth.grads(n, 1, k, std=1e-3, bf16=True)
    st = oracle.state_zeros("f32", n)
    if _start_barrier is not None:
        _start_barrier.wait(timeout=300)   # a lost worker fails the pool, not hangs it
    done = 0
    t = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        t += 1
        oracle.step("adamw", "f32", oracle.make_hp(lr=3e-4, weight_decay=0.1, step=t), p, g, **st)
        done += n
    return t, done, time.perf_counter() - t0


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(budget_s=12.0):
    """The oracle on the host: one process per core of this process's CPU
    share (at most 16), each on its own 2^24-element slice, then one process
    alone.  The workers are forked, so this runs before the process touches
    the GPU, and before it uses torch's CPU thread pool (the inputs' BF16
    cast), which a forked child could not use."""
    import multiprocessing
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    ctx = multiprocessing.get_context("fork")
    with ctx.Pool(workers, initializer=_set_barrier, initargs=(ctx.Barrier(workers),)) as pool:
        res = pool.starmap(_oracle_steps, [(k, budget_s) for k in range(workers)], chunksize=1)
    steps, done, dt = _oracle_steps(0, budget_s)
    single = done / dt / 1e9
    rate = sum(d / s for _, d, s in res) / 1e9          # the workers' intervals overlap
    return {"value": rate, "unit": "Gelem/s", "cores": workers, "kind": "oracle",
            "sample": f"AdamW (fp32 p/m/v, bf16 g) on 2^24-element slices of the Llama-7B-shaped list's "
                      f"synthetic inputs, C oracle: {workers} processes x ~{budget_s:.0f} s "
                      f"({sum(r[0] for r in res)} steps); one process alone: {steps} steps in {dt:.1f} s",
            "bytes_per_element": 26, "GBps": rate * 26, "cpu_model": _cpu_model(),
            "single_core": {"value": single, "unit": "Gelem/s", "cores": 1, "GBps": single * 26}}


def calibrate(torch, osa, n=1 << 30, reps=3):
    """The calibration copy: n fp32 read and n written per launch."""
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty(n, dtype=torch.float32, device="cuda")
    osa.opt_debug_stream([src], [dst])
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        osa.opt_debug_stream([src], [dst])
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    # the runtime's device-to-device copy of the same buffer, beside it
    dst.copy_(src)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms_d2d = a.elapsed_time(b) / reps
    return {"kernel": "debug_stream_kernel (1 read, 1 write)", "bytes_read": 4 * n, "bytes_written": 4 * n,
            "ms": ms, "GBps": 8 * n / ms / 1e6,
            "d2d_copy": {"how": "torch copy_ of the same fp32 buffer (device to device)", "ms": ms_d2d,
                         "GBps": 8 * n / ms_d2d / 1e6}}


# ---------------------------------------------------------------------------
# profile summaries (from rocprofv3 csv output)

HEADLINE_KERNEL = "step_ew_kernel<0, 1, 0, 0, true>"
CALIB_KERNEL = "debug_stream_kernel"


def summarize_profiles(trace_dir, fetch_dir, write_dir, cmd_trace, cmd_fetch, cmd_write):
    """Write profiles/step_ew_adamw_llama7b_{trace,counters}.txt and
    profiles/step_counters.json from the csv files of three rocprofv3 runs:
    --kernel-trace --stats, --pmc FETCH_SIZE and --pmc WRITE_SIZE (counter
    values are KiB per dispatch).  The calibration copy kernel moves a known
    number of bytes, and its counter readings give the scale factors."""
    import csv
    import glob
    import statistics

    def one(pattern):
        files = glob.glob(pattern, recursive=True)
        if not files:
            raise SystemExit(f"no file matches {pattern}")
        return files[0]

    stats = list(csv.DictReader(open(one(os.path.join(trace_dir, "**", "*kernel_stats.csv")))))
    head = [r for r in stats if HEADLINE_KERNEL in r["Name"]][0]
    calib = [r for r in stats if CALIB_KERNEL in r["Name"]]
    # the bench line the traced run printed, if kept next to the trace
    live = None
    for cand in glob.glob(os.path.join(trace_dir, "..", "trace_bench.json")):
        try:
            live = json.loads(open(cand).read().strip().splitlines()[-1])
        except (ValueError, IndexError):
            live = None

    def counters(d, name):
        rows = list(csv.DictReader(open(one(os.path.join(d, "**", "*counter_collection.csv")))))
        pick = lambda k: [float(r["Counter_Value"]) for r in rows if k in r["Kernel_Name"] and r["Counter_Name"] == name]
        return pick(HEADLINE_KERNEL), pick(CALIB_KERNEL)

    f_step, f_cal = counters(fetch_dir, "FETCH_SIZE")
    w_step, w_cal = counters(write_dir, "WRITE_SIZE")
    n_cal = 1 << 30
    cal_bytes = 4 * n_cal                      # read and also written per launch
    kib = 1024.0
    fetch_scale = cal_bytes / (statistics.median(f_cal) * kib)
    write_scale = cal_bytes / (statistics.median(w_cal) * kib)
    rd = statistics.median(f_step) * kib * fetch_scale
    wr = statistics.median(w_step) * kib * write_scale
    elems = sum(n for _, n in __import__("synth").llama7b_shapes())
    alg_r, alg_w = 14 * elems, 12 * elems
    avg_ms = float(head["AverageNs"]) / 1e6
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "step_ew_adamw_llama7b_trace.txt"), "w") as f:
        f.write("rocprofv3 kernel statistics: AdamW step over the Llama-7B-shaped list (290 tensors,\n"
                f"6,738,411,520 elements; fp32 p/m/v, bf16 g), and the calibration copy kernel if it ran.\n"
                f"command: {cmd_trace}\n\n")
        f.write(f"{'kernel':48s} {'calls':>6s} {'avg ms':>10s} {'min ms':>10s} {'max ms':>10s}\n")
        for r in [head] + calib:
            nm = HEADLINE_KERNEL if r is head else CALIB_KERNEL
            f.write(f"{nm:48s} {r['Calls']:>6s} {float(r['AverageNs'])/1e6:10.3f} "
                    f"{float(r['MinNs'])/1e6:10.3f} {float(r['MaxNs'])/1e6:10.3f}\n")
        f.write(f"\nstep kernel: {alg_r + alg_w:.4e} algorithmic bytes per launch / {avg_ms:.3f} ms = "
                f"{(alg_r + alg_w) / avg_ms / 1e6:.0f} GB/s ({(alg_r + alg_w) / avg_ms / 1e6 / PEAK_GBPS:.1%} of 8 TB/s)\n")
        if live is not None:
            lm = live["roofline"]["launch_ms"]
            f.write(f"the same run's bench line (HIP events on the launch stream, timed steps only): "
                    f"{lm:.3f} ms per launch, {live['roofline']['achieved']:.0f} GB/s, "
                    f"value {live['value']:.1f} Gelem/s\n")
    with open(os.path.join(ROOT, "profiles", "step_ew_adamw_llama7b_counters.txt"), "w") as f:
        f.write("rocprofv3 HBM byte counters (KiB per dispatch), one counter per run.\n"
                f"commands:\n  {cmd_fetch}\n  {cmd_write}\n\n")
        f.write(f"calibration copy (debug_stream_kernel, 2^30 fp32 read + written = {cal_bytes} B each way):\n"
                f"  FETCH_SIZE {statistics.median(f_cal):.1f} KiB -> scale {fetch_scale:.4f}\n"
                f"  WRITE_SIZE {statistics.median(w_cal):.1f} KiB -> scale {write_scale:.4f}\n")
        f.write(f"step kernel ({HEADLINE_KERNEL}), per launch:\n"
                f"  FETCH_SIZE {statistics.median(f_step):.1f} KiB x scale = {rd:.4e} B (algorithmic reads {alg_r:.4e} B, ratio {rd / alg_r:.4f})\n"
                f"  WRITE_SIZE {statistics.median(w_step):.1f} KiB x scale = {wr:.4e} B (algorithmic writes {alg_w:.4e} B, ratio {wr / alg_w:.4f})\n"
                f"  HBM traffic {rd + wr:.4e} B per launch vs {alg_r + alg_w:.4e} B algorithmic\n")
    summary = {"kernel_source_hash": kernel_hash(), "fetch_scale": fetch_scale, "write_scale": write_scale,
               "workloads": {"adamw_f32_llama7b": {"kernel": HEADLINE_KERNEL, "hbm_bytes_per_launch": rd + wr,
                                                   "read_bytes": rd, "write_bytes": wr,
                                                   "trace_avg_ms": avg_ms}},
               "commands": [cmd_trace, cmd_fetch, cmd_write]}
    with open(COUNTERS, "w") as f:
        json.dump(summary, f, indent=1)
    print(open(os.path.join(ROOT, "profiles", "step_ew_adamw_llama7b_counters.txt")).read())


OUR_KERNELS = ("step_", "gnorm_", "unorm_", "norm_group", "round_cast")


def summarize_rows_counters(base):
    """profiles/bench_rows_counters.txt: HBM bytes per step of each bench row
    from two rocprofv3 runs per row (--pmc FETCH_SIZE, then WRITE_SIZE; KiB
    per dispatch), scaled by the same run's calibration copy, against the
    row's algorithmic bytes per step.  A row's kernels are this library's
    kernels in its run (the rows run one per process), each dispatched once
    per step."""
    import csv
    import glob
    import statistics
    kib = 1024.0
    cal_bytes = 4.0 * (1 << 30)
    lines = []
    for rdir in sorted(glob.glob(os.path.join(base, "*", ""))):
        row = os.path.basename(os.path.normpath(rdir))
        try:
            info = json.loads(open(os.path.join(rdir, "bench.json")).read().strip().splitlines()[-1])["rows"][0]
        except (OSError, ValueError, IndexError, KeyError):
            continue
        per = {}
        for counter, sub_ in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
            files = glob.glob(os.path.join(rdir, sub_, "**", "*counter_collection.csv"), recursive=True)
            if not files:
                break
            vals = {}
            for r in csv.DictReader(open(files[0])):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"].replace("void ", "").replace("optstep::", "")
                name = name[:name.index(">(") + 1] if ">(" in name else name.split("(")[0]
                vals.setdefault(name, []).append(float(r["Counter_Value"]))
            cal = [v for k, v in vals.items() if CALIB_KERNEL in k]
            if not cal:
                break
            scale = cal_bytes / (statistics.median(cal[0]) * kib)
            per[counter] = {k: statistics.median(v) * kib * scale for k, v in vals.items()
                            if k.startswith(OUR_KERNELS)}
        if len(per) != 2:
            continue
        rd, wr = sum(per["FETCH_SIZE"].values()), sum(per["WRITE_SIZE"].values())
        alg = info["bytes_per_element"] * info["elements"]
        kernels = ", ".join(sorted(set(per["FETCH_SIZE"]) | set(per["WRITE_SIZE"])))
        lines.append((row, info["elements"], info["bytes_per_element"], alg, rd, wr, kernels))
    if not lines:
        raise SystemExit(f"no complete row under {base}")
    with open(os.path.join(ROOT, "profiles", "bench_rows_counters.txt"), "w") as f:
        f.write("rocprofv3 HBM byte counters per bench row: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each\n"
                "scaled by what it reads for the calibration copy in the same run (2^30 fp32 read + written),\n"
                "summed over this library's kernels of one step, against the row's algorithmic bytes per step.\n"
                f"commands, per row R (each a process of its own):\n"
                f"  rocprofv3 --pmc FETCH_SIZE --output-format csv -d {base}/R/fetch -o c -- python bench.py "
                "--rows-only --rows R --no-cpu --calibrate --steps 2 --warmup 1 > " f"{base}/R/bench.json\n"
                f"  rocprofv3 --pmc WRITE_SIZE --output-format csv -d {base}/R/write -o c -- python bench.py "
                "--rows-only --rows R --no-cpu --calibrate --steps 2 --warmup 1\n\n")
        f.write(f"{'row':26s} {'elements':>14s} {'B/elem':>8s} {'algorithmic':>12s} {'read':>12s} {'written':>12s} "
                f"{'ratio':>7s}  kernels\n")
        for row, n, bpe, alg, rd, wr, kernels in lines:
            f.write(f"{row:26s} {n:14,d} {bpe:8.4g} {alg:12.4e} {rd:12.4e} {wr:12.4e} {(rd + wr) / alg:7.4f}  "
                    f"{kernels}\n")
    print(f"wrote profiles/bench_rows_counters.txt ({len(lines)} rows)")


ACTIVITY_PASSES = {
    "A": "VALUBusy LDSBankConflict OccupancyPercent MemUnitStalled",
    "B": "SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_SALU SQ_WAVES SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR SQ_BUSY_CYCLES "
         "SQ_WAIT_INST_ANY GRBM_GUI_ACTIVE",
}


ACTIVITY_REGEX = "step_|gnorm_|round_cast|norm_group"


def summarize_rows_activity(base):
    """profiles/bench_rows_activity.txt: per bench row, what the step kernel
    keeps busy -- VALU issue (VALUBusy: share of the kernel's cycles the SIMDs
    issue vector ALU work), VALU instructions per element, LDS bank-conflict
    stall share, occupancy, memory-unit stall share -- from two rocprofv3
    counter passes per row (A and B), medians over the row's dispatches of
    its dominant kernel (the one the shader sequencers are busy longest in)."""
    import csv
    import glob
    import statistics
    lines = []
    for rdir in sorted(glob.glob(os.path.join(base, "*", ""))):
        row = os.path.basename(os.path.normpath(rdir))
        try:
            info = json.loads(open(os.path.join(rdir, "bench.json")).read().strip().splitlines()[-1])["rows"][0]
        except (OSError, ValueError, IndexError, KeyError):
            continue
        per = {}
        for p in ACTIVITY_PASSES:
            files = glob.glob(os.path.join(rdir, p, "**", "*counter_collection.csv"), recursive=True)
            if not files:
                break
            for r in csv.DictReader(open(files[0])):
                name = r["Kernel_Name"].replace("void ", "").replace("optstep::", "")
                if not name.startswith(OUR_KERNELS):
                    continue
                name = name[:name.index(">(") + 1] if ">(" in name else name.split("(")[0]
                per.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        need = ("VALUBusy", "SQ_INSTS_VALU", "SQ_WAVES", "SQ_BUSY_CYCLES")
        per = {k: v for k, v in per.items() if all(c in v for c in need)}
        if not per:
            continue
        # the row's dominant kernel: the one its SQs are busy longest in
        kname = max(per, key=lambda k: statistics.median(per[k]["SQ_BUSY_CYCLES"]))
        m = {c: statistics.median(v) for c, v in per[kname].items()}
        lines.append((row, kname, info["elements"], m))
    if not lines:
        raise SystemExit(f"no complete row under {base}")
    with open(os.path.join(ROOT, "profiles", "bench_rows_activity.txt"), "w") as f:
        f.write("rocprofv3 activity counters of each bench row's dominant kernel (medians over its dispatches).\n"
                "VALUBusy: % of the kernel's cycles the SIMDs spend issuing vector ALU work; VALU/elem: vector\n"
                "instructions (each for 64 lanes) x 64 / elements, i.e. per-element VALU work; LDSconfl: % of\n"
                "cycles LDS is stalled on bank conflicts; Occ: % of the maximum waves resident; MemStall: % of\n"
                "cycles the memory unit is stalled.\n"
                "commands, per row R (each a process of its own):\n")
        for p, ctr in ACTIVITY_PASSES.items():
            f.write(f"  rocprofv3 --pmc {ctr} --kernel-include-regex '{ACTIVITY_REGEX}' --output-format csv -d {base}/R/{p} -o c "
                    f"-- python bench.py --rows-only --rows R --no-cpu --steps 2 --warmup 1 > {base}/R/bench.json\n")
        f.write(f"\n{'row':24s} {'VALUBusy':>8s} {'VALU/elem':>9s} {'LDS/elem':>8s} {'LDSconfl':>8s} {'Occ':>6s} "
                f"{'MemStall':>8s}  kernel\n")
        for row, kname, n, m in lines:
            valu = m["SQ_INSTS_VALU"] * 64 / n
            lds = m.get("SQ_INSTS_LDS", 0.0) * 64 / n
            f.write(f"{row:24s} {m['VALUBusy']:8.1f} {valu:9.1f} {lds:8.2f} {m.get('LDSBankConflict', 0.0):8.2f} "
                    f"{m.get('OccupancyPercent', 0.0):6.1f} {m.get('MemUnitStalled', 0.0):8.2f}  {kname}\n")
    print(open(os.path.join(ROOT, "profiles", "bench_rows_activity.txt")).read())


def summarize_rows_trace(trace_dir, cmd):
    """profiles/bench_rows_kernel_stats.txt: per-kernel time statistics of a
    rocprofv3 --kernel-trace --stats run over every bench row."""
    import csv
    import glob
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = list(csv.DictReader(open(files[0])))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = os.path.join(ROOT, "profiles", "bench_rows_kernel_stats.txt")
    with open(out, "w") as f:
        f.write("rocprofv3 kernel statistics over every bench row (template arguments: optimizer\n"
                "0 AdamW 1 AdEMAMix 2 momentum 5 Lion; gradient 0 fp32 1 bf16 2 fp16; state format 0 fp32\n"
                "1 BF16-RN 2 BF16-SR 3 8-bit 4 FP8-RN 5 FP8-SR 6 FP4-RN 7 FP4-SR; parameter 0 fp32 1 bf16\n"
                "2 fp16; true: a call with no gradient scale, skip_zeros or state reset).\n"
                f"command: {cmd}\n\n")
        f.write(f"{'kernel':70s} {'calls':>6s} {'avg ms':>9s} {'min ms':>9s} {'max ms':>9s}\n")
        for r in rows:
            nm = r["Name"].replace("optstep::", "")
            nm = nm.split("(")[0] if len(nm) > 70 else nm
            f.write(f"{nm[:70]:70s} {r['Calls']:>6s} {float(r['AverageNs'])/1e6:9.3f} "
                    f"{float(r['MinNs'])/1e6:9.3f} {float(r['MaxNs'])/1e6:9.3f}\n")
    print(open(out).read())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the warmup also lets the device leave its idle clocks: on MI355X the
    # step runs about 2 % slower for the first 1-2 s of sustained load
    # (Llama-7B-shaped AdamW 28.01 ms per step in the first second, 27.38
    # from the second on); 100 steps of the headline take about 2.7 s
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--rows", default="all", help="'all', 'none', or comma-separated workload names")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    ap.add_argument("--calibrate", action="store_true",
                    help="with --rows-only: also run the plain copy kernel (2^30 fp32 read + written, 3 launches) "
                         "whose HBM counters scale the step kernels' (the default run always does)")
    ap.add_argument("--rounds", type=int, default=7,
                    help="interleaved rounds over every row, the headline included (after the headline's own "
                         "warmup + timed steps)")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ summaries from three rocprofv3 output folders and exit")
    ap.add_argument("--rows-only", action="store_true",
                    help="time only the rows given by --rows (no headline, no CPU leg) and print them as one "
                         "JSON line; for per-row profiling runs")
    ap.add_argument("--summarize-rows-counters", metavar="DIR",
                    help="write profiles/bench_rows_counters.txt from per-row rocprofv3 counter runs under DIR "
                         "(DIR/<row>/{fetch,write}/ and DIR/<row>/bench.json) and exit")
    ap.add_argument("--summarize-rows-activity", metavar="DIR",
                    help="write profiles/bench_rows_activity.txt from per-row rocprofv3 activity-counter runs under "
                         "DIR (DIR/<row>/{A,B}/ and DIR/<row>/bench.json) and exit")
    ap.add_argument("--summarize-rows-trace", metavar="TRACE_DIR",
                    help="write profiles/bench_rows_kernel_stats.txt from a rocprofv3 run over all rows and exit")
    args = ap.parse_args()

    # the commands the summaries record: the profiling runs that wrote the
    # folders given (the trace run's bench line sits beside its folder)
    def trace_cmd(d):
        line = os.path.join(os.path.dirname(os.path.normpath(d)), "trace_bench.json")
        return (f"rocprofv3 --kernel-trace --stats --output-format csv -d {d} -o trace -- "
                f"python bench.py --no-cpu > {line}")

    def pmc_cmd(counter, d, name):
        return (f"rocprofv3 --pmc {counter} --output-format csv -d {d} -o {name} -- "
                "python bench.py --rows none --no-cpu --calibrate --steps 2 --warmup 1")

    if args.summarize_rows_trace:
        summarize_rows_trace(args.summarize_rows_trace, trace_cmd(args.summarize_rows_trace))
        return
    if args.summarize_rows_counters:
        summarize_rows_counters(args.summarize_rows_counters)
        return
    if args.summarize_rows_activity:
        summarize_rows_activity(args.summarize_rows_activity)
        return
    if args.summarize_profiles:
        tdir, fdir, wdir = args.summarize_profiles
        summarize_profiles(tdir, fdir, wdir, cmd_trace=trace_cmd(tdir), cmd_fetch=pmc_cmd("FETCH_SIZE", fdir, "fetch"),
                           cmd_write=pmc_cmd("WRITE_SIZE", wdir, "write"))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the step is "
              "element-wise: each GPU would run this same launch on its own shard, with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    if args.rows_only:
        import torch
        import optimizer_step_amd as osa
        import synth
        osa.lib()
        rows = [time_workload(name, max(args.steps, 20), max(args.warmup, 5), torch, osa, synth)
                for name in (r for r in args.rows.split(",") if r and r not in ("all", "none"))]
        out = {"rows": rows}
        if args.calibrate:
            out["calibration"] = calibrate(torch, osa)
        print(json.dumps(out), flush=True)
        return

    # the CPU baseline first: its workers are forked, which must happen
    # before this process initialises the GPU
    cpu = None if args.no_cpu else cpu_baseline()
    if cpu is not None:
        print(f"[bench] CPU oracle: {cpu['value']:.3f} Gelem/s on {cpu['cores']} cores, "
              f"{cpu['single_core']['value']:.3f} on 1", file=sys.stderr, flush=True)

    import torch
    import optimizer_step_amd as osa
    import synth
    osa.lib()
    head = "adamw_f32_llama7b"
    print(f"[bench] headline {head}: {args.warmup} warmup + {args.steps} timed steps", file=sys.stderr, flush=True)
    head_row = Row(head, torch, osa, synth)
    main_row = head_row.summary([head_row.run(args.warmup, args.steps)])
    print(f"[bench] {head}: {main_row['gelem_per_s']:.1f} Gelem/s, {main_row['achieved_GBps']:.0f} GB/s",
          file=sys.stderr, flush=True)

    others = ["adamw_q8_1g", "ademamix_f32_268m", "adamw_f32_unorm_268m", "adamw_bf16_1g", "adamw_bf16_sr_1g",
              "adamw_bf16p_bf16_sr_1g", "adamw_bf16p_f32_1g",
              "adamw_fp8_rn_1g", "adamw_fp8_sr_1g", "adamw_fp4_rn_1g", "adamw_fp4_sr_1g",
              "gradnorm_bf16_llama7b", "adamw_f32_clip_llama7b", "momentum_f32_1g", "lion_f32_1g",
              "cast_bf16_sr_1g"]
    if args.rows == "none":
        others = []
    elif args.rows != "all":
        others = [r for r in args.rows.split(",") if r]
    # every row resident at once (about 210 GB of the 288 GB), the rows over
    # the Llama-shaped list on the headline's own buffers
    rows = [head_row]
    for name in others:
        share = head_row.share if synth.WORKLOADS[name]["sizes"] == synth.WORKLOADS[head]["sizes"] else None
        rows.append(Row(name, torch, osa, synth, share=share))
    calib = calibrate(torch, osa)
    print(f"[bench] calibration copy: {calib['GBps']:.0f} GB/s (runtime D2D copy {calib['d2d_copy']['GBps']:.0f}); "
          f"{args.rounds} interleaved rounds over "
          f"{len(rows)} rows", file=sys.stderr, flush=True)
    protocol = interleaved_rounds(rows, args.rounds, torch) if args.rounds > 0 else []
    for r in protocol:
        print(f"[bench] {r['workload']}: median {r['ms_median']:.3f} ms, {r['achieved_GBps']:.0f} GB/s "
              f"({r['frac_of_peak']:.1%}), round medians {r['round_medians_ms']}", file=sys.stderr, flush=True)
    cast = [r for r in rows if r.opt == "cast"]
    if cast:
        c = cast[0]
        torch_ms = torch_cast_ms(torch, c.x, 5, 20)
        for r in protocol:
            if r["workload"] == c.name:
                r["torch_nearest_cast_ms"] = torch_ms

    traffic = counter_traffic(head, main_row["elements"])
    gb_launch = main_row["bytes_per_element"] * main_row["elements"]
    head_rounds = protocol[0] if protocol else None
    out = {
        "metric": METRIC,
        "value": main_row["gelem_per_s"],
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_row["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "AdamW, Llama-7B-shaped list (290 tensors, 6,738,411,520 elements), "
                               "fp32 params, bf16 grads ~N(0,1e-3), fp32 m/v, lr 3e-4, wd 0.1",
                   "tensors": main_row["tensors"], "elements": main_row["elements"],
                   "launches_per_step": 1, "bytes_per_element": main_row["bytes_per_element"]},
        "roofline": {"bound": "hbm", "achieved": main_row["achieved_GBps"], "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": main_row["achieved_GBps"] / PEAK_GBPS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": gb_launch,
                     "kernel": "step_ew_kernel<AdamW, bf16 grad, fp32 states, fp32 params, plain>",
                     "launch_ms": main_row["launch_ms"]},
        "cpu_baseline": cpu,
        "gbps_achieved": main_row["achieved_GBps"],
        "frac_of_peak": main_row["frac_of_peak"],
        "ms_median": main_row["ms_median"], "ms_p10": main_row["ms_p10"], "ms_p90": main_row["ms_p90"],
        "samples_ms": main_row["samples_ms"],
        "headline_rounds": None if head_rounds is None else
            {k: head_rounds[k] for k in ("steps", "ms_median", "ms_p10", "ms_p90", "achieved_GBps",
                                         "frac_of_peak", "round_medians_ms", "rounds")},
        "calibration": calib,
        "rows": protocol[1:],
    }
    print(json.dumps(out), flush=True)


def torch_cast_ms(torch, x, warmup, steps):
    """torch's built-in nearest FP32 -> BF16 cast over the same array."""
    for _ in range(warmup):
        x.to(torch.bfloat16)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        x.to(torch.bfloat16)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


if __name__ == "__main__":
    main()
