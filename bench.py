"""Benchmark of the per-rank ZeRO-2 optimizer-shard step on one MI355X.

One step = one pass of the whole shard step over one batch of synthetic
gradients already resident in HBM: ring-order W-way fp32 sum, average,
unscale, overflow check, AdamW, cast into the gather buffer (the fused
kernel), then the commit or skip with its loss-scaler update on the device
(zs_step_device: the commit kernel), steps queued back to back. The same
step with the decision taken on the host (zs_step_commit: 4-byte flag
readback, scaler on the host, one wait per step) is reported beside it
under `host_commit`. Inputs come from the seeded generator, on the device.

Prints ONE JSON line (rank 0). `value` is parameters updated per second of
the chosen workload; the HBM side of the metric is in `hbm_gbps`,
`hbm_pct_of_peak` and `roofline`. `roofline.achieved` is the algorithmic
bytes of one fused launch ((2W + 12) read + 14 written per parameter, plus
4 read per parameter for an accumulated micro-batch input) divided by that
launch's average duration measured with HIP events on the launch stream.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload
on this host's cores. Beside the headline, on the same workload: the step
with its decision on the host (`host_commit`), with bf16 partial sums on
the ring (`wire_bf16`), the ZeRO-Offload variant (`offload`), and one full
ring all-gather of the 16-bit parameters over W replicas (`all_gather`).
`copy_ceiling_gbps` is the read + write rate of libzscopy's plain 4 GiB
copy timed in the same run (the fastest copy shape found on MI355X), and
`hbm_pct_of_copy_ceiling` the step's HBM rate against it; the runtime's
device-to-device memcpy is reported beside it (`memcpy_d2d_gbps`).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--workload NAME] [--also NAME,...] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E peak (vendor figure)
DEFAULT_WORKLOAD = "gpt2s-w8"   # GPT-2-small-shaped flat model, W = 8
DEFAULT_ALSO = "7p5b-shard-w64,7b-full-w1,1p3b-w4-acc4-fp16"
KERNEL_SRC = os.path.join(ROOT, "sharded_mixed_precision_zs_amd", "csrc", "zs_kernels.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_step_traffic.md")
ALL_GATHER_LARGE = "1p3b-w4-acc4-fp16"  # 4 replicas of 1.3e9 params: beyond any cache
EVENT_EVERY_MAX = 16   # at most one launch in 16 is bracketed by HIP events
EVENT_SAMPLES = 20     # ... and at least this many are, where the steps allow
METRIC = "params updated/sec per ZeRO-2 shard step + achieved HBM GB/s (% of peak)"


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


class HipEvents:
    """Raw hipEvent_t handles (libamdhip64 through ctypes). The library's
    zs_step_commit records them on the launch stream immediately before and
    after the fused kernel."""

    def __init__(self):
        import ctypes
        self.C = ctypes
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = self.C.c_void_p()
        if self.lib.hipEventCreate(self.C.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def elapsed_ms(self, start, stop):
        ms = self.C.c_float()
        if self.lib.hipEventElapsedTime(self.C.byref(ms), start, stop) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)


def kernel_source_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_traffic(workload):
    """HBM bytes per fused launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    m = re.search(rf"traffic_bytes_per_launch\[{re.escape(workload)}\]:\s*([0-9.eE+]+)", text)
    return float(m.group(1)) if m else None


def _time_copy(torch, copy, nbytes, reps):
    """Average ms of copy(src, dst) over `reps` calls between two 4-byte-
    aligned device buffers of nbytes, timed with events on the current
    stream after three untimed calls."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        copy(a, b)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        copy(a, b)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del a, b
    torch.cuda.empty_cache()
    return ms


def copy_rates_gbps(torch, gib=4, reps=10):
    """Read + write rate of two plain device copies of `gib` GiB: the copy
    kernel of libzscopy (16 bytes per lane, the shape that streamed fastest
    on MI355X: the practical ceiling) and the runtime's device-to-device
    memcpy (the copy the counter calibration uses)."""
    import ctypes
    from sharded_mixed_precision_zs_amd import build as pkg_build
    if not os.path.exists(pkg_build.COPY):
        raise RuntimeError(f"{pkg_build.COPY} is not built: run the package build first")
    lib = ctypes.CDLL(pkg_build.COPY)  # after torch: it shares torch's HIP runtime
    lib.zs_copy_ceiling.restype = ctypes.c_int
    lib.zs_copy_ceiling.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                    ctypes.c_void_p]
    lib.zs_copy_last_error.restype = ctypes.c_char_p
    nbytes = gib << 30

    def kernel_copy(a, b):
        rc = lib.zs_copy_ceiling(a.data_ptr(), b.data_ptr(), nbytes,
                                 torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"zs_copy_ceiling returned {rc}: "
                               f"{lib.zs_copy_last_error().decode()}")

    rates = {}
    for name, copy in (("ceiling", kernel_copy), ("memcpy", lambda a, b: b.copy_(a))):
        rates[name] = 2 * nbytes / (_time_copy(torch, copy, nbytes, reps) * 1e-3) / 1e9
    return rates


def pad_elems(n, align_bytes=256):
    """Row length (16-bit elements) rounded up to a multiple of align_bytes."""
    per = align_bytes // 2
    return -(-n // per) * per


def replicas_for(wl, bytes_per_step):
    """Independent shard copies cycled through so a step never finds its
    inputs in the 256 MB last-level cache (whole working set >= 1 GB)."""
    return max(1, min(8, -(-(1 << 30) // max(bytes_per_step, 1))))


def run_workload(name, steps, warmup, torch, wire=0, device_commit=True):
    from sharded_mixed_precision_zs_amd import shard, synth

    wl = synth.WORKLOADS[name]
    n, W, A = wl.n, wl.world, wl.accum
    rd, wr = wl.bytes_per_param()
    # bytes of the fused launch alone (the last micro-batch) and of the step
    fused_rd = 2 * W + 12 + (4 if A > 1 else 0)
    fused_bytes = (fused_rd + 14) * n
    step_bytes = (rd + wr) * n
    R = replicas_for(wl, step_bytes)
    log(f"{name}: n={n} W={W} A={A} replicas={R} step bytes={step_bytes / 1e9:.3f} GB")
    opt = shard.AdamW(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay)
    reps = []
    for r in range(R):
        st = shard.ShardState(n, W, wl.rank, wl.offset, wl.offset + n, wl.param_dtype,
                              wl.grad_dtype, opt, wl.loss_scale, dynamic=wl.dynamic_scale,
                              growth_interval=wl.scale_interval, accumulate=A > 1,
                              wire_dtype=wire, device_commit=device_commit)
        synth.dev_state(wl, wl.offset, st.master, st.m, st.v)
        # one row per worker, rows padded to 256 B like separate allocations
        grads = torch.empty((A, W, pad_elems(n)), dtype=torch.int16, device="cuda")
        views = [[grads[j, k, :n] for k in range(W)] for j in range(A)]
        for j in range(A):
            for k in range(W):
                synth.dev_grad(wl, k, 1 + r, j, wl.offset, views[j][k], scale=wl.loss_scale)
        reps.append((st, views))
    for st, g in reps:
        st.bind(g[A - 1], acc_in=st.acc if A > 1 else None)
    torch.cuda.synchronize()
    hip = HipEvents()

    def one_step(i, events=None):
        st, g = reps[i % R]
        for j in range(A - 1):
            st.reduce_micro(g[j], first=(j == 0))
        ev = events if events is not None else (None, None)
        if device_commit:
            st.step_device(ev_start=ev[0], ev_stop=ev[1])
            return 0
        return st.step(ev_start=ev[0], ev_stop=ev[1])

    def committed_so_far():
        return sum(int(st.sync_scaler().step_t) for st, _ in reps) if device_commit else 0

    for i in range(warmup):
        one_step(i)
    torch.cuda.synchronize()
    # HIP events bracket the fused kernel on every k-th timed step: each
    # record puts a gap of a few us between kernels, which the step time
    # would carry, so k is as large as EVENT_SAMPLES samples allow (up to 16)
    every = max(1, min(EVENT_EVERY_MAX, steps // EVENT_SAMPLES))
    timed = list(range(0, steps, every))
    evs = {i: (hip.create(), hip.create()) for i in timed}
    committed = -committed_so_far()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        committed += one_step(warmup + i, evs.get(i))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    committed += committed_so_far()
    kern_ms = [hip.elapsed_ms(*evs[i]) for i in timed]
    for s, e in evs.values():
        hip.destroy(s)
        hip.destroy(e)
    kern_avg = sum(kern_ms) / len(kern_ms)
    kern_med = sorted(kern_ms)[len(kern_ms) // 2]
    ms_per_step = elapsed * 1e3 / steps
    res = dict(workload=name, commit="device" if device_commit else "host", n=n, world=W,
               accum=A, replicas=R,
               ms_per_step=ms_per_step, params_per_s=n / (ms_per_step * 1e-3),
               step_bytes=step_bytes, hbm_gbps=step_bytes / (ms_per_step * 1e-3) / 1e9,
               fused_kernel_ms=kern_avg, fused_bytes=fused_bytes,
               fused_gbps=fused_bytes / (kern_avg * 1e-3) / 1e9, committed=committed,
               kernel_ms_min=min(kern_ms), kernel_ms_max=max(kern_ms),
               kernel_ms_median=kern_med, kernel_samples=len(kern_ms), event_every=every)
    del reps
    torch.cuda.empty_cache()
    return res


def run_offload(name, steps, warmup, torch):
    """The ZeRO-Offload variant on the same workload: the ring reduction on
    the GPU, the fp32 gradient to the host, AdamW + cast on the host cores,
    the 16-bit parameters back (reported beside the fused GPU step)."""
    from sharded_mixed_precision_zs_amd import shard, synth

    wl = synth.WORKLOADS[name]
    n, W, A = wl.n, wl.world, wl.accum
    threads = min(16, len(os.sched_getaffinity(0)))
    off = shard.OffloadShard(n, W, wl.rank, wl.offset, wl.offset + n, wl.param_dtype,
                             wl.grad_dtype, shard.AdamW(wl.lr, wl.beta1, wl.beta2, wl.eps,
                                                        wl.weight_decay),
                             wl.loss_scale, dynamic=wl.dynamic_scale,
                             growth_interval=wl.scale_interval, threads=threads)
    m = torch.empty(n, dtype=torch.float32, device="cuda")
    v = torch.empty(n, dtype=torch.float32, device="cuda")
    master = torch.empty(n, dtype=torch.float32, device="cuda")
    synth.dev_state(wl, wl.offset, master, m, v)
    off.master.copy_(master.cpu())
    off.m.copy_(m.cpu())
    off.v.copy_(v.cpu())
    del master, m, v
    grads = torch.empty((A, W, pad_elems(n)), dtype=torch.int16, device="cuda")
    views = [[grads[j, k, :n] for k in range(W)] for j in range(A)]
    for j in range(A):
        for k in range(W):
            synth.dev_grad(wl, k, 1, j, wl.offset, views[j][k], scale=wl.loss_scale)
    torch.cuda.synchronize()

    def one():
        for j in range(A - 1):
            off.reduce_micro(views[j], first=(j == 0))
        return off.step(views[A - 1], first=(A == 1))

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return dict(workload=name, params_per_s=n / (ms * 1e-3), ms_per_step=ms, host_threads=threads,
                pieces=off.pieces, pcie_bytes_per_step=6 * n, hbm_state_bytes_saved=12 * n)


def run_all_gather(name, reps, torch):
    """One full ring all-gather (W - 1 zs_all_gather_step calls) over W
    replicas of the workload's flat 16-bit parameter buffer on one GPU.
    Each step copies one chunk per replica: 2 bytes read and 2 written per
    element moved."""
    from sharded_mixed_precision_zs_amd import synth
    from sharded_mixed_precision_zs_amd import zeroshard as zs

    wl = synth.WORKLOADS[name]
    W, phi = wl.world, wl.phi
    chunk = -(-phi // W)
    row = pad_elems(phi)
    buf = torch.zeros((W, row), dtype=torch.int16, device="cuda")
    replicas = [buf[k, :phi] for k in range(W)]

    def gather():
        for step in range(1, W):
            zs.zs_all_gather_step(replicas, phi, step, sigma=0)

    gather()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        gather()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    moved = 4 * (W - 1) * sum(min(chunk, max(0, phi - c * chunk)) for c in range(W))
    del buf, replicas
    torch.cuda.empty_cache()
    gbps = moved / (ms * 1e-3) / 1e9
    # each step reads the chunks the step before wrote: 2*phi bytes over all
    # replicas, which the 256 MB last-level cache can hold for small models
    cached = 2 * phi <= (256 << 20)
    out = dict(workload=name, world=W, phi=phi, steps=W - 1, ms_per_gather=ms,
               bytes_per_gather=moved, gbps=gbps)
    if cached:
        out["note"] = (f"each step reads the chunks the step before wrote ({2 * phi / 1e6:.0f} MB "
                       "over all replicas, within the 256 MB last-level cache), so this is not "
                       "an HBM rate")
    else:
        out["roofline_frac"] = gbps / PEAK_HBM_GBPS
    return out


def cpu_model():
    """The host CPU's model string (Linux), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(name, target_s=25.0):
    """The CPU oracle (as it stands) on a bounded sample of the workload."""
    import numpy as np

    import oracle
    from sharded_mixed_precision_zs_amd import synth

    wl = synth.WORKLOADS[name]
    threads = min(16, len(os.sched_getaffinity(0)))
    kw = dict(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
              weight_decay=wl.weight_decay, loss_scale=wl.loss_scale, step_t=1)

    def timed(ns, reps, threads=threads):
        # distinct inputs for up to the workload's step count, then cycled
        distinct = []
        for r in range(min(reps, wl.steps)):
            micro = [[synth.host_grad(wl, k, 1 + r, j, wl.offset, ns) for k in range(wl.world)]
                     for j in range(wl.accum)]
            distinct.append(micro)
        master, m, v = synth.host_state(wl, wl.offset, ns)
        acc = np.empty(ns, np.float32) if wl.accum > 1 else None
        t0 = time.perf_counter()
        for r in range(reps):
            micro = distinct[r % len(distinct)]
            for j, parts in enumerate(micro[:-1]):
                oracle.reduce_avg(parts, wl.rank, wl.grad_dtype, acc, j > 0, wl.loss_scale)
            oracle.shard_step(micro[-1], wl.rank, wl.grad_dtype, wl.param_dtype, master, m, v,
                              acc_in=acc, threads=threads, **kw)
        return time.perf_counter() - t0

    probe = min(wl.n, 1 << 21)
    dt = timed(probe, 2) / 2
    # host memory bound on the sample: ~6 GB of generated inputs and state
    cap = (6 << 30) // (2 * wl.world * wl.accum + 30)
    want = int(probe * target_s / max(dt, 1e-6))
    ns = int(min(wl.n, cap, max(probe, want)))
    reps = max(1, min(1000, int(want // ns)))
    dt = timed(ns, reps)
    # one thread, on a smaller sample (about a third of the time budget)
    dt1 = timed(probe, 1, threads=1)
    reps1 = max(1, min(100, int(target_s / 3 / max(dt1, 1e-6))))
    dt1 = timed(probe, reps1, threads=1)
    return dict(value=ns * reps / dt, unit="params/s", cores=threads, kind="oracle",
                sample=f"{ns} params of the {name} rank-{wl.rank} partition (W={wl.world}, "
                       f"{wl.accum} micro-batch(es)) x {reps} step(s), {threads} threads, "
                       f"{dt:.1f} s",
                value_1_thread=probe * reps1 / dt1,
                sample_1_thread=f"{probe} params x {reps1} step(s), 1 thread, {dt1:.1f} s",
                cpu_model=cpu_model(), host_cpus_machine=os.cpu_count(),
                host_cpus_available=len(os.sched_getaffinity(0)))


def world_sweep(worlds, n, steps, warmup, torch):
    """The fused step at one shard size for several worker counts W: the
    read/write mix goes from 14:14 bytes per parameter (W = 1) to
    (2W + 12):14. Each W gets its own n (n + 4096 W), so a kernel trace of
    the sweep can be split by grid size. Returns one record per W."""
    import dataclasses

    from sharded_mixed_precision_zs_amd import synth

    out = []
    base = synth.WORKLOADS[DEFAULT_WORKLOAD]
    for w in worlds:
        nw = n + 4096 * w
        name = f"sweep-w{w}"
        synth.WORKLOADS[name] = dataclasses.replace(base, name=name, world=w, phi=w * nw,
                                                    description=f"world sweep, W={w}")
        r = run_workload(name, steps, warmup, torch)
        log(json.dumps(r))
        out.append(dict(world=w, n=nw, fused_kernel_ms=r["fused_kernel_ms"],
                        fused_gbps=r["fused_gbps"], roofline_frac=r["fused_gbps"] / PEAK_HBM_GBPS,
                        bytes_per_param_read=2 * w + 12, bytes_per_param_written=14,
                        ms_per_step=r["ms_per_step"]))
        del synth.WORKLOADS[name]
    return out


def side_leg(name, fn, torch):
    """Run a leg reported beside the headline; a failure (for instance too
    little free device memory for a 7B state) is recorded in the JSON line
    as {"error": ...} instead of taking the headline down with it."""
    try:
        return fn()
    except (RuntimeError, MemoryError, OSError, ValueError) as e:
        log(f"{name} failed: {type(e).__name__}: {e}")
        torch.cuda.empty_cache()
        return {"error": f"{type(e).__name__}: {e}"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1,
                    help="GPUs to use; only 1 is supported (one rank's shard on one MI355X)")
    ap.add_argument("--steps", type=int, default=320, help="timed steps of the headline workload")
    ap.add_argument("--warmup", type=int, default=5, help="untimed steps before the timed ones")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="headline workload (a key of synth.WORKLOADS)")
    ap.add_argument("--also", default=DEFAULT_ALSO,
                    help="comma-separated extra workloads reported under 'other_workloads'")
    ap.add_argument("--wire", choices=["fp32", "bf16", "fp16"], default="fp32",
                    help="precision of the ring's partial sums (default fp32)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the CPU oracle (cpu_baseline)")
    ap.add_argument("--no-offload", action="store_true",
                    help="skip the ZeRO-Offload (host update) leg")
    ap.add_argument("--no-copy-ceiling", action="store_true",
                    help="skip timing the plain copies (copy_ceiling_gbps, memcpy_d2d_gbps)")
    ap.add_argument("--sweep-world", default="",
                    help="comma-separated W values: time the fused step at one shard size for "
                         "each and print that table as the JSON line instead")
    ap.add_argument("--sweep-n", type=int, default=1 << 25,
                    help="shard size of the --sweep-world runs")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this benchmark runs on one GPU: the shard step takes one "
                          "rank's real share on one MI355X; multi-GPU runs are not part of it"}))
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    from sharded_mixed_precision_zs_amd import synth  # noqa: F401  (fails loudly if unbuilt)
    from sharded_mixed_precision_zs_amd import zeroshard  # noqa: F401

    if args.sweep_world:
        worlds = [int(x) for x in args.sweep_world.split(",") if x]
        sweep = world_sweep(worlds, args.sweep_n, args.steps, args.warmup, torch)
        print(json.dumps({"metric": "fused step HBM GB/s by worker count", "unit": "GB/s",
                          "peak": PEAK_HBM_GBPS, "sweep": sweep}))
        return
    copies = {} if args.no_copy_ceiling else side_leg("copy_ceiling",
                                                       lambda: copy_rates_gbps(torch), torch)
    if "error" in copies:
        copies = {}
    ceiling = copies.get("ceiling")
    if copies:
        log(f"plain copy ceiling {ceiling:.0f} GB/s; runtime memcpy {copies['memcpy']:.0f} GB/s")
    wire = {"fp32": 0, "bf16": 1, "fp16": 2}[args.wire]
    main_res = run_workload(args.workload, args.steps, args.warmup, torch, wire)
    log(json.dumps(main_res))
    host_res = run_workload(args.workload, args.steps, args.warmup, torch, wire,
                            device_commit=False)
    log(json.dumps(host_res))
    # the beyond-core legs on the same workload: the fused step with bf16
    # partial sums on the wire, and the ring all-gather of the parameters
    wire_bf16 = None
    if args.wire == "fp32":
        r = side_leg("wire_bf16", lambda: run_workload(args.workload, max(3, args.steps // 2), 2,
                                                        torch, 1), torch)
        log(json.dumps(r))
        wire_bf16 = r if "error" in r else dict(
            workload=args.workload, ms_per_step=r["ms_per_step"],
            params_per_s=r["params_per_s"], fused_kernel_ms=r["fused_kernel_ms"],
            fused_gbps=r["fused_gbps"], roofline_frac=r["fused_gbps"] / PEAK_HBM_GBPS)
    all_gather = []
    for name in dict.fromkeys([args.workload, ALL_GATHER_LARGE]):
        r = side_leg(f"all_gather {name}", lambda: run_all_gather(name, 10, torch), torch)
        log(json.dumps(r))
        all_gather.append(r if "error" not in r else dict(workload=name, error=r["error"]))
    # the host-side legs run before the large workloads, which churn
    # hundreds of GB of device memory
    offload = None
    if not args.no_offload:
        offload = side_leg("offload", lambda: run_offload(args.workload, max(10, args.steps // 2),
                                                          2, torch), torch)
        log(json.dumps(offload))
    cpu = None if args.no_cpu_baseline else side_leg("cpu_baseline",
                                                     lambda: cpu_baseline(args.workload), torch)
    others = []
    for name in [x for x in args.also.split(",") if x and x != args.workload]:
        r = side_leg(name, lambda: run_workload(name, max(3, args.steps // 2), 2, torch, wire),
                     torch)
        log(json.dumps(r))
        if "error" in r:
            others.append(dict(workload=name, error=r["error"]))
            continue
        others.append(dict(workload=name, params_per_s=r["params_per_s"],
                           ms_per_step=r["ms_per_step"], hbm_gbps=r["hbm_gbps"],
                           fused_kernel_ms=r["fused_kernel_ms"], fused_gbps=r["fused_gbps"],
                           roofline_frac=r["fused_gbps"] / PEAK_HBM_GBPS))

    from sharded_mixed_precision_zs_amd import synth as s
    wl = s.WORKLOADS[args.workload]
    traffic = recorded_traffic(args.workload)
    out = {
        "metric": METRIC,
        "value": main_res["params_per_s"],
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded counter-based generator, generated in HBM)",
        "config": {"workload": args.workload, "description": wl.description,
                   "phi": wl.phi, "world": wl.world, "rank": wl.rank, "shard_params": wl.n,
                   "grad_dtype": "bf16" if wl.grad_dtype == 0 else "fp16",
                   "param_dtype": "bf16" if wl.param_dtype == 0 else "fp16",
                   "micro_batches": wl.accum, "replicas": main_res["replicas"],
                   "wire": args.wire},
        "hbm_gbps": main_res["hbm_gbps"],
        "hbm_pct_of_peak": 100.0 * main_res["hbm_gbps"] / PEAK_HBM_GBPS,
        "copy_ceiling_gbps": ceiling,
        "memcpy_d2d_gbps": copies.get("memcpy"),
        "hbm_pct_of_copy_ceiling": 100.0 * main_res["hbm_gbps"] / ceiling if ceiling else None,
        "roofline": {"bound": "hbm", "achieved": main_res["fused_gbps"],
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": main_res["fused_gbps"] / PEAK_HBM_GBPS,
                     "traffic": traffic,
                     "kernel": "zs::fused_kernel", "kernel_ms": main_res["fused_kernel_ms"],
                     "kernel_ms_median": main_res["kernel_ms_median"],
                     "kernel_samples": main_res["kernel_samples"],
                     "event_every": main_res["event_every"],
                     "algorithmic_bytes_per_launch": main_res["fused_bytes"]},
        "cpu_baseline": cpu,
        "other_workloads": others,
        "host_commit": {"ms_per_step": host_res["ms_per_step"],
                        "params_per_s": host_res["params_per_s"],
                        "fused_kernel_ms": host_res["fused_kernel_ms"]},
        "offload": offload,
        "wire_bf16": wire_bf16,
        "all_gather": all_gather,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
