"""Benchmark of the per-rank ZeRO-2 optimizer-shard step on one MI355X.

One step = one pass of the whole shard step over one batch of synthetic
gradients already resident in HBM: ring-order W-way fp32 sum, average,
unscale, overflow check, AdamW, cast into the gather buffer (the fused
kernel), then the commit or skip with its loss-scaler update on the device
(zs_step_device: the commit kernel), steps queued back to back. Inputs come
from the seeded generator, on the device.

The headline workload is the 7B model's full state on one rank (W = 1,
7e9 parameters, 196 GB moved per step); the 7.5B model's rank-0 shard at
W = 64 and the other workloads are reported in the same line, each with its
own roofline object (`roofline_by_workload`).

Prints ONE JSON line. `value` is parameters updated per second of the
headline workload: n / (wall time of K steps queued back to back, with no
timing events among them) -- `ms_per_step`. `roofline.achieved` is the
algorithmic bytes of one fused launch ((2W + 12) read + 14 written per
parameter, plus 4 read per parameter for an accumulated micro-batch input)
divided by that launch's average duration, measured with HIP events that the
library records on the launch stream right around the kernel, in a second
pass of K steps. `roofline.traffic` is the HBM bytes per launch from the
committed rocprofv3 request-counter passes (profiles/fused_step_traffic.md),
when they were taken on the current kernel source. `ceilings` are the rates
of libzscopy's measurement kernels in the same run: a plain copy, read-only
and write-only streams, and the step's own mix of streams with no arithmetic
(the wave probe, in the fused kernel's launch shapes).
`read_write_harmonic_gbps` combines the headline step's read-only and
write-only stream rates at its read:write bytes; `stream_bounds` does the
same for the W = 64 shard and sets each fused rate against it and against
the no-arithmetic mix. `cpu_baseline` times the CPU oracle on a bounded
sample of the headline workload on this host's cores.

Beside the headline: the step with its decision on the host (`host_commit`),
with bf16 partial sums on the ring (`wire_bf16`, on the W = 64 shard), the
W = 64 shard with libzeroshard's write windows switched off
(`write_windows_off`), the ZeRO-Offload variant (`offload`), and a full ring
all-gather of the 16-bit parameters over W replicas (`all_gather`).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--also NAME,...] [--no-cpu-baseline] [--no-ceilings] ...
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

PEAK_HBM_GBPS = 8000.0           # MI355X HBM3E peak (vendor figure)
DEFAULT_WORKLOAD = "7b-full-w1"  # the 7B model's full state on one rank, W = 1
DEFAULT_ALSO = "7p5b-shard-w64,1p3b-w4-acc4-fp16,gpt2s-w8,mlp9-w3"
WIRE_WORKLOAD = "7p5b-shard-w64"       # the bf16-wire leg: the most partial sums
WINDOW_WORKLOAD = "7p5b-shard-w64"     # the same step timed without write windows
HOST_LEG_WORKLOAD = "gpt2s-w8"         # the ZeRO-Offload leg (host memory bound)
ALL_GATHER_WORKLOADS = ("1p3b-w4-acc4-fp16", "gpt2s-w8")
KERNEL_SRC = os.path.join(ROOT, "sharded_mixed_precision_zs_amd", "csrc", "zs_kernels.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_step_traffic.md")
CPU_WINDOW = 1 << 26     # oracle window for workloads too large for host memory
METRIC = "params updated/sec per ZeRO-2 shard step + achieved HBM GB/s (% of peak)"


def log(msg):
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def kernel_source_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_traffic(workload, kernel=None):
    """HBM bytes per fused launch of `workload` from the committed rocprofv3
    request-counter summary, if it was taken on the current kernel source
    and (when `kernel` is given) on that kernel instance; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    if kernel is not None:
        row = re.search(rf"^\| `([^`]+)` \({re.escape(workload)}\) \|", text, re.M)
        if not row or row.group(1) != kernel:
            return None
    m = re.search(rf"traffic_bytes_per_launch\[{re.escape(workload)}\]:\s*([0-9.eE+]+)", text)
    return float(m.group(1)) if m else None


def fused_bytes_per_param(world, accum):
    """Algorithmic (read, write) bytes per parameter of one fused launch."""
    return 2 * world + 12 + (4 if accum > 1 else 0), 14


FUSED_MANY_TILES = 20000   # 2048-element tiles
# fp32 state layout of every ShardState the benchmark builds ("split": master,
# m and v as three arrays; "grouped": one array of 1024-element groups of
# each); --state-layout sets it
STATE_LAYOUT = "grouped"


# write windows of the grouped rolling shape (libzeroshard's policy):
# W >= 40 and at least 4 GB of model bytes per launch, a 30.72 us period
# with its last eighth open for stores; ZS_FUSED_WRITE_WINDOW overrides it
WINDOW_WORLD, WINDOW_BYTES = 40, 4e9
WINDOW_PERIOD_US, WINDOW_OPEN = 30.72, 0.125


def write_window_of(world, n, accum=1, state_layout="grouped"):
    """{period_us, open_fraction} of the write windows libzeroshard uses
    for a 16-byte-aligned shard of n parameters over `world` workers (either
    state layout), or None."""
    if world < 5:
        return None
    env = os.environ.get("ZS_FUSED_WRITE_WINDOW", "")
    if env == "off":
        return None
    if env:
        period, frac = (float(x) for x in env.split(","))
        return {"period_us": period, "open_fraction": frac}
    rd, wr = fused_bytes_per_param(world, accum)
    if world < WINDOW_WORLD or (rd + wr) * n < WINDOW_BYTES:
        return None
    return {"period_us": WINDOW_PERIOD_US, "open_fraction": WINDOW_OPEN}


def fused_shape(world, n, state_layout="split"):
    """(threads per block, vectors per thread, zs::kShape* access shape,
    blocks per CU; 0 = no cap) of the fused kernel that zs_step_fused
    launches for a 16-byte-aligned shard of n parameters over `world`
    workers: 4-element vectors, non-temporal state loads and stores.
    Split state: 256-thread blocks with two vectors per thread at W = 3 (3
    or 4 per CU by the shard's size), one-wave blocks otherwise: one vector
    at 12 per CU for W = 1 and 16 for W = 2, then as the grouped state from
    W = 4 on. Grouped state: one-wave blocks throughout; one
    vector per thread at 12 blocks per CU for W = 1 and 16 for W = 2, 3;
    two from W = 4 on: the batched sum at 12 per CU for W = 4, the rolling
    sum (shape 6) at 8 per CU up to W = 12 and 6 beyond, uncapped when the
    launch takes write windows."""
    if state_layout == "grouped":
        if world == 1:
            return 64, 1, 5, 12
        if world <= 3:
            return 64, 1, 5, 16
        if world == 4:
            return 64, 2, 5, 12
        if write_window_of(world, n) is not None:
            return 64, 2, 6, 0
        return 64, 2, 6, 8 if world <= 12 else 6
    if world == 1:
        return (256, 2, 5, 2) if os.environ.get("ZS_FUSED_W1") == "block256" else (64, 1, 5, 12)
    if world == 2:
        return 64, 1, 5, 16
    if world == 3:
        return 256, 2, 5, 3 if n // 2048 >= FUSED_MANY_TILES else 4
    if world == 4:
        return 64, 2, 5, 12
    if write_window_of(world, n) is not None:
        return 64, 2, 6, 0
    return 64, 2, 6, 8 if world <= 12 else 6


def fused_instance(wl, wire=0, state_layout="split"):
    """Template instance of zs::fused_kernel that a 16-byte-aligned shard of
    this workload launches (the name rocprofv3 shows)."""
    t, u, shape, _ = fused_shape(wl.world, wl.n, state_layout)
    return (f"zs::fused_kernel<4, {u}, {str(wl.world > 1).lower()}, "
            f"{str(wl.accum > 1).lower()}, {wl.grad_dtype}, {wl.param_dtype}, {wire}, {shape}, "
            f"{t}, {str(state_layout == 'grouped').lower()}>")


def timing_events(torch, count):
    """`count` pairs of timing events, each recorded once so that its raw
    hipEvent_t exists (the library re-records it around the kernel)."""
    pairs = []
    for _ in range(count):
        pair = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        for ev in pair:
            ev.record()
        pairs.append(pair)
    torch.cuda.synchronize()
    return pairs


# ---- ceilings: libzscopy's measurement kernels -------------------------------

def _copylib():
    import ctypes as C
    from sharded_mixed_precision_zs_amd import build as pkg_build
    if not os.path.exists(pkg_build.COPY):
        raise RuntimeError(f"{pkg_build.COPY} is not built: run the package build first")
    lib = C.CDLL(pkg_build.COPY)
    lib.zs_copy_ceiling.restype = C.c_int
    lib.zs_copy_ceiling.argtypes = [C.c_void_p, C.c_void_p, C.c_uint64, C.c_void_p]
    lib.zs_copy_last_error.restype = C.c_char_p
    lib.zs_copy_shape.restype = C.c_int
    lib.zs_copy_shape.argtypes = [C.c_int, C.c_void_p, C.c_void_p, C.c_uint64, C.c_uint32,
                                  C.c_void_p]
    lib.zs_copy_shape_name.restype = C.c_char_p
    lib.zs_copy_shape_tile_bytes.restype = C.c_uint64
    lib.zs_stream_probe.restype = C.c_int
    lib.zs_stream_probe.argtypes = [C.c_void_p, C.c_uint32, C.c_void_p, C.c_uint32, C.c_void_p,
                                    C.c_uint32, C.c_void_p, C.c_uint64, C.c_uint32, C.c_uint32,
                                    C.c_void_p, C.c_uint32, C.c_void_p]
    lib.zs_wave_probe.restype = C.c_int
    lib.zs_wave_probe.argtypes = [C.c_void_p, C.c_uint32, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_uint64, C.c_uint32, C.c_uint32, C.c_double, C.c_double,
                                  C.c_void_p, C.c_uint32, C.c_void_p]
    return lib


def _time_calls(torch, fn, reps, warm=2):
    """Average ms of fn() over `reps` calls on the current stream, timed with
    events after `warm` untimed calls."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def copy_rates_gbps(torch, gib=4, reps=10):
    """Read + write rate of two plain device copies of `gib` GiB: libzscopy's
    copy kernel (16 bytes per lane, the copy shape that streamed fastest on
    MI355X) and the runtime's device-to-device memcpy."""
    lib = _copylib()
    nbytes = gib << 30
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)

    def kernel_copy():
        rc = lib.zs_copy_ceiling(a.data_ptr(), b.data_ptr(), nbytes,
                                 torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"zs_copy_ceiling returned {rc}: "
                               f"{lib.zs_copy_last_error().decode()}")

    rates = {name: 2 * nbytes / (_time_calls(torch, fn, reps) * 1e-3) / 1e9
             for name, fn in (("ceiling", kernel_copy), ("memcpy", lambda: b.copy_(a)))}
    del a, b
    torch.cuda.empty_cache()
    return rates


COPY_SWEEP_CAPS = (0, 2, 4)            # one tile per block: residency caps (0: none)
COPY_SWEEP_PERSISTENT = (2, 4, 8)      # persistent grids: blocks per CU


def copy_shape_sweep(torch, gib=4, reps=10, rounds=3):
    """Read + write rate of every copy shape of libzscopy over `gib` GiB,
    interleaved over `rounds`: shapes with one tile per block at each cap
    of COPY_SWEEP_CAPS, persistent shapes at each grid of
    COPY_SWEEP_PERSISTENT. Bytes are checked once per configuration."""
    lib = _copylib()
    nbytes = gib << 30
    a = torch.randint(-(1 << 31), 1 << 31, (nbytes // 4,), dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    configs = []
    for i in range(lib.zs_copy_shape_count()):
        name = lib.zs_copy_shape_name(i).decode()
        for k in (COPY_SWEEP_PERSISTENT if "persistent" in name else COPY_SWEEP_CAPS):
            configs.append((i, name, k))

    def runner(i, k):
        def go():
            rc = lib.zs_copy_shape(i, a.data_ptr(), b.data_ptr(), nbytes, k,
                                   torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"zs_copy_shape({i}) returned {rc}: "
                                   f"{lib.zs_copy_last_error().decode()}")
        return go

    for i, name, k in configs:
        b.zero_()
        runner(i, k)()
        torch.cuda.synchronize()
        if not torch.equal(a, b):
            raise RuntimeError(f"copy shape {name} (blocks per CU {k}) did not copy exactly")
    times = {c: [] for c in range(len(configs))}
    for _ in range(rounds):
        for c, (i, _, k) in enumerate(configs):
            times[c].append(_time_calls(torch, runner(i, k), reps))
    out = []
    for c, (i, name, k) in enumerate(configs):
        ms = sum(times[c]) / rounds
        gbps = 2 * nbytes / (ms * 1e-3) / 1e9
        out.append(dict(shape=i, name=name, blocks_per_cu=k, ms=ms, ms_rounds=times[c],
                        gbps=gbps, frac_of_peak=gbps / PEAK_HBM_GBPS))
        log(f"copy shape {name} k={k}: {ms:.4f} ms ({gbps:.0f} GB/s)")
    del a, b
    torch.cuda.empty_cache()
    return dict(bytes_each_way=nbytes, reps_per_round=reps, rounds=rounds, results=out)


# (name, 16-bit input streams, grouped fp32 state read, state written,
#  16-bit output, vectors per thread, blocks per CU (0: no cap), write
#  windows, shard size): the wave probe in the fused kernel's launch shapes
#  (W = 1: one vector per thread, 12 blocks per CU; W = 64: two, no cap and
#  the write windows, or its best cap without them)
N_W1 = 1 << 30                 # 1 G parameters: 28 GB for the W = 1 mix
N_W64 = 117_186_560            # the 7.5B shard rounded down to the 4096-element tile
WINDOW_W64 = (WINDOW_PERIOD_US, WINDOW_OPEN)
PROBES = (
    ("step_mix_w1", 1, True, True, True, 1, 12, None, N_W1),
    ("read_only_w1_streams", 1, True, False, False, 1, 12, None, N_W1),
    ("write_only_w1_streams", 0, False, True, True, 1, 12, None, N_W1),
    ("step_mix_w64", 64, True, True, True, 2, 0, WINDOW_W64, N_W64),
    ("step_mix_w64_no_windows", 64, True, True, True, 2, 6, None, N_W64),
    ("read_only_w64_streams", 64, True, False, False, 2, 0, None, N_W64),
    ("read_only_w64_grads", 64, False, False, False, 2, 0, None, N_W64),
    ("write_only_w64_streams", 0, False, True, True, 2, 0, None, N_W64),
    ("w64_grads_plus_param_store", 64, False, False, True, 2, 0, None, N_W64),
)


# per shard size: the probes of its streams read alone, written alone, and
# all of them in the fused kernel's launch shape
BOUND_PROBES = {
    1: ("read_only_w1_streams", "write_only_w1_streams", "step_mix_w1"),
    64: ("read_only_w64_streams", "write_only_w64_streams", "step_mix_w64"),
}


def stream_bounds(ceilings, roofs):
    """For each measured workload whose streams the probes carry (W = 1 and
    W = 64): the time its reads alone plus its writes alone take (the two
    phases back to back, no read/write turnaround in between) as a rate,
    and the fused kernel's rate against that and against the probe of the
    same mix in the same launch shape."""
    from sharded_mixed_precision_zs_amd import synth
    out = {}
    for name, roof in roofs.items():
        wl = synth.WORKLOADS.get(name)
        names = BOUND_PROBES.get(wl.world) if wl is not None and wl.accum == 1 else None
        if not names or not all(k in ceilings for k in names) or not roof:
            continue
        rd, wr = fused_bytes_per_param(wl.world, wl.accum)
        r_alone, w_alone, mix = (ceilings[k]["gbps"] for k in names)
        phased = (rd + wr) / (rd / r_alone + wr / w_alone)
        out[name] = dict(read_only_gbps=r_alone, write_only_gbps=w_alone,
                         phased_gbps=phased, phased_frac_of_peak=phased / PEAK_HBM_GBPS,
                         no_arithmetic_mix_gbps=mix, fused_gbps=roof["achieved"],
                         fused_pct_of_phased=100.0 * roof["achieved"] / phased,
                         fused_pct_of_no_arithmetic_mix=100.0 * roof["achieved"] / mix,
                         probes=list(names))
    return out


def stream_ceilings(torch, reps=8, names=None):
    """Rates of the wave probe in the shapes above: for each, HBM bytes per
    launch (2 per element of each 16-bit stream, 12 per element of the state
    read or written) over the average launch time. step_mix_w1 and
    step_mix_w64 carry the fused step's own streams in its own launch shape
    (residency cap, write windows), with integer folds in place of the
    arithmetic."""
    import ctypes as C
    lib = _copylib()
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    out = {}
    for name, w, sin, sout, p16, vecs, cap, window, n in PROBES:
        if names is not None and name not in names:
            continue
        row = -(-n // 128) * 128
        g = torch.empty((max(w, 1), row), dtype=torch.int16, device="cuda").random_()
        st_in = torch.empty(3 * n, dtype=torch.int32, device="cuda").random_() if sin else None
        st_out = torch.empty(3 * n, dtype=torch.int32, device="cuda") if sout else None
        o16 = torch.empty(n, dtype=torch.int16, device="cuda") if p16 else None
        gp = (C.c_void_p * 64)(*[g[k].data_ptr() for k in range(w)])
        period, share = window or (0.0, 0.0)

        def launch():
            rc = lib.zs_wave_probe(gp, w, st_in.data_ptr() if sin else None,
                                   st_out.data_ptr() if sout else None,
                                   o16.data_ptr() if p16 else None, n, vecs, cap, period, share,
                                   sink.data_ptr(), 0x6D2B79F5,
                                   torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"zs_wave_probe({name}) returned {rc}: "
                                   f"{lib.zs_copy_last_error().decode()}")

        ms = _time_calls(torch, launch, reps)
        rd, wr = 2 * w + (12 if sin else 0), (12 if sout else 0) + (2 if p16 else 0)
        gbps = (rd + wr) * n / (ms * 1e-3) / 1e9
        out[name] = dict(gbps=gbps, frac_of_peak=gbps / PEAK_HBM_GBPS, ms=ms, n=n,
                         read_bytes_per_param=rd, write_bytes_per_param=wr,
                         blocks_per_cu=cap or None,
                         write_window=(dict(period_us=period, open_fraction=share)
                                       if window else None),
                         kernel=f"wave_probe<{vecs}, {str(sin).lower()}, {str(sout).lower()}, "
                                f"{str(p16).lower()}>")
        log(f"ceiling {name}: {gbps:.0f} GB/s ({ms:.3f} ms)")
        del g, st_in, st_out, o16
        torch.cuda.empty_cache()
    return out


# (W, shard size, vectors per thread, caps): the wave probe's step mixes
PROBE_SWEEP = ((64, N_W64, 2, (0, 4, 6, 8, 12, 16)), (1, N_W1 // 2, 1, (0, 8, 12, 16)))


def probe_sweep(torch, rounds=3, reps=6):
    """The wave probe's W = 64 and W = 1 step mixes (all streams read and
    written, no arithmetic) at each residency cap, with and without the
    write windows the library uses at W = 64, interleaved over `rounds`."""
    import ctypes as C
    lib = _copylib()
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    cases, keep = [], []
    for w, n, vecs, caps in PROBE_SWEEP:
        g = torch.empty((w, -(-n // 128) * 128), dtype=torch.int16, device="cuda").random_()
        si = torch.empty(3 * n, dtype=torch.int32, device="cuda").random_()
        so = torch.empty(3 * n, dtype=torch.int32, device="cuda")
        o16 = torch.empty(n, dtype=torch.int16, device="cuda")
        gp = (C.c_void_p * 64)(*[g[k].data_ptr() for k in range(w)])
        keep.append((g, si, so, o16, gp))
        for cap in caps:
            for win in (None, WINDOW_W64):
                def launch(w=w, n=n, vecs=vecs, cap=cap, win=win, b=keep[-1]):
                    period, share = win or (0.0, 0.0)
                    rc = lib.zs_wave_probe(b[4], w, b[1].data_ptr(), b[2].data_ptr(),
                                           b[3].data_ptr(), n, vecs, cap, period, share,
                                           sink.data_ptr(), 0x6D2B79F5,
                                           torch.cuda.current_stream().cuda_stream)
                    if rc != 0:
                        raise RuntimeError(f"zs_wave_probe returned {rc}: "
                                           f"{lib.zs_copy_last_error().decode()}")
                cases.append(dict(world=w, n=n, vecs_per_thread=vecs, blocks_per_cu=cap or None,
                                  write_window=(dict(period_us=win[0], open_fraction=win[1])
                                                if win else None), fn=launch))
    times = [[] for _ in cases]
    for _ in range(rounds):
        for c, case in enumerate(cases):
            times[c].append(_time_calls(torch, case["fn"], reps))
    out = []
    for c, case in enumerate(cases):
        ms = sum(times[c]) / rounds
        gbps = (2 * case["world"] + 26) * case["n"] / (ms * 1e-3) / 1e9
        rec = {k: v for k, v in case.items() if k != "fn"}
        rec.update(ms=ms, ms_rounds=times[c], gbps=gbps, frac_of_peak=gbps / PEAK_HBM_GBPS)
        out.append(rec)
        log(f"probe W={case['world']} cap={case['blocks_per_cu']} "
            f"windows={'on' if case['write_window'] else 'off'}: {ms:.3f} ms ({gbps:.0f} GB/s)")
    del keep
    torch.cuda.empty_cache()
    return out


# ---- the shard step ------------------------------------------------------------

def pad_elems(n, align_bytes=256):
    """Row length (16-bit elements) rounded up to a multiple of align_bytes."""
    per = align_bytes // 2
    return -(-n // per) * per


def replicas_for(wl, bytes_per_step):
    """Independent shard copies cycled through so a step never finds its
    inputs in the 256 MB last-level cache (whole working set >= 1 GB)."""
    return max(1, min(128, -(-(1 << 30) // max(bytes_per_step, 1))))


def run_workload(name, steps, warmup, torch, wire=0, device_commit=True, event_pass=True,
                 state_layout=None):
    """Time `steps` steps of one workload queued back to back (no events),
    then (event_pass) the fused kernel alone over another `steps` steps,
    each bracketed by HIP events."""
    from sharded_mixed_precision_zs_amd import shard, synth

    wl = synth.WORKLOADS[name]
    layout = state_layout or STATE_LAYOUT
    n, W, A = wl.n, wl.world, wl.accum
    rd, wr = wl.bytes_per_param()
    frd, fwr = fused_bytes_per_param(W, A)
    fused_bytes = (frd + fwr) * n
    step_bytes = (rd + wr) * n
    R = replicas_for(wl, step_bytes)
    log(f"{name}: n={n} W={W} A={A} replicas={R} step bytes={step_bytes / 1e9:.3f} GB "
        f"commit={'device' if device_commit else 'host'} wire={wire} state={layout}")
    opt = shard.AdamW(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay)
    reps = []
    for r in range(R):
        st = shard.ShardState(n, W, wl.rank, wl.offset, wl.offset + n, wl.param_dtype,
                              wl.grad_dtype, opt, wl.loss_scale, dynamic=wl.dynamic_scale,
                              growth_interval=wl.scale_interval, accumulate=A > 1,
                              wire_dtype=wire, device_commit=device_commit,
                              state_layout=layout)
        st.fill_state(lambda first, count, *t: synth.dev_state(wl, wl.offset + first, *t))
        # one row per worker, rows padded to 256 B like separate allocations
        grads = torch.empty((A, W, pad_elems(n)), dtype=torch.int16, device="cuda")
        views = [[grads[j, k, :n] for k in range(W)] for j in range(A)]
        for j in range(A):
            for k in range(W):
                synth.dev_grad(wl, k, 1 + r % max(1, wl.steps), j, wl.offset, views[j][k],
                               scale=wl.loss_scale)
        reps.append((st, views))
    for st, g in reps:
        st.bind(g[A - 1], acc_in=st.acc if A > 1 else None)
    torch.cuda.synchronize()

    def one_step(i, events=None):
        st, g = reps[i % R]
        for j in range(A - 1):
            st.reduce_micro(g[j], first=(j == 0))
        ev = (events[0].cuda_event, events[1].cuda_event) if events else (None, None)
        if device_commit:
            st.step_device(ev_start=ev[0], ev_stop=ev[1])
            return 0
        return st.step(ev_start=ev[0], ev_stop=ev[1])

    def committed_so_far():
        return sum(int(st.sync_scaler().step_t) for st, _ in reps) if device_commit else 0

    for i in range(warmup):
        one_step(i)
    committed = -committed_so_far()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        committed += one_step(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    committed += committed_so_far()
    ms_per_step = elapsed * 1e3 / steps
    res = dict(workload=name, commit="device" if device_commit else "host", n=n, world=W,
               accum=A, replicas=R, wire=wire, state_layout=layout, ms_per_step=ms_per_step,
               params_per_s=n / (ms_per_step * 1e-3), step_bytes=step_bytes,
               hbm_gbps=step_bytes / (ms_per_step * 1e-3) / 1e9, committed=committed,
               fused_bytes=fused_bytes, write_window=write_window_of(W, n, A, layout))
    if event_pass:
        evs = timing_events(torch, steps)
        for i in range(steps):
            one_step(warmup + steps + i, evs[i])
        torch.cuda.synchronize()
        kern = sorted(s.elapsed_time(e) for s, e in evs)
        avg = sum(kern) / len(kern)
        res.update(fused_kernel_ms=avg, kernel_ms_median=kern[len(kern) // 2],
                   kernel_ms_min=kern[0], kernel_ms_max=kern[-1], kernel_samples=len(kern),
                   fused_gbps=fused_bytes / (avg * 1e-3) / 1e9)
    del reps
    torch.cuda.empty_cache()
    return res


def roofline_of(res, wl, wire=0):
    """The roofline object of one workload's fused kernel."""
    kernel = fused_instance(wl, wire, res["state_layout"])
    traffic = recorded_traffic(res["workload"], kernel) if wire == 0 else None
    rd, wr = fused_bytes_per_param(wl.world, wl.accum)
    return {"bound": "hbm", "achieved": res["fused_gbps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": res["fused_gbps"] / PEAK_HBM_GBPS, "traffic": traffic,
            "traffic_over_algorithmic": traffic / res["fused_bytes"] if traffic else None,
            "kernel": kernel, "kernel_ms": res["fused_kernel_ms"],
            "kernel_ms_median": res["kernel_ms_median"],
            "kernel_samples": res["kernel_samples"], "event_every": 1,
            "algorithmic_bytes_per_launch": res["fused_bytes"],
            "bytes_per_param": {"read": rd, "write": wr}, "shard_params": wl.n}


def run_offload(name, steps, warmup, torch):
    """The ZeRO-Offload variant on a workload: the ring reduction on the GPU,
    the fp32 gradient to the host, AdamW + cast on the host cores, the 16-bit
    parameters back."""
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

    ms = _time_calls(torch, gather, reps, warm=1)
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


# ---- the CPU oracle as a baseline ------------------------------------------------

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


def cpu_windows(wl, cap):
    """Flat starts (within the shard) and size of the oracle's sample: the
    whole shard when it fits `cap` parameters, else three windows of
    CPU_WINDOW parameters at the head, the middle and the tail."""
    if wl.n <= cap:
        return [0], wl.n
    L = min(CPU_WINDOW, cap // 3)
    return [0, (wl.n // 2) // 4096 * 4096, wl.n - L], L


def cpu_baseline(name, target_s=15.0):
    """The CPU oracle (as it stands) on a bounded sample of the workload:
    params/s, the step's rate if the whole shard ran at the sample's rate."""
    import numpy as np

    import oracle
    from sharded_mixed_precision_zs_amd import synth

    wl = synth.WORKLOADS[name]
    threads = min(16, len(os.sched_getaffinity(0)))
    kw = dict(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
              weight_decay=wl.weight_decay, loss_scale=wl.loss_scale, step_t=1)
    # host memory bound on the sample: ~6 GB of generated inputs and state
    cap = (6 << 30) // (2 * wl.world * wl.accum + 30)
    starts, L = cpu_windows(wl, cap)
    extrapolated = len(starts) > 1 or L < wl.n

    def inputs(first, ns, r):
        micro = [[synth.host_grad(wl, k, 1 + r, j, wl.offset + first, ns)
                  for k in range(wl.world)] for j in range(wl.accum)]
        return micro, synth.host_state(wl, wl.offset + first, ns)

    def timed(sets, reps, threads):
        acc = np.empty(sets[0][1][0].size, np.float32) if wl.accum > 1 else None
        t0 = time.perf_counter()
        for r in range(reps):
            micro, (master, m, v) = sets[r % len(sets)]
            for j, parts in enumerate(micro[:-1]):
                oracle.reduce_avg(parts, wl.rank, wl.grad_dtype, acc, j > 0, wl.loss_scale)
            oracle.shard_step(micro[-1], wl.rank, wl.grad_dtype, wl.param_dtype, master, m, v,
                              acc_in=acc, threads=threads, **kw)
        return time.perf_counter() - t0

    probe = min(L, 1 << 21)
    dt = timed([inputs(starts[0], probe, 0)], 2, threads) / 2
    want = int(probe * target_s / max(dt, 1e-6))
    ns = int(min(L, max(probe, want)))
    if extrapolated:
        ns = L
        sets = [inputs(s, L, r) for r, s in enumerate(starts)]
    else:
        sets = [inputs(starts[0], ns, r) for r in range(min(max(1, want // ns), wl.steps))]
    reps = max(1, min(1000, int(want // ns)))
    dt = timed(sets, reps, threads)
    # one thread, on a smaller sample (about a quarter of the time budget)
    one = [inputs(starts[0], probe, 0)]
    dt1 = timed(one, 1, 1)
    reps1 = max(1, min(100, int(target_s / 4 / max(dt1, 1e-6))))
    dt1 = timed(one, reps1, 1)
    rate = ns * reps / dt
    where = (f"{len(starts)} windows of {L} params (flat offsets {', '.join(map(str, starts))} "
             f"of the {wl.n}-param shard)" if extrapolated else
             f"{ns} params of the {name} rank-{wl.rank} partition")
    out = dict(value=rate, unit="params/s", cores=threads, kind="oracle",
               sample=f"{where} (W={wl.world}, {wl.accum} micro-batch(es)) x {reps} step(s), "
                      f"{threads} threads, {dt:.1f} s",
               value_1_thread=probe * reps1 / dt1,
               sample_1_thread=f"{probe} params x {reps1} step(s), 1 thread, {dt1:.1f} s",
               cpu_model=cpu_model(), host_cpus_machine=os.cpu_count(),
               host_cpus_available=len(os.sched_getaffinity(0)))
    if extrapolated:
        out.update(extrapolated=True,
                   extrapolated_step_s=wl.n / rate,
                   extrapolation=f"linear: the update is elementwise, so the whole "
                                 f"{wl.n}-param step takes n / value at the windows' rate")
    return out


def world_sweep(worlds, n, steps, warmup, torch):
    """The fused step at one shard size for several worker counts W: the
    read/write mix goes from 14:14 bytes per parameter (W = 1) to
    (2W + 12):14. Each W gets its own n (n + 4096 W), so a kernel trace of
    the sweep can be split by grid size. Returns one record per W."""
    import dataclasses

    from sharded_mixed_precision_zs_amd import synth

    out = []
    base = synth.WORKLOADS["gpt2s-w8"]
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


# The variant sweep: per workload, (variant id, residency cap, persistent
# blocks per CU). Ids 0 and 5 are the production shapes (libzsvariants).
VARIANT_SWEEP = {
    "7b-full-w1": [(49, 2, 0), (59, 2, 0), (49, 3, 0), (43, 2, 0), (42, 2, 0), (44, 4, 0), (45, 2, 0),
                   (0, 2, 0), (0, 3, 0), (0, 4, 0), (0, 0, 0), (1, 2, 0), (2, 2, 0), (3, 2, 0),
                   (4, 2, 2), (12, 0, 3), (13, 0, 3), (14, 0, 1),
                   (30, 8, 0), (30, 0, 0), (31, 4, 0), (32, 1, 0), (33, 1, 0)],
    "gpt2s-w8": [(53, 4, 0), (58, 4, 0), (64, 16, 0), (70, 16, 0), (53, 3, 0), (52, 0, 0), (50, 3, 0), (50, 0, 0), (41, 3, 0),
                 (51, 3, 0), (38, 3, 0), (46, 6, 0), (47, 3, 0),
                 (5, 3, 0), (5, 0, 0), (5, 2, 0), (5, 4, 0), (6, 3, 0), (7, 3, 0), (8, 3, 0),
                 (9, 3, 0), (10, 3, 3), (11, 3, 0), (15, 0, 3), (16, 0, 3),
                 (23, 3, 0), (25, 3, 0), (26, 8, 0), (27, 6, 0), (28, 2, 0), (29, 0, 0)],
    "7p5b-shard-w64": [(64, 12, 0), (70, 12, 0), (64, 8, 0), (64, 16, 0), (55, 6, 0), (57, 6, 0),
                       (55, 0, 0), (56, 3, 0), (53, 3, 0), (51, 0, 0), (50, 0, 0),
                       (40, 0, 0), (39, 0, 0), (38, 0, 0), (34, 0, 0), (47, 0, 0), (48, 0, 0),
                       (5, 0, 0), (5, 5, 0), (5, 3, 0), (6, 0, 0), (7, 0, 0), (8, 0, 0),
                       (9, 0, 0), (10, 0, 5), (11, 0, 0), (15, 0, 3), (16, 0, 3), (17, 0, 1),
                       (18, 0, 3), (19, 0, 2), (20, 0, 2), (21, 0, 1), (22, 0, 2),
                       (23, 0, 0), (24, 0, 0), (25, 0, 0), (26, 0, 0), (27, 0, 0), (28, 0, 0),
                       (29, 0, 0)],
}
VARIANT_N_MAX = 1 << 30   # W = 1: the first 2^30 parameters of the 7B state (3 sets fit HBM)


def _variantlib():
    import ctypes as C
    from sharded_mixed_precision_zs_amd import build as pkg_build
    if not os.path.exists(pkg_build.VARIANTS):
        raise RuntimeError(f"{pkg_build.VARIANTS} is not built: run the package build first")
    lib = C.CDLL(pkg_build.VARIANTS)
    lib.zs_variant_name.restype = C.c_char_p
    lib.zs_variant_name.argtypes = [C.c_int]
    lib.zs_variant_tile.argtypes = [C.c_int]
    lib.zs_variant_multi.argtypes = [C.c_int]
    lib.zs_variant_last_error.restype = C.c_char_p
    lib.zs_variant_launch.restype = C.c_int
    lib.zs_variant_launch.argtypes = [C.c_int, C.c_void_p, C.c_uint32, C.c_uint32, C.c_void_p]
    return lib


def variant_sweep(name, plan, reps, torch, rounds=3):
    """Time libzeroshard's fused step (zs_step_fused) and the variants of
    `plan` on one workload, interleaved over `rounds`, after checking that
    each variant writes the production kernel's bits. The shard is cut to a
    multiple of every variant's tile (and to VARIANT_N_MAX parameters)."""
    import ctypes as C

    from sharded_mixed_precision_zs_amd import synth
    from sharded_mixed_precision_zs_amd import zeroshard as zs

    lib = _variantlib()
    wl = synth.WORKLOADS[name]
    W = wl.world
    tile = max(lib.zs_variant_tile(v) for v, _, _ in plan)
    n = min(wl.n, VARIANT_N_MAX) // tile * tile
    bytes_per = 2 * W + 12 + 14
    R = replicas_for(wl, bytes_per * n)
    f32 = dict(dtype=torch.float32, device="cuda")
    reps_sets = []
    for r in range(R):
        grads = torch.empty((W, pad_elems(n)), dtype=torch.int16, device="cuda")
        views = [grads[k, :n] for k in range(W)]
        for k in range(W):
            synth.dev_grad(wl, k, 1 + r, 0, wl.offset, views[k], scale=wl.loss_scale)
        sin = [torch.empty(n, **f32) for _ in range(3)]
        synth.dev_state(wl, wl.offset, *sin)
        sout = [torch.empty(n, **f32) for _ in range(3)]
        par = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        hp = zs.hparams(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay, wl.loss_scale, 1)
        args = zs.StepArgs(views, 0, n, *sin, *sout, par, 0, flag, hp,
                           grad_dtype=wl.grad_dtype, param_dtype=wl.param_dtype)
        # StepArgs keeps raw addresses only: the replica holds its tensors
        reps_sets.append((args, sout, par, (grads, views, sin, flag)))
    torch.cuda.synchronize()

    def prod(i):
        zs.zs_step_fused(reps_sets[i % R][0])

    def variant(v, cap, per):
        def go(i):
            a = reps_sets[i % R][0]
            rc = lib.zs_variant_launch(v, C.addressof(a.args), cap, per,
                                       torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"zs_variant_launch({v}) returned {rc}: "
                                   f"{lib.zs_variant_last_error().decode()}")
        return go

    # bits: production into replica 0's outputs, saved; each variant must match
    prod(0)
    torch.cuda.synchronize()
    _, sout0, par0, _ = reps_sets[0]
    ref = [x.clone() for x in sout0] + [par0.clone()]
    for v, cap, per in plan:
        for x in sout0 + [par0]:
            x.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32).fill_(-1)
        variant(v, cap, per)(0)
        torch.cuda.synchronize()
        for what, x, y in zip(("master", "m", "v", "params"), sout0 + [par0], ref):
            xi = x.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32)
            yi = y.view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32)
            if not torch.equal(xi, yi):
                bad = torch.nonzero(xi != yi).flatten()
                i = int(bad[0])
                raise RuntimeError(f"variant {v} ({lib.zs_variant_name(v).decode()}) differs from "
                                   f"the production kernel: {bad.numel()} {what} elements, first "
                                   f"at {i}: {int(xi[i])} vs {int(yi[i])}")
    del ref
    configs = [("libzeroshard zs_step_fused", None, None, None, prod)]
    configs += [(lib.zs_variant_name(v).decode(), v, cap, per, variant(v, cap, per))
                for v, cap, per in plan]
    times = {i: [] for i in range(len(configs))}
    for _ in range(rounds):
        for i, (_, _, _, _, fn) in enumerate(configs):
            ms = _time_calls(torch, lambda it=iter(range(10 ** 9)): fn(next(it)), reps)
            times[i].append(ms)
    base = sum(times[0]) / rounds
    out = []
    for i, (label, v, cap, per, _) in enumerate(configs):
        ms = sum(times[i]) / rounds
        out.append(dict(config=label, variant=v, blocks_per_cu=cap, persistent_per_cu=per or None,
                        ms=ms, ms_rounds=times[i], gbps=bytes_per * n / (ms * 1e-3) / 1e9,
                        vs_production=base / ms, bit_exact=True))
        log(f"variants {name}: {label} cap={cap} persist={per}: {ms:.4f} ms "
            f"({out[-1]['gbps']:.0f} GB/s, x{base / ms:.4f})")
    del reps_sets
    torch.cuda.empty_cache()
    return dict(workload=name, n=n, world=W, replicas=R, bytes_per_param=bytes_per,
                reps_per_round=reps, rounds=rounds, results=out)


# Shards of the tile-depth sweep: W workers over n parameters (the 7.5B
# shard's hyper-parameters and generator), a GPT-2-sized and a 7.5B-sized n.
SHAPE_GRID = [(W, n) for n in (15_554_976, 117_187_500) for W in (2, 3, 4, 8, 12, 16, 24, 32, 64)]


def shape_plan(world):
    """Alternatives to zs_step_fused's own launch at W = `world`, all with
    4-element vectors and non-temporal state loads and stores: four vectors
    per thread in 256-thread blocks (3 per CU to W = 8, uncapped above, 16
    loads ahead from W = 16); two vectors in 256-thread blocks at 3 and 4
    per CU; one vector, 16 ahead, 256-thread blocks at 6 per CU; and in
    one-wave blocks, one vector at 16 per CU and two vectors at 8, 12 and
    16 per CU."""
    prev = (50, 3, 0) if world <= 8 else (50, 0, 0) if world < 16 else (51, 0, 0)
    return [prev, (53, 3, 0), (53, 4, 0), (55, 6, 0), (66, 16, 0), (64, 8, 0), (64, 12, 0),
            (64, 16, 0)]


def shape_sweep(torch, rounds=3):
    """variant_sweep over SHAPE_GRID: for each shard, the launch the library
    picks against shape_plan's alternatives, bits checked, interleaved."""
    import dataclasses

    from sharded_mixed_precision_zs_amd import synth

    base = synth.WORKLOADS["7p5b-shard-w64"]
    out = []
    for W, n in SHAPE_GRID:
        name = f"shape-w{W}-n{n}"
        synth.WORKLOADS[name] = dataclasses.replace(
            base, name=name, world=W, phi=W * n,
            description=f"{W} workers' bf16 gradients over a {n}-parameter shard")
        try:
            reps = max(4, min(100, int(2e10 / ((2 * W + 26) * n))))
            r = variant_sweep(name, shape_plan(W), reps, torch, rounds=rounds)
        finally:
            del synth.WORKLOADS[name]
        t, u, shape, cap = fused_shape(W, r["n"])
        r["production"] = {"threads_per_block": t, "vectors_per_thread": u, "access_shape": shape,
                           "blocks_per_cu": cap}
        out.append(r)
    return out


GROUPED_WORLDS = (1, 4, 5, 8, 16, 24, 32, 36, 40, 48, 64)
GROUPED_N = 117_187_500
# (W, n) cases of the grouped sweep: every W of GROUPED_WORLDS on the 7.5B
# shard's size, then smaller W = 64 shards around the write windows' floor,
# then W = 1 on 1 G parameters (28 GB per launch)
GROUPED_CASES = tuple((w, GROUPED_N) for w in GROUPED_WORLDS) + \
    tuple((64, n) for n in (10_000_000, 20_000_000, 33_816_576)) + ((1, 1_000_000_000),)


def grouped_plan(world, layout="grouped"):
    """(label, environment) of each launch the layout sweep times at `world`
    workers: libzeroshard's own launch first, then the same kernel with its
    measurement overrides (every one computes the same bits)."""
    plan = [("production", {})]
    if layout == "split" and world == 1:
        return plan + [(f"cap {c}", {"ZS_FUSED_BLOCKS_PER_CU": str(c)}) for c in (8, 16)] + [
            ("256-thread blocks, 2 vectors per thread, 2 per CU (the earlier launch)",
             {"ZS_FUSED_W1": "block256"})]
    if layout == "split" and world <= 3:
        return plan + [(f"cap {c}", {"ZS_FUSED_BLOCKS_PER_CU": str(c)}) for c in (2, 4, 8)]
    if world == 1:
        return plan + [(f"cap {c}", {"ZS_FUSED_BLOCKS_PER_CU": str(c)}) for c in (8, 16, 0)]
    if world == 4:
        return plan + [(f"cap {c}", {"ZS_FUSED_BLOCKS_PER_CU": str(c)}) for c in (8, 16)]
    off = {"ZS_FUSED_WRITE_WINDOW": "off"}
    plan.append(("batched sum, cap %d%s" % (16 if world <= 16 else 12,
                                            " (the earlier launch)" if layout == "grouped" else ""),
                 {"ZS_FUSED_SUM": "batched", "ZS_FUSED_BLOCKS_PER_CU": "16" if world <= 16 else "12",
                  **off}))
    plan += [(f"rolling sum, cap {c}, no windows", {"ZS_FUSED_BLOCKS_PER_CU": str(c), **off})
             for c in (4, 6, 8, 12)]
    plan.append((f"rolling sum, uncapped, windows {WINDOW_PERIOD_US} us / {WINDOW_OPEN}",
                 {"ZS_FUSED_BLOCKS_PER_CU": "0",
                  "ZS_FUSED_WRITE_WINDOW": f"{WINDOW_PERIOD_US},{WINDOW_OPEN}"}))
    if world >= WINDOW_WORLD:
        for period, share in ((20.48, 0.125), (40.96, 0.125), (30.72, 0.09375), (30.72, 0.15625)):
            plan.append((f"rolling sum, uncapped, windows {period} us / {share}",
                         {"ZS_FUSED_BLOCKS_PER_CU": "0",
                          "ZS_FUSED_WRITE_WINDOW": f"{period},{share}"}))
        plan.append((f"rolling sum, 16 per CU, windows {WINDOW_PERIOD_US} us / {WINDOW_OPEN}",
                     {"ZS_FUSED_BLOCKS_PER_CU": "16",
                      "ZS_FUSED_WRITE_WINDOW": f"{WINDOW_PERIOD_US},{WINDOW_OPEN}"}))
    return plan


def grouped_sweep(torch, cases=GROUPED_CASES, rounds=3, layout="grouped"):
    """libzeroshard's fused step with the grouped (or split) state for each
    (W, n) of `cases`: its own launch against the same kernel under the
    measurement overrides of grouped_plan (cap, batched sum, write windows),
    each launch's output checked bit for bit against the production
    launch's, timed interleaved over `rounds`. Random inputs (bf16
    gradients N(0, 1e-3), master N(0, 0.02), m N(0, 1e-4), v |N(0, 1e-3)|)."""
    from sharded_mixed_precision_zs_amd import zeroshard as zs

    hp = zs.hparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01,
                    loss_scale=1.0, step_t=1)
    saved = {k: os.environ.get(k) for k in ("ZS_FUSED_BLOCKS_PER_CU", "ZS_FUSED_SUM",
                                            "ZS_FUSED_WRITE_WINDOW", "ZS_FUSED_W1")}

    def setenv(env):
        for k in saved:
            os.environ.pop(k, None)
        os.environ.update(env)

    out = []
    try:
        for W, n in cases:
            g = torch.empty((W, pad_elems(n)), dtype=torch.int16, device="cuda")
            for k in range(W):
                g[k, :n].view(torch.bfloat16).copy_(
                    torch.empty(n, dtype=torch.float32, device="cuda").normal_(0, 1e-3))
            grads = [g[k, :n].view(torch.bfloat16) for k in range(W)]
            grouped = layout == "grouped"
            L = zs.grouped_len(n) if grouped else 3 * n
            sin = torch.empty(L, dtype=torch.float32, device="cuda").normal_(0, 0.02)
            sv = sin.view(-1, 3, 1024) if grouped else sin.view(3, 1, n)
            sv[:, 1, :].mul_(5e-3) if grouped else sv[1].mul_(5e-3)
            sv[:, 2, :].abs_().mul_(0.05) if grouped else sv[2].abs_().mul_(0.05)
            sout = torch.empty_like(sin)
            gather = torch.empty(n, dtype=torch.bfloat16, device="cuda")
            flag = torch.zeros(1, dtype=torch.int32, device="cuda")
            if grouped:
                args = zs.StepArgs(grads, 0, n, sin, None, None, sout, None, None, gather, 0,
                                   flag, hp, state_layout=zs.ZS_STATE_GROUPED)
            else:
                args = zs.StepArgs(grads, 0, n, sin[:n], sin[n:2 * n], sin[2 * n:], sout[:n],
                                   sout[n:2 * n], sout[2 * n:], gather, 0, flag, hp)
            plan = grouped_plan(W, layout)
            ref = None
            for label, env in plan:
                setenv(env)
                sout.zero_()
                zs.zs_step_fused(args)
                torch.cuda.synchronize()
                got = (sout.view(torch.int32).clone(), gather.view(torch.int16).clone())
                if ref is None:
                    ref = got
                elif not (torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])):
                    raise RuntimeError(f"W={W} {label}: bits differ from the production launch")
            del ref, got
            reps = max(4, min(50, int(2e10 / ((2 * W + 26) * n))))
            times = {label: [] for label, _ in plan}
            for _ in range(rounds):
                for label, env in plan:
                    setenv(env)
                    times[label].append(_time_calls(torch, lambda: zs.zs_step_fused(args), reps))
            rows = []
            for label, _ in plan:
                ms = sum(times[label]) / rounds
                gbps = (2 * W + 26) * n / (ms * 1e-3) / 1e9
                rows.append(dict(launch=label, ms=ms, ms_rounds=times[label], gbps=gbps,
                                 frac_of_peak=gbps / PEAK_HBM_GBPS))
                log(f"{layout} W={W} n={n} {label}: {ms:.4f} ms ({gbps:.0f} GB/s)")
            setenv({})
            t, u, shape, cap = fused_shape(W, n, layout)
            out.append(dict(world=W, n=n, layout=layout, reps=reps, rounds=rounds, results=rows,
                            production={"threads_per_block": t, "vectors_per_thread": u,
                                        "access_shape": shape, "blocks_per_cu": cap,
                                        "write_window": write_window_of(W, n)}))
            del g, grads, sin, sout, gather, args
            torch.cuda.empty_cache()
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return out


def phase_sweep(torch, reps=10, rounds=2):
    """Reads and writes of the 7.5B shard's step separated in time, with the
    stream probe: per chunk of the shard, a read-only probe kernel (the 64
    gradient and 3 state streams) then a write-only one (the 3 fp32 and the
    16-bit output streams), back to back on one stream, for 1 to 64 chunks;
    beside them the mixed probe and the read-only and write-only passes over
    the whole shard. What a kernel that kept a chunk's outputs on chip until
    the chunk's reads were done could at best reach, by chunk count."""
    import ctypes as C
    lib = _copylib()
    n, W = N_W64, 64
    g = torch.empty((W, n), dtype=torch.int16, device="cuda").random_()
    ins = [torch.empty(n, dtype=torch.int32, device="cuda").random_() for _ in range(3)]
    outs = [torch.empty(n, dtype=torch.int32, device="cuda") for _ in range(3)]
    o16 = torch.empty(n, dtype=torch.int16, device="cuda")
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")

    def ptrs(ts, off, es):
        return (C.c_void_p * 64)(*[t.data_ptr() + off * es for t in ts])

    def probe(c0, cn, reads, writes):
        rc = lib.zs_stream_probe(ptrs([g[k] for k in range(W)] if reads else [], c0, 2),
                                 W if reads else 0, ptrs(ins if reads else [], c0, 4),
                                 3 if reads else 0, ptrs(outs if writes else [], c0, 4),
                                 3 if writes else 0, o16.data_ptr() + 2 * c0 if writes else None,
                                 cn, 2, 0, sink.data_ptr(), 0x6D2B79F5,
                                 torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"zs_stream_probe returned {rc}")

    def chunked(chunks, phased, reads=True, writes=True):
        size = -(-n // chunks // 4096) * 4096
        c0 = 0
        while c0 < n:
            cn = min(size, n - c0)
            if phased:
                probe(c0, cn, True, False)
                probe(c0, cn, False, True)
            else:
                probe(c0, cn, reads, writes)
            c0 += cn

    legs = [("mixed, whole shard", lambda: chunked(1, False)),
            ("reads only, whole shard", lambda: chunked(1, False, writes=False)),
            ("writes only, whole shard", lambda: chunked(1, False, reads=False))]
    legs += [(f"phased, {k} chunk(s)", (lambda k=k: chunked(k, True))) for k in (1, 2, 4, 8, 16, 64)]
    times = {name: [] for name, _ in legs}
    for _ in range(rounds):
        for name, fn in legs:
            times[name].append(_time_calls(torch, fn, reps))
    per_param = {"reads only, whole shard": 140, "writes only, whole shard": 14}
    out = []
    for name, t in times.items():
        ms = sum(t) / len(t)
        b = per_param.get(name, 154)
        out.append(dict(leg=name, ms=ms, ms_rounds=t, bytes_per_param=b,
                        gbps=b * n / (ms * 1e-3) / 1e9))
        log(f"phases: {name}: {ms:.4f} ms ({out[-1]['gbps']:.0f} GB/s)")
    del g, ins, outs, o16
    torch.cuda.empty_cache()
    return dict(n=n, world=W, bytes_per_param=154, reps=reps, rounds=rounds, legs=out)


def side_leg(name, fn, torch):
    """Run a leg reported beside the headline; a failure (for instance too
    little free device memory) is recorded in the JSON line as
    {"error": ...} instead of taking the headline down with it."""
    try:
        return fn()
    except (RuntimeError, MemoryError, OSError, ValueError) as e:
        log(f"{name} failed: {type(e).__name__}: {e}")
        torch.cuda.empty_cache()
        return {"error": f"{type(e).__name__}: {e}"}


def without_write_windows(fn):
    """fn() with libzeroshard's write windows switched off."""
    old = os.environ.get("ZS_FUSED_WRITE_WINDOW")
    os.environ["ZS_FUSED_WRITE_WINDOW"] = "off"
    try:
        return fn()
    finally:
        if old is None:
            del os.environ["ZS_FUSED_WRITE_WINDOW"]
        else:
            os.environ["ZS_FUSED_WRITE_WINDOW"] = old


def summary(res, wl, wire=0):
    """The record of one workload in the JSON line."""
    out = dict(workload=res["workload"], params_per_s=res["params_per_s"],
               ms_per_step=res["ms_per_step"], hbm_gbps=res["hbm_gbps"],
               hbm_pct_of_peak=100.0 * res["hbm_gbps"] / PEAK_HBM_GBPS,
               replicas=res["replicas"], committed=res["committed"],
               write_window=res.get("write_window"))
    if "fused_gbps" in res:
        out["roofline"] = roofline_of(res, wl, wire)
    return out


def main():
    global STATE_LAYOUT
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1,
                    help="GPUs to use; only 1 is supported (one rank's shard on one MI355X)")
    ap.add_argument("--steps", type=int, default=20, help="timed steps of each workload")
    ap.add_argument("--warmup", type=int, default=5, help="untimed steps before the timed ones")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="headline workload (a key of synth.WORKLOADS)")
    ap.add_argument("--also", default=DEFAULT_ALSO,
                    help="comma-separated workloads reported beside the headline")
    ap.add_argument("--state-layout", choices=("split", "grouped"), default=STATE_LAYOUT,
                    help="fp32 state layout of the timed shards")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the CPU oracle (cpu_baseline)")
    ap.add_argument("--no-offload", action="store_true",
                    help="skip the ZeRO-Offload (host update) leg")
    ap.add_argument("--no-ceilings", "--no-copy-ceiling", dest="no_ceilings", action="store_true",
                    help="skip the copy and stream-probe ceilings")
    ap.add_argument("--ceilings", default="",
                    help="comma-separated stream-probe names to run (default: all)")
    ap.add_argument("--no-host-commit", action="store_true",
                    help="skip the host-commit flow of the headline")
    ap.add_argument("--no-side-legs", action="store_true",
                    help="skip the bf16-wire and all-gather legs")
    ap.add_argument("--sweep-world", default="",
                    help="comma-separated W values: time the fused step at one shard size for "
                         "each and print that table as the JSON line instead")
    ap.add_argument("--sweep-n", type=int, default=1 << 25,
                    help="shard size of the --sweep-world runs")
    ap.add_argument("--sweep-probe", action="store_true",
                    help="the wave probe's W = 64 and W = 1 step mixes by residency cap, with "
                         "and without write windows")
    ap.add_argument("--sweep-phases", action="store_true",
                    help="time the 7.5B shard's reads and writes separated in time (stream "
                         "probe, 1 to 64 chunks) and print that table as the JSON line instead")
    ap.add_argument("--sweep-copy", action="store_true",
                    help="time libzscopy's copy shapes (vectors per lane, non-temporal loads "
                         "and stores, block size, persistent grids, residency caps) over 4 GiB "
                         "and print that table as the JSON line instead")
    ap.add_argument("--sweep-grouped", action="store_true",
                    help="time libzeroshard's grouped-state fused step against its measurement "
                         "overrides (caps, batched sum, write windows) over W = "
                         + ", ".join(map(str, GROUPED_WORLDS)) + " on the 7.5B shard's size and "
                         "three smaller W = 64 shards, and print that table as the JSON line "
                         "instead")
    ap.add_argument("--sweep-split", action="store_true",
                    help="the same sweep as --sweep-grouped with the split state layout")
    ap.add_argument("--sweep-shapes", action="store_true",
                    help="time the fused step's tile depths and residency caps against "
                         "libzeroshard's own launch over a grid of W and shard sizes and print "
                         "that table as the JSON line instead")
    ap.add_argument("--sweep-variants", default="",
                    help="comma-separated workloads (of " + ", ".join(VARIANT_SWEEP) + "): time "
                         "the fused kernel's shapes of libzsvariants against libzeroshard's and "
                         "print that table as the JSON line instead")
    args = ap.parse_args()
    STATE_LAYOUT = args.state_layout
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this benchmark runs on one GPU: the shard step takes one "
                          "rank's real share on one MI355X; multi-GPU runs are not part of it"}))
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    from sharded_mixed_precision_zs_amd import synth
    from sharded_mixed_precision_zs_amd import zeroshard  # noqa: F401  (fails loudly if unbuilt)

    if args.sweep_world:
        worlds = [int(x) for x in args.sweep_world.split(",") if x]
        sweep = world_sweep(worlds, args.sweep_n, args.steps, args.warmup, torch)
        print(json.dumps({"metric": "fused step HBM GB/s by worker count", "unit": "GB/s",
                          "peak": PEAK_HBM_GBPS, "sweep": sweep}))
        return
    if args.sweep_probe:
        print(json.dumps({"metric": "wave-probe step mix GB/s by residency cap and write windows",
                          "unit": "GB/s", "peak": PEAK_HBM_GBPS, "probe": probe_sweep(torch)}))
        return
    if args.sweep_phases:
        print(json.dumps({"metric": "7.5B-shard step mix, reads and writes separated in time",
                          "unit": "ms", "phases": phase_sweep(torch)}))
        return
    if args.sweep_copy:
        print(json.dumps({"metric": "plain copy, read + write GB/s by copy shape", "unit": "GB/s",
                          "peak": PEAK_HBM_GBPS, "copies": copy_shape_sweep(torch)}))
        return
    if args.sweep_grouped:
        print(json.dumps({"metric": "grouped-state fused step by launch setting, ms per launch",
                          "unit": "ms", "sweeps": grouped_sweep(torch)}))
        return
    if args.sweep_split:
        print(json.dumps({"metric": "split-state fused step by launch setting, ms per launch",
                          "unit": "ms", "sweeps": grouped_sweep(torch, layout="split")}))
        return
    if args.sweep_shapes:
        print(json.dumps({"metric": "fused step tile depth and residency by W and shard size, "
                          "ms per launch", "unit": "ms", "sweeps": shape_sweep(torch)}))
        return
    if args.sweep_variants:
        res = [variant_sweep(w, VARIANT_SWEEP[w], max(4, args.steps), torch)
               for w in args.sweep_variants.split(",") if w]
        print(json.dumps({"metric": "fused step kernel shapes, ms per launch", "unit": "ms",
                          "sweeps": res}))
        return
    K, Wm = args.steps, args.warmup
    also = [x for x in args.also.split(",") if x and x != args.workload]
    # the host-side offload leg first: it measured slower after the large
    # workloads' hundreds of GB of device allocations
    offload = None
    if not args.no_offload:
        offload = side_leg("offload", lambda: run_offload(HOST_LEG_WORKLOAD, max(10, K), 2, torch),
                           torch)
        log(json.dumps(offload))
    copies, ceilings = {}, {}
    if not args.no_ceilings:
        copies = side_leg("copy_ceiling", lambda: copy_rates_gbps(torch), torch)
        names = set(x for x in args.ceilings.split(",") if x) or None
        ceilings = side_leg("stream_ceilings", lambda: stream_ceilings(torch, names=names), torch)
    copy_ceiling = copies.get("ceiling")
    # the workloads beside the headline, smallest memory first
    others, roofs = [], {}
    for name in also:
        wl = synth.WORKLOADS[name]
        k = max(K, 200) if wl.n < (1 << 20) else K
        r = side_leg(name, lambda: run_workload(name, k, 2, torch), torch)
        log(json.dumps(r))
        if "error" in r:
            others.append(dict(workload=name, error=r["error"]))
            continue
        rec = summary(r, wl)
        others.append(rec)
        roofs[name] = rec["roofline"]
    wire_bf16, all_gather, windows_off = None, [], None
    if not args.no_side_legs:
        if WIRE_WORKLOAD in synth.WORKLOADS:
            wl = synth.WORKLOADS[WIRE_WORKLOAD]
            r = side_leg("wire_bf16", lambda: run_workload(WIRE_WORKLOAD, K, 2, torch, wire=1),
                         torch)
            log(json.dumps(r))
            wire_bf16 = r if "error" in r else summary(r, wl, wire=1)
        if WINDOW_WORKLOAD in synth.WORKLOADS and roofs.get(WINDOW_WORKLOAD):
            r = side_leg("write_windows_off", lambda: without_write_windows(
                lambda: run_workload(WINDOW_WORKLOAD, K, 2, torch)), torch)
            log(json.dumps(r))
            if "error" not in r:
                on = roofs[WINDOW_WORKLOAD]
                windows_off = dict(workload=WINDOW_WORKLOAD, kernel_ms_on=on["kernel_ms"],
                                   kernel_ms_off=r["fused_kernel_ms"],
                                   gbps_on=on["achieved"], gbps_off=r["fused_gbps"],
                                   speedup=r["fused_kernel_ms"] / on["kernel_ms"],
                                   ms_per_step_off=r["ms_per_step"])
            else:
                windows_off = r
        for name in ALL_GATHER_WORKLOADS:
            r = side_leg(f"all_gather {name}", lambda: run_all_gather(name, 10, torch), torch)
            log(json.dumps(r))
            all_gather.append(r if "error" not in r else dict(workload=name, error=r["error"]))
    # the headline: device commit, then host commit, on fresh buffers each
    main_res = run_workload(args.workload, K, Wm, torch)
    log(json.dumps(main_res))
    host_res = None
    if not args.no_host_commit:
        host_res = side_leg("host_commit", lambda: run_workload(args.workload, K, 2, torch,
                                                                device_commit=False), torch)
        log(json.dumps(host_res))

    # the CPU oracle last, so the GPU legs run back to back from the start
    cpu = None if args.no_cpu_baseline else side_leg("cpu_baseline",
                                                     lambda: cpu_baseline(args.workload), torch)
    log(f"cpu_baseline: {json.dumps(cpu)}")

    wl = synth.WORKLOADS[args.workload]
    head = summary(main_res, wl)
    roofs[args.workload] = head["roofline"]
    # the headline mix's own streams alone: read-only and write-only probe
    # rates, and their harmonic combination at the step's read:write bytes
    alone = {1: ("read_only_w1_streams", "write_only_w1_streams")}.get(wl.world)
    harmonic = None
    if alone and all(k in ceilings for k in alone):
        rd, wr = fused_bytes_per_param(wl.world, wl.accum)
        harmonic = (rd + wr) / (rd / ceilings[alone[0]]["gbps"] + wr / ceilings[alone[1]]["gbps"])
    bounds = stream_bounds(ceilings, roofs)
    out = {
        "metric": METRIC,
        "value": main_res["params_per_s"],
        "unit": "params/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
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
                   "micro_batches": wl.accum, "replicas": main_res["replicas"], "wire": "fp32",
                   "state_layout": main_res["state_layout"]},
        "hbm_gbps": main_res["hbm_gbps"],
        "hbm_pct_of_peak": 100.0 * main_res["hbm_gbps"] / PEAK_HBM_GBPS,
        "copy_ceiling_gbps": copy_ceiling,
        "memcpy_d2d_gbps": copies.get("memcpy"),
        "hbm_pct_of_copy_ceiling": (100.0 * main_res["hbm_gbps"] / copy_ceiling
                                    if copy_ceiling else None),
        "read_write_harmonic_gbps": harmonic,
        "fused_pct_of_read_write_harmonic": (100.0 * main_res["fused_gbps"] / harmonic
                                             if harmonic else None),
        "roofline": head["roofline"],
        "roofline_by_workload": roofs,
        "ceilings": ceilings,
        "stream_bounds": bounds,
        "cpu_baseline": cpu,
        "other_workloads": others,
        "host_commit": (None if host_res is None else host_res if "error" in host_res else
                        dict(ms_per_step=host_res["ms_per_step"],
                             params_per_s=host_res["params_per_s"],
                             fused_kernel_ms=host_res.get("fused_kernel_ms"))),
        "offload": offload,
        "wire_bf16": wire_bf16,
        "write_windows_off": windows_off,
        "all_gather": all_gather,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
