"""Randomized GPU parity: seeded random configurations of the fused step
(with the decision on the host and on the device; with the split and the
grouped state, the latter with write windows forced on at random), of the
reduction, of the unfused check / update / cast chain, of the ring
all-gather and of the pipelined offload step, each against the oracle
through the C ABI.

Every case draws the worker count (1 to 64), a ragged size, the rank, the
gradient and parameter dtypes, the precision of the ring's partial sums,
an accumulated micro-batch input or none, the loss scale (powers of two
and others), the step index, the AdamW settings (within their valid
ranges), the gather offset and misaligned gradient starts (so every vector
width of the kernels runs), and sometimes one non-finite gradient value.
Bars as in the fixed parity tests: the flag bit-exact; fp32 state within
1e-6 relative, 16-bit parameters within 1 ulp (and, as there, every
element bit-identical); the reduced gradient bit-exact; inputs never
written.
"""
import numpy as np
import pytest

import oracle
from gpu_util import (F32, announce, assert_bits_equal, assert_offload_matches_oracle,
                      assert_rel, assert_ulp16, down16, down32, oracle_offload_update, up16,
                      up32)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DT = {"bf16": 0, "fp16": 1}
WIRES = [None, "bf16", "fp16"]
WIRE_CODE = {None: 0, "bf16": 1, "fp16": 2}


@pytest.fixture(scope="module")
def zs(hip_built):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sharded_mixed_precision_zs_amd import zeroshard
    return zeroshard


def _rand16(rng, n, sigma, dtype):
    x = (rng.standard_normal(n) * sigma).astype(F32)
    if dtype == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    return x.astype(np.float16).view(np.uint16)


def _draw(rng):
    world = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 13, 16, 31, 64]))
    n = int(rng.integers(1, 200_000 if rng.random() < 0.2 else 20_000))
    scale = float(rng.choice([1.0, 2.0 ** int(rng.integers(0, 17)), 3.0, 1000.0]))
    gdt = str(rng.choice(["bf16", "fp16"]))
    if gdt == "fp16":
        scale = min(scale, 1024.0)   # keeps N(0, 1e-3) * scale sums inside fp16
    return dict(
        world=world, n=n, rank=int(rng.integers(0, world)), gdt=gdt,
        pdt=str(rng.choice(["bf16", "fp16"])), wire=WIRES[int(rng.integers(0, 3))],
        acc=bool(rng.random() < 0.3), scale=scale, t=int(rng.integers(1, 5000)),
        lr=float(10 ** rng.uniform(-5, -2)), beta1=float(rng.uniform(0.8, 0.99)),
        beta2=float(rng.uniform(0.9, 0.9999)), eps=float(rng.choice([0.0, 1e-8, 1e-6])),
        weight_decay=float(rng.uniform(0.0, 0.1)), off=int(rng.integers(0, 10)),
        shifts=[int(x) for x in rng.integers(0, 4, world)],
        inject=bool(rng.random() < 0.1))


def _upload_grads(g16, shifts, dtype):
    """Each worker's buffer starts `shift` elements into its allocation, so
    some start off the 16-byte boundary."""
    out = []
    for g, s in zip(g16, shifts):
        pad = np.zeros(s, np.uint16)
        out.append(up16(np.concatenate([pad, g]), dtype)[s:])
    return out


@pytest.mark.parametrize("case", range(200))
def test_fused_step_random_configuration(zs, case):
    rng = np.random.default_rng(5000 + case)
    c = _draw(rng)
    W, n, gdt, pdt = c["world"], c["n"], c["gdt"], c["pdt"]
    announce(f"fuzz fused #{case}: " + ", ".join(f"{k}={v}" for k, v in c.items()
                                                 if k != "shifts"))
    g16 = [_rand16(rng, n, 1e-3 * c["scale"], gdt) for _ in range(W)]
    if c["inject"]:
        bad = 0x7F80 if gdt == "bf16" else 0x7C00
        g16[int(rng.integers(0, W))][int(rng.integers(0, n))] = bad | (1 if rng.random() < 0.5 else 0)
    master = (rng.standard_normal(n) * 0.02).astype(F32)
    m = (rng.standard_normal(n) * 1e-4).astype(F32)
    v = rng.uniform(0, 1e-6, n).astype(F32)
    acc = (rng.standard_normal(n) * c["scale"] * 1e-3).astype(F32) if c["acc"] else None
    hp = dict(lr=c["lr"], beta1=c["beta1"], beta2=c["beta2"], eps=c["eps"],
              weight_decay=c["weight_decay"])
    dg = _upload_grads(g16, c["shifts"], gdt)
    din = [up32(x) for x in (master, m, v)]
    dout = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3)]
    gather = torch.full((n + c["off"] + 3,), 7, dtype=torch.int16, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = zs.StepArgs(dg, c["rank"], n, *din, *dout, gather, c["off"], flag,
                       zs.hparams(**hp, loss_scale=c["scale"], step_t=c["t"]),
                       acc_in=up32(acc) if acc is not None else None, grad_dtype=DT[gdt],
                       param_dtype=DT[pdt], wire_dtype=WIRE_CODE[c["wire"]])
    zs.zs_step_fused(args)
    f, mo, mmo, vo, po = oracle.shard_step(g16, c["rank"], gdt, pdt, master, m, v,
                                           step_t=c["t"], acc_in=acc, loss_scale=c["scale"],
                                           threads=4, wire=c["wire"], **hp)
    assert int(flag.item()) == f
    assert f == (1 if c["inject"] else 0)
    for d, x in zip(din, (master, m, v)):
        assert_bits_equal(down32(d), x, "inputs untouched")
    if f == 0:
        # within the bars, and in fact bit-identical (same operations, same order)
        for got, want, what in zip(dout, (mo, mmo, vo), ("master", "m", "v")):
            assert assert_rel(down32(got), want, 1e-6, f"#{case} {what}") == 0
        gb = down16(gather)
        off = c["off"]
        assert np.all(gb[:off] == 7) and np.all(gb[off + n:] == 7)
        assert assert_ulp16(gb[off:off + n], po, pdt, 1, f"#{case} params") == 0


SENTINEL = np.uint32(0x7FC0DEAD).view(F32)  # a NaN no arithmetic produces


@pytest.mark.parametrize("case", range(60))
def test_fused_step_random_grouped(zs, case, monkeypatch):
    """The grouped state layout (operands aligned for 4-element vectors, so
    every W >= 5 takes the rolling sum) with write windows forced on in
    about half the cases, against the oracle; the slots past n of the last
    group stay untouched."""
    rng = np.random.default_rng(7000 + case)
    c = _draw(rng)
    W, n, gdt, pdt = c["world"], c["n"], c["gdt"], c["pdt"]
    off = 4 * int(rng.integers(0, 3))
    windows = rng.random() < 0.5
    if windows:
        monkeypatch.setenv("ZS_FUSED_WRITE_WINDOW",
                           f"{float(rng.choice([1.28, 2.56, 5.12]))},{float(rng.choice([0.125, 0.25]))}")
    announce(f"fuzz fused grouped #{case}: W={W} n={n} rank={c['rank']} {gdt}/{pdt} "
             f"wire={c['wire']} acc={c['acc']} windows={windows} inject={c['inject']}")
    g16 = [_rand16(rng, n, 1e-3 * c["scale"], gdt) for _ in range(W)]
    if c["inject"]:
        bad = 0x7F80 if gdt == "bf16" else 0x7C00
        g16[int(rng.integers(0, W))][int(rng.integers(0, n))] = bad
    state = [(rng.standard_normal(n) * 0.02).astype(F32), (rng.standard_normal(n) * 1e-4).astype(F32),
             rng.uniform(0, 1e-6, n).astype(F32)]
    acc = (rng.standard_normal(n) * c["scale"] * 1e-3).astype(F32) if c["acc"] else None
    hp = dict(lr=c["lr"], beta1=c["beta1"], beta2=c["beta2"], eps=c["eps"],
              weight_decay=c["weight_decay"])
    G = -(-n // 1024)
    buf = np.full((G, 3, 1024), SENTINEL, dtype=F32)
    for k, x in enumerate(state):
        flat = np.full(G * 1024, SENTINEL, dtype=F32)
        flat[:n] = x
        buf[:, k, :] = flat.reshape(G, 1024)
    gin = up32(buf.ravel())
    gout = up32(np.full(G * 3072, SENTINEL, dtype=F32))
    gather = torch.full((n + off + 8,), 7, dtype=torch.int16, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = zs.StepArgs([up16(g, gdt) for g in g16], c["rank"], n, gin, None, None, gout, None,
                       None, gather, off, flag,
                       zs.hparams(**hp, loss_scale=c["scale"], step_t=c["t"]),
                       acc_in=up32(acc) if acc is not None else None, grad_dtype=DT[gdt],
                       param_dtype=DT[pdt], wire_dtype=WIRE_CODE[c["wire"]],
                       state_layout=zs.ZS_STATE_GROUPED)
    zs.zs_step_fused(args)
    f, mo, mmo, vo, po = oracle.shard_step(g16, c["rank"], gdt, pdt, *state, step_t=c["t"],
                                           acc_in=acc, loss_scale=c["scale"], threads=4,
                                           wire=c["wire"], **hp)
    assert int(flag.item()) == f == (1 if c["inject"] else 0)
    assert_bits_equal(down32(gin), buf.ravel(), "input set untouched")
    out = down32(gout).reshape(G, 3, 1024)
    for k, (want, what) in enumerate(zip((mo, mmo, vo), ("master", "m", "v"))):
        flat = out[:, k, :].ravel()
        assert_bits_equal(flat[n:], np.full(G * 1024 - n, SENTINEL, dtype=F32), f"{what} past n")
        if f == 0:
            assert assert_rel(flat[:n], want, 1e-6, f"#{case} {what}") == 0
    gb = down16(gather)
    assert np.all(gb[:off] == 7) and np.all(gb[off + n:] == 7)
    if f == 0:
        assert assert_ulp16(gb[off:off + n], po, pdt, 1, f"#{case} params") == 0


@pytest.mark.parametrize("case", range(100))
def test_reduce_random_configuration(zs, case):
    rng = np.random.default_rng(9000 + case)
    c = _draw(rng)
    W, n, gdt = c["world"], c["n"], c["gdt"]
    announce(f"fuzz reduce #{case}: W={W} n={n} {gdt} wire={c['wire']} acc={c['acc']} "
             f"scale={c['scale']} inject={c['inject']}")
    g16 = [_rand16(rng, n, 1e-3 * c["scale"], gdt) for _ in range(W)]
    if c["inject"]:
        g16[int(rng.integers(0, W))][int(rng.integers(0, n))] = 0x7F80 if gdt == "bf16" else 0x7C00
    start = (rng.standard_normal(n) * c["scale"] * 1e-3).astype(F32)
    out = up32(start) if c["acc"] else torch.zeros(n, dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    zs.zs_reduce_scatter_avg(_upload_grads(g16, c["shifts"], gdt), DT[gdt], W, c["rank"], n,
                             out, accumulate=c["acc"], overflow_flag=flag,
                             loss_scale=c["scale"], wire_dtype=WIRE_CODE[c["wire"]])
    ref = start.copy() if c["acc"] else np.zeros(n, F32)
    f = oracle.reduce_avg(g16, c["rank"], gdt, ref, c["acc"], c["scale"], wire=c["wire"])
    assert int(flag.item()) == f
    assert_bits_equal(down32(out), ref, f"#{case} reduced gradient")


@pytest.mark.parametrize("case", range(100))
def test_unfused_chain_random_configuration(zs, case):
    """zs_check_overflow, zs_adamw_step and zs_cast_gather on a random
    averaged gradient partition (sometimes with a non-finite value) at a
    random misaligned start, with random AdamW settings and loss scale:
    the flag, the updated state and the 16-bit parameters equal the
    oracle's; a set flag makes both later calls leave everything as it was."""
    rng = np.random.default_rng(13000 + case)
    c = _draw(rng)
    n, pdt = c["n"], c["pdt"]
    skew = int(rng.integers(0, 4))            # misaligns every fp32 operand
    announce(f"fuzz unfused #{case}: n={n} {pdt} scale={c['scale']} t={c['t']} skew={skew} "
             f"inject={c['inject']}")
    a = (rng.standard_normal(n) * 1e-3 * c["scale"]).astype(F32)
    if c["inject"]:
        a[int(rng.integers(0, n))] = np.inf if rng.random() < 0.5 else np.nan
    state = [(rng.standard_normal(n) * s).astype(F32) for s in (0.02, 1e-4, 1e-6)]
    state[2] = np.abs(state[2])

    def dev32(x):
        buf = torch.empty(n + skew, dtype=torch.float32, device="cuda")
        buf[skew:].copy_(torch.from_numpy(x))
        return buf[skew:]

    da = dev32(a)
    dst = [dev32(x) for x in state]
    gather = torch.full((n + c["off"] + 3,), 7, dtype=torch.int16, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    hp = dict(lr=c["lr"], beta1=c["beta1"], beta2=c["beta2"], eps=c["eps"],
              weight_decay=c["weight_decay"])
    zs.zs_check_overflow(da, n, c["scale"], flag)
    zs.zs_adamw_step(*dst, da, n, zs.hparams(**hp, loss_scale=c["scale"], step_t=c["t"]), flag)
    zs.zs_cast_gather(dst[0], gather, DT[pdt], c["off"], n, flag)
    f = oracle.check_overflow(a, c["scale"])
    assert int(flag.item()) == f == (1 if c["inject"] else 0)
    gb = down16(gather)
    off = c["off"]
    assert np.all(gb[:off] == 7) and np.all(gb[off + n:] == 7)
    if f:
        for d, x, what in zip(dst, state, ("master", "m", "v")):
            assert_bits_equal(down32(d), x, f"#{case} skipped {what}")
        assert np.all(gb == 7)
        return
    ref = [x.copy() for x in state]
    oracle.adamw(*ref, a, c["scale"], t=c["t"], **hp)
    for d, want, what in zip(dst, ref, ("master", "m", "v")):
        assert assert_rel(down32(d), want, 1e-6, f"#{case} {what}") == 0
    want_p = oracle.float_to_half(ref[0], pdt)
    assert assert_ulp16(gb[off:off + n], want_p, pdt, 1, f"#{case} params") == 0


@pytest.mark.parametrize("case", range(60))
def test_all_gather_random_configuration(zs, case):
    """zs_all_gather_step over a random worker count and flat length (also
    shorter than W, so some chunks are empty), a random sigma and, for some
    cases, replicas starting off the 16-byte boundary (the one-element
    path): every replica equals the oracle's ring simulation after every
    step."""
    rng = np.random.default_rng(17000 + case)
    world = int(rng.choice([2, 3, 4, 5, 7, 8, 13, 16, 31, 64]))
    phi = int(rng.integers(1, 3 * world if rng.random() < 0.2 else 60_000))
    sigma = int(rng.integers(0, world))
    shift = int(rng.integers(0, 4)) if rng.random() < 0.4 else 0
    announce(f"fuzz all-gather #{case}: W={world} phi={phi} sigma={sigma} shift={shift}")
    P = -(-phi // world)
    data = rng.integers(0, 1 << 16, size=(world, phi), dtype=np.uint64).astype(np.uint16)
    reps = []
    for k in range(world):
        buf = torch.zeros(phi + shift, dtype=torch.int16, device="cuda")
        buf[shift:].copy_(torch.from_numpy(data[k].view(np.int16)))
        reps.append(buf[shift:].view(torch.bfloat16))
    ref = np.zeros((world, world * P), F32)
    ref[:, :phi] = np.stack([oracle.half_to_float(d, "bf16") for d in data])
    for step in range(1, world):
        zs.zs_all_gather_step(reps, phi, step, sigma=sigma)
        want = oracle.ring_all_gather(ref.copy(), sigma, step)[:, :phi]
        got = np.stack([oracle.half_to_float(down16(r.view(torch.int16)), "bf16") for r in reps])
        assert_bits_equal(got, want, f"#{case} after step {step}")


@pytest.mark.parametrize("case", range(40))
def test_offload_step_random_configuration(zs, case):
    """zs_offload_step (GPU check, gradient in pieces, host update per piece,
    parameters back per piece) against the oracle's check, AdamW update and
    cast on the same random gradient -- and, beside it, against zs_cpu_step
    (the host update without the pipeline): random size, piece count,
    thread count, AdamW settings, loss scale and parameter dtype, sometimes
    a non-finite value (then nothing is written)."""
    rng = np.random.default_rng(21000 + case)
    c = _draw(rng)
    n, pdt = c["n"], c["pdt"]
    pieces = int(rng.choice([1, 2, 7, 16, 64, 1024]))
    threads = int(rng.integers(1, 17))
    announce(f"fuzz offload #{case}: n={n} {pdt} pieces={pieces} threads={threads} "
             f"scale={c['scale']} inject={c['inject']}")
    a = (rng.standard_normal(n) * 1e-3 * c["scale"]).astype(F32)
    if c["inject"]:
        a[int(rng.integers(0, n))] = np.inf
    state = [(rng.standard_normal(n) * s).astype(F32) for s in (0.02, 1e-4, 1e-6)]
    state[2] = np.abs(state[2])
    hp = zs.hparams(c["lr"], c["beta1"], c["beta2"], c["eps"], c["weight_decay"], c["scale"],
                    c["t"])
    ref = [x.copy() for x in state]
    ref_p = np.full(n, 7, np.uint16)
    ref_flag = zs.zs_cpu_step(*ref, a, hp, ref_p, DT[pdt], 1)
    host = [torch.from_numpy(x.copy()) for x in state]
    tdt = torch.bfloat16 if pdt == "bf16" else torch.float16
    params_dev = torch.full((n,), 7, dtype=torch.int16, device="cuda")
    grad_dev = torch.from_numpy(a).cuda()
    torch.cuda.synchronize()
    ok = zs.zs_offload_step(grad_dev, torch.empty(n, dtype=torch.float32, pin_memory=True), *host,
                            torch.empty(n, dtype=tdt, pin_memory=True), params_dev.view(tdt), hp,
                            torch.zeros(1, dtype=torch.int32, device="cuda"),
                            torch.zeros(1, dtype=torch.int32, pin_memory=True), DT[pdt], threads,
                            pieces)
    torch.cuda.synchronize()
    want = oracle_offload_update(*state, a, c["scale"], c["lr"], c["beta1"], c["beta2"],
                                 c["eps"], c["weight_decay"], c["t"], pdt)
    assert ok == (want[0] == 0) == (ref_flag == 0) == (not c["inject"])
    got_p = down16(params_dev)
    assert assert_offload_matches_oracle([x.numpy() for x in host], got_p, want, pdt,
                                         f"#{case}") == 0
    if not ok:
        assert np.all(got_p == 7), "a skipped step writes no parameters"
    for got, ref_x, what in zip(host, ref, ("master", "m", "v")):
        assert_bits_equal(got.numpy(), ref_x, f"#{case} {what} vs zs_cpu_step")
    assert np.array_equal(got_p, ref_p)


@pytest.mark.parametrize("case", range(100))
def test_device_step_random_configuration(zs, case):
    """zs_step_device (fused pass + commit kernel, the scale and bias
    corrections read from a device scaler) over the same random
    configurations, with non-finite values injected more often: a commit
    writes the oracle's step and advances the scaler by the commit rule; a
    skip restores the output set to the input set and the parameters to the
    cast of the input master, and applies the skip rule."""
    rng = np.random.default_rng(31000 + case)
    c = _draw(rng)
    c["inject"] = bool(rng.random() < 0.35)
    W, n, gdt, pdt = c["world"], c["n"], c["gdt"], c["pdt"]
    interval = int(rng.choice([0, 1, 2, 5, 2000]))
    clean0 = int(rng.integers(0, max(interval, 1)))
    dynamic = bool(rng.random() < 0.7)
    announce(f"fuzz device #{case}: " + ", ".join(f"{k}={v}" for k, v in c.items()
                                                  if k != "shifts")
             + f", interval={interval}, clean={clean0}, dynamic={dynamic}")
    g16 = [_rand16(rng, n, 1e-3 * c["scale"], gdt) for _ in range(W)]
    if c["inject"]:
        bad = 0x7F80 if gdt == "bf16" else 0x7C00
        g16[int(rng.integers(0, W))][int(rng.integers(0, n))] = bad | (1 if rng.random() < 0.5 else 0)
    master = (rng.standard_normal(n) * 0.02).astype(F32)
    m = (rng.standard_normal(n) * 1e-4).astype(F32)
    v = rng.uniform(0, 1e-6, n).astype(F32)
    acc = (rng.standard_normal(n) * c["scale"] * 1e-3).astype(F32) if c["acc"] else None
    hp = dict(lr=c["lr"], beta1=c["beta1"], beta2=c["beta2"], eps=c["eps"],
              weight_decay=c["weight_decay"])
    dg = _upload_grads(g16, c["shifts"], gdt)
    din = [up32(x) for x in (master, m, v)]
    dout = [torch.full((n,), 5.0, dtype=torch.float32, device="cuda") for _ in range(3)]
    gather = torch.full((n + c["off"] + 3,), 7, dtype=torch.int16, device="cuda")
    unused = torch.zeros(1, dtype=torch.int32, device="cuda")
    ls = zs.zs_loss_scaler(scale=c["scale"], clean_steps=clean0, growth_interval=interval,
                           dynamic=1 if dynamic else 0, step_t=c["t"] - 1, skipped=3)
    dev = zs.device_scaler_upload(zs.zs_device_scaler_make(ls, c["beta1"], c["beta2"]))
    # loss_scale and step_t here are placeholders: the device scaler supplies both
    args = zs.StepArgs(dg, c["rank"], n, *din, *dout, gather, c["off"], unused,
                       zs.hparams(**hp, loss_scale=1.0, step_t=1),
                       acc_in=up32(acc) if acc is not None else None, grad_dtype=DT[gdt],
                       param_dtype=DT[pdt], wire_dtype=WIRE_CODE[c["wire"]])
    zs.zs_step_device(args, dev)
    d = zs.device_scaler_read(dev)
    f, mo, mmo, vo, po = oracle.shard_step(g16, c["rank"], gdt, pdt, master, m, v,
                                           step_t=c["t"], acc_in=acc, loss_scale=c["scale"],
                                           threads=4, wire=c["wire"], **hp)
    assert f == (1 if c["inject"] else 0)
    assert (d.last_flag, d.epoch) == (f, 1)
    for x, want in zip(din, (master, m, v)):
        assert_bits_equal(down32(x), want, "inputs untouched")
    gb = down16(gather)
    off = c["off"]
    assert np.all(gb[:off] == 7) and np.all(gb[off + n:] == 7)
    if f == 0:
        for got, want, what in zip(dout, (mo, mmo, vo), ("master", "m", "v")):
            assert_bits_equal(down32(got), want, f"#{case} {what}")
        assert np.array_equal(gb[off:off + n], po)
        clean = clean0 + 1
        grow = dynamic and interval and clean >= interval
        assert d.step_t == c["t"] and d.skipped == 3
        assert d.clean_steps == (0 if grow else clean)
        assert d.scale == np.float32(c["scale"] * 2.0 if grow else c["scale"])
    else:
        for got, want, what in zip(dout, (master, m, v), ("master", "m", "v")):
            assert_bits_equal(down32(got), want, f"#{case} restored {what}")
        assert np.array_equal(gb[off:off + n], oracle.float_to_half(master, pdt))
        assert d.step_t == c["t"] - 1 and d.skipped == 4 and d.clean_steps == 0
        assert d.scale == np.float32(c["scale"] * 0.5 if dynamic else c["scale"])
