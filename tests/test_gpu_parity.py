"""GPU parity: every libzeroshard entry point against the CPU oracle, through
the C ABI, on the same seeded inputs.

Bars: bit-exact for the overflow flag, offsets and the summed/averaged fp32
gradient; |rel err| <= 1e-6 for fp32 master, m, v; <= 1 ulp for the 16-bit
parameters (the design performs the oracle's exact operation sequence, so
the tests also report how many elements are not bit-identical).
"""
import numpy as np
import pytest

import oracle
from gpu_util import (F32, announce, assert_bits_equal, assert_rel, assert_ulp16, down16,
                      down32, up16, up32)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def zs(hip_built):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sharded_mixed_precision_zs_amd import zeroshard
    return zeroshard


@pytest.fixture(scope="module")
def synth(hip_built):
    from sharded_mixed_precision_zs_amd import synth as s
    return s


def rand16(rng, shape, sigma, dtype):
    x = (rng.standard_normal(shape) * sigma).astype(F32)
    if dtype == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    return x.astype(np.float16).view(np.uint16)


DT = {"bf16": 0, "fp16": 1}
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _flag():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


# ---- the input generator's device twin ------------------------------------------

def test_device_generator_matches_host(zs, synth):
    for name, worker, step, micro, first, scale in (
            ("gpt2s-w8", 3, 2, 0, 123_457, None),
            ("1p3b-w4-acc4-fp16", 1, 3, 2, 7, 2.0 ** 15),
            ("7b-full-w1", 0, 1, 0, 6_999_000_000, None)):
        wl = synth.WORKLOADS[name]
        announce(f"generator {name} first={first}")
        n = 100_003
        out = torch.empty(n, dtype=torch.int16, device="cuda")
        synth.dev_grad(wl, worker, step, micro, first, out, scale=scale)
        np.testing.assert_array_equal(down16(out), synth.host_grad(wl, worker, step, micro,
                                                                   first, n, scale=scale))
        t = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3)]
        synth.dev_state(wl, first, *t)
        torch.cuda.synchronize()
        for got, want in zip(t, synth.host_state(wl, first, n)):
            assert_bits_equal(down32(got), want, f"{name} state")


# ---- zs_reduce_scatter_avg ---------------------------------------------------------

@pytest.mark.parametrize("world", [1, 2, 3, 5, 8, 63, 64])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_reduce_scatter_avg(zs, world, dtype):
    rng = np.random.default_rng(world * 7 + DT[dtype])
    n = 3000 + 37 * world + 5
    for off in (0, 1, 2, 4):                       # element offsets: all vector widths
        for rank in sorted({0, world - 1}):
            announce(f"reduce W={world} {dtype} n={n} off={off} rank={rank}")
            g16 = [rand16(rng, n + off, 1.0, dtype) for _ in range(world)]
            dev = [up16(g, dtype) for g in g16]
            views = [d[off:] for d in dev]
            out = torch.empty(n + 1, dtype=torch.float32, device="cuda")[1:] if off else \
                torch.empty(n, dtype=torch.float32, device="cuda")
            flag = _flag()
            zs.zs_reduce_scatter_avg(views, None, world, rank, n, out, False, flag, 1024.0)
            ref = np.empty(n, F32)
            parts = [g[off:] for g in g16]
            rflag = oracle.reduce_avg(parts, rank, dtype, ref, False, 1024.0)
            got = down32(out)
            assert_bits_equal(got, ref, "mean")
            assert int(flag.item()) == rflag == 0
            # a second micro-batch accumulates
            g2 = [rand16(rng, n, 1.0, dtype) for _ in range(world)]
            zs.zs_reduce_scatter_avg([up16(g, dtype) for g in g2], None, world, rank, n, out,
                                     True, flag, 1024.0)
            oracle.reduce_avg(g2, rank, dtype, ref, True, 1024.0)
            assert_bits_equal(down32(out), ref, "accumulated mean")


def test_reduce_flag_positions(zs):
    rng = np.random.default_rng(1)
    world, n = 3, 4099
    base = [rand16(rng, n, 1.0, "bf16") for _ in range(world)]
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    ref = np.empty(n, F32)
    positions = list(range(0, 70)) + list(range(2040, 2060)) + list(range(n - 70, n))
    specials = [0x7F80, 0xFF80, 0x7FC0]
    announce(f"reduce flag positions n={n}")
    for i, pos in enumerate(positions):
        parts = [b.copy() for b in base]
        parts[i % world][pos] = specials[i % 3]
        flag = _flag()
        zs.zs_reduce_scatter_avg([up16(p, "bf16") for p in parts], None, world, 0, n, out,
                                 False, flag, 1024.0)
        rflag = oracle.reduce_avg(parts, 0, "bf16", ref, False, 1024.0)
        assert int(flag.item()) == rflag == 1, pos
        assert_bits_equal(down32(out), ref, f"mean with special at {pos}")


# ---- zs_check_overflow ----------------------------------------------------------

def test_check_overflow(zs):
    rng = np.random.default_rng(2)
    n = 10_007
    a = (rng.standard_normal(n) * 100).astype(F32)
    for scale in (1.0, 1024.0, 3.0, 0.25):
        for pos, val in [(None, None), (0, np.inf), (n - 1, -np.inf), (5000, np.nan),
                         (8, F32(2.0 ** 126)), (n - 3, F32(-3e38))]:
            x = a.copy()
            if pos is not None:
                x[pos] = val
            announce(f"check scale={scale} pos={pos}")
            flag = _flag()
            zs.zs_check_overflow(up32(x), n, scale, flag)
            assert int(flag.item()) == oracle.check_overflow(x, scale), (scale, pos)
    flag = _flag()
    flag.fill_(1)
    zs.zs_check_overflow(up32(a), n, 1.0, flag)
    assert int(flag.item()) == 1  # never cleared by a call


# ---- zs_adamw_step ---------------------------------------------------------------

@pytest.mark.parametrize("scale,t", [(1.0, 1), (1024.0, 5), (3.0, 1000), (65536.0, 2)])
def test_adamw_step(zs, scale, t):
    rng = np.random.default_rng(int(scale) + t)
    for n, off in ((10_001, 0), (4097, 1), (33, 2), (1, 0)):
        announce(f"adamw n={n} off={off} scale={scale} t={t}")
        master = (rng.standard_normal(n) * 0.02).astype(F32)
        m = (rng.standard_normal(n) * 1e-4).astype(F32)
        v = rng.uniform(0, 1e-6, n).astype(F32)
        a = (rng.standard_normal(n) * 1e-3 * scale).astype(F32)
        dm, dmm, dv, da = [up32(np.concatenate([np.zeros(off, F32), x]))[off:]
                           for x in (master, m, v, a)]
        hp = zs.hparams(**HP, loss_scale=scale, step_t=t)
        zs.zs_adamw_step(dm, dmm, dv, da, n, hp)
        oracle.adamw(master, m, v, a, scale, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"],
                     HP["weight_decay"], t)
        for got, want, what in ((dm, master, "master"), (dmm, m, "m"), (dv, v, "v")):
            nbits = assert_rel(down32(got), want, 1e-6, what)
            assert nbits == 0, f"{what}: {nbits} not bit-identical"


def test_adamw_step_is_gated_by_the_flag(zs):
    rng = np.random.default_rng(3)
    n = 5000
    xs = [(rng.standard_normal(n)).astype(F32) for _ in range(4)]
    dev = [up32(x) for x in xs]
    flag = _flag()
    flag.fill_(1)
    announce("adamw gated")
    zs.zs_adamw_step(dev[0], dev[1], dev[2], dev[3], n, zs.hparams(**HP, loss_scale=1.0,
                                                                   step_t=1), flag)
    for d, x in zip(dev, xs):
        assert_bits_equal(down32(d), x, "untouched")


# ---- zs_cast_gather -------------------------------------------------------------

def _cast_patterns():
    low = sorted({(h << 12) | l for h in range(16) for l in (0, 1, 0x7FF, 0x800, 0xFFF)}
                 | {0x7FFF, 0x8000, 0x8001, 0xFFFF})
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    return (hi[:, None] | np.array(low, np.uint32)[None, :]).ravel().view(F32)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_cast_gather(zs, dtype):
    x = _cast_patterns()
    n = x.size
    ref = oracle.float_to_half(x, dtype)
    for off in (0, 3, 8):
        announce(f"cast {dtype} n={n} off={off}")
        buf = torch.full((n + off + 5,), 7, dtype=torch.int16, device="cuda")
        zs.zs_cast_gather(up32(x), buf, DT[dtype], off, n)
        got = down16(buf)
        assert np.all(got[:off] == 7) and np.all(got[off + n:] == 7)
        nd = assert_ulp16(got[off:off + n], ref, dtype, 0, "cast")
        assert nd == 0
    flag = _flag()
    flag.fill_(1)
    buf = torch.full((n,), 7, dtype=torch.int16, device="cuda")
    zs.zs_cast_gather(up32(x), buf, DT[dtype], 0, n, flag)
    assert np.all(down16(buf) == 7)


# ---- zs_step_fused ------------------------------------------------------------------

def _fused_case(zs, rng, world, rank, n, gdt, pdt, with_acc, off, scale=1024.0, t=3,
                inject=None):
    g16 = [rand16(rng, n, 1e-3 * scale, gdt) for _ in range(world)]
    if inject is not None:
        w, pos, val = inject
        g16[w][pos] = val
    master = (rng.standard_normal(n) * 0.02).astype(F32)
    m = (rng.standard_normal(n) * 1e-4).astype(F32)
    v = rng.uniform(0, 1e-6, n).astype(F32)
    acc = (rng.standard_normal(n) * scale * 1e-3).astype(F32) if with_acc else None
    pad = np.zeros(off, np.uint16)
    dg = [up16(np.concatenate([pad, g]), gdt)[off:] for g in g16]
    din = [up32(x) for x in (master, m, v)]
    dout = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3)]
    gather = torch.full((n + off + 3,), 7, dtype=torch.int16, device="cuda")
    flag = _flag()
    hp = zs.hparams(**HP, loss_scale=scale, step_t=t)
    args = zs.StepArgs(dg, rank, n, *din, *dout, gather, off, flag, hp,
                       acc_in=up32(acc) if with_acc else None, grad_dtype=DT[gdt],
                       param_dtype=DT[pdt])
    zs.zs_step_fused(args)
    ref = oracle.shard_step(g16, rank, gdt, pdt, master, m, v, step_t=t, acc_in=acc,
                            loss_scale=scale, threads=4, **HP)
    return dict(flag=int(flag.item()), out=[down32(d) for d in dout], gather=down16(gather),
                din=din, ins=(master, m, v), ref=ref, off=off, n=n)


@pytest.mark.parametrize("world", [1, 3, 8, 64])
@pytest.mark.parametrize("gdt,pdt", [("bf16", "bf16"), ("fp16", "fp16"), ("bf16", "fp16")])
def test_step_fused(zs, world, gdt, pdt):
    rng = np.random.default_rng(world + 100 * DT[gdt] + 10 * DT[pdt])
    for n, off, with_acc, rank in ((20_011, 0, False, 0), (5003, 2, True, world - 1),
                                   (777, 1, False, world // 2), (8, 0, True, 0)):
        announce(f"fused W={world} {gdt}/{pdt} n={n} off={off} acc={with_acc} rank={rank}")
        r = _fused_case(zs, rng, world, rank, n, gdt, pdt, with_acc, off)
        rflag, rm, rmm, rv, rp = r["ref"]
        assert r["flag"] == rflag == 0
        for got, want, what in zip(r["out"], (rm, rmm, rv), ("master", "m", "v")):
            assert assert_rel(got, want, 1e-6, what) == 0
        g = r["gather"]
        assert np.all(g[:off] == 7) and np.all(g[off + n:] == 7)
        assert assert_ulp16(g[off:off + n], rp, pdt, 1, "params") == 0


SENTINEL = np.uint32(0x7FC0DEAD).view(F32)  # a NaN no arithmetic produces


def _grouped(arrs, n):
    """master, m, v (n floats each) in the grouped state layout, the slots
    past n in the last group holding SENTINEL."""
    G = -(-n // 1024)
    buf = np.full((G, 3, 1024), SENTINEL, dtype=F32)
    for k, x in enumerate(arrs):
        flat = np.full(G * 1024, SENTINEL, dtype=F32)
        flat[:n] = x
        buf[:, k, :] = flat.reshape(G, 1024)
    return buf.ravel()


def _ungrouped(buf, n):
    b = buf.reshape(-1, 3, 1024)
    return [b[:, k, :].ravel()[:n] for k in range(3)], [b[:, k, :].ravel()[n:] for k in range(3)]


def _fused_case_grouped(zs, rng, world, rank, n, gdt, pdt, with_acc, scale=1024.0, t=3,
                        inject=None, wire=None):
    g16 = [rand16(rng, n, 1e-3 * scale, gdt) for _ in range(world)]
    if inject is not None:
        w, pos, val = inject
        g16[w][pos] = val
    master = (rng.standard_normal(n) * 0.02).astype(F32)
    m = (rng.standard_normal(n) * 1e-4).astype(F32)
    v = rng.uniform(0, 1e-6, n).astype(F32)
    acc = (rng.standard_normal(n) * scale * 1e-3).astype(F32) if with_acc else None
    dg = [up16(g, gdt) for g in g16]
    gin = up32(_grouped((master, m, v), n))
    gout = up32(np.full(zs.grouped_len(n), SENTINEL, dtype=F32))
    gather = torch.full((n + 8,), 7, dtype=torch.int16, device="cuda")
    flag = _flag()
    hp = zs.hparams(**HP, loss_scale=scale, step_t=t)
    args = zs.StepArgs(dg, rank, n, gin, None, None, gout, None, None, gather, 0, flag, hp,
                       acc_in=up32(acc) if with_acc else None, grad_dtype=DT[gdt],
                       param_dtype=DT[pdt], state_layout=zs.ZS_STATE_GROUPED,
                       wire_dtype=WIRE[wire] if wire else 0)
    zs.zs_step_fused(args)
    ref = oracle.shard_step(g16, rank, gdt, pdt, master, m, v, step_t=t, acc_in=acc,
                            loss_scale=scale, threads=4, wire=wire, **HP)
    return dict(flag=int(flag.item()), gout=down32(gout), gin=down32(gin), gather=down16(gather),
                ins=(master, m, v), ref=ref, n=n)


# W = 4 takes the batched sum; from W = 5 on the rolling sum, whose last
# round holds (W - 1) mod 4 workers: 5, 9, 13, 17 -> 0; 6, 10 -> 1; 7 -> 2;
# 8, 64 -> 3 (and 13 and 64 run at the 6-blocks-per-CU shape, 5 to 12 at 8)
@pytest.mark.parametrize("world", [1, 3, 4, 5, 6, 7, 8, 10, 13, 17, 64])
@pytest.mark.parametrize("gdt,pdt", [("bf16", "bf16"), ("fp16", "fp16"), ("bf16", "fp16")])
def test_step_fused_grouped_state(zs, world, gdt, pdt):
    """The grouped state layout writes the oracle's state and parameters bit
    for bit, ragged shards and accumulated micro-batches included, and
    leaves the slots past n of its last group alone."""
    rng = np.random.default_rng(7 + world + 100 * DT[gdt] + 10 * DT[pdt])
    for n, with_acc, rank in ((20_011, False, 0), (5003, True, world - 1), (777, False, world // 2),
                              (8, True, 0), (3 * 1024 + 5, False, 0), (4096, True, 0)):
        announce(f"fused grouped W={world} {gdt}/{pdt} n={n} acc={with_acc} rank={rank}")
        r = _fused_case_grouped(zs, rng, world, rank, n, gdt, pdt, with_acc)
        rflag, rm, rmm, rv, rp = r["ref"]
        assert r["flag"] == rflag == 0
        got, tails = _ungrouped(r["gout"], n)
        for g, want, what in zip(got, (rm, rmm, rv), ("master", "m", "v")):
            assert assert_rel(g, want, 1e-6, what) == 0
        for tail in tails:
            assert_bits_equal(tail, np.full(tail.size, SENTINEL, dtype=F32), "slots past n")
        g = r["gather"]
        assert np.all(g[n:] == 7)
        assert assert_ulp16(g[:n], rp, pdt, 1, "params") == 0


@pytest.mark.parametrize("world", [4, 6, 64])
@pytest.mark.parametrize("wire", ["bf16", "fp16"])
def test_step_fused_grouped_wire(zs, world, wire):
    """The grouped layout with 16-bit partial sums on the ring equals the
    oracle's ring with the same wire rounding."""
    gdt = "bf16" if wire == "bf16" else "fp16"
    rng = np.random.default_rng(31 + world + 7 * WIRE[wire])
    for n, with_acc in ((12_345, False), (4097, True)):
        announce(f"fused grouped wire={wire} W={world} n={n} acc={with_acc}")
        r = _fused_case_grouped(zs, rng, world, 0, n, gdt, gdt, with_acc, t=2, wire=wire)
        rflag, rm, rmm, rv, rp = r["ref"]
        assert r["flag"] == rflag == 0
        got, _ = _ungrouped(r["gout"], n)
        for g, want, what in zip(got, (rm, rmm, rv), ("master", "m", "v")):
            assert assert_rel(g, want, 1e-6, what) == 0
        assert assert_ulp16(r["gather"][:n], rp, gdt, 1, "params") == 0


@pytest.mark.parametrize("world,window", [(5, "2.56,0.25"), (8, "2.56,0.25"), (64, "2.56,0.25"),
                                          (8, "30.72,0.001"), (8, "0.2,0.5")])
def test_step_fused_grouped_write_windows(zs, world, window, monkeypatch):
    """With write windows forced on (a 2.56 us period, a quarter of it
    open, so that even a small shard's launch spans many periods; or the
    production period with an open part below the 16-tick floor, which the
    library widens; or a period under the 64-tick floor, which means no
    windows) the rolling grouped step still writes the oracle's state and
    parameters: the windows only delay the stores."""
    monkeypatch.setenv("ZS_FUSED_WRITE_WINDOW", window)
    rng = np.random.default_rng(57 + world)
    for n, with_acc, gdt in ((200_003, False, "bf16"), (33_333, True, "fp16")):
        announce(f"fused grouped write windows {window} W={world} n={n} acc={with_acc}")
        r = _fused_case_grouped(zs, rng, world, world - 1, n, gdt, gdt, with_acc)
        rflag, rm, rmm, rv, rp = r["ref"]
        assert r["flag"] == rflag == 0
        got, _ = _ungrouped(r["gout"], n)
        for g, want, what in zip(got, (rm, rmm, rv), ("master", "m", "v")):
            assert assert_rel(g, want, 1e-6, what) == 0
        assert assert_ulp16(r["gather"][:n], rp, gdt, 1, "params") == 0


def test_step_fused_grouped_skip_and_alignment(zs):
    """A skipped grouped step leaves the input buffer as it was; a grouped
    step whose gather slice is not aligned for 4-element vectors is refused."""
    rng = np.random.default_rng(11)
    n = 9000
    announce("fused grouped skip")
    r = _fused_case_grouped(zs, rng, 4, 1, n, "fp16", "fp16", True, scale=65536.0,
                            inject=(2, 4321, 0x7E00))
    assert r["flag"] == r["ref"][0] == 1
    assert_bits_equal(r["gin"], _grouped(r["ins"], n), "input set after a skipped step")
    g16 = [rand16(rng, 64, 1.0, "bf16") for _ in range(2)]
    gin = up32(np.zeros(zs.grouped_len(64), F32))
    gout = up32(np.zeros(zs.grouped_len(64), F32))
    gather = torch.zeros(80, dtype=torch.int16, device="cuda")
    args = zs.StepArgs([up16(g, "bf16") for g in g16], 0, 64, gin, None, None, gout, None, None,
                       gather, 1, _flag(), zs.hparams(**HP, loss_scale=1.0, step_t=1),
                       grad_dtype=DT["bf16"], param_dtype=DT["bf16"],
                       state_layout=zs.ZS_STATE_GROUPED)
    with pytest.raises(zs.ZsError) as e:
        zs.zs_step_fused(args)
    assert e.value.status == zs.ZS_ERR_UNSUPPORTED


def test_step_fused_skip_leaves_the_input_set(zs):
    rng = np.random.default_rng(5)
    n = 9000
    announce("fused skip")
    r = _fused_case(zs, rng, 4, 1, n, "fp16", "fp16", True, 0, scale=65536.0,
                    inject=(2, 4321, 0x7E00))
    assert r["flag"] == r["ref"][0] == 1
    for d, x in zip(r["din"], r["ins"]):
        assert_bits_equal(down32(d), x, "input set after a skipped step")


def test_step_fused_equals_unfused(zs):
    rng = np.random.default_rng(6)
    world, rank, n = 8, 3, 100_003
    announce("fused vs unfused")
    g16 = [rand16(rng, n, 1e-3 * 65536, "bf16") for _ in range(world)]
    dg = [up16(g, "bf16") for g in g16]
    state = [(rng.standard_normal(n) * s).astype(F32) for s in (0.02, 1e-4, 1e-6)]
    state[2] = np.abs(state[2])
    hp = zs.hparams(**HP, loss_scale=65536.0, step_t=2)
    # fused
    din = [up32(x) for x in state]
    dout = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3)]
    gf = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    flag = _flag()
    zs.zs_step_fused(zs.StepArgs(dg, rank, n, *din, *dout, gf, 0, flag, hp))
    # unfused, in place, bucketed: the partition in three ranges, last first
    du = [up32(x) for x in state]
    gpart = torch.empty(n, dtype=torch.float32, device="cuda")
    gu = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    flag2 = _flag()
    cuts = [0, 30_000, 70_001, n]
    for lo, hi in reversed(list(zip(cuts[:-1], cuts[1:]))):
        zs.zs_reduce_scatter_avg([d[lo:hi] for d in dg], None, world, rank, hi - lo,
                                 gpart[lo:hi], False, flag2, 65536.0)
    zs.zs_adamw_step(*du, gpart, n, hp, flag2)
    zs.zs_cast_gather(du[0], gu, None, 0, n, flag2)
    assert int(flag.item()) == int(flag2.item()) == 0
    for a, b in zip(dout, du):
        assert_bits_equal(down32(a), down32(b), "fused vs unfused")
    assert np.array_equal(down16(gf), down16(gu))


# ---- zs_step_commit ---------------------------------------------------------------

def test_step_commit_commits_skips_and_times(zs):
    import ctypes as C
    rng = np.random.default_rng(8)
    world, rank, n = 4, 1, 50_000
    hip = C.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
    hip.hipEventDestroy.argtypes = [C.c_void_p]
    ev = [C.c_void_p(), C.c_void_p()]
    for e in ev:
        assert hip.hipEventCreate(C.byref(e)) == 0
    master = (rng.standard_normal(n) * 0.02).astype(F32)
    m = np.zeros(n, F32)
    v = np.zeros(n, F32)
    sets = [[up32(x) for x in (master, m, v)],
            [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3)]]
    gather = [torch.zeros(n, dtype=torch.float16, device="cuda") for _ in range(2)]
    flags = torch.zeros(8, dtype=torch.int32, device="cuda")
    host_flag = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    scaler = zs.zs_loss_scaler(scale=65536.0, clean_steps=0, growth_interval=2, dynamic=1,
                               step_t=0, skipped=0)
    ref = oracle.Scaler(65536.0, 2)
    state = (master, m, v)
    cur = 0
    for step, inject in enumerate([False, True, False, False, True], start=1):
        announce(f"step_commit step {step} inject={inject}")
        g16 = [rand16(rng, n, 1e-3 * ref.scale, "fp16") for _ in range(world)]
        if inject:
            g16[step % world][123 + step] = 0x7C00
        dg = [up16(g, "fp16") for g in g16]
        args = zs.StepArgs(dg, rank, n, *sets[cur], *sets[1 - cur], gather[1 - cur], 0,
                           flags[step:step + 1], zs.hparams(**HP, loss_scale=1.0, step_t=999))
        ok = zs.zs_step_commit(args, scaler, host_flag, None, ev[0].value, ev[1].value)
        f, mo, mmo, vo, po = oracle.shard_step(g16, rank, "fp16", "fp16", *state,
                                               loss_scale=ref.scale, step_t=ref.t + 1, **HP)
        assert ok == (f == 0) and ok == (not inject)
        ref.update(f)
        assert (scaler.scale, scaler.step_t, scaler.skipped, scaler.clean_steps) == \
            (ref.scale, ref.t, ref.skipped, ref.clean)
        ms = C.c_float()
        assert hip.hipEventElapsedTime(C.byref(ms), ev[0], ev[1]) == 0
        assert 0.0 < ms.value < 1000.0
        if ok:
            cur = 1 - cur
            state = (mo, mmo, vo)
            assert assert_ulp16(down16(gather[cur]), po, "fp16", 1, "params") == 0
        for got, want in zip(sets[cur], state):
            assert_bits_equal(down32(got), want, f"state after step {step}")
    for e in ev:
        hip.hipEventDestroy(e)


# ---- exhaustive conversions on the device ------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_cast_all_fp32_patterns(zs, dtype):
    """Every one of the 2^32 fp32 bit patterns through zs_cast_gather's
    hardware round-to-nearest-even convert, against the oracle (NaN by class)."""
    chunk = 1 << 28
    out = torch.empty(chunk, dtype=torch.int16, device="cuda")
    for c in range(1 << 32 >> 28):
        announce(f"cast all patterns {dtype} chunk {c}")
        x = torch.arange(c * chunk, (c + 1) * chunk, dtype=torch.int64, device="cuda")
        x = x.to(torch.int32).view(torch.float32)
        zs.zs_cast_gather(x, out, DT[dtype], 0, chunk)
        got = down16(out)
        del x
        host = np.arange(c * chunk, (c + 1) * chunk, dtype=np.uint64).astype(np.uint32).view(F32)
        want = oracle.float_to_half(host, dtype)
        assert assert_ulp16(got, want, dtype, 0, f"{dtype} chunk {c}") == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_widen_all_16bit_patterns(zs, dtype):
    """Every 16-bit pattern widened by the kernels (W = 1: the sum is the
    value itself, the average divides by 1) against the oracle."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    out = torch.empty(bits.size, dtype=torch.float32, device="cuda")
    flag = _flag()
    announce(f"widen all {dtype} patterns")
    zs.zs_reduce_scatter_avg([up16(bits, dtype)], None, 1, 0, bits.size, out, False, flag, 1.0)
    assert_bits_equal(down32(out), oracle.half_to_float(bits, dtype), f"widen {dtype}")
    assert int(flag.item()) == 1  # the NaN and inf patterns raise the flag


# ---- 16-bit wire mode -------------------------------------------------------------

WIRE = {"fp32": 0, "bf16": 1, "fp16": 2}


@pytest.mark.parametrize("world", [2, 3, 8, 64])
@pytest.mark.parametrize("dtype,wire", [("bf16", "bf16"), ("fp16", "fp16"), ("fp16", "bf16"),
                                        ("bf16", "fp16")])
def test_reduce_scatter_avg_wire(zs, world, dtype, wire):
    rng = np.random.default_rng(world + 10 * WIRE[wire])
    n = 5000 + 13 * world
    for off in (0, 1):
        rank = world - 1 if off else 0
        announce(f"reduce wire={wire} W={world} {dtype} off={off}")
        g16 = [rand16(rng, n + off, 1.0, dtype) for _ in range(world)]
        views = [up16(g, dtype)[off:] for g in g16]
        out = torch.empty(n, dtype=torch.float32, device="cuda")
        flag = _flag()
        zs.zs_reduce_scatter_avg(views, None, world, rank, n, out, False, flag, 1.0,
                                 wire_dtype=WIRE[wire])
        ref = np.empty(n, F32)
        rflag = oracle.reduce_avg([g[off:] for g in g16], rank, dtype, ref, False, 1.0, wire=wire)
        assert_bits_equal(down32(out), ref, f"wire {wire} mean")
        assert int(flag.item()) == rflag


@pytest.mark.parametrize("world", [1, 4, 64])
@pytest.mark.parametrize("wire", ["bf16", "fp16"])
def test_step_fused_wire(zs, world, wire):
    rng = np.random.default_rng(world + 7)
    gdt = "bf16" if wire == "bf16" else "fp16"
    for n, with_acc in ((20_011, False), (4099, True)):
        announce(f"fused wire={wire} W={world} n={n} acc={with_acc}")
        g16 = [rand16(rng, n, 1e-3 * 1024, gdt) for _ in range(world)]
        master = (rng.standard_normal(n) * 0.02).astype(F32)
        m = (rng.standard_normal(n) * 1e-4).astype(F32)
        v = rng.uniform(0, 1e-6, n).astype(F32)
        acc = (rng.standard_normal(n) * 1.0).astype(F32) if with_acc else None
        dout = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3)]
        gather = torch.zeros(n, dtype=torch.int16, device="cuda")
        flag = _flag()
        args = zs.StepArgs([up16(g, gdt) for g in g16], 0, n, *[up32(x) for x in (master, m, v)],
                           *dout, gather, 0, flag, zs.hparams(**HP, loss_scale=1024.0, step_t=2),
                           acc_in=up32(acc) if with_acc else None, grad_dtype=DT[gdt],
                           param_dtype=DT[gdt], wire_dtype=WIRE[wire])
        zs.zs_step_fused(args)
        f, mo, mmo, vo, po = oracle.shard_step(g16, 0, gdt, gdt, master, m, v, loss_scale=1024.0,
                                               step_t=2, acc_in=acc, wire=wire, **HP)
        assert int(flag.item()) == f
        for got, want, what in zip(dout, (mo, mmo, vo), ("master", "m", "v")):
            assert assert_rel(down32(got), want, 1e-6, what) == 0
        assert assert_ulp16(down16(gather), po, gdt, 1, "params") == 0


# ---- ring all-gather of the parameters --------------------------------------------

def test_all_gather_replays_the_three_gpu_example(zs):
    """[Notes] 二: after the scatter-reduce GPU k holds the total of chunk
    k+1 (sigma = 1); the golden file lists which totals each GPU holds after
    each all-gather step."""
    from conftest import golden_rows
    L, W = 1000, 3
    totals = [up16(np.full(L, bits, np.uint16), "bf16") for bits in (0x3F80, 0x4000, 0x4040)]
    reps = [torch.zeros(W * L, dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    for k in range(W):
        c = (k + 1) % W
        reps[k][c * L:(c + 1) * L] = totals[c]
    names = {"A": 0, "B": 1, "C": 2}
    for step in (1, 2):
        announce(f"all-gather example step {step}")
        zs.zs_all_gather_step(reps, W * L, step, sigma=1)
        for row in golden_rows("ring_three_gpu_example.txt"):
            if row[0] == "all_gather" and int(row[1]) == step:
                gpu, c = int(row[2]), names[row[3]]
                got = down16(reps[gpu][c * L:(c + 1) * L].view(torch.int16))
                assert np.all(got == down16(totals[c].view(torch.int16))), (step, row)
    for k in range(W):  # every GPU holds every total
        for c in range(W):
            assert torch.equal(reps[k][c * L:(c + 1) * L], totals[c])


@pytest.mark.parametrize("world,phi,sigma", [(2, 100_000, 0), (3, 100_003, 1), (5, 77_777, 0),
                                             (8, 1 << 20, 0), (64, 1_000_001, 0), (64, 64 * 4096, 1)])
def test_all_gather_matches_the_oracle(zs, world, phi, sigma):
    rng = np.random.default_rng(world + phi)
    P = -(-phi // world)
    announce(f"all-gather W={world} phi={phi} sigma={sigma}")
    data = rng.integers(0, 1 << 16, size=(world, phi), dtype=np.uint64).astype(np.uint16)
    reps = [up16(data[k], "bf16") for k in range(world)]

    def oracle_after(steps):
        ref = np.zeros((world, world * P), F32)
        ref[:, :phi] = np.stack([oracle.half_to_float(d, "bf16") for d in data])
        return oracle.ring_all_gather(np.ascontiguousarray(ref), sigma, steps)[:, :phi]

    for step in range(1, world):
        zs.zs_all_gather_step(reps, phi, step, sigma=sigma)
        if step in (1, world // 2, world - 1):
            got = np.stack([oracle.half_to_float(down16(r.view(torch.int16)), "bf16")
                            for r in reps])
            assert_bits_equal(got, oracle_after(step), f"after step {step}")


@pytest.mark.parametrize("W,phi", [(4, 4 * 50_003 + 3), (4, 9), (5, 13), (7, 6995), (64, 64 * 1009 - 17)])
def test_sharded_step_over_all_ranks_then_all_gather(zs, W, phi):
    """A whole ZeRO-2 step for W ranks on one GPU: every rank's fused step
    on its own partition (gradients reduced in that rank's ring order), then
    the ring all-gather; every replica must hold the oracle's parameters.
    phi = 9, W = 4 leaves the last rank an empty partition (P = 3); 13 over
    5 leaves it one element; 6995 over 7 a ragged one."""
    rng = np.random.default_rng(77 + phi)
    P = -(-phi // W)
    announce(f"sharded step W={W} phi={phi}")
    grads = [rand16(rng, phi, 1e-3 * 1024, "bf16") for _ in range(W)]
    master = (rng.standard_normal(phi) * 0.02).astype(F32)
    dgrads = [up16(g, "bf16") for g in grads]
    reps = [torch.zeros(phi, dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    flags = torch.zeros(W, dtype=torch.int32, device="cuda")
    want = np.empty(phi, np.uint16)
    for r in range(W):
        p, off, cnt = oracle.partition(phi, W, r)
        # an empty partition still passes valid (one-element) buffers
        room = max(cnt, 1)
        mst = np.zeros(room, F32)
        mst[:cnt] = master[off:off + cnt]
        din = [up32(mst), up32(np.zeros(room, F32)), up32(np.zeros(room, F32))]
        dout = [torch.empty(room, dtype=torch.float32, device="cuda") for _ in range(3)]
        args = zs.StepArgs([g[min(off, phi - 1):] for g in dgrads], r, cnt, *din, *dout, reps[r],
                           min(off, phi), flags[r:r + 1],
                           zs.hparams(**HP, loss_scale=1024.0, step_t=1))
        zs.zs_step_fused(args)
        if cnt == 0:
            continue
        f, mo, mmo, vo, po = oracle.shard_step([g[off:off + cnt] for g in grads], r, "bf16",
                                               "bf16", master[off:off + cnt],
                                               np.zeros(cnt, F32), np.zeros(cnt, F32),
                                               loss_scale=1024.0, step_t=1, **HP)
        want[off:off + cnt] = po
    for step in range(1, W):
        zs.zs_all_gather_step(reps, phi, step)
    assert not flags.any()
    for k in range(W):
        assert np.array_equal(down16(reps[k].view(torch.int16)), want), k


def test_step_fused_vector_widths_agree(zs):
    """The same step at element offsets 0, 4, 2 and 1 of the gradient and
    gather buffers takes the 8-, 4-, 2- and 1-element vector paths (different
    grids and tile shapes); every result is bit-identical."""
    rng = np.random.default_rng(11)
    world, rank, n = 5, 2, 50_021
    g16 = [rand16(rng, n, 1e-3 * 1024.0, "bf16") for _ in range(world)]
    state = [(rng.standard_normal(n) * 0.02).astype(F32), (rng.standard_normal(n) * 1e-4).astype(F32),
             rng.uniform(0, 1e-6, n).astype(F32)]
    hp = zs.hparams(**HP, loss_scale=1024.0, step_t=4)
    results = []
    for off in (0, 4, 2, 1):
        announce(f"vector widths: offset {off}")
        pad = np.zeros(off, np.uint16)
        dg = [up16(np.concatenate([pad, g]), "bf16")[off:] for g in g16]
        din = [up32(x) for x in state]
        dout = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3)]
        gather = torch.zeros(n + off, dtype=torch.int16, device="cuda")
        flag = _flag()
        zs.zs_step_fused(zs.StepArgs(dg, rank, n, *din, *dout, gather, off, flag, hp,
                                     grad_dtype=0, param_dtype=0))
        assert int(flag.item()) == 0
        results.append(([down32(d) for d in dout], down16(gather)[off:]))
    for outs, params in results[1:]:
        for a, b in zip(outs, results[0][0]):
            assert_bits_equal(a, b, "vector width")
        assert np.array_equal(params, results[0][1])


@pytest.mark.parametrize("eps", [1e-8, 0.0])
def test_step_fused_special_state_values(zs, eps):
    """master, m and v drawn from special values (signed zeros, subnormals,
    values near the fp32 maximum, infinities, NaN) with ordinary gradients:
    the kernel's IEEE behaviour (subnormals kept, correctly rounded divide
    and square root, inf and NaN propagation, 0/0 when eps = 0) equals the
    oracle's element for element; NaN compared by class."""
    rng = np.random.default_rng(int(eps == 0.0) + 31)
    world, rank, n = 3, 1, 4099
    specials = np.array([0.0, -0.0, 1e-45, -1e-45, 1.17549421e-38, 5.877e-39, 1e-30, 3.4e38,
                         -3.4e38, 1.7e38, np.inf, -np.inf, np.nan, 1.0, -1.0, 1e-3], F32)
    master = specials[rng.integers(0, specials.size, n)]
    m = specials[rng.integers(0, specials.size, n)]
    v = np.abs(specials[rng.integers(0, specials.size, n)])
    g16 = [rand16(rng, n, 1e-3 * 1024.0, "bf16") for _ in range(world)]
    hp = dict(HP, eps=eps)
    announce(f"special state values eps={eps}")
    din = [up32(x) for x in (master, m, v)]
    dout = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3)]
    gather = torch.zeros(n, dtype=torch.int16, device="cuda")
    flag = _flag()
    zs.zs_step_fused(zs.StepArgs([up16(g, "bf16") for g in g16], rank, n, *din, *dout, gather, 0,
                                 flag, zs.hparams(**hp, loss_scale=1024.0, step_t=2),
                                 grad_dtype=0, param_dtype=0))
    f, mo, mmo, vo, po = oracle.shard_step(g16, rank, "bf16", "bf16", master, m, v,
                                           loss_scale=1024.0, step_t=2, **hp)
    assert int(flag.item()) == f == 0      # the flag looks at gradients only
    for got, want, what in zip(dout, (mo, mmo, vo), ("master", "m", "v")):
        assert_bits_equal(down32(got), want, what)
    assert assert_ulp16(down16(gather), po, "bf16", 0, "params") == 0


def test_flag_ring_wraps_on_the_steps_stream(zs):
    """ShardState's host-commit flow takes a fresh zeroed flag slot per step
    from a ring of 256 and re-zeroes the ring on the stream of the step that
    wraps it. Step 5 overflows (slot 4 set); step 261 reuses slot 4 with
    finite gradients and must commit; step 100 overflows through
    launch()/finish(), whose flag readback must be ordered after the step on
    its stream. Steps run on a side stream through step() and
    launch()/finish() alternately; the final state equals the same schedule
    on the default stream, bit for bit."""
    from sharded_mixed_precision_zs_amd import shard
    world, n, steps = 2, 1024, 300
    rng = np.random.default_rng(31)
    g16 = [rand16(rng, n, 1e-3 * 1024, "bf16") for _ in range(world)]
    state = [(rng.standard_normal(n) * s).astype(F32) for s in (0.02, 1e-4, 1e-6)]
    state[2] = np.abs(state[2])

    def run(stream):
        st = shard.ShardState(n, world, 0, 0, n, zs.ZS_BF16, zs.ZS_BF16, shard.AdamW(**HP),
                              1024.0)
        for dst, x in zip((st.master, st.m, st.v), state):
            dst.copy_(torch.from_numpy(x))
        good = [up16(g, "bf16") for g in g16]
        bad = [g.clone() for g in good]
        bad[1][77] = float("inf")
        torch.cuda.synchronize()
        outcome = []
        for step in range(1, steps + 1):
            grads = bad if step in (5, 100) else good
            if step % 2:
                outcome.append(st.step(grads, stream=stream))
            else:
                outcome.append(st.finish(st.launch(grads, stream=stream), stream=stream))
        torch.cuda.synchronize()
        return st, outcome

    announce("flag ring wrap on a side stream")
    side, got = run(torch.cuda.Stream())
    assert got[4] is False and got[99] is False and got[260] is True
    assert got.count(False) == 2 and side.t == steps - 2 and side.scaler.skipped == 2
    announce("flag ring wrap on the default stream")
    ref, want = run(None)
    assert got == want
    for a, b, what in ((side.master, ref.master, "master"), (side.m, ref.m, "m"),
                       (side.v, ref.v, "v")):
        assert_bits_equal(down32(a), down32(b), f"flag ring {what}")
    assert np.array_equal(down16(side.params), down16(ref.params))
