"""The device-resident commit or skip (zs_step_device) on the GPU.

The decision of dynamic loss scaling (skip a step whose unscaled gradient is
not finite, adjust the scale) runs in a kernel against a scaler kept in
device memory, so steps queue back to back with no host round trip. These
tests check that it changes nothing else: queued device steps equal the
host-synchronous flow bit for bit (skipped steps included), the bias
corrections formed on the device from the running beta powers equal the
oracle's at every step t, the scaler follows the oracle's rule, and a step
captured in a HIP graph replays to the eager result.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from gpu_util import F32, announce, assert_bits_equal, assert_rel, assert_ulp16, down16, down32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def env(hip_built):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sharded_mixed_precision_zs_amd import shard, synth, zeroshard
    return zeroshard, synth, shard


def _make(env, wl, device_commit, **kw):
    zs, synth, shard = env
    n = wl.n
    opt = shard.AdamW(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay)
    st = shard.ShardState(n, wl.world, 0, 0, n, wl.param_dtype, wl.grad_dtype, opt,
                          kw.pop("loss_scale", wl.loss_scale), accumulate=wl.accum > 1,
                          device_commit=device_commit, **kw)
    st.fill_state(lambda first, count, *t: synth.dev_state(wl, first, *t))
    grads = torch.empty((wl.world, -(-n // 128) * 128), dtype=torch.int16, device="cuda")
    return st, [grads[k, :n] for k in range(wl.world)]


def _same_state(a, b, what):
    for k, name in enumerate(("master", "m", "v")):
        assert_bits_equal(down32(a.state(k)), down32(b.state(k)), f"{what} {name}")
    assert np.array_equal(down16(a.params.view(torch.int16)), down16(b.params.view(torch.int16))), \
        f"{what} params"


@pytest.mark.parametrize("wire", [0, 1])
def test_queued_device_steps_equal_host_commit(env, wire):
    """Six steps queued without any synchronization (gradients regenerated
    on the same stream between them), one of them hit by injected inf/NaN,
    against the host-synchronous zs_step_commit flow; fp32 and bf16 ring
    partials."""
    zs, synth, shard = env
    wl = dataclasses.replace(synth.WORKLOADS["gpt2s-w8"], phi=8 * 250_003, steps=6,
                             inject_steps=(3,), inject_rate=1e-3, name="queued")
    host, gh = _make(env, wl, False, wire_dtype=wire)
    dev, gd = _make(env, wl, True, wire_dtype=wire)
    announce(f"queued device steps vs host commit, wire {wire}")
    committed = []
    for step in range(1, wl.steps + 1):
        for k in range(wl.world):
            synth.dev_grad(wl, k, step, 0, 0, gh[k], scale=wl.loss_scale)
            synth.dev_grad(wl, k, step, 0, 0, gd[k], scale=wl.loss_scale)
        committed.append(host.step(gh))
        dev.step_device(gd)
    assert committed == [True, True, False, True, True, True]
    d = dev.sync_scaler()
    # six steps run (epoch 6); the third (epoch 2) overflowed; the last ran at epoch 5
    assert (d.step_t, d.skipped, d.last_flag) == (5, 1, 0)
    assert (d.epoch, d.flag_epoch, d.checked_epoch) == (6, 3, 5)
    assert d.scale == wl.loss_scale
    _same_state(host, dev, "queued")


@pytest.mark.parametrize("windows", [None, "2.56,0.25"])
@pytest.mark.parametrize("device_commit", [False, True])
def test_grouped_state_equals_split(env, device_commit, windows, monkeypatch):
    """Six steps over a shard whose length is not a multiple of the group
    (the third skipped for an injected inf/NaN) with the grouped state
    layout equal the split layout bit for bit: the state, the parameters
    and the scaler, through both commit flows, and state_dict round trips;
    also with the grouped step's write windows forced on (a 2.56 us period
    with a quarter open), which only delay its stores."""
    zs, synth, shard = env
    if windows:
        monkeypatch.setenv("ZS_FUSED_WRITE_WINDOW", windows)
    wl = dataclasses.replace(synth.WORKLOADS["gpt2s-w8"], phi=8 * 250_003, steps=6,
                             inject_steps=(3,), inject_rate=1e-3, name="grouped")
    split, gs = _make(env, wl, device_commit)
    grouped, gg = _make(env, wl, device_commit, state_layout="grouped")
    announce(f"grouped vs split state, device commit {device_commit}")
    _same_state(split, grouped, "initial")
    for step in range(1, wl.steps + 1):
        for k in range(wl.world):
            synth.dev_grad(wl, k, step, 0, 0, gs[k], scale=wl.loss_scale)
            synth.dev_grad(wl, k, step, 0, 0, gg[k], scale=wl.loss_scale)
        if device_commit:
            split.step_device(gs)
            grouped.step_device(gg)
        else:
            assert split.step(gs) == grouped.step(gg)
    if device_commit:
        a, b = split.sync_scaler(), grouped.sync_scaler()
        assert (a.step_t, a.skipped, a.scale) == (b.step_t, b.skipped, b.scale) == \
            (5, 1, wl.loss_scale)
    _same_state(split, grouped, "after six steps")
    sd = grouped.state_dict()
    for k, key in enumerate(("master", "m", "v")):
        assert_bits_equal(sd[key].numpy(), down32(split.state(k)), f"state_dict {key}")
    grouped.load_state_dict(split.state_dict())
    _same_state(split, grouped, "after load_state_dict")


def test_skip_restores_state_and_params(env):
    """A skipped device step leaves the output set equal to the input set and
    the gather slice equal to the cast of the kept master weights."""
    zs, synth, shard = env
    wl = dataclasses.replace(synth.WORKLOADS["mlp9-w3"], phi=3 * 40_009, steps=2,
                             inject_steps=(2,), inject_rate=1e-3, name="skip")
    st, g = _make(env, wl, True, dynamic=True, growth_interval=4)
    for step in (1, 2):
        for k in range(wl.world):
            synth.dev_grad(wl, k, step, 0, 0, g[k], scale=st.loss_scale)
        if step == 2:
            before = [down32(x).copy() for x in (st.master, st.m, st.v)]
        st.step_device(g)
        d = st.sync_scaler()
    assert d.last_flag == 1 and d.skipped == 1 and d.step_t == 1
    assert d.scale == wl.loss_scale * 0.5
    for got, want, name in zip((st.master, st.m, st.v), before, ("master", "m", "v")):
        assert_bits_equal(down32(got), want, f"kept {name}")
    want = oracle.float_to_half(before[0], wl.param_dtype)
    assert np.array_equal(down16(st.params.view(torch.int16)), want)


@pytest.mark.parametrize("lr,b1,b2", [(1e-3, 0.9, 0.999), (3e-4, 0.9, 0.95), (2e-2, 0.8, 0.9999)])
def test_bias_corrections_match_oracle_every_step(env, lr, b1, b2):
    """1500 committed steps: the fp32 bias corrections the device forms from
    its running beta powers equal the oracle's (formed from t repeated
    products on the host) at every t, and the final state equals the
    oracle's 1500-step run bit for bit."""
    zs, synth, shard = env
    wl = dataclasses.replace(synth.WORKLOADS["mlp9-w3"], phi=2 * 4099, world=2, lr=lr,
                             beta1=b1, beta2=b2, loss_scale=1.0, name="consts")
    st, g = _make(env, wl, True)
    for k in range(wl.world):
        synth.dev_grad(wl, k, 1, 0, 0, g[k], scale=1.0)
    st.bind(g)
    parts = [synth.host_grad(wl, k, 1, 0, 0, wl.n, scale=1.0) for k in range(wl.world)]
    master, m, v = synth.host_state(wl, 0, wl.n)
    announce(f"bias corrections lr={lr} b1={b1} b2={b2}")
    steps = 1500
    for t in range(1, steps + 1):
        st.step_device()
        d = st.sync_scaler()
        k = oracle.adamw_consts(lr, b1, b2, wl.eps, wl.weight_decay, t)
        assert (np.float32(d.last_alpha), np.float32(d.last_bc2)) == \
            (np.float32(k["alpha"]), np.float32(k["b2"])), f"t={t}"
        f, master, m, v, p = oracle.shard_step(parts, 0, wl.grad_dtype, wl.param_dtype, master,
                                               m, v, lr=lr, beta1=b1, beta2=b2, eps=wl.eps,
                                               weight_decay=wl.weight_decay, loss_scale=1.0,
                                               step_t=t)
        assert f == 0 and d.last_flag == 0
    assert d.step_t == steps
    for got, want, name in ((st.master, master, "master"), (st.m, m, "m"), (st.v, v, "v")):
        assert_bits_equal(down32(got), want, f"after {steps} steps: {name}")
    assert np.array_equal(down16(st.params.view(torch.int16)), p)


def test_scale_growth_to_infinity_then_skip(env):
    """Growth every 2 clean steps from 2^126: 2^127 after step 2, inf after
    step 4 (no cap, as the host rule); a step that finds the scale not
    finite is skipped, counted in bad_scale, and changes no state."""
    zs, synth, shard = env
    wl = dataclasses.replace(synth.WORKLOADS["mlp9-w3"], phi=10_007, world=1, name="growth")
    st, g = _make(env, wl, True, loss_scale=2.0 ** 126, dynamic=True, growth_interval=2)
    for k in range(wl.world):
        synth.dev_grad(wl, k, 1, 0, 0, g[k], scale=1.0)
    st.bind(g)
    parts = [synth.host_grad(wl, 0, 1, 0, 0, wl.n, scale=1.0)]
    master, m, v = synth.host_state(wl, 0, wl.n)
    hs = oracle.Scaler(2.0 ** 126, 2)
    scales = []
    for step in range(1, 5):
        scales.append(st.loss_scale)
        assert st.loss_scale == hs.scale
        st.step_device()
        d = st.sync_scaler()
        f, master, m, v, p = oracle.shard_step(parts, 0, wl.grad_dtype, wl.param_dtype, master,
                                               m, v, lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2,
                                               eps=wl.eps, weight_decay=wl.weight_decay,
                                               loss_scale=hs.scale, step_t=hs.t + 1)
        hs.update(f)
        assert f == 0 and d.last_flag == 0
        for got, want, name in ((st.master, master, "master"), (st.m, m, "m"), (st.v, v, "v")):
            assert_bits_equal(down32(got), want, f"step {step}: {name}")
    assert scales == [2.0 ** 126, 2.0 ** 126, 2.0 ** 127, 2.0 ** 127]
    assert d.scale == float("inf") and d.bad_scale == 0
    st.step_device()
    d = st.sync_scaler()
    assert (d.last_flag, d.bad_scale, d.skipped, d.step_t) == (1, 1, 1, 4)
    for got, want, name in ((st.master, master, "master"), (st.m, m, "m"), (st.v, v, "v")):
        assert_bits_equal(down32(got), want, f"bad-scale step: {name}")
    assert np.array_equal(down16(st.params.view(torch.int16)), p)


def test_empty_shard_commits(env):
    """An empty partition commits, also right after a skipped step (it has no
    fused pass, so the previous step's overflow mark must not count)."""
    zs, synth, shard = env
    wl = dataclasses.replace(synth.WORKLOADS["mlp9-w3"], phi=3, world=4, name="empty")
    assert wl.n == 1
    st, g = _make(env, wl, True)
    a = st._args(g, None).args
    a.n = 0
    zs.zs_step_device(a, st.dev)
    d = st.sync_scaler()
    assert (d.step_t, d.skipped, d.last_flag, d.epoch) == (1, 0, 0, 1)
    # a skipped step on the one-element shard, then an empty one
    for k in range(wl.world):
        g[k].fill_(0x7F80)                      # +inf (bf16) from every worker
    a.n = 1
    zs.zs_step_device(a, st.dev)
    d = st.sync_scaler()
    assert (d.step_t, d.skipped, d.last_flag, d.epoch, d.flag_epoch) == (1, 1, 1, 2, 2)
    a.n = 0
    zs.zs_step_device(a, st.dev)
    d = st.sync_scaler()
    assert (d.step_t, d.skipped, d.last_flag, d.epoch) == (2, 1, 0, 3)


@pytest.mark.parametrize("windows", [None, "2.56,0.25"])
def test_graph_capture_replays_match_eager(env, windows, monkeypatch):
    """Two device steps (one per direction of the ping-pong sets) captured in
    a graph; three replays, with eager work and synchronizations between
    them, each equal to two eager steps; also with write windows forced on
    for both the eager and the captured steps (the captured launches keep
    the window they were recorded with)."""
    zs, synth, shard = env
    if windows:
        monkeypatch.setenv("ZS_FUSED_WRITE_WINDOW", windows)
    wl = dataclasses.replace(synth.WORKLOADS["gpt2s-w8"], phi=8 * 100_003, name="graph")
    eager, ge = _make(env, wl, True)
    graph, gg = _make(env, wl, True)
    for k in range(wl.world):
        synth.dev_grad(wl, k, 1, 0, 0, ge[k], scale=wl.loss_scale)
        synth.dev_grad(wl, k, 1, 0, 0, gg[k], scale=wl.loss_scale)
    eager.bind(ge)
    graph.bind(gg)
    torch.cuda.synchronize()
    announce("graph capture of two device steps")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            graph.step_device()
            graph.step_device()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # capture enqueued nothing: the graph shard is still at its initial state
    assert graph.sync_scaler().step_t == 0
    for r in range(3):
        eager.step_device()
        eager.step_device()
        junk = torch.arange(1 << 20, device="cuda", dtype=torch.float32).sum()
        g.replay()
        torch.cuda.synchronize()
        assert float(junk) > 0
        _same_state(eager, graph, f"replay {r}")
        de, dg = eager.sync_scaler(), graph.sync_scaler()
        assert (dg.step_t, dg.skipped, dg.epoch) == (de.step_t, 0, de.epoch) == \
            (2 * (r + 1), 0, 2 * (r + 1))


@pytest.mark.parametrize("off,n", [(0, 40_000), (3, 40_003)])
def test_skip_restore_on_misaligned_slices(env, off, n):
    """Skip through zs_step_device with the gather slice at an odd offset and
    a ragged length (the commit kernel's narrow vector path): the output set
    equals the input set and the slice holds the fp16 cast of master_in;
    elements outside the slice are untouched."""
    zs, synth, shard = env
    rng = np.random.default_rng(off + n)
    world = 3
    g = (rng.standard_normal((world, n)) * 64.0).astype(np.float16)
    g[1, n // 2] = np.inf
    dg = [torch.from_numpy(g[k].copy()).cuda() for k in range(world)]
    state = [(rng.standard_normal(n) * s).astype(F32) for s in (0.02, 1e-4, 1e-6)]
    state[2] = np.abs(state[2])
    din = [torch.from_numpy(x.copy()).cuda() for x in state]
    dout = [torch.full((n,), 5.0, dtype=torch.float32, device="cuda") for _ in range(3)]
    gather = torch.full((n + off + 5,), 0x1234, dtype=torch.int16, device="cuda")
    host = zs.zs_loss_scaler(scale=1024.0, clean_steps=0, growth_interval=0, dynamic=1,
                             step_t=0, skipped=0)
    dev = zs.device_scaler_upload(zs.zs_device_scaler_make(host, 0.9, 0.999))
    args = zs.StepArgs(dg, 0, n, *din, *dout, gather, off, None,
                       zs.hparams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01,
                                  loss_scale=1.0, step_t=1),
                       grad_dtype=zs.ZS_FP16, param_dtype=zs.ZS_FP16)
    announce(f"skip restore off={off} n={n}")
    zs.zs_step_device(args, dev)
    d = zs.device_scaler_read(dev)
    assert (d.last_flag, d.skipped, d.step_t, d.scale) == (1, 1, 0, 512.0)
    for got, want, name in zip(dout, state, ("master", "m", "v")):
        assert_bits_equal(down32(got), want, f"restored {name}")
    gb = down16(gather)
    assert np.all(gb[:off] == 0x1234) and np.all(gb[off + n:] == 0x1234)
    assert np.array_equal(gb[off:off + n], oracle.float_to_half(state[0], "fp16"))


def test_long_run_matches_the_oracle(env):
    """2000 device-commit steps with fresh gradients every step, a dynamic
    scale growing every 50 clean steps and injected inf/NaN at steps 100,
    777 and 1500: the whole state equals the oracle's run bit for bit at
    several points and at the end, and the scaler follows the oracle's."""
    zs, synth, shard = env
    wl = dataclasses.replace(synth.WORKLOADS["gpt2s-w8"], phi=4 * 65_537, world=4, steps=2000,
                             inject_steps=(100, 777, 1500), inject_rate=1e-3, loss_scale=1024.0,
                             name="long")
    n = wl.n
    st, g = _make(env, wl, True, dynamic=True, growth_interval=50)
    master, m, v = synth.host_state(wl, 0, n)
    hs = oracle.Scaler(1024.0, 50)
    hp = dict(lr=wl.lr, beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps, weight_decay=wl.weight_decay)
    announce("long run: 2000 device-commit steps")
    for step in range(1, wl.steps + 1):
        scale = hs.scale
        for k in range(wl.world):
            synth.dev_grad(wl, k, step, 0, 0, g[k], scale=scale)
        st.step_device(g)
        parts = [synth.host_grad(wl, k, step, 0, 0, n, scale=scale) for k in range(wl.world)]
        f, mo, mmo, vo, po = oracle.shard_step(parts, 0, wl.grad_dtype, wl.param_dtype, master, m,
                                               v, loss_scale=scale, step_t=hs.t + 1, threads=8,
                                               **hp)
        hs.update(f)
        if f == 0:
            master, m, v = mo, mmo, vo
        d = st.sync_scaler()
        assert (d.last_flag, d.scale, d.step_t, d.skipped) == (f, hs.scale, hs.t, hs.s.skipped), step
        if step in (1, 101, 778, 1000, 1501, wl.steps):
            for got, want, name in ((st.master, master, "master"), (st.m, m, "m"), (st.v, v, "v")):
                assert_bits_equal(down32(got), want, f"step {step}: {name}")
    assert hs.s.skipped == 3 and hs.t == 1997


def test_hyperparameters_follow_opt_every_step(env):
    """A learning-rate schedule (with eps and weight decay changing too) and
    a change of betas at step 3 reach every step path of ShardState: step()
    (host commit), step_device() (device commit, where the beta change
    re-forms beta^t on the device) and launch()/finish(). Every step of every
    path matches the oracle run on that path's previous state with the
    step's settings, and the three paths agree bit for bit."""
    zs, synth, shard = env
    rng = np.random.default_rng(23)
    world, n, scale = 3, 5003, 1024.0
    sched = [(1e-3, 0.9, 0.999, 1e-8, 0.01), (5e-4, 0.9, 0.999, 1e-8, 0.02),
             (2e-4, 0.85, 0.99, 1e-7, 0.02), (1e-4, 0.85, 0.99, 0.0, 0.0)]
    g16 = [[((rng.standard_normal(n) * 1e-3 * scale).astype(F32).view(np.uint32) >> 16)
            .astype(np.uint16) for _ in range(world)] for _ in sched]
    init = [(rng.standard_normal(n) * s).astype(F32) for s in (0.02, 1e-4, 1e-6)]
    init[2] = np.abs(init[2])

    def make(device_commit):
        st = shard.ShardState(n, world, 0, 0, n, zs.ZS_BF16, zs.ZS_BF16, shard.AdamW(*sched[0]),
                              scale, device_commit=device_commit)
        for dst, x in zip((st.master, st.m, st.v), init):
            dst.copy_(torch.from_numpy(x))
        return st

    paths = {"step": make(False), "step_device": make(True), "launch": make(False)}
    grads = torch.empty((world, n), dtype=torch.bfloat16, device="cuda")
    for i, (lr, b1, b2, eps, wd) in enumerate(sched):
        announce(f"hyper-parameter schedule, step {i + 1}")
        for k in range(world):
            grads[k].copy_(torch.from_numpy(g16[i][k].view(np.int16)).view(torch.bfloat16))
        gl = [grads[k] for k in range(world)]
        outs = {}
        for name, st in paths.items():
            prev = [down32(x).copy() for x in (st.master, st.m, st.v)]
            st.opt.lr, st.opt.beta1, st.opt.beta2 = lr, b1, b2
            st.opt.eps, st.opt.weight_decay = eps, wd
            if name == "step":
                assert st.step(gl)
            elif name == "step_device":
                st.step_device(gl)
                assert st.sync_scaler().last_flag == 0
            else:
                assert st.finish(st.launch(gl))
            f, mo, mmo, vo, po = oracle.shard_step(g16[i], 0, "bf16", "bf16", *prev, lr=lr,
                                                   beta1=b1, beta2=b2, eps=eps, weight_decay=wd,
                                                   loss_scale=scale, step_t=i + 1)
            assert f == 0
            got = [down32(x) for x in (st.master, st.m, st.v)]
            for g_, w_, what in zip(got, (mo, mmo, vo), ("master", "m", "v")):
                assert_rel(g_, w_, 1e-6, f"{name} step {i + 1} {what}")
            p = down16(st.params.view(torch.int16))
            assert_ulp16(p, po, "bf16", 1, f"{name} step {i + 1} params")
            outs[name] = got + [p]
        for name in ("step_device", "launch"):
            for a, b in zip(outs["step"], outs[name]):
                assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8)), \
                    f"{name} differs from step at step {i + 1}"
    assert all(st.t == len(sched) for st in paths.values())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_schedule_device_equals_host(env, seed):
    """60 steps with a learning rate that changes every step, dynamic loss
    scaling with a growth interval of 3 and non-finite gradients injected on
    about 15 % of the steps (so the scale halves and doubles many times):
    the queued device-commit flow ends in the same state, parameters and
    scaler as the host-commit flow, bit for bit."""
    zs, synth, shard = env
    rng = np.random.default_rng(700 + seed)
    world, n, steps = 4, 30_011, 60
    gdt = ("bf16", "fp16", "bf16")[seed]
    code = zs.ZS_BF16 if gdt == "bf16" else zs.ZS_FP16
    init = [(rng.standard_normal(n) * s).astype(F32) for s in (0.02, 1e-4, 1e-6)]
    init[2] = np.abs(init[2])

    def make(device_commit):
        st = shard.ShardState(n, world, 0, 0, n, code, code, shard.AdamW(1e-3, 0.9, 0.999, 1e-8, 0.01),
                              2.0 ** 10, dynamic=True, growth_interval=3, device_commit=device_commit)
        for dst, x in zip((st.master, st.m, st.v), init):
            dst.copy_(torch.from_numpy(x))
        return st

    host, dev = make(False), make(True)
    gh = torch.empty((world, n), dtype=torch.int16, device="cuda")
    gd = torch.empty((world, n), dtype=torch.int16, device="cuda")
    lhs, lds = [gh[k] for k in range(world)], [gd[k] for k in range(world)]
    tdt = torch.bfloat16 if gdt == "bf16" else torch.float16
    announce(f"random schedule, seed {seed} ({gdt})")
    committed = 0
    for step in range(steps):
        lr = float(10 ** rng.uniform(-4, -2.5))
        host.opt.lr = dev.opt.lr = lr
        # both flows draw the same gradient, scaled by the host scaler's scale
        # (the device scaler follows the same rule, checked at the end)
        g = (torch.from_numpy(rng.standard_normal((world, n)).astype(F32) * 1e-3) *
             host.loss_scale).to(tdt).view(torch.int16)
        if rng.random() < 0.15:
            g[int(rng.integers(0, world)), int(rng.integers(0, n))] = 0x7F80 if gdt == "bf16" else 0x7C00
        gh.copy_(g)
        gd.copy_(g)
        committed += host.step([x.view(tdt) for x in lhs])
        dev.step_device([x.view(tdt) for x in lds])
    d = dev.sync_scaler()
    assert (d.step_t, d.skipped) == (host.scaler.step_t, host.scaler.skipped) == (committed,
                                                                                 steps - committed)
    assert d.scale == host.loss_scale and d.clean_steps == host.scaler.clean_steps
    assert steps - committed >= 3 and committed >= 30   # both paths exercised
    _same_state(host, dev, f"random schedule {seed}")


def test_shard_capture_replays_match_eager(env):
    """ShardState.capture(): each replay runs two device steps (one per
    direction of the ping-pong sets) on whatever the gradient buffers hold;
    three replays, with the gradients refilled in place before each, equal
    six eager steps on the same fills, bit for bit."""
    zs, synth, shard = env
    wl = dataclasses.replace(synth.WORKLOADS["mlp9-w3"], phi=3 * 50_001, name="capture")
    graph, gg = _make(env, wl, True)
    ref, rg = _make(env, wl, True)
    announce("ShardState.capture")
    replay = graph.capture(gg)
    torch.cuda.synchronize()
    assert graph.sync_scaler().step_t == 0      # capturing ran nothing
    for r in range(3):
        for k in range(wl.world):
            synth.dev_grad(wl, k, r + 1, 0, 0, gg[k], scale=wl.loss_scale)
            synth.dev_grad(wl, k, r + 1, 0, 0, rg[k], scale=wl.loss_scale)
        replay()
        ref.step_device(rg)
        ref.step_device(rg)
    torch.cuda.synchronize()
    _same_state(ref, graph, "capture replays")
    d = graph.sync_scaler()
    assert (d.step_t, d.epoch) == (6, 6) and graph.cur == ref.cur


def test_two_shards_on_two_streams_equal_each_alone(env):
    """Two shards with their own device scalers stepping on two streams at
    the same time (gradients generated and steps queued on each shard's
    stream, launches interleaved, no synchronization in between; one shard
    takes a skip): each ends bit-identical to the same shard stepped alone on
    the default stream. Disjoint buffers on different streams share nothing
    in the library."""
    zs, synth, shard = env
    base = synth.WORKLOADS["gpt2s-w8"]
    wls = [dataclasses.replace(base, phi=8 * 300_007, steps=5, inject_steps=(2,),
                               inject_rate=1e-3, name="stream-a", seed=21),
           dataclasses.replace(base, phi=8 * 200_003, steps=5, name="stream-b", seed=22)]
    announce("two shards on two streams against each alone")

    def run(wl, st, grads, stream=None):
        for step in range(1, wl.steps + 1):
            for k in range(wl.world):
                synth.dev_grad(wl, k, step, 0, 0, grads[k], scale=wl.loss_scale, stream=stream)
            st.step_device(grads, stream=stream)

    alone = []
    for wl in wls:
        st, g = _make(env, wl, True)
        run(wl, st, g)
        alone.append(st)
    pairs = [_make(env, wl, True) for wl in wls]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for step in range(1, 6):
        for wl, (st, g), s in zip(wls, pairs, streams):
            for k in range(wl.world):
                synth.dev_grad(wl, k, step, 0, 0, g[k], scale=wl.loss_scale, stream=s)
            st.step_device(g, stream=s)
    torch.cuda.synchronize()
    for (st, _), ref, wl in zip(pairs, alone, wls):
        d, r = st.sync_scaler(), ref.sync_scaler()
        assert (d.step_t, d.skipped, d.epoch) == (r.step_t, r.skipped, r.epoch)
        assert d.skipped == (1 if wl.inject_steps else 0)
        _same_state(ref, st, wl.name)
