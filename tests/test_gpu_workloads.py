"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (ShardState -> zs_step_fused, one flag readback per step).

Inputs are generated on the device by the seeded generator; the oracle
regenerates the same values on the host. The two smaller workloads are
compared element for element over the whole partition; the 7.5B-shard, 7B
and 1.3B workloads on sampled windows (head, tail and seeded random
offsets): the update is elementwise, so each window's state evolves
independently across steps and the oracle can follow it alone. The overflow
flag is global: the oracle's window flag must equal the GPU flag, which
holds because non-finite values only come from injection (the generator's
samples are bounded) and injection at 1e-3 over the windows' inputs is
certain to hit them.
"""
import numpy as np
import pytest

import oracle
from gpu_util import (F32, announce, assert_bits_equal, assert_offload_matches_oracle,
                      assert_rel, assert_ulp16, down16, down32, oracle_offload_update)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

WINDOW = 1 << 16
# Window sizes of the large workloads: as large as the host-side generation
# and oracle allow within seconds per step (64 workers' gradients are
# generated per element of the 7.5B shard's windows).
WINDOW_7P5B = 1 << 21
WINDOW_7B = 1 << 22
WINDOW_1P3B = 1 << 20
# Element offsets where 32-bit address arithmetic would wrap in the 7e9-
# element arrays: fp32 byte offsets 2^31 .. 2^34 (elements 2^29 .. 2^32),
# 16-bit byte offsets 2^31 .. 2^33 and element indices 2^31, 2^32.
BOUNDARIES_7B = (1 << 29, 1 << 30, 1 << 31, 1 << 32)


@pytest.fixture(scope="module")
def env(hip_built):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sharded_mixed_precision_zs_amd import shard, synth, zeroshard
    return zeroshard, synth, shard


def _windows(n, count, seed, window=WINDOW, straddle=()):
    """Head, tail, middle and seeded random windows of `window` elements,
    plus one window centred on each offset in `straddle`."""
    if n <= 4 * window:
        return [(0, n)]
    rng = np.random.default_rng(seed)
    starts = {0, n - window, (n // 2) - window // 2}
    starts |= {b - window // 2 for b in straddle if window // 2 <= b <= n - window // 2}
    while len(starts) < count + len(straddle):
        starts.add(int(rng.integers(0, n - window)))
    return [(s, window) for s in sorted(starts)]


def run_workload(env, name, windows=None, gather_full=False, device_commit=False, wl=None,
                 state_layout="split"):
    """device_commit: steps through zs_step_device (commit or skip decided on
    the device); the host reads the device scaler back after each step only
    to check it and to scale the next step's synthetic gradients.
    state_layout: ShardState's fp32 state layout ("split" or "grouped")."""
    zs, synth, shard = env
    wl = wl if wl is not None else synth.WORKLOADS[name]
    n, off, W, A = wl.n, wl.offset, wl.world, wl.accum
    wins = windows if windows is not None else [(0, n)]
    announce(f"workload {name}: n={n} W={W} A={A} steps={wl.steps} windows={len(wins)} "
             f"device_commit={device_commit} state={state_layout}")
    st = shard.ShardState(n, W, wl.rank, off, (W * wl.chunk) if gather_full else off + n,
                          wl.param_dtype, wl.grad_dtype,
                          shard.AdamW(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay),
                          wl.loss_scale, dynamic=wl.dynamic_scale,
                          growth_interval=wl.scale_interval, accumulate=A > 1,
                          device_commit=device_commit, state_layout=state_layout)
    st.fill_state(lambda first, count, *t: synth.dev_state(wl, off + first, *t))
    # one row per worker, padded to 256 B like separate allocations
    row = -(-n // 128) * 128
    grads = torch.empty((W, row), dtype=torch.int16, device="cuda")
    gviews = [grads[k, :n] for k in range(W)]
    gdt = wl.grad_dtype
    # host-side oracle state per window
    hs = [list(synth.host_state(wl, off + s, L)) for s, L in wins]
    hscaler = oracle.Scaler(wl.loss_scale, wl.scale_interval if wl.dynamic_scale else 10 ** 9)
    for step in range(1, wl.steps + 1):
        scale = hscaler.scale
        assert scale == st.loss_scale
        announce(f"  {name} step {step} scale={scale} t={st.t}")
        accs = [None] * len(wins)
        for j in range(A):
            for k in range(W):
                synth.dev_grad(wl, k, step, j, off, gviews[k], scale=scale)
            parts_w = [[synth.host_grad(wl, k, step, j, off + s, L, scale=scale)
                        for k in range(W)] for s, L in wins]
            if j < A - 1:
                st.reduce_micro(gviews, first=(j == 0))
                for i, (s, L) in enumerate(wins):
                    if accs[i] is None:
                        accs[i] = np.empty(L, F32)
                    oracle.reduce_avg(parts_w[i], wl.rank, gdt, accs[i], j > 0, scale)
            else:
                if device_commit:
                    st.step_device(gviews, acc_in=st.acc if A > 1 else None)
                    committed = st.sync_scaler().last_flag == 0
                else:
                    committed = st.step(gviews, acc_in=st.acc if A > 1 else None)
                rflag = 0
                outs = []
                for i, (s, L) in enumerate(wins):
                    f, mo, mmo, vo, po = oracle.shard_step(
                        parts_w[i], wl.rank, gdt, wl.param_dtype, *hs[i], lr=wl.lr,
                        beta1=wl.beta1, beta2=wl.beta2, eps=wl.eps,
                        weight_decay=wl.weight_decay, loss_scale=scale, step_t=hscaler.t + 1,
                        acc_in=accs[i], threads=16)
                    rflag |= f
                    outs.append((mo, mmo, vo, po))
                assert st.last_flag == rflag, f"step {step}: gpu flag {st.last_flag} oracle {rflag}"
                assert committed == (rflag == 0)
                hscaler.update(rflag)
                if rflag == 0:
                    for i in range(len(wins)):
                        hs[i] = list(outs[i][:3])
                # compare the current set (committed or kept) with the oracle's
                nonbit = 0
                for i, (s, L) in enumerate(wins):
                    for k, what in enumerate(("master", "m", "v")):
                        nonbit += assert_rel(down32(st.state(k, s, L)), hs[i][k], 1e-6,
                                             f"{name} step {step} {what} window {s}")
                    if rflag == 0:
                        nonbit += assert_ulp16(down16(st.params[s:s + L].view(torch.int16)),
                                               outs[i][3], wl.param_dtype, 1,
                                               f"{name} step {step} params window {s}")
                    elif device_commit:
                        # skipped on the device: the gather slice holds the
                        # cast of the kept master weights
                        nonbit += assert_ulp16(down16(st.params[s:s + L].view(torch.int16)),
                                               oracle.float_to_half(hs[i][0], wl.param_dtype),
                                               wl.param_dtype, 0,
                                               f"{name} step {step} kept params window {s}")
                assert nonbit == 0, f"{name} step {step}: {nonbit} elements not bit-identical"
    assert (st.t, st.loss_scale, int(st.scaler.skipped)) == (hscaler.t, hscaler.scale,
                                                              hscaler.skipped)
    return st


def test_mlp9_w3_full(env):
    run_workload(env, "mlp9-w3", gather_full=True)


def test_mlp9_w3_last_rank_full(env):
    # rank 2 of 3 owns the ragged tail [699052, 2^20) at an offset that is
    # not 16-byte aligned: the narrower vector path of the same kernel.
    zs, synth, shard = env
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["mlp9-w3"], name="mlp9-w3-r2", rank=2)
    synth.WORKLOADS[wl.name] = wl
    try:
        assert wl.n == 349_524 and wl.offset == 699_052
        run_workload(env, wl.name, gather_full=True)
    finally:
        del synth.WORKLOADS[wl.name]


def test_gpt2s_w8_full(env):
    run_workload(env, "gpt2s-w8")


@pytest.mark.parametrize("device_commit", [False, True])
def test_gpt2s_w8_full_grouped_state(env, device_commit):
    run_workload(env, "gpt2s-w8", device_commit=device_commit, state_layout="grouped")


def test_1p3b_w4_acc4_windows_grouped_state(env):
    zs, synth, shard = env
    wl = synth.WORKLOADS["1p3b-w4-acc4-fp16"]
    run_workload(env, wl.name, windows=_windows(wl.n, 6, 4, WINDOW_1P3B), state_layout="grouped")
    torch.cuda.empty_cache()


# One shard per branch of the split layout's launch rule (block size,
# vectors per thread, sum and blocks per CU follow W, and at W = 3 the
# shard's size): W = 1 and 2 (one-wave blocks, one vector per thread, 12
# and 16 per CU); W = 3 under and at 20 000 2048-element tiles and a half
# (256-thread blocks, two vectors, 4 and 3 per CU); W = 4 (one-wave blocks,
# two vectors, the batched sum); W = 6 and 13 (the rolling sum at 8 and 6
# per CU, tails of 1 and 0 workers); W = 40 below the write windows' size
# floor. Each n is ragged against every tile. (The windows themselves run
# in the 7.5B-shard tests below.)
TILE_RULE_CASES = [(1, 1_000_003), (2, 1_000_003), (3, 1_000_003), (3, 40_961_029),
                   (4, 1_000_003), (6, 1_000_003), (13, 1_000_003), (40, 1_000_003)]


@pytest.mark.parametrize("world,n", TILE_RULE_CASES)
def test_each_launch_shape_matches_the_oracle(env, world, n):
    zs, synth, shard = env
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["gpt2s-w8"], name=f"shape-w{world}-n{n}",
                             world=world, phi=world * n, steps=2, bucket=0)
    assert wl.n == n and wl.offset == 0
    wins = _windows(n, 4, world) if n > 4 * WINDOW else None
    run_workload(env, wl.name, windows=wins, wl=wl)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("device_commit", [False, True])
def test_7p5b_shard_w64_windows(env, device_commit):
    zs, synth, shard = env
    wl = synth.WORKLOADS["7p5b-shard-w64"]
    run_workload(env, wl.name, windows=_windows(wl.n, 8, 2, WINDOW_7P5B),
                 device_commit=device_commit)


@pytest.mark.parametrize("device_commit", [False, True])
def test_7b_full_w1_windows(env, device_commit):
    zs, synth, shard = env
    wl = synth.WORKLOADS["7b-full-w1"]
    wins = _windows(wl.n, 8, 3, WINDOW_7B, straddle=BOUNDARIES_7B)
    for b in BOUNDARIES_7B:
        assert any(s < b < s + L for s, L in wins), b
    run_workload(env, wl.name, windows=wins, device_commit=device_commit)


def test_7p5b_shard_w64_windows_grouped_state(env):
    zs, synth, shard = env
    wl = synth.WORKLOADS["7p5b-shard-w64"]
    torch.cuda.empty_cache()
    run_workload(env, wl.name, windows=_windows(wl.n, 8, 5, WINDOW_7P5B), state_layout="grouped")
    torch.cuda.empty_cache()


def test_7b_full_w1_windows_grouped_state(env):
    zs, synth, shard = env
    wl = synth.WORKLOADS["7b-full-w1"]
    torch.cuda.empty_cache()
    wins = _windows(wl.n, 8, 6, WINDOW_7B, straddle=BOUNDARIES_7B)
    run_workload(env, wl.name, windows=wins, device_commit=True, state_layout="grouped")
    torch.cuda.empty_cache()


FLAG_CHUNK = 1 << 28


def _oracle_flag_over(gview, wl, scale):
    """The oracle's overflow flag (ring sum, average, unscale, check) over a
    whole single-worker gradient on the device, streamed to the host in
    chunks of FLAG_CHUNK elements."""
    n = gview.numel()
    out = np.empty(FLAG_CHUNK, F32)
    flag = 0
    for c0 in range(0, n, FLAG_CHUNK):
        c1 = min(n, c0 + FLAG_CHUNK)
        bits = gview[c0:c1].cpu().numpy().view(np.uint16)
        flag |= oracle.reduce_avg([bits], 0, wl.grad_dtype, out[:c1 - c0], False, scale)
    return flag


def test_7p5b_flag_covers_the_whole_partition(env):
    """The 7.5B shard's flag (64 workers) at full size against the oracle's
    ring sum, average, unscale and check of every element of the partition,
    the 64 gradients streamed to the host in chunks; then one NaN planted in
    the last worker's last element is found and the step skipped."""
    zs, synth, shard = env
    wl = synth.WORKLOADS["7p5b-shard-w64"]
    n, off, W = wl.n, wl.offset, wl.world
    torch.cuda.empty_cache()
    st = shard.ShardState(n, W, wl.rank, off, off + n, wl.param_dtype, wl.grad_dtype,
                          shard.AdamW(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay),
                          wl.loss_scale)
    synth.dev_state(wl, off, st.master, st.m, st.v)
    row = -(-n // 128) * 128
    grads = torch.empty((W, row), dtype=torch.int16, device="cuda")
    gv = [grads[k, :n] for k in range(W)]
    for k in range(W):
        synth.dev_grad(wl, k, 1, 0, off, gv[k], scale=wl.loss_scale)
    announce("7.5B whole-partition flag: clean step")
    assert st.step(gv) and st.last_flag == 0
    announce("7.5B whole-partition flag: oracle over all elements")
    chunk = 1 << 24
    out = np.empty(chunk, F32)
    flag = 0
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        parts = [g[c0:c1].cpu().numpy().view(np.uint16) for g in gv]
        flag |= oracle.reduce_avg(parts, wl.rank, wl.grad_dtype, out[:c1 - c0], False,
                                  wl.loss_scale)
    assert flag == 0
    gv[W - 1][n - 1] = 0x7FC0  # bf16 quiet NaN
    kept = st.v[n - 256:].clone()
    announce("7.5B whole-partition flag: NaN in the last element")
    assert not st.step(gv) and st.last_flag == 1
    parts = [g[n - 4096:].cpu().numpy().view(np.uint16) for g in gv]
    assert oracle.reduce_avg(parts, wl.rank, wl.grad_dtype, np.empty(4096, F32), False,
                             wl.loss_scale) == 1
    assert torch.equal(st.v[n - 256:], kept)
    assert st.t == 1 and int(st.scaler.skipped) == 1
    del st, grads, gv
    torch.cuda.empty_cache()


def test_7b_flag_covers_the_whole_gradient(env):
    """The fused step's overflow flag at the 7B workload's full size equals
    the oracle's check of all 7e9 gradient elements (streamed to the host),
    and one +inf planted past element 2^32 is found: that step is skipped and
    the kept set is left as it was."""
    zs, synth, shard = env
    wl = synth.WORKLOADS["7b-full-w1"]
    n, off = wl.n, wl.offset
    torch.cuda.empty_cache()
    st = shard.ShardState(n, 1, wl.rank, off, off + n, wl.param_dtype, wl.grad_dtype,
                          shard.AdamW(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay),
                          wl.loss_scale)
    synth.dev_state(wl, off, st.master, st.m, st.v)
    g = torch.empty(n, dtype=torch.int16, device="cuda")
    synth.dev_grad(wl, 0, 1, 0, off, g, scale=wl.loss_scale)
    announce("7b whole-gradient flag: clean step")
    assert st.step([g]) and st.last_flag == 0
    announce("7b whole-gradient flag: oracle over all elements")
    assert _oracle_flag_over(g, wl, wl.loss_scale) == 0
    p = (1 << 32) + 12_345
    g[p] = 0x7F80  # bf16 +inf
    kept = st.master[p - 64:p + 64].clone()
    announce("7b whole-gradient flag: +inf past element 2^32")
    assert not st.step([g]) and st.last_flag == 1
    c0 = p // FLAG_CHUNK * FLAG_CHUNK
    assert _oracle_flag_over(g[c0:c0 + FLAG_CHUNK], wl, wl.loss_scale) == 1
    assert torch.equal(st.master[p - 64:p + 64], kept)
    assert st.t == 1 and int(st.scaler.skipped) == 1
    del st, g
    torch.cuda.empty_cache()


@pytest.mark.parametrize("device_commit", [False, True])
def test_1p3b_w4_acc4_fp16_windows(env, device_commit):
    zs, synth, shard = env
    wl = synth.WORKLOADS["1p3b-w4-acc4-fp16"]
    st = run_workload(env, wl.name, windows=_windows(wl.n, 6, 4, WINDOW_1P3B),
                      device_commit=device_commit)
    # two injected steps skipped: 2^16 -> 2^15 -> 2^14, eight steps committed
    assert st.loss_scale == 2.0 ** 14 and st.t == 8


def test_gpt2s_w8_full_device_commit(env):
    run_workload(env, "gpt2s-w8", device_commit=True)


def test_1p3b_schedule_device_commit(env):
    """The dynamic-scaler schedule (fp16, W=4, four micro-batches, injected
    inf/NaN at steps 3 and 7) with commit or skip on the device, the whole
    partition compared with the oracle after every step."""
    zs, synth, shard = env
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["1p3b-w4-acc4-fp16"], phi=4 * 200_003,
                             name="1p3b-device-commit")
    st = run_workload(env, wl.name, device_commit=True, wl=wl)
    assert st.loss_scale == 2.0 ** 14 and st.t == 8 and int(st.scaler.skipped) == 2


@pytest.mark.parametrize("device_commit", [False, True])
def test_checkpoint_resume_is_bit_identical(env, tmp_path, device_commit):
    """k steps, save, reload into a fresh shard, continue: identical bits to
    an uninterrupted run (dynamic scaler and skipped steps included), with
    the commit decided on the host or on the device."""
    zs, synth, shard = env
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["1p3b-w4-acc4-fp16"], phi=4 * 300_007,
                             inject_steps=(2, 5), steps=7, name="resume-case")
    n, W, A = wl.n, wl.world, wl.accum
    opt = shard.AdamW(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay)

    def fresh():
        st = shard.ShardState(n, W, 0, 0, n, wl.param_dtype, wl.grad_dtype, opt, wl.loss_scale,
                              dynamic=True, growth_interval=2, accumulate=True,
                              device_commit=device_commit)
        synth.dev_state(wl, 0, st.master, st.m, st.v)
        return st

    grads = torch.empty((W, -(-n // 128) * 128), dtype=torch.int16, device="cuda")
    g = [grads[k, :n] for k in range(W)]

    def run(st, steps):
        for step in steps:
            for j in range(A):
                for k in range(W):
                    synth.dev_grad(wl, k, step, j, 0, g[k], scale=st.loss_scale)
                if j < A - 1:
                    st.reduce_micro(g, first=(j == 0))
                elif device_commit:
                    st.step_device(g, acc_in=st.acc)
                    st.sync_scaler()   # the next step's gradients use the scale
                else:
                    st.step(g, acc_in=st.acc)

    announce(f"checkpoint/resume, device_commit={device_commit}")
    ref = fresh()
    run(ref, range(1, 8))
    a = fresh()
    run(a, range(1, 4))
    path = tmp_path / "shard.pt"
    torch.save(a.state_dict(), path)
    del a
    b = fresh()
    b.load_state_dict(torch.load(path, weights_only=True))
    run(b, range(4, 8))
    for x, y in ((b.master, ref.master), (b.m, ref.m), (b.v, ref.v)):
        assert_bits_equal(down32(x), down32(y), "resumed state")
    assert np.array_equal(down16(b.params.view(torch.int16)), down16(ref.params.view(torch.int16)))
    assert (b.t, b.loss_scale, int(b.scaler.skipped)) == (ref.t, ref.loss_scale,
                                                          int(ref.scaler.skipped))
    assert int(ref.scaler.skipped) == 2


@pytest.mark.parametrize("name,phi", [("gpt2s-w8", 8 * 250_003), ("1p3b-w4-acc4-fp16", 4 * 200_001)])
def test_offload_equals_fused(env, name, phi):
    """The ZeRO-Offload variant (reduce on the GPU, update on the host)
    follows the oracle step by step over the whole partition (its host state
    and device parameters after every step, skipped steps included), and
    the fused GPU step produces the same bits."""
    zs, synth, shard = env
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS[name], phi=phi, name=name + "-offload",
                             steps=6, inject_steps=(3,) if name.startswith("1p3b") else ())
    n, W, A = wl.n, wl.world, wl.accum
    opt = shard.AdamW(wl.lr, wl.beta1, wl.beta2, wl.eps, wl.weight_decay)
    kw = dict(dynamic=wl.dynamic_scale, growth_interval=wl.scale_interval)
    gpu = shard.ShardState(n, W, 0, 0, n, wl.param_dtype, wl.grad_dtype, opt, wl.loss_scale,
                           accumulate=A > 1, **kw)
    off = shard.OffloadShard(n, W, 0, 0, n, wl.param_dtype, wl.grad_dtype, opt, wl.loss_scale,
                             threads=8, **kw)
    synth.dev_state(wl, 0, gpu.master, gpu.m, gpu.v)
    off.master.copy_(gpu.master.cpu())
    off.m.copy_(gpu.m.cpu())
    off.v.copy_(gpu.v.cpu())
    grads = torch.empty((W, -(-n // 128) * 128), dtype=torch.int16, device="cuda")
    g = [grads[k, :n] for k in range(W)]
    hs = list(synth.host_state(wl, 0, n))          # the oracle's state
    hscaler = oracle.Scaler(wl.loss_scale, wl.scale_interval if wl.dynamic_scale else 10 ** 9)
    skipped = 0
    for step in range(1, wl.steps + 1):
        announce(f"offload vs oracle and fused {name} step {step}")
        assert gpu.loss_scale == off.loss_scale == hscaler.scale
        scale = hscaler.scale
        acc = np.empty(n, F32) if A > 1 else None
        for j in range(A):
            for k in range(W):
                synth.dev_grad(wl, k, step, j, 0, g[k], scale=scale)
            parts = [synth.host_grad(wl, k, step, j, 0, n, scale=scale) for k in range(W)]
            if j < A - 1:
                gpu.reduce_micro(g, first=(j == 0))
                off.reduce_micro(g, first=(j == 0))
                oracle.reduce_avg(parts, 0, wl.grad_dtype, acc, j > 0, scale)
            else:
                ok1 = gpu.step(g, acc_in=gpu.acc if A > 1 else None)
                ok2 = off.step(g, first=(A == 1))
                f, mo, mmo, vo, po = oracle.shard_step(
                    parts, 0, wl.grad_dtype, wl.param_dtype, *hs, lr=wl.lr, beta1=wl.beta1,
                    beta2=wl.beta2, eps=wl.eps, weight_decay=wl.weight_decay, loss_scale=scale,
                    step_t=hscaler.t + 1, acc_in=acc, threads=8)
                assert ok1 == ok2 == (f == 0)
        hscaler.update(f)
        skipped += f
        if f == 0:
            hs = [mo, mmo, vo]
        torch.cuda.synchronize()
        nonbit = assert_offload_matches_oracle(
            [off.master.numpy(), off.m.numpy(), off.v.numpy()],
            down16(off.params.view(torch.int16)), (f, hs, po if f == 0 else None),
            wl.param_dtype, f"{name} step {step}")
        assert nonbit == 0, f"{name} step {step}: {nonbit} elements not bit-identical"
    assert (off.t, off.loss_scale) == (hscaler.t, hscaler.scale)
    assert skipped == len(wl.inject_steps)
    torch.cuda.synchronize()
    for x, y in ((gpu.master, off.master), (gpu.m, off.m), (gpu.v, off.v)):
        assert_bits_equal(down32(x), y.numpy(), f"{name} offload state")
    assert np.array_equal(down16(gpu.params.view(torch.int16)), down16(off.params.view(torch.int16)))
    assert (gpu.t, gpu.loss_scale) == (off.t, off.loss_scale)


@pytest.mark.parametrize("n,pieces,threads", [(1, 1, 1), (4099, 3, 2), (200_003, 16, 0),
                                              (65_536, 1024, 4), (100_000, 7, 16)])
def test_offload_step_equals_cpu_step(env, n, pieces, threads):
    """zs_offload_step (GPU check, gradient in pieces, host update as the
    pieces land, parameters copied back per piece) leaves the host state and
    the device parameters as the oracle's check, AdamW update and cast of
    the same gradient -- and exactly as zs_cpu_step -- for ragged sizes,
    more pieces than elements per thread, and any thread count; a gradient
    with one non-finite value is skipped with nothing written; the call
    runs on a side stream."""
    zs, synth, shard = env
    rng = np.random.default_rng(n + pieces)
    grad = (rng.standard_normal(n) * 3e-3 * 1024).astype(F32)
    state = [(rng.standard_normal(n) * s).astype(F32) for s in (0.02, 1e-4, 1e-6)]
    state[2] = np.abs(state[2])
    hp = zs.hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1024.0, 3)
    # reference: the host update alone
    ref = [x.copy() for x in state]
    ref_p = np.zeros(n, np.uint16)
    assert zs.zs_cpu_step(*ref, grad, hp, ref_p, zs.ZS_BF16, 1) == 0
    host = [torch.from_numpy(x.copy()) for x in state]
    grad_dev = torch.from_numpy(grad).cuda()
    params_dev = torch.full((n + 16,), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    grad_host = torch.empty(n, dtype=torch.float32, pin_memory=True)
    params_host = torch.empty(n, dtype=torch.bfloat16, pin_memory=True)
    flag_dev = torch.full((1,), 5, dtype=torch.int32, device="cuda")
    flag_host = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()   # the fills above ran on the default stream
    announce(f"offload step n={n} pieces={pieces} threads={threads}")
    ok = zs.zs_offload_step(grad_dev, grad_host, *host, params_host, params_dev[8:8 + n], hp,
                            flag_dev, flag_host, zs.ZS_BF16, threads, pieces, stream=side)
    side.synchronize()
    assert ok and int(flag_host[0]) == 0
    p = down16(params_dev.view(torch.int16))
    want = oracle_offload_update(*state, grad, 1024.0, 1e-3, 0.9, 0.999, 1e-8, 0.01, 3, "bf16")
    assert want[0] == 0
    assert assert_offload_matches_oracle([x.numpy() for x in host], p[8:8 + n], want, "bf16",
                                         "offload step") == 0
    for got, ref_x, what in zip(host, ref, ("master", "m", "v")):
        assert_bits_equal(got.numpy(), ref_x, f"offload step {what} vs zs_cpu_step")
    assert np.array_equal(p[8:8 + n], ref_p) and np.all(p[:8] == 7) and np.all(p[8 + n:] == 7)
    # a non-finite gradient value: skipped, nothing written
    bad = grad.copy()
    bad[n // 2] = np.inf
    grad_dev.copy_(torch.from_numpy(bad))
    before = [x.numpy().copy() for x in host]
    params_dev[8:8 + n].view(torch.int16).fill_(3)
    torch.cuda.synchronize()
    announce(f"offload step skip n={n}")
    ok = zs.zs_offload_step(grad_dev, grad_host, *host, params_host, params_dev[8:8 + n], hp,
                            flag_dev, flag_host, zs.ZS_BF16, threads, pieces, stream=side)
    side.synchronize()
    assert not ok and int(flag_host[0]) == 1
    want = oracle_offload_update(*before, bad, 1024.0, 1e-3, 0.9, 0.999, 1e-8, 0.01, 3, "bf16")
    assert want[0] == 1
    assert assert_offload_matches_oracle([x.numpy() for x in host], None, want, "bf16",
                                         "skipped offload step") == 0
    for got, ref_x in zip(host, before):
        assert_bits_equal(got.numpy(), ref_x, "skipped offload step")
    assert np.all(down16(params_dev.view(torch.int16))[8:8 + n] == 3)
