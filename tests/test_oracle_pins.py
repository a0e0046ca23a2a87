"""Pins of the CPU oracle to what the pages and the mathematics fix (CPU only).

Each test checks the oracle against something other than itself: values the
pages print (tests/golden/, each line cited), closed forms, exact integer
arithmetic, special cases with a known answer, or a library routine
(torch.optim.AdamW). They are chosen so a plausible slip in the oracle -- a
dropped or reordered term, a wrong sign, a missing bias correction, a check
before instead of after the unscale -- fails at least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from conftest import golden_rows

F32 = np.float32


def to_bf16_bits(x):
    """Bits of fp32 values that are exactly representable in bf16."""
    u = np.asarray(x, F32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not representable in bf16"
    return (u >> 16).astype(np.uint16)


def rand_bf16(rng, shape, scale=1.0):
    """Random bf16 bit patterns of N(0, scale) samples (truncated)."""
    x = (rng.standard_normal(shape) * scale).astype(F32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def test_fp_environment():
    assert oracle._load().zso_fp_env_ok() == 1


# ---- a1: partition ------------------------------------------------------------

def test_partition_properties_exhaustive():
    for phi in list(range(0, 130)) + [1000, 1023, 1024, 1025, 1999]:
        for w in range(1, 18):
            chunk = -(-phi // w) if phi else 0
            covered = []
            for r in range(w):
                p, off, cnt = oracle.partition(phi, w, r)
                assert p == max(chunk, 0)
                assert off == r * p
                assert 0 <= cnt <= p
                covered.extend(range(off, off + cnt))
            # contiguous, disjoint, covering: exactly 0..phi-1 in order
            assert covered == list(range(phi))


def test_partition_of_the_workloads():
    # 2^20 / 3 rounded up; exact divisions for the GPT-2-small shape at W = 8
    # and the 7.5B model at N = 64; W = 1 keeps everything.
    assert oracle.partition(2 ** 20, 3, 0) == (349_526, 0, 349_526)
    assert oracle.partition(2 ** 20, 3, 2) == (349_526, 699_052, 349_524)
    assert oracle.partition(124_439_808, 8, 0) == (15_554_976, 0, 15_554_976)
    assert oracle.partition(7_500_000_000, 64, 0)[2] == 117_187_500
    assert oracle.partition(7_000_000_000, 1, 0) == (7_000_000_000, 0, 7_000_000_000)
    assert oracle.partition(1_300_000_000, 4, 0)[2] == 325_000_000
    with pytest.raises(ValueError):
        oracle.partition(10, 0, 0)
    with pytest.raises(ValueError):
        oracle.partition(10, 3, 3)


# ---- a2: the ring, against the pages' three-GPU example -----------------------

NAMES = {c: i for i, c in enumerate("ABC")}


def _example_bufs(values):
    """bufs[k] = [A_k, B_k, C_k] with values[(chunk, gpu)]."""
    b = np.zeros((3, 3), F32)
    for (c, k), v in values.items():
        b[k, c] = v
    return b


def _rows(phase):
    return [r for r in golden_rows("ring_three_gpu_example.txt") if r[0] == phase]


def _contrib(tokens):
    return [(NAMES[t[0]], int(t[1])) for t in tokens]


def test_ring_example_contributor_sets():
    # Distinct powers of two: every partial sum is exact and names its terms.
    vals = {(c, k): F32(2.0 ** (3 * c + k)) for c in range(3) for k in range(3)}
    start = _example_bufs(vals)
    for step in (1, 2):
        before = start.copy()
        if step == 2:
            oracle.ring_reduce_scatter(before, sigma=1, steps=1)
        bufs = start.copy()
        oracle.ring_reduce_scatter(bufs, sigma=1, steps=step)
        touched = set()
        for _, s, gpu, chunk, *terms in _rows("scatter_reduce"):
            if int(s) != step:
                continue
            gpu, c = int(gpu), NAMES[chunk]
            touched.add((gpu, c))
            assert bufs[gpu, c] == sum(float(vals[t]) for t in _contrib(terms)), (step, gpu, chunk)
        for k in range(3):
            for c in range(3):
                if (k, c) not in touched:  # copies the step does not touch
                    assert bufs[k, c] == before[k, c], (step, k, c)
    # the rank that ends holding each chunk, in the page's labelling
    assert [oracle.ring_held_chunk(3, k, 1) for k in range(3)] == [1, 2, 0]
    total = {c: sum(float(vals[(c, k)]) for k in range(3)) for c in range(3)}
    for step in (1, 2):
        bufs = _example_bufs(vals)
        oracle.ring_reduce_scatter(bufs, sigma=1, steps=2)
        oracle.ring_all_gather(bufs, sigma=1, steps=step)
        for _, s, gpu, chunk, *terms in _rows("all_gather"):
            if int(s) == step:
                assert bufs[int(gpu), NAMES[chunk]] == total[NAMES[chunk]]
    # after both phases every GPU holds every total
    assert np.all(bufs == np.array([[total[c] for c in range(3)]] * 3, F32))


def test_ring_example_addition_order():
    # Random fp32 values: fp32 addition is not associative, so the bits only
    # match when the oracle adds the terms in the page's order.
    rng = np.random.default_rng(7)
    for trial in range(200):
        vals = {(c, k): F32(rng.standard_normal() * 10.0 ** rng.integers(-3, 4))
                for c in range(3) for k in range(3)}
        for steps in (1, 2):
            bufs = _example_bufs(vals)
            oracle.ring_reduce_scatter(bufs, sigma=1, steps=steps)
            for _, s, gpu, chunk, *terms in _rows("scatter_reduce"):
                if int(s) != steps:
                    continue
                acc = None
                for t in _contrib(terms):
                    acc = vals[t] if acc is None else F32(acc + vals[t])
                assert bufs[int(gpu), NAMES[chunk]].view(np.uint32) == F32(acc).view(np.uint32)


def test_ring_order_witness():
    # (2^24 + 1) - 2^24 = 0 in fp32 (the tie rounds to even), while
    # 2^24 + (1 - 2^24) = 1: the page's order (A0 to GPU1, then on to GPU2)
    # gives 0 for parameter A.
    vals = {(c, k): F32(0) for c in range(3) for k in range(3)}
    vals[(0, 0)], vals[(0, 1)], vals[(0, 2)] = F32(2 ** 24), F32(1), F32(-(2 ** 24))
    bufs = _example_bufs(vals)
    oracle.ring_reduce_scatter(bufs, sigma=1, steps=2)
    assert bufs[2, 0] == 0.0


@pytest.mark.parametrize("world", [1, 2, 3, 4, 5, 8, 13])
def test_ring_simulation_equals_chunk_trace(world):
    rng = np.random.default_rng(world)
    L = 37
    g16 = rand_bf16(rng, (world, world * L), 1e-3)
    bufs = oracle.half_to_float(g16, "bf16").reshape(world, world * L).copy()
    oracle.ring_reduce_scatter(bufs, sigma=0, steps=world - 1)
    for r in range(world):
        assert oracle.ring_held_chunk(world, r, 0) == r
        parts = [g16[k, r * L:(r + 1) * L] for k in range(world)]
        trace = oracle.ring_chunk_sum(parts, r, "bf16")
        np.testing.assert_array_equal(bufs[r, r * L:(r + 1) * L].view(np.uint32), trace.view(np.uint32))


@pytest.mark.parametrize("world", [1, 2, 3, 7, 31, 64])
def test_ring_sum_brute_force_integers(world):
    # Integers |x| <= 256 are exact in bf16 and their sums (< 2^24) exact in
    # fp32, so the ring sum must equal the integer sum.
    rng = np.random.default_rng(100 + world)
    n = 1031
    ints = rng.integers(-256, 257, size=(world, n))
    parts = [to_bf16_bits(ints[k].astype(F32)) for k in range(world)]
    for r in {0, world - 1, world // 2}:
        s = oracle.ring_chunk_sum(parts, r, "bf16")
        np.testing.assert_array_equal(s.astype(np.int64), ints.sum(axis=0))


# ---- a3/a4: average and accumulation -------------------------------------------

@pytest.mark.parametrize("world", [1, 2, 3, 5, 7, 8, 64])
def test_average_is_correctly_rounded_quotient(world):
    # fp32(s / W) via binary64: rounding twice is innocuous for division when
    # 53 >= 2*24 + 2, so this is the correctly rounded fp32 quotient.
    rng = np.random.default_rng(200 + world)
    n = 4099
    parts = [rand_bf16(rng, n, 1.0) for _ in range(world)]
    s = oracle.ring_chunk_sum(parts, 0, "bf16")
    out = np.empty(n, F32)
    flag = oracle.reduce_avg(parts, 0, "bf16", out, accumulate=False, loss_scale=1.0)
    assert flag == 0
    expect = (s.astype(np.float64) / world).astype(F32)
    np.testing.assert_array_equal(out.view(np.uint32), expect.view(np.uint32))


def test_accumulation_adds_in_micro_batch_order():
    rng = np.random.default_rng(5)
    n, world = 2000, 4
    acc = np.empty(n, F32)
    expect = None
    for j in range(4):
        parts = [rand_bf16(rng, n, 1.0) for _ in range(world)]
        oracle.reduce_avg(parts, 1, "bf16", acc, accumulate=(j > 0), loss_scale=1.0)
        a = (oracle.ring_chunk_sum(parts, 1, "bf16").astype(np.float64) / world).astype(F32)
        expect = a if expect is None else (expect + a).astype(F32)
        np.testing.assert_array_equal(acc.view(np.uint32), expect.view(np.uint32))


def test_data_parallel_equivalence_closed_form():
    # Lecture 7, "数学等价性": averaging the W worker means (each over B/W
    # samples) gives the mean over the whole batch. Dyadic values keep every
    # quantity exact, so the oracle must hit the exact batch mean.
    rng = np.random.default_rng(11)
    world, per = 4, 4
    B, n = world * per, 257
    samples = rng.integers(-8, 9, size=(B, n))
    parts = []
    for k in range(world):
        g_k = samples[k * per:(k + 1) * per].sum(axis=0).astype(F32) / F32(per)
        parts.append(to_bf16_bits(g_k))
    out = np.empty(n, F32)
    oracle.reduce_avg(parts, 0, "bf16", out, accumulate=False, loss_scale=1.0)
    for i in range(n):
        assert Fraction(float(out[i])) == Fraction(int(samples[:, i].sum()), B)


# ---- a5: unscale and overflow flag ----------------------------------------------

def test_flag_each_position_and_kind():
    n, world = 4099, 3
    rng = np.random.default_rng(3)
    base = [rand_bf16(rng, n, 1.0) for _ in range(world)]
    out = np.empty(n, F32)
    assert oracle.reduce_avg(base, 0, "bf16", out, False, 1024.0) == 0
    assert oracle.check_overflow(out, 1024.0) == 0
    specials = [0x7F80, 0xFF80, 0x7FC0]  # +inf, -inf, NaN
    for pos in range(n):
        k = pos % world
        parts = [b.copy() for b in base]
        parts[k][pos] = specials[pos % 3]
        assert oracle.reduce_avg(parts, 0, "bf16", out, False, 1024.0) == 1, pos
    # +inf and -inf in two workers at one index sum to NaN: still flagged
    parts = [b.copy() for b in base]
    parts[0][17], parts[2][17] = 0x7F80, 0xFF80
    assert oracle.reduce_avg(parts, 0, "bf16", out, False, 1.0) == 1
    assert np.isnan(out[17])


def test_flag_is_taken_after_the_unscale():
    # A finite average that overflows only once divided by a scale < 1.
    big = to_bf16_bits(np.full(8, 2.0 ** 126, F32))  # sum 2^127, mean 2^126
    parts = [big, big]
    out = np.empty(8, F32)
    assert oracle.reduce_avg(parts, 0, "bf16", out, False, 1.0) == 0
    assert np.all(np.isfinite(out))
    assert oracle.reduce_avg(parts, 0, "bf16", out, False, 0.25) == 1
    assert oracle.check_overflow(out, 0.25) == 1
    assert oracle.check_overflow(out, 1.0) == 0


def test_shard_step_flag_is_taken_after_the_unscale():
    # The whole step flags the unscaled gradient too: a finite average of
    # 2^126 is fine at S = 1 and overflows at S = 1/4.
    big = to_bf16_bits(np.full(8, 2.0 ** 126, F32))
    z = np.zeros(8, F32)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step_t=1)
    assert oracle.shard_step([big, big], 0, "bf16", "bf16", z, z, z, loss_scale=1.0, **hp)[0] == 0
    assert oracle.shard_step([big, big], 0, "bf16", "bf16", z, z, z, loss_scale=0.25, **hp)[0] == 1


# ---- a7: AdamW ------------------------------------------------------------------

def _ulp(x):
    return np.spacing(np.abs(F32(x)))


def test_adamw_first_step_is_lr_sign_g():
    # With m = v = 0, t = 1, no decay and eps = 0, Adam's first step moves
    # each weight by exactly lr against the sign of its gradient.
    rng = np.random.default_rng(1)
    n = 10000
    g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 3, n)).astype(F32)
    g[g == 0] = F32(1e-3)
    lr = 1e-3
    master = np.zeros(n, F32)
    m = np.zeros(n, F32)
    v = np.zeros(n, F32)
    oracle.adamw(master, m, v, g, 1.0, lr, 0.9, 0.999, 0.0, 0.0, 1)
    err = np.abs(master.astype(np.float64) + lr * np.sign(g))
    assert np.all(err <= 8 * _ulp(lr))


def test_adamw_first_step_decay_is_decoupled():
    # First step (m = v = 0, t = 1, eps = 0) with a large decay: the decay
    # multiplies the old weight only, theta'' = theta (1 - lr wd) - lr sign(g),
    # not (theta - lr sign(g)) (1 - lr wd), which differs by lr^2 wd.
    rng = np.random.default_rng(3)
    n = 5000
    theta = rng.uniform(-1, 1, n).astype(F32)
    g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 2, n)).astype(F32)
    g[g == 0] = F32(1.0)
    lr, wd = 0.1, 0.5
    master, m, v = theta.copy(), np.zeros(n, F32), np.zeros(n, F32)
    oracle.adamw(master, m, v, g, 1.0, lr, 0.9, 0.999, 0.0, wd, 1)
    lr32, wd32 = float(F32(lr)), float(F32(wd))
    want = theta.astype(np.float64) * (1.0 - lr32 * wd32) - lr32 * np.sign(g)
    assert np.all(np.abs(master - want) <= 16 * _ulp(np.maximum(np.abs(want), lr)))


def test_adamw_zero_gradient_is_pure_decay():
    rng = np.random.default_rng(2)
    n = 5000
    theta = (rng.standard_normal(n) * 0.02).astype(F32)
    master, m, v = theta.copy(), np.zeros(n, F32), np.zeros(n, F32)
    lr, wd = 1e-3, 0.1
    oracle.adamw(master, m, v, np.zeros(n, F32), 1.0, lr, 0.9, 0.999, 1e-8, wd, 7)
    exact = theta.astype(np.float64) * (1.0 - float(F32(lr)) * float(F32(wd)))
    assert np.all(np.abs(master - exact) <= 2 * _ulp(master))
    assert np.all(m == 0) and np.all(v == 0)
    assert np.all(np.abs(master) < np.abs(theta))  # decay shrinks, never grows


def test_adamw_bias_correction_constant_gradient():
    # A constant gradient g makes the bias-corrected moments g and g^2 at
    # every t, so each update is lr * g / (|g| + eps) for t = 1 .. 1000.
    g = np.array([1e-2, -1e-3, 0.5, -2.0, 1e-5], F32)
    lr, eps = 1e-3, 1e-8
    m = np.zeros(g.size, F32)
    v = np.zeros(g.size, F32)
    want = -float(F32(lr)) * g.astype(np.float64) / (np.abs(g.astype(np.float64)) + eps)
    for t in range(1, 1001):
        master = np.zeros(g.size, F32)  # read off this step's update alone
        oracle.adamw(master, m, v, g, 1.0, lr, 0.9, 0.999, eps, 0.0, t)
        np.testing.assert_allclose(master, want, rtol=2e-5, err_msg=f"t={t}")


def test_adamw_unscales_before_the_update():
    rng = np.random.default_rng(4)
    n = 3000
    g = (rng.standard_normal(n) * 1e-3).astype(F32)
    res = []
    for scale in (1.0, 1024.0):
        master = (rng.standard_normal(n) * 0.02).astype(F32) if not res else res[0][3].copy()
        if not res:
            start = master.copy()
        master = start.copy()
        m, v = np.zeros(n, F32), np.zeros(n, F32)
        oracle.adamw(master, m, v, (g * F32(scale)).astype(F32), scale, 1e-3, 0.9, 0.999,
                     1e-8, 0.01, 1)
        res.append((master, m, v, start))
    for a, b in zip(res[0][:3], res[1][:3]):
        np.testing.assert_array_equal(a, b)


def test_adamw_matches_torch_optim_adamw():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    n = 20000
    lr, b1, b2, eps, wd = [float(F32(x)) for x in (1e-3, 0.9, 0.999, 1e-8, 0.01)]
    theta0 = (rng.standard_normal(n) * 0.02).astype(F32)
    p = torch.nn.Parameter(torch.from_numpy(theta0.copy()))
    opt = torch.optim.AdamW([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd,
                            foreach=False, fused=False)
    master, m, v = theta0.copy(), np.zeros(n, F32), np.zeros(n, F32)
    for t in range(1, 8):
        g = (rng.standard_normal(n) * 1e-3).astype(F32)
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        oracle.adamw(master, m, v, g, 1.0, lr, b1, b2, eps, wd, t)
        st = opt.state[p]
        for ours, ref in ((master, p.detach().numpy()), (m, st["exp_avg"].numpy()),
                          (v, st["exp_avg_sq"].numpy())):
            np.testing.assert_allclose(ours, ref, rtol=1e-6, atol=1e-6 * float(np.abs(ref).max()))


# ---- whole step: composition, threads, skip ---------------------------------

def _step_inputs(rng, world, n, dtype="bf16"):
    parts = [rand_bf16(rng, n, 1e-3 * 1024) if dtype == "bf16" else
             (rng.standard_normal(n) * 1e-3 * 1024).astype(np.float16).view(np.uint16)
             for _ in range(world)]
    master = (rng.standard_normal(n) * 0.02).astype(F32)
    m = (rng.standard_normal(n) * 1e-4).astype(F32)
    v = rng.uniform(0, 1e-6, n).astype(F32)
    return parts, master, m, v


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("with_acc", [False, True])
def test_shard_step_is_the_composition(dtype, with_acc):
    rng = np.random.default_rng(21)
    world, n, rank = 5, 3001, 2
    parts, master, m, v = _step_inputs(rng, world, n, dtype)
    acc = (rng.standard_normal(n) * 1.0).astype(F32) if with_acc else None
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, loss_scale=1024.0)
    flag, mo, mmo, vo, po = oracle.shard_step(parts, rank, dtype, dtype, master, m, v,
                                              step_t=3, acc_in=acc, **hp)
    a = acc.copy() if with_acc else np.empty(n, F32)
    f2 = oracle.reduce_avg(parts, rank, dtype, a, accumulate=with_acc, loss_scale=1024.0)
    m2, mm2, v2 = master.copy(), m.copy(), v.copy()
    oracle.adamw(m2, mm2, v2, a, 1024.0, 1e-3, 0.9, 0.999, 1e-8, 0.01, 3)
    assert flag == f2 == 0
    for x, y in ((mo, m2), (mmo, mm2), (vo, v2)):
        np.testing.assert_array_equal(x.view(np.uint32), y.view(np.uint32))
    np.testing.assert_array_equal(po, oracle.float_to_half(m2, dtype))


def test_shard_step_thread_count_invariance():
    rng = np.random.default_rng(22)
    parts, master, m, v = _step_inputs(rng, 3, 10007)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, loss_scale=1024.0,
              step_t=1)
    ref = oracle.shard_step(parts, 0, "bf16", "bf16", master, m, v, threads=1, **hp)
    for t in (2, 3, 8, 64):
        got = oracle.shard_step(parts, 0, "bf16", "bf16", master, m, v, threads=t, **hp)
        assert got[0] == ref[0]
        for x, y in zip(got[1:], ref[1:]):
            np.testing.assert_array_equal(x, y)


def test_shard_step_flags_injected_values():
    rng = np.random.default_rng(23)
    parts, master, m, v = _step_inputs(rng, 4, 999, "fp16")
    parts[3][500] = 0x7E00  # NaN
    flag, *_ = oracle.shard_step(parts, 0, "fp16", "fp16", master, m, v, lr=1e-3, beta1=0.9,
                                 beta2=0.999, eps=1e-8, weight_decay=0.01, loss_scale=65536.0,
                                 step_t=1)
    assert flag == 1


# ---- a6: the dynamic scaler (reading: halve on overflow, double after 4 clean) ----

def test_scaler_schedule_with_two_overflows():
    s = oracle.Scaler(2.0 ** 16, 4)
    scales = []
    for step in range(1, 11):
        scales.append(s.scale)
        s.update(step in (3, 7))
    assert scales == [2.0 ** 16] * 3 + [2.0 ** 15] * 4 + [2.0 ** 14] * 3
    assert (s.scale, s.t, s.skipped, s.clean) == (2.0 ** 14, 8, 2, 3)


def test_scaler_doubles_after_interval_clean_steps():
    s = oracle.Scaler(1024.0, 4)
    seen = []
    for _ in range(12):
        seen.append(s.scale)
        s.update(False)
    assert seen == [1024.0] * 4 + [2048.0] * 4 + [4096.0] * 4
    assert s.scale == 8192.0 and s.t == 12 and s.clean == 0
    s.update(True)
    assert s.scale == 4096.0 and s.t == 12 and s.clean == 0


# ---- accounting against the printed numbers ----------------------------------

def test_model_state_memory_matches_the_pages():
    for psi, ngpu, stage, value, unit, digits, *src in golden_rows("model_state_memory.txt"):
        got = oracle.model_state_bytes(float(psi), float(ngpu), int(stage))
        if unit == "GB":
            got /= 1e9
        assert round(got, int(digits)) == float(value), " ".join(src)


def test_memory_savings_match_the_pages():
    full = oracle.model_state_bytes(1.0, 8.0, 0)
    for stage, pct, tol, *src in golden_rows("memory_savings.txt"):
        saved = 100.0 * (1.0 - oracle.model_state_bytes(1.0, 8.0, int(stage)) / full)
        assert abs(saved - float(pct)) <= float(tol), " ".join(src)


def test_ring_time_estimate_matches_the_pages():
    for msg, world, beta, secs, digits, *src in golden_rows("ring_comm_time.txt"):
        limit = oracle.ring_allreduce_time(float(msg), 1e15, 0.0, float(beta))
        assert round(limit, int(digits)) == float(secs), " ".join(src)
        exact = oracle.ring_allreduce_time(float(msg), float(world), 0.0, float(beta))
        assert exact < limit


# ---- 16-bit wire (partials rounded at every hop) ------------------------------------

def test_wire_bf16_witnesses():
    # W = 2, rank 0: the sum is G1 then + G0 (the owner's term last).
    one = to_bf16_bits(np.array([1.0, 1.0, 1.0078125, 1.0], F32))
    tiny = to_bf16_bits(np.array([2.0 ** -8, 3 * 2.0 ** -9, 2.0 ** -8, -2.0 ** -9], F32))
    parts = [tiny, one]  # worker 0 = owner, worker 1 = successor
    fp32 = oracle.ring_chunk_sum(parts, 0, "bf16")
    wire = oracle.ring_chunk_sum(parts, 0, "bf16", wire="bf16")
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even -> 1
    # 1 + 3*2^-9 is above the tie -> 1 + 2^-7
    # 1.0078125 + 2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: even -> 1 + 2^-6
    # 1 - 2^-9 is a tie between 1 - 2^-8 and 1 (spacing 2^-8 below 1): even -> 1
    np.testing.assert_array_equal(wire, np.array([1.0, 1.0078125, 1.015625, 1.0], F32))
    np.testing.assert_array_equal(fp32, np.array([1.00390625, 1.005859375, 1.01171875,
                                                  0.998046875], F32))


def test_wire_rounds_the_first_term_too():
    # fp16 gradients on a bf16 wire, W = 2, rank 0: the successor's value
    # goes on the wire (rounded to bf16) before the owner's term is added.
    # 1 + 2^-10 rounds to 1 on the wire; 1 + 2^-8 is then a tie -> even = 1.
    # 1 + 3*2^-10 rounds to 1; 1 + 2^-9 is below the tie -> 1.
    # Without the first rounding both would give 1 + 5*2^-10 -> 1 + 2^-7.
    owner = np.array([2.0 ** -8, 2.0 ** -9], np.float16).view(np.uint16)
    succ = np.array([1.0 + 2.0 ** -10, 1.0 + 3 * 2.0 ** -10], np.float16).view(np.uint16)
    got = oracle.ring_chunk_sum([owner, succ], 0, "fp16", wire="bf16")
    np.testing.assert_array_equal(got, np.array([1.0, 1.0], F32))
    a = np.empty(2, F32)
    oracle.reduce_avg([owner, succ], 0, "fp16", a, False, 1.0, wire="bf16")
    np.testing.assert_array_equal(a, np.array([0.5, 0.5], F32))


@pytest.mark.parametrize("wire,dtype,u", [("bf16", "bf16", 2.0 ** -8), ("fp16", "fp16", 2.0 ** -11)])
@pytest.mark.parametrize("world", [2, 8, 64])
def test_wire_rounding_bound_and_format(wire, dtype, u, world):
    rng = np.random.default_rng(world)
    n = 20000
    if dtype == "bf16":
        parts = [rand_bf16(rng, n, 1.0) for _ in range(world)]
    else:
        parts = [(rng.standard_normal(n)).astype(np.float16).view(np.uint16) for _ in range(world)]
    vals = np.stack([oracle.half_to_float(p, dtype).astype(np.float64) for p in parts])
    exact = vals.sum(axis=0)                         # |x| <= 2^16 terms: exact in binary64
    got = oracle.ring_chunk_sum(parts, 0, dtype, wire=wire)
    # every partial is rounded once (relative error <= u) after one fp32 add
    # (<= 2^-24): |error| <= W (u + 2^-24)(1 + u) * sum|x|
    bound = world * (u + 2.0 ** -24) * (1 + u) * np.abs(vals).sum(axis=0)
    assert np.all(np.abs(got.astype(np.float64) - exact) <= bound)
    # the result is a value of the wire format
    assert np.array_equal(oracle.half_to_float(oracle.float_to_half(got, wire), wire), got)
    # and the rounding is real: most sums differ from the fp32-wire ones
    fp32 = oracle.ring_chunk_sum(parts, 0, dtype)
    assert np.mean(got != fp32) > 0.5
    assert np.array_equal(oracle.ring_chunk_sum(parts, 0, dtype, wire="fp32"), fp32)


def test_wire_is_exact_when_every_partial_fits():
    rng = np.random.default_rng(12)
    ints = rng.integers(-8, 9, size=(16, 999))   # partial sums stay below 2^7
    parts = [to_bf16_bits(ints[k].astype(F32)) for k in range(16)]
    got = oracle.ring_chunk_sum(parts, 3, "bf16", wire="bf16")
    np.testing.assert_array_equal(got.astype(np.int64), ints.sum(axis=0))


def test_fp16_wire_overflow_raises_the_flag():
    big = np.full(5, 60000.0, np.float16).view(np.uint16)
    out = np.empty(5, F32)
    assert oracle.reduce_avg([big, big], 0, "fp16", out, False, 1.0) == 0
    assert np.all(out == 60000.0)                    # fp32 partials: 120000 / 2
    assert oracle.reduce_avg([big, big], 0, "fp16", out, False, 1.0, wire="fp16") == 1
    assert np.all(np.isinf(out))                     # 120000 overflows binary16


def test_shard_step_carries_the_wire():
    rng = np.random.default_rng(31)
    parts = [rand_bf16(rng, 3000, 1.0) for _ in range(8)]
    master = (rng.standard_normal(3000) * 0.02).astype(F32)
    z = np.zeros(3000, F32)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, loss_scale=1.0,
              step_t=1)
    f, mo, mmo, vo, po = oracle.shard_step(parts, 2, "bf16", "bf16", master, z, z, wire="bf16",
                                           **hp)
    a = np.empty(3000, F32)
    oracle.reduce_avg(parts, 2, "bf16", a, False, 1.0, wire="bf16")
    m2, mm2, v2 = master.copy(), z.copy(), z.copy()
    oracle.adamw(m2, mm2, v2, a, 1.0, 1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    np.testing.assert_array_equal(mo, m2)
    np.testing.assert_array_equal(mmo, mm2)
