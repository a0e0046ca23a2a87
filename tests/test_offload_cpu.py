"""The ZeRO-Offload host update (zs_cpu_step) against the oracle (CPU only).

zs_cpu_step is product code that runs on the host: AdamW and the 16-bit
cast on CPU memory, AVX-512 where available. It must equal the oracle's
arithmetic bit for bit (fp32 state) and the oracle's round-to-nearest-even
casts (16-bit parameters, NaN by class).
"""
import numpy as np
import pytest

import oracle

F32 = np.float32


@pytest.fixture(scope="module")
def zs(hip_built):
    from sharded_mixed_precision_zs_amd import zeroshard
    return zeroshard


HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _inputs(rng, n, scale):
    master = (rng.standard_normal(n) * 0.02).astype(F32)
    m = (rng.standard_normal(n) * 1e-4).astype(F32)
    v = rng.uniform(0, 1e-6, n).astype(F32)
    a = (rng.standard_normal(n) * 1e-3 * scale).astype(F32)
    return master, m, v, a


def _nan_class_equal(x, y):
    return np.array_equal(np.isnan(x), np.isnan(y)) and \
        np.array_equal(x[~np.isnan(x)].view(np.uint32), y[~np.isnan(y)].view(np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("n,threads", [(1, 1), (15, 1), (16, 1), (100_003, 1), (100_003, 3),
                                       (1_000_000, 0)])
def test_cpu_step_matches_oracle(zs, dtype, n, threads):
    rng = np.random.default_rng(n + threads)
    for scale, t in ((1.0, 1), (1024.0, 7), (3.0, 300)):
        master, m, v, a = _inputs(rng, n, scale)
        got = [x.copy() for x in (master, m, v)]
        params = np.full(n, 7, np.uint16)
        hp = zs.hparams(**HP, loss_scale=scale, step_t=t)
        flag = zs.zs_cpu_step(*got, a, hp, params, zs.ZS_BF16 if dtype == "bf16" else zs.ZS_FP16,
                              threads)
        assert flag == 0
        oracle.adamw(master, m, v, a, scale, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"],
                     HP["weight_decay"], t)
        for x, y in zip(got, (master, m, v)):
            assert _nan_class_equal(x, y)
        assert np.array_equal(params, oracle.float_to_half(master, dtype))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_cpu_step_special_values_and_casts(zs, dtype):
    """Masters chosen to land on rounding ties, subnormals and overflow of the
    16-bit format; the update itself is made the identity (lr = wd = 0)."""
    rng = np.random.default_rng(5)
    pats = np.concatenate([
        (np.arange(1 << 16, dtype=np.uint32) << 16) | 0x8000,      # bf16 ties
        (np.arange(1 << 16, dtype=np.uint32) << 16) | 0x7FFF,
        rng.integers(0, 1 << 32, 1 << 18, dtype=np.uint64).astype(np.uint32),
    ]).view(F32)
    n = pats.size
    master = pats.copy()
    m = np.zeros(n, F32)
    v = np.zeros(n, F32)
    a = np.zeros(n, F32)
    params = np.empty(n, np.uint16)
    hp = zs.hparams(0.0, 0.9, 0.999, 1e-8, 0.0, 1.0, 1)
    zs.zs_cpu_step(master, m, v, a, hp, params, zs.ZS_BF16 if dtype == "bf16" else zs.ZS_FP16, 4)
    want = oracle.float_to_half(pats, dtype)
    nanmask = 0x7F80 if dtype == "bf16" else 0x7C00
    frac = 0x007F if dtype == "bf16" else 0x03FF

    def isnan(b):
        b = b.astype(np.int32)
        return ((b & nanmask) == nanmask) & ((b & frac) != 0)
    assert np.array_equal(isnan(params), isnan(want))
    assert np.array_equal(params[~isnan(want)], want[~isnan(want)])


def test_cpu_step_skips_on_overflow(zs):
    rng = np.random.default_rng(6)
    n = 50_000
    master, m, v, a = _inputs(rng, n, 1.0)
    for pos, val in ((0, np.inf), (n - 1, -np.inf), (31_337, np.nan)):
        x = a.copy()
        x[pos] = val
        st = [y.copy() for y in (master, m, v)]
        params = np.full(n, 7, np.uint16)
        assert zs.zs_cpu_step(*st, x, zs.hparams(**HP, loss_scale=1.0, step_t=1), params,
                              zs.ZS_BF16, 2) == 1
        for y, z in zip(st, (master, m, v)):
            assert np.array_equal(y.view(np.uint32), z.view(np.uint32))
        assert np.all(params == 7)


def test_cpu_step_rejects_bad_arguments(zs):
    x = np.zeros(10, F32)
    p = np.zeros(10, np.uint16)
    with pytest.raises(zs.ZsError):
        zs.zs_cpu_step(x, x.copy(), x.copy(), x.copy(), zs.hparams(**HP, loss_scale=0.0, step_t=1),
                       p, zs.ZS_BF16)
    with pytest.raises(zs.ZsError):
        zs.zs_cpu_step(x, x.copy(), x.copy(), x.copy(), zs.hparams(**HP, loss_scale=1.0, step_t=0),
                       p, zs.ZS_BF16)
    with pytest.raises(zs.ZsError):
        zs.zs_cpu_step(x, x.copy(), x.copy(), x.copy(), zs.hparams(**HP, loss_scale=1.0, step_t=1),
                       p, 9)
    # the message names what the host update checks, not an earlier call's error
    bad = dict(HP, beta1=1.0)
    with pytest.raises(zs.ZsError, match="hyper-parameter out of range"):
        zs.zs_cpu_update(x, x.copy(), x.copy(), x.copy(), zs.hparams(**bad, loss_scale=1.0, step_t=1),
                         p, zs.ZS_BF16)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("n,threads", [(1, 1), (4099, 2), (200_003, 0)])
def test_cpu_update_equals_cpu_step(zs, dtype, n, threads):
    """zs_cpu_update is zs_cpu_step's update pass alone: the same bits on
    finite gradients, in pieces or whole."""
    rng = np.random.default_rng(n)
    master, m, v, a = _inputs(rng, n, 1024.0)
    hp = zs.hparams(**HP, loss_scale=1024.0, step_t=9)
    code = zs.ZS_BF16 if dtype == "bf16" else zs.ZS_FP16
    ref = [x.copy() for x in (master, m, v)]
    pref = np.empty(n, np.uint16)
    assert zs.zs_cpu_step(*ref, a, hp, pref, code, threads) == 0
    got = [x.copy() for x in (master, m, v)]
    pgot = np.empty(n, np.uint16)
    cuts = sorted({0, n // 3, n // 2, n})
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        zs.zs_cpu_update(*(x[lo:hi] for x in got), a[lo:hi], hp, pgot[lo:hi], code, threads)
    for x, y in zip(got, ref):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert np.array_equal(pgot, pref)
    with pytest.raises(zs.ZsError):
        zs.zs_cpu_update(*got, a, zs.hparams(**HP, loss_scale=0.0, step_t=1), pgot, code)


def test_bias_correction_powers_continue_exactly(zs):
    """The host forms beta^t by t repeated products and continues the
    product from the previous call when t grows: t = 1 .. 3000 in order,
    then a jump back to t = 7 and forward to 5000, each equal bit for bit
    to the oracle's from-scratch products."""
    rng = np.random.default_rng(9)
    n = 64
    master, m, v, a = _inputs(rng, n, 1.0)
    for t in list(range(1, 3001)) + [7, 5000]:
        got = [x.copy() for x in (master, m, v)]
        p = np.empty(n, np.uint16)
        zs.zs_cpu_update(*got, a, zs.hparams(**HP, loss_scale=1.0, step_t=t), p, zs.ZS_BF16, 1)
        want = [x.copy() for x in (master, m, v)]
        oracle.adamw(*want, a, 1.0, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"],
                     HP["weight_decay"], t)
        for x, y in zip(got, want):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), t


def test_concurrent_callers_share_the_pool_safely(zs):
    """Host threads calling zs_cpu_step at the same time (ctypes releases the
    GIL, so the calls overlap) on disjoint buffers: the library serialises
    them on its one worker pool, and every result equals the oracle's."""
    import threading

    n, callers, rounds = 200_003, 6, 4
    rng = np.random.default_rng(77)
    jobs = []
    for k in range(callers):
        master, m, v, a = _inputs(rng, n, 1024.0)
        jobs.append(dict(inp=(master, m, v, a), got=[master.copy(), m.copy(), v.copy()],
                         params=np.zeros(n, np.uint16), t=1 + k))
    errors = []

    def work(job):
        try:
            for r in range(rounds):
                hp = zs.hparams(**HP, loss_scale=1024.0, step_t=job["t"] + r)
                if zs.zs_cpu_step(*job["got"], job["inp"][3], hp, job["params"], zs.ZS_BF16,
                                  1 + job["t"] % 4) != 0:
                    errors.append("flag")
        except Exception as e:  # noqa: BLE001 (reported below)
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(j,)) for j in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for job in jobs:
        master, m, v, a = (x.copy() for x in job["inp"])
        for r in range(rounds):
            oracle.adamw(master, m, v, a, 1024.0, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"],
                         HP["weight_decay"], job["t"] + r)
        for x, y in zip(job["got"], (master, m, v)):
            assert _nan_class_equal(x, y)
        assert np.array_equal(job["params"], oracle.float_to_half(master, "bf16"))
