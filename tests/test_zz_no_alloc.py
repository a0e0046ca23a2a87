"""zs_step_commit_noalloc, the entry point for callers that cannot allocate,
against zs_step_commit through the C ABI.

Both run the same kernels on the same seeded inputs, so every output is
compared bit for bit: the fp32 state, the 16-bit parameters (also on a
skipped step, where the caller discards them), the committed flag and the
scaler. Consecutive calls share the library's one overflow word: the first
call overflows and leaves it at 1, the next ones are smaller and clean, so
they commit only if each call clears the word. Committed steps are also held
to the oracle (fp32 state bit-exact, parameters within 1 ulp).
"""
import numpy as np
import pytest

import oracle
from gpu_util import F32, announce, assert_bits_equal, assert_ulp16, down16, down32, up16, up32

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)

# (world, rank, n, dtype, inject): each call smaller than, or as large as, the
# one before; a ragged n in each, and a W = 1 call for the other kernel shape.
CALLS = [
    (4, 1, 300_007, "fp16", True),
    (4, 2, 70_001, "fp16", False),
    (1, 0, 20_483, "bf16", False),
    (8, 5, 20_483, "bf16", True),
    (3, 0, 4_099, "fp16", False),
]


@pytest.fixture(scope="module")
def zs(hip_built):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sharded_mixed_precision_zs_amd import zeroshard
    return zeroshard


def rand16(rng, n, sigma, dtype):
    x = (rng.standard_normal(n) * sigma).astype(F32)
    if dtype == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    return x.astype(np.float16).view(np.uint16)


def bits16(t):
    return down16(t)


def scaler_fields(s):
    return (s.scale, s.clean_steps, s.growth_interval, s.dynamic, s.step_t, s.skipped)


def test_noalloc_commit_equals_commit(zs):
    rng = np.random.default_rng(20261202)
    host_flag = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    make = lambda: zs.zs_loss_scaler(scale=32768.0, clean_steps=0, growth_interval=2,
                                      dynamic=1, step_t=0, skipped=0)
    sc_ref, sc_new = make(), make()
    ref = oracle.Scaler(32768.0, 2)
    # the caller's own overflow word, which the new entry point must not touch
    ignored = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    for call, (world, rank, n, dtype, inject) in enumerate(CALLS):
        announce(f"noalloc call {call}: world={world} rank={rank} n={n} {dtype} "
                 f"inject={inject}")
        g16 = [rand16(rng, n, 1e-3 * ref.scale, dtype) for _ in range(world)]
        if inject:
            g16[call % world][n // 3] = 0x7C00 if dtype == "fp16" else 0x7F80
        master = (rng.standard_normal(n) * 0.02).astype(F32)
        m = (rng.standard_normal(n) * 1e-4).astype(F32)
        v = np.abs(rng.standard_normal(n) * 1e-7).astype(F32)
        dg = [up16(g, dtype) for g in g16]
        sin = [up32(x) for x in (master, m, v)]
        outs = {}
        for side in ("ref", "new"):
            sout = [torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
                    for _ in range(3)]
            gather = torch.zeros(n, dtype=torch.float16 if dtype == "fp16" else torch.bfloat16,
                                 device="cuda")
            flag = torch.zeros(1, dtype=torch.int32, device="cuda") if side == "ref" else ignored
            args = zs.StepArgs(dg, rank, n, *sin, *sout, gather, 0, flag,
                               zs.hparams(**HP, loss_scale=1.0, step_t=999))
            if side == "ref":
                ok = zs.zs_step_commit(args, sc_ref, host_flag)
            else:
                ok = zs.zs_step_commit_noalloc(args, sc_new, host_flag)
            torch.cuda.synchronize()
            outs[side] = (ok, int(host_flag.item()), [down32(t) for t in sout], bits16(gather))
        ok_r, hf_r, st_r, p_r = outs["ref"]
        ok_n, hf_n, st_n, p_n = outs["new"]
        assert ok_r == ok_n == (not inject), (call, ok_r, ok_n)
        assert hf_r == hf_n == (1 if inject else 0)
        assert scaler_fields(sc_ref) == scaler_fields(sc_new)
        for a, b, name in zip(st_r, st_n, ("master", "m", "v")):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"call {call} {name}"
        assert np.array_equal(p_r, p_n), f"call {call} params"
        assert int(ignored.item()) == 7, "the caller's overflow_flag was written"
        f, mo, mmo, vo, po = oracle.shard_step(g16, rank, dtype, dtype, master, m, v,
                                               loss_scale=ref.scale, step_t=ref.t + 1, **HP)
        assert f == (1 if inject else 0)
        ref.update(f)
        assert (sc_new.scale, sc_new.step_t, sc_new.skipped, sc_new.clean_steps) == \
            (ref.scale, ref.t, ref.skipped, ref.clean)
        if not inject:
            for got, want, name in zip(st_n, (mo, mmo, vo), ("master", "m", "v")):
                assert_bits_equal(got, want, f"call {call} {name} vs oracle")
            assert assert_ulp16(p_n, po, dtype, 1, f"call {call} params vs oracle") == 0


def test_noalloc_commit_accepts_null_flag_and_empty_shard(zs):
    """a->overflow_flag NULL is accepted; n == 0 commits without a launch."""
    host_flag = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    sc = zs.zs_loss_scaler(scale=1024.0, clean_steps=0, growth_interval=1000, dynamic=1,
                           step_t=4, skipped=0)
    rng = np.random.default_rng(5)
    for n in (0, 2_049):
        announce(f"noalloc null flag n={n}")
        g = [up16(rand16(rng, max(n, 1), 1.0, "bf16"), "bf16") for _ in range(2)]
        sin = [up32(np.zeros(max(n, 1), F32)) for _ in range(3)]
        sout = [torch.empty(max(n, 1), dtype=torch.float32, device="cuda") for _ in range(3)]
        gather = torch.empty(max(n, 1), dtype=torch.bfloat16, device="cuda")
        args = zs.StepArgs(g, 1, n, *sin, *sout, gather, 0, None,
                           zs.hparams(**HP, loss_scale=1.0, step_t=1))
        t0 = sc.step_t
        assert zs.zs_step_commit_noalloc(args, sc, host_flag) is True
        assert sc.step_t == t0 + 1
    torch.cuda.synchronize()


def test_noalloc_commit_refusals(zs):
    """Refused calls leave the scaler unchanged."""
    host_flag = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    n = 1_000
    g = [up16(np.zeros(n, np.uint16), "fp16")]
    sin = [up32(np.zeros(n, F32)) for _ in range(3)]
    sout = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3)]
    gather = torch.empty(n, dtype=torch.float16, device="cuda")
    args = zs.StepArgs(g, 0, n, *sin, *sout, gather, 0, None,
                       zs.hparams(**HP, loss_scale=1.0, step_t=1))
    bad_scale = zs.zs_loss_scaler(scale=float("inf"), clean_steps=0, growth_interval=2,
                                  dynamic=1, step_t=0, skipped=0)
    with pytest.raises(zs.ZsError) as e:
        zs.zs_step_commit_noalloc(args, bad_scale, host_flag)
    assert e.value.status == zs.ZS_ERR_INVALID_ARG
    alias = zs.StepArgs(g, 0, n, *sin, sin[0], sout[1], sout[2], gather, 0, None,
                        zs.hparams(**HP, loss_scale=1.0, step_t=1))
    sc = zs.zs_loss_scaler(scale=8.0, clean_steps=0, growth_interval=2, dynamic=1, step_t=0,
                           skipped=0)
    with pytest.raises(zs.ZsError) as e:
        zs.zs_step_commit_noalloc(alias, sc, host_flag)
    assert e.value.status == zs.ZS_ERR_ALIAS
    assert (sc.scale, sc.step_t, sc.skipped) == (8.0, 0, 0)
    torch.cuda.synchronize()
