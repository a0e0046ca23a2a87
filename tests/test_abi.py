"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and its host-only logic (partition, scaler, argument validation
that returns before any launch) behaves as documented. No GPU work is done.
"""
import ctypes as C
import os
import re

import pytest

import oracle
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "zeroshard.h")


@pytest.fixture(scope="module")
def zs(hip_built):
    from sharded_mixed_precision_zs_amd import zeroshard
    return zeroshard


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zs_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("zs_reduce_scatter_avg", "zs_check_overflow", "zs_adamw_step",
                     "zs_cast_gather", "zs_step_fused", "zs_partition", "zs_scaler_update",
                     "zs_abi_version", "zs_status_string", "zs_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol(zs):
    lib = C.CDLL(zs.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert zs.zs_abi_version() == zs.ZS_ABI_VERSION == 7
    # the binding's zs_step_args matches the header's layout (the C driver
    # under tests/sanitize asserts the same size and offsets at compile time)
    assert C.sizeof(zs.zs_step_args) == 152
    assert zs.zs_step_args.wire_dtype.offset == 140
    assert zs.zs_step_args.state_layout.offset == 144


def test_status_strings(zs):
    assert zs.zs_status_string(zs.ZS_OK) == "ZS_OK"
    assert zs.zs_status_string(zs.ZS_ERR_ALIAS) == "ZS_ERR_ALIAS"
    assert zs.zs_status_string(99) == "ZS_UNKNOWN_STATUS"


def test_partition_matches_oracle(zs):
    for phi in (0, 1, 2, 3, 7, 100, 1001, 2 ** 20, 124_439_808, 7_500_000_000):
        for w in (1, 2, 3, 4, 7, 8, 64):
            for r in sorted({0, 1 % w, w // 2, w - 1}):
                assert zs.zs_partition(phi, w, r) == oracle.partition(phi, w, r)
    with pytest.raises(zs.ZsError) as e:
        zs.zs_partition(10, 0, 0)
    assert e.value.status == zs.ZS_ERR_INVALID_ARG
    with pytest.raises(zs.ZsError):
        zs.zs_partition(10, 4, 4)


def test_scaler_matches_oracle(zs):
    rng = __import__("numpy").random.default_rng(0)
    flags = [int(x) for x in rng.random(200) < 0.15]
    ours = zs.zs_loss_scaler(scale=65536.0, clean_steps=0, growth_interval=4, dynamic=1,
                             step_t=0, skipped=0)
    ref = oracle.Scaler(65536.0, 4)
    for f in flags:
        zs.zs_scaler_update(ours, f)
        ref.update(f)
        assert (ours.scale, ours.clean_steps, ours.step_t, ours.skipped) == \
            (ref.scale, ref.clean, ref.t, ref.skipped)
    static = zs.zs_loss_scaler(scale=1024.0, clean_steps=0, growth_interval=0, dynamic=0,
                               step_t=0, skipped=0)
    for f in (0, 1, 0, 0, 0, 0, 0):
        zs.zs_scaler_update(static, f)
    assert static.scale == 1024.0 and static.step_t == 6 and static.skipped == 1


# Raw C calls with fake, never-dereferenced addresses: every case below must
# be rejected on the host before anything is enqueued.
FAKE = 0x7F0000000000


def _raw(zs):
    return zs._lib


def test_reduce_rejects_bad_arguments(zs):
    lib = _raw(zs)
    arr = (C.c_void_p * 3)(FAKE, FAKE + 4096, FAKE + 8192)
    ok_out = C.c_void_p(FAKE + 65536)
    cases = [
        (None, 0, 3, 0, 10, ok_out, 1.0),           # null worker array
        (arr, 0, 3, 0, 10, None, 1.0),               # null output
        (arr, 0, 0, 0, 10, ok_out, 1.0),             # world 0
        (arr, 0, 65, 0, 10, ok_out, 1.0),            # world > 64
        (arr, 0, 3, 3, 10, ok_out, 1.0),             # rank >= world
        (arr, 7, 3, 0, 10, ok_out, 1.0),             # bad dtype
        (arr, 0, 3, 0, 10, ok_out, 0.0),             # zero scale
        (arr, 0, 3, 0, 10, ok_out, float("inf")),    # inf scale
        (arr, 0, 3, 0, 10, ok_out, float("nan")),    # nan scale
    ]
    for a, dt, w, r, n, out, s in cases:
        st = lib.zs_reduce_scatter_avg(a, dt, 0, w, r, n, out, 0, None, s, None)
        assert st == zs.ZS_ERR_INVALID_ARG, (w, r, dt, s)
        assert zs.zs_last_error()
    nulls = (C.c_void_p * 3)(FAKE, None, FAKE)
    assert lib.zs_reduce_scatter_avg(nulls, 0, 0, 3, 0, 10, ok_out, 0, None, 1.0, None) == \
        zs.ZS_ERR_INVALID_ARG
    # n == 0 is a no-op
    for wire in (-1, 3):                             # bad wire dtype
        assert lib.zs_reduce_scatter_avg(arr, 0, wire, 3, 0, 10, ok_out, 0, None, 1.0, None) == \
            zs.ZS_ERR_INVALID_ARG
    assert lib.zs_reduce_scatter_avg(arr, 0, 0, 3, 0, 0, ok_out, 0, None, 1.0, None) == zs.ZS_OK


def test_other_entry_points_reject_bad_arguments(zs):
    lib = _raw(zs)
    hp = zs.hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
    bad_t = zs.hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 0)
    p = C.c_void_p(FAKE)
    E = zs.ZS_ERR_INVALID_ARG
    assert lib.zs_check_overflow(None, 10, 1.0, p, None) == E
    assert lib.zs_check_overflow(p, 10, 1.0, None, None) == E
    assert lib.zs_check_overflow(p, 10, -1.0, p, None) == E
    assert lib.zs_adamw_step(p, p, None, p, 10, C.byref(hp), None, None) == E
    assert lib.zs_adamw_step(p, p, p, p, 10, C.byref(bad_t), None, None) == E
    assert lib.zs_adamw_step(p, p, p, p, 10, None, None, None) == E
    assert lib.zs_cast_gather(None, p, 0, 0, 10, None, None) == E
    assert lib.zs_cast_gather(p, p, 5, 0, 10, None, None) == E
    assert lib.zs_check_overflow(p, 0, 1.0, p, None) == zs.ZS_OK
    assert lib.zs_adamw_step(p, p, p, p, 0, C.byref(hp), None, None) == zs.ZS_OK
    assert lib.zs_cast_gather(p, p, 0, 0, 0, None, None) == zs.ZS_OK


def _fused_args(zs, n=1000, **over):
    grads = (C.c_void_p * 2)(FAKE, FAKE + 0x100000)
    a = zs.zs_step_args()
    a.world, a.rank, a.n = 2, 0, n
    a.grad_dtype = a.param_dtype = zs.ZS_BF16
    a.worker_grads = C.cast(grads, C.POINTER(C.c_void_p))
    base = FAKE + 0x1000000
    a.master_in, a.m_in, a.v_in = base, base + 0x100000, base + 0x200000
    a.master_out, a.m_out, a.v_out = base + 0x300000, base + 0x400000, base + 0x500000
    a.gather_buf, a.gather_offset = base + 0x600000, 0
    a.overflow_flag = base + 0x700000
    a.hp = zs.hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
    for k, v in over.items():
        setattr(a, k, v)
    return a, grads


def test_fused_rejects_aliasing_and_bad_arguments(zs):
    lib = _raw(zs)
    base = FAKE + 0x1000000
    for field, addr in (("master_out", base), ("m_out", base + 0x100000 + 40),
                        ("v_out", base + 0x200000 - 8), ("gather_buf", base + 0x100)):
        a, keep = _fused_args(zs, **{field: addr})
        assert lib.zs_step_fused(C.byref(a), None) == zs.ZS_ERR_ALIAS, field
    a, keep = _fused_args(zs, m_out=base + 0x300000 + 100)       # two outputs overlap
    assert lib.zs_step_fused(C.byref(a), None) == zs.ZS_ERR_ALIAS
    a, keep = _fused_args(zs, master_out=FAKE + 8)                # output on a gradient
    assert lib.zs_step_fused(C.byref(a), None) == zs.ZS_ERR_ALIAS
    a, keep = _fused_args(zs, acc_in=base + 0x400000)             # output on acc_in
    assert lib.zs_step_fused(C.byref(a), None) == zs.ZS_ERR_ALIAS
    for field, val in (("world", 0), ("world", 65), ("rank", 2), ("grad_dtype", 3),
                       ("overflow_flag", None), ("master_in", None), ("wire_dtype", 5)):
        a, keep = _fused_args(zs, **{field: val})
        assert lib.zs_step_fused(C.byref(a), None) == zs.ZS_ERR_INVALID_ARG, field
    a, keep = _fused_args(zs)
    a.hp.step_t = 0
    assert lib.zs_step_fused(C.byref(a), None) == zs.ZS_ERR_INVALID_ARG
    a, keep = _fused_args(zs, n=0)
    assert lib.zs_step_fused(C.byref(a), None) == zs.ZS_OK
    assert lib.zs_step_fused(None, None) == zs.ZS_ERR_INVALID_ARG


def test_fused_grouped_layout_rules(zs):
    """The grouped state layout: m and v pointers must be NULL, the layout
    code must be known, the state buffers overlap by their grouped size
    (whole groups of 1024 elements, 12 KB each), and every operand must be
    aligned for 4-element vectors; all refused before anything runs."""
    lib = _raw(zs)
    base = FAKE + 0x1000000
    G = dict(state_layout=zs.ZS_STATE_GROUPED, m_in=None, v_in=None, m_out=None, v_out=None)
    for field, val in (("m_in", base + 0x100000), ("v_out", base + 0x500000)):
        a, keep = _fused_args(zs, **{**G, field: val})
        assert lib.zs_step_fused(C.byref(a), None) == zs.ZS_ERR_INVALID_ARG, field
    a, keep = _fused_args(zs, state_layout=2)
    assert lib.zs_step_fused(C.byref(a), None) == zs.ZS_ERR_INVALID_ARG
    a, keep = _fused_args(zs)  # split with a NULL m_in is still refused
    a.m_in = None
    assert lib.zs_step_fused(C.byref(a), None) == zs.ZS_ERR_INVALID_ARG
    # n = 1000: one group, 12288 bytes; 8 KB past master_in overlaps it
    # (split arrays of 4000 bytes would not)
    a, keep = _fused_args(zs, **G, master_out=base + 0x2000)
    assert lib.zs_step_fused(C.byref(a), None) == zs.ZS_ERR_ALIAS
    a, keep = _fused_args(zs, **G, master_out=base + 0x300000, gather_buf=base + 0x2f00)
    assert lib.zs_step_fused(C.byref(a), None) == zs.ZS_ERR_ALIAS
    for field, addr in (("master_in", base + 4), ("master_out", base + 0x300008),
                        ("gather_buf", base + 0x600002)):
        a, keep = _fused_args(zs, **{**G, field: addr})
        assert lib.zs_step_fused(C.byref(a), None) == zs.ZS_ERR_UNSUPPORTED, field
    assert zs.grouped_len(1) == 3072 and zs.grouped_len(1024) == 3072
    assert zs.grouped_len(1025) == 6144 and zs.grouped_len(0) == 0


def test_step_commit_rejects_bad_arguments(zs):
    lib = _raw(zs)
    a, keep = _fused_args(zs)
    good = zs.zs_loss_scaler(scale=1024.0, clean_steps=0, growth_interval=4, dynamic=1,
                             step_t=0, skipped=0)
    hf = C.c_uint32(0)
    ok = C.c_int(7)
    E = zs.ZS_ERR_INVALID_ARG
    assert lib.zs_step_commit(None, C.byref(good), C.byref(hf), None, None, None, C.byref(ok)) == E
    assert lib.zs_step_commit(C.byref(a), None, C.byref(hf), None, None, None, C.byref(ok)) == E
    assert lib.zs_step_commit(C.byref(a), C.byref(good), None, None, None, None, C.byref(ok)) == E
    assert lib.zs_step_commit(C.byref(a), C.byref(good), C.byref(hf), None, None, None, None) == E
    for bad_scale in (0.0, -1.0, float("inf"), float("nan")):
        sc = zs.zs_loss_scaler(scale=bad_scale, clean_steps=0, growth_interval=4, dynamic=1,
                               step_t=0, skipped=0)
        assert lib.zs_step_commit(C.byref(a), C.byref(sc), C.byref(hf), None, None, None,
                                  C.byref(ok)) == E
    alias, keep2 = _fused_args(zs, master_out=FAKE + 0x1000000)
    assert lib.zs_step_commit(C.byref(alias), C.byref(good), C.byref(hf), None, None, None,
                              C.byref(ok)) == zs.ZS_ERR_ALIAS
    # every error left the scaler untouched; n == 0 commits an empty step
    assert (good.scale, good.step_t, good.skipped) == (1024.0, 0, 0)
    empty, keep3 = _fused_args(zs, n=0)
    assert lib.zs_step_commit(C.byref(empty), C.byref(good), C.byref(hf), None, None, None,
                              C.byref(ok)) == zs.ZS_OK
    assert ok.value == 1 and good.step_t == 1


def test_all_gather_step_rejects_bad_arguments(zs):
    lib = _raw(zs)
    reps = (C.c_void_p * 3)(FAKE, FAKE + 0x100000, FAKE + 0x200000)
    E = zs.ZS_ERR_INVALID_ARG
    assert lib.zs_all_gather_step(None, 3, 1000, 0, 1, None) == E
    assert lib.zs_all_gather_step(reps, 0, 1000, 0, 1, None) == E
    assert lib.zs_all_gather_step(reps, 65, 1000, 0, 1, None) == E
    assert lib.zs_all_gather_step(reps, 3, 1000, 3, 1, None) == E    # sigma >= world
    assert lib.zs_all_gather_step(reps, 3, 1000, 0, 0, None) == E    # step 0
    assert lib.zs_all_gather_step(reps, 3, 1000, 0, 3, None) == E    # step >= world
    nul = (C.c_void_p * 3)(FAKE, None, FAKE + 0x200000)
    assert lib.zs_all_gather_step(nul, 3, 1000, 0, 1, None) == E
    close = (C.c_void_p * 3)(FAKE, FAKE + 1000, FAKE + 0x200000)  # 2*phi bytes overlap
    assert lib.zs_all_gather_step(close, 3, 1000, 0, 1, None) == zs.ZS_ERR_ALIAS
    assert lib.zs_all_gather_step(reps, 3, 0, 0, 1, None) == zs.ZS_OK  # phi == 0


def test_device_scaler_layout_and_image(zs):
    """The host image of the device scaler: fields copied from the host
    scaler, beta powers formed by t+1 repeated binary64 products, and the
    bias corrections they give equal the oracle's for step t+1."""
    assert C.sizeof(zs.zs_device_scaler) == 88
    assert zs.zs_device_scaler.beta1_t.offset == 32 and zs.zs_device_scaler.epoch.offset == 48
    assert zs.zs_device_scaler.checked_epoch.offset == 64 and zs.zs_device_scaler.last_alpha.offset == 80
    import numpy as np
    for b1, b2, lr, t in ((0.9, 0.999, 1e-3, 0), (0.9, 0.95, 3e-4, 7), (0.8, 0.9999, 1e-2, 1234)):
        host = zs.zs_loss_scaler(scale=2.0 ** 15, clean_steps=3, growth_interval=4, dynamic=1,
                                 step_t=t, skipped=2)
        img = zs.zs_device_scaler_make(host, b1, b2)
        assert (img.scale, img.clean_steps, img.growth_interval, img.dynamic, img.step_t,
                img.skipped) == (2.0 ** 15, 3, 4, 1, t, 2)
        assert (img.epoch, img.flag_epoch, img.checked_epoch, img.last_flag, img.bad_scale) == \
            (0, 0, 0, 0, 0)
        p1 = p2 = 1.0
        for _ in range(t + 1):
            p1 *= float(np.float32(b1))
            p2 *= float(np.float32(b2))
        assert (img.beta1_t, img.beta2_t) == (p1, p2)
        k = oracle.adamw_consts(lr, b1, b2, 1e-8, 0.01, t + 1)
        lr64 = float(np.float32(lr))
        assert np.float32(lr64 / (1.0 - img.beta1_t)) == np.float32(k["alpha"])
        assert np.float32(np.sqrt(1.0 - img.beta2_t)) == np.float32(k["b2"])
    for bad in (0.0, -2.0, float("inf"), float("nan")):
        with pytest.raises(zs.ZsError):
            zs.zs_device_scaler_make(zs.zs_loss_scaler(scale=bad, clean_steps=0,
                                                       growth_interval=0, dynamic=0, step_t=0,
                                                       skipped=0), 0.9, 0.999)


def test_device_step_rejects_bad_arguments(zs):
    """Argument errors return before anything is enqueued (no GPU needed)."""
    lib = _raw(zs)
    a, keep = _fused_args(zs)
    E = zs.ZS_ERR_INVALID_ARG
    dev = C.c_void_p(FAKE + 0x7000000)
    assert lib.zs_step_device(C.byref(a), None, None, None, None) == E
    assert lib.zs_step_device(C.byref(a), C.c_void_p(FAKE + 0x7000004), None, None, None) == E
    assert lib.zs_step_device(None, dev, None, None, None) == E
    bad, keep2 = _fused_args(zs, grad_dtype=5)
    assert lib.zs_step_device(C.byref(bad), dev, None, None, None) == E
    alias, keep3 = _fused_args(zs, master_out=FAKE + 0x1000000)
    assert lib.zs_step_device(C.byref(alias), dev, None, None, None) == zs.ZS_ERR_ALIAS
    good, keep4 = _fused_args(zs)
    inside = C.c_void_p(good.m_out + 64)          # the scaler inside an output
    assert lib.zs_step_device(C.byref(good), inside, None, None, None) == zs.ZS_ERR_ALIAS
    # the scaler inside an input: master_in, m_in, v_in, acc_in or a gradient
    for field, offset in (("master_in", 0), ("m_in", 3992), ("v_in", 16)):
        inside = C.c_void_p(getattr(good, field) + offset)
        assert lib.zs_step_device(C.byref(good), inside, None, None, None) == \
            zs.ZS_ERR_ALIAS, field
    acc, keep5 = _fused_args(zs, acc_in=FAKE + 0x1800000)
    inside = C.c_void_p(FAKE + 0x1800000 + 8)
    assert lib.zs_step_device(C.byref(acc), inside, None, None, None) == zs.ZS_ERR_ALIAS
    for g in (FAKE, FAKE + 0x100000 + 1992):       # each worker's 2 n bytes
        assert lib.zs_step_device(C.byref(good), C.c_void_p(g), None, None, None) == \
            zs.ZS_ERR_ALIAS


def test_huge_sizes_are_refused_before_any_arithmetic(zs):
    """Counts and offsets above 2^48 return ZS_ERR_UNSUPPORTED (byte extents
    are 4 n and must not wrap around in the overlap checks)."""
    lib = _raw(zs)
    U = zs.ZS_ERR_UNSUPPORTED
    huge = 1 << 62
    arr = (C.c_void_p * 2)(FAKE, FAKE + 4096)
    out = C.c_void_p(FAKE + 65536)
    assert lib.zs_reduce_scatter_avg(arr, 0, 0, 2, 0, huge, out, 0, None, 1.0, None) == U
    assert lib.zs_check_overflow(out, huge, 1.0, out, None) == U
    hp = zs.hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
    assert lib.zs_adamw_step(out, out, out, out, huge, C.byref(hp), None, None) == U
    assert lib.zs_cast_gather(out, out, 0, 0, huge, None, None) == U
    assert lib.zs_cast_gather(out, out, 0, huge, 10, None, None) == U
    a, keep = _fused_args(zs, n=huge)
    assert lib.zs_step_fused(C.byref(a), None) == U
    b, keep2 = _fused_args(zs, gather_offset=huge)
    assert lib.zs_step_fused(C.byref(b), None) == U
    reps = (C.c_void_p * 2)(FAKE, FAKE + 0x100000)
    assert lib.zs_all_gather_step(reps, 2, huge, 0, 1, None) == U
    x = (C.c_float * 1)()
    h = (C.c_uint16 * 1)()
    ovf = C.c_uint32(0)
    assert lib.zs_cpu_step(x, x, x, x, huge, C.byref(hp), h, 0, 1, C.byref(ovf)) == U
    assert lib.zs_cpu_update(x, x, x, x, huge, C.byref(hp), h, 0, 1) == U


BAD_HPARAMS = [
    dict(beta1=1.0), dict(beta1=-0.1), dict(beta2=1.0), dict(beta2=float("nan")),
    dict(lr=float("nan")), dict(lr=-1e-3), dict(lr=float("inf")),
    dict(eps=-1e-8), dict(eps=float("nan")),
    dict(weight_decay=-0.01), dict(weight_decay=float("inf")),
]


def _hp(zs, **over):
    kw = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, loss_scale=1.0,
              step_t=1)
    kw.update(over)
    return zs.hparams(**kw)


@pytest.mark.parametrize("bad", BAD_HPARAMS, ids=lambda d: ",".join(f"{k}={v}" for k, v in d.items()))
def test_hyperparameters_out_of_range_are_refused(zs, bad):
    """A beta outside [0, 1) or a negative or non-finite lr, eps or weight
    decay would make every parameter inf or NaN with no overflow reported:
    each entry point that takes them refuses before any launch."""
    lib = _raw(zs)
    E = zs.ZS_ERR_INVALID_ARG
    hp = _hp(zs, **bad)
    p = C.c_void_p(FAKE)
    assert lib.zs_adamw_step(p, p, p, p, 10, C.byref(hp), None, None) == E
    a, keep = _fused_args(zs)
    a.hp = hp
    assert lib.zs_step_fused(C.byref(a), None) == E
    assert lib.zs_step_device(C.byref(a), C.c_void_p(FAKE + 0x7000000), None, None, None) == E
    sc = zs.zs_loss_scaler(scale=1024.0, clean_steps=0, growth_interval=4, dynamic=1,
                           step_t=0, skipped=0)
    hf, ok = C.c_uint32(0), C.c_int(7)
    assert lib.zs_step_commit(C.byref(a), C.byref(sc), C.byref(hf), None, None, None,
                              C.byref(ok)) == E
    assert (sc.scale, sc.step_t, sc.skipped) == (1024.0, 0, 0)
    x = (C.c_float * 4)(0.5, 0.0, 0.0, 0.25)
    h = (C.c_uint16 * 4)()
    ovf = C.c_uint32(9)
    assert lib.zs_cpu_step(x, x, x, x, 4, C.byref(hp), h, 0, 1, C.byref(ovf)) == E
    assert lib.zs_cpu_update(x, x, x, x, 4, C.byref(hp), h, 0, 1) == E
    assert list(x) == [0.5, 0.0, 0.0, 0.25] and ovf.value == 9    # nothing written
    if "beta1" in bad or "beta2" in bad:
        host = zs.zs_loss_scaler(scale=1.0, clean_steps=0, growth_interval=0, dynamic=0,
                                 step_t=0, skipped=0)
        with pytest.raises(zs.ZsError):
            zs.zs_device_scaler_make(host, hp.beta1, hp.beta2)


def test_hyperparameter_range_edges_are_accepted(zs):
    """beta = 0 and lr = eps = weight_decay = 0 are valid settings."""
    lib = _raw(zs)
    hp = _hp(zs, lr=0.0, beta1=0.0, beta2=0.0, eps=0.0, weight_decay=0.0)
    p = C.c_void_p(FAKE)
    assert lib.zs_adamw_step(p, p, p, p, 0, C.byref(hp), None, None) == zs.ZS_OK
    a, keep = _fused_args(zs, n=0)
    a.hp = hp
    assert lib.zs_step_fused(C.byref(a), None) == zs.ZS_OK
    x = (C.c_float * 4)(0.5, 0.0, 0.0, 0.25)
    h = (C.c_uint16 * 4)()
    ovf = C.c_uint32(9)
    assert lib.zs_cpu_step(x, x, x, x, 4, C.byref(hp), h, 0, 1, C.byref(ovf)) == zs.ZS_OK
    assert ovf.value == 0
    zs.zs_device_scaler_make(zs.zs_loss_scaler(scale=1.0, clean_steps=0, growth_interval=0,
                                               dynamic=0, step_t=0, skipped=0), 0.0, 0.0)


def test_offload_step_rejects_bad_arguments(zs):
    """zs_offload_step refuses bad arguments before any HIP call, and an
    empty partition commits without touching the GPU."""
    lib = _raw(zs)
    E = zs.ZS_ERR_INVALID_ARG
    hp = _hp(zs)
    n = 1000
    host = FAKE + 0x40000000
    gd, pd, fd = FAKE, FAKE + 0x100000, FAKE + 0x200000
    gh, ms, m, v, ph, fh = (host + i * 0x100000 for i in range(6))
    ok = C.c_int(7)

    def call(*, n=n, hp=hp, dtype=0, pieces=16, threads=1, **over):
        a = dict(gd=gd, gh=gh, ms=ms, m=m, v=v, ph=ph, pd=pd, fd=fd, fh=fh)
        a.update(over)
        return lib.zs_offload_step(a["gd"], a["gh"], a["ms"], a["m"], a["v"], a["ph"], a["pd"], n,
                                   C.byref(hp) if hp is not None else None, dtype, a["fd"],
                                   a["fh"], threads, pieces, None, C.byref(ok))

    for field in ("gd", "gh", "ms", "m", "v", "ph", "pd", "fd", "fh"):
        assert call(**{field: None}) == E, field
    assert call(hp=None) == E
    assert call(dtype=4) == E
    assert call(pieces=0) == E and call(pieces=1025) == E
    assert call(hp=_hp(zs, step_t=0)) == E
    assert call(hp=_hp(zs, loss_scale=float("inf"))) == E
    assert call(hp=_hp(zs, beta1=1.0)) == E
    assert call(m=ms + 8) == E                       # host buffers overlap
    assert call(ph=v + 4 * n - 2) == E
    assert call(n=1 << 50) == zs.ZS_ERR_UNSUPPORTED
    assert lib.zs_offload_step(gd, gh, ms, m, v, ph, pd, n, C.byref(hp), 0, fd, fh, 1, 16, None,
                               None) == E            # no committed
    assert call(n=0) == zs.ZS_OK and ok.value == 1
