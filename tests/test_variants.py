"""libzsvariants: the fused kernel's alternative shapes that bench.py times
against libzeroshard's (measurement only). A shape is only worth timing if it
computes the step exactly, so each variant is checked against the oracle on
the GPU; its argument checks run on the CPU (no HIP call before them)."""
import ctypes as C

import numpy as np
import pytest

import oracle
from gpu_util import F32, assert_bits_equal, down16, down32, up16, up32

FAKE = 0x7F0000000000


@pytest.fixture(scope="module")
def vlib(hip_built):
    lib = C.CDLL(hip_built.VARIANTS)
    lib.zs_variant_name.restype = C.c_char_p
    lib.zs_variant_name.argtypes = [C.c_int]
    lib.zs_variant_last_error.restype = C.c_char_p
    lib.zs_variant_launch.restype = C.c_int
    lib.zs_variant_launch.argtypes = [C.c_int, C.c_void_p, C.c_uint32, C.c_uint32, C.c_void_p]
    return lib


@pytest.fixture(scope="module")
def zs(hip_built):
    from sharded_mixed_precision_zs_amd import zeroshard
    return zeroshard


def _args(zs, world, n, base=FAKE, **over):
    grads = (C.c_void_p * world)(*[base + k * 0x1000000 for k in range(world)])
    a = zs.zs_step_args()
    a.world, a.rank, a.n = world, 0, n
    a.grad_dtype = a.param_dtype = zs.ZS_BF16
    a.worker_grads = C.cast(grads, C.POINTER(C.c_void_p))
    s = base + 0x40000000
    a.master_in, a.m_in, a.v_in = s, s + 0x1000000, s + 0x2000000
    a.master_out, a.m_out, a.v_out = s + 0x3000000, s + 0x4000000, s + 0x5000000
    a.gather_buf, a.gather_offset = s + 0x6000000, 0
    a.overflow_flag = s + 0x7000000
    a.hp = zs.hparams(1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0, 1)
    for k, v in over.items():
        setattr(a, k, v)
    return a, grads


def test_catalogue(vlib):
    count = vlib.zs_variant_count()
    assert count >= 12
    names = [vlib.zs_variant_name(i).decode() for i in range(count)]
    assert len(set(names)) == count
    assert vlib.zs_variant_name(count) is None and vlib.zs_variant_name(-1) is None
    assert [vlib.zs_variant_multi(i) for i in (0, 5)] == [0, 1]
    assert vlib.zs_variant_tile(0) == 2048 and vlib.zs_variant_tile(5) == 4096
    splits = [i for i in range(count) if "split" in names[i]]
    assert splits and all(vlib.zs_variant_tile(i) in (2048, 4096) for i in splits)
    assert vlib.zs_variant_tile(count) == 0 and vlib.zs_variant_multi(count) == -1


def test_refusals_before_any_launch(vlib, zs):
    E = zs.ZS_ERR_INVALID_ARG
    a, k1 = _args(zs, 1, 4096)
    assert vlib.zs_variant_launch(99, C.addressof(a), 0, 0, None) == E
    assert vlib.zs_variant_launch(5, C.addressof(a), 0, 0, None) == E        # W > 1 variant, W = 1
    b, k2 = _args(zs, 4, 4096)
    assert vlib.zs_variant_launch(0, C.addressof(b), 0, 0, None) == E        # W = 1 variant, W = 4
    c, k3 = _args(zs, 4, 4096 + 2048)
    assert vlib.zs_variant_launch(5, C.addressof(c), 0, 0, None) == E        # ragged for the tile
    for field, val in (("grad_dtype", zs.ZS_FP16), ("wire_dtype", 1), ("acc_in", FAKE + 64),
                       ("master_out", None), ("m_in", FAKE + 0x40000004)):
        d, k4 = _args(zs, 4, 4096, **{field: val})
        assert vlib.zs_variant_launch(5, C.addressof(d), 0, 0, None) == E, field
    assert vlib.zs_variant_launch(5, C.addressof(b), 33, 0, None) == E       # cap out of range
    assert vlib.zs_variant_launch(10, C.addressof(b), 0, 0, None) == E       # persistent, no grid
    assert vlib.zs_variant_launch(5, None, 0, 0, None) == E
    assert vlib.zs_variant_last_error().decode()


@pytest.mark.gpu
@pytest.mark.parametrize("world", [1, 5, 14, 39])
def test_every_variant_computes_the_step(vlib, zs, world):
    """Each variant of the world's family writes the oracle's state and
    parameters bit for bit, at several residency caps; the persistent and
    split variants walk several tiles per block (n is 600 of the smaller
    tiles, against a grid of at most 2 blocks per CU)."""
    import torch
    rng = np.random.default_rng(world)
    n = 600 * 2048
    g16 = [((rng.standard_normal(n) * 1e-3).astype(F32).view(np.uint32) >> 16).astype(np.uint16)
           for _ in range(world)]
    master = (rng.standard_normal(n) * 0.02).astype(F32)
    m = (rng.standard_normal(n) * 1e-4).astype(F32)
    v = rng.uniform(0, 1e-6, n).astype(F32)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    f, mo, mmo, vo, po = oracle.shard_step(g16, 0, "bf16", "bf16", master, m, v, loss_scale=1.0,
                                           step_t=3, threads=4, **hp)
    assert f == 0
    grads = [up16(g, "bf16") for g in g16]
    din = [up32(x) for x in (master, m, v)]
    # grouped layout: [master | m | v] per 1024-element group
    din_g = up32(np.stack([x.reshape(-1, 1024) for x in (master, m, v)], axis=1).ravel())
    for vid in range(vlib.zs_variant_count()):
        if vlib.zs_variant_multi(vid) != (1 if world > 1 else 0):
            continue
        name_v = vlib.zs_variant_name(vid).decode()
        if "phased" in name_v:
            continue  # test_phased_variants_walk_several_chunks
        grouped = "grouped state" in name_v
        for cap in (0, 2, 5):
            if grouped:
                dout_g = torch.full((3 * n,), 7.0, dtype=torch.float32, device="cuda")
                ins, outs = [din_g] * 3, [dout_g] * 3
            else:
                outs = [torch.full((n,), 7.0, dtype=torch.float32, device="cuda") for _ in range(3)]
                ins = din
            par = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
            flag = torch.zeros(1, dtype=torch.int32, device="cuda")
            args = zs.StepArgs(grads, 0, n, *ins, *outs, par, 0, flag,
                               zs.hparams(**hp, loss_scale=1.0, step_t=3))
            rc = vlib.zs_variant_launch(vid, C.addressof(args.args), cap, 2,
                                        torch.cuda.current_stream().cuda_stream)
            assert rc == 0, vlib.zs_variant_last_error().decode()
            torch.cuda.synchronize()
            what = f"variant {vid} ({name_v}) cap {cap}"
            assert int(flag.item()) == 0, what
            if grouped:
                g3 = down32(dout_g).reshape(-1, 3, 1024)
                got3 = [g3[:, k, :].ravel() for k in range(3)]
            else:
                got3 = [down32(x) for x in outs]
            for got, want, name in zip(got3, (mo, mmo, vo), ("master", "m", "v")):
                assert_bits_equal(got, want, f"{what} {name}")
            assert np.array_equal(down16(par), po), what


@pytest.mark.gpu
def test_phased_variants_walk_several_chunks(vlib, zs):
    """The phase-separated variants (cooperative grid, reads and writes in
    separate chunk-wide phases) write the oracle's bits over a shard of two
    to three chunks, the last one partial, at one block per CU."""
    import torch
    world, n = 6, 2200 * 2048
    rng = np.random.default_rng(77)
    g16 = [((rng.standard_normal(n) * 1e-3).astype(F32).view(np.uint32) >> 16).astype(np.uint16)
           for _ in range(world)]
    master = (rng.standard_normal(n) * 0.02).astype(F32)
    m = (rng.standard_normal(n) * 1e-4).astype(F32)
    v = rng.uniform(0, 1e-6, n).astype(F32)
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    f, mo, mmo, vo, po = oracle.shard_step(g16, 2, "bf16", "bf16", master, m, v, loss_scale=8.0,
                                           step_t=5, threads=8, **hp)
    grads = [up16(g, "bf16") for g in g16]
    din = [up32(x) for x in (master, m, v)]
    phased = [i for i in range(vlib.zs_variant_count())
              if "phased" in vlib.zs_variant_name(i).decode()]
    assert phased
    for vid in phased:
        dout = [torch.full((n,), 7.0, dtype=torch.float32, device="cuda") for _ in range(3)]
        par = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
        flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        args = zs.StepArgs(grads, 2, n, *din, *dout, par, 0, flag,
                           zs.hparams(**hp, loss_scale=8.0, step_t=5))
        rc = vlib.zs_variant_launch(vid, C.addressof(args.args), 0, 1,
                                    torch.cuda.current_stream().cuda_stream)
        assert rc == 0, vlib.zs_variant_last_error().decode()
        torch.cuda.synchronize()
        what = f"variant {vid} ({vlib.zs_variant_name(vid).decode()})"
        assert int(flag.item()) == f == 0, what
        for got, want, name in zip(dout, (mo, mmo, vo), ("master", "m", "v")):
            assert_bits_equal(down32(got), want, f"{what} {name}")
        assert np.array_equal(down16(par), po), what
