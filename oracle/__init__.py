"""CPU oracle of the per-rank ZeRO-2 optimizer-shard step (ctypes over liboracle.so).

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package. It shares no
code with the GPU library; the two meet only through the seeded input
generator, which holds none of the step's arithmetic.

Every function works on numpy arrays (16-bit floats travel as ``uint16`` bit
patterns). The C sources (``zs_oracle.c``) cite the pages each step follows.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

BF16 = 0
FP16 = 1
_DTYPES = {"bf16": BF16, "fp16": FP16, BF16: BF16, FP16: FP16}
WIRE_FP32, WIRE_BF16, WIRE_FP16 = 0, 1, 2
_WIRES = {"fp32": 0, "bf16": 1, "fp16": 2, 0: 0, 1: 1, 2: 2, None: 0}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # ZSO_ORACLE_LIB: load another build of the oracle (the mutation test
    # points it at copies with planted mistakes)
    path = os.environ.get("ZSO_ORACLE_LIB")
    if path is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        path = _build.LIB
    lib = C.CDLL(path)
    u16p = C.POINTER(C.c_uint16)
    f32p = C.POINTER(C.c_float)
    u64p = C.POINTER(C.c_uint64)
    lib.zso_fp_env_ok.restype = C.c_int
    lib.zso_partition.argtypes = [C.c_uint64, C.c_uint32, C.c_uint32, u64p, u64p, u64p]
    lib.zso_partition.restype = C.c_int
    lib.zso_half_to_float.argtypes = [C.c_uint16, C.c_int]
    lib.zso_half_to_float.restype = C.c_float
    lib.zso_float_to_half.argtypes = [C.c_float, C.c_int]
    lib.zso_float_to_half.restype = C.c_uint16
    lib.zso_halves_to_floats.argtypes = [u16p, f32p, C.c_uint64, C.c_int]
    lib.zso_floats_to_halves.argtypes = [f32p, u16p, C.c_uint64, C.c_int]
    lib.zso_ring_reduce_scatter.argtypes = [C.c_uint32, C.c_uint64, C.c_int, C.c_uint32, f32p]
    lib.zso_ring_reduce_scatter.restype = C.c_int
    lib.zso_ring_all_gather.argtypes = [C.c_uint32, C.c_uint64, C.c_int, C.c_uint32, f32p]
    lib.zso_ring_all_gather.restype = C.c_int
    lib.zso_ring_held_chunk.argtypes = [C.c_uint32, C.c_uint32, C.c_int]
    lib.zso_ring_held_chunk.restype = C.c_uint32
    lib.zso_ring_chunk_sum.argtypes = [C.c_uint32, C.c_uint32, C.POINTER(u16p), C.c_int, C.c_uint64, f32p]
    lib.zso_reduce_avg.argtypes = [C.c_uint32, C.c_uint32, C.POINTER(u16p), C.c_int, C.c_uint64,
                                   f32p, C.c_int, C.c_float]
    lib.zso_reduce_avg.restype = C.c_uint32
    lib.zso_reduce_avg_wire.argtypes = [C.c_uint32, C.c_uint32, C.POINTER(u16p), C.c_int, C.c_int,
                                        C.c_uint64, f32p, C.c_int, C.c_float]
    lib.zso_reduce_avg_wire.restype = C.c_uint32
    lib.zso_ring_chunk_sum_wire.argtypes = [C.c_uint32, C.c_uint32, C.POINTER(u16p), C.c_int,
                                            C.c_int, C.c_uint64, f32p]
    lib.zso_check_overflow.argtypes = [f32p, C.c_uint64, C.c_float]
    lib.zso_check_overflow.restype = C.c_uint32
    lib.zso_adamw_consts_make.argtypes = [C.c_float] * 5 + [C.c_uint32, C.POINTER(AdamWConsts)]
    lib.zso_adamw.argtypes = [f32p, f32p, f32p, f32p, C.c_uint64, C.c_float, C.POINTER(AdamWConsts)]
    lib.zso_shard_step.argtypes = [C.POINTER(_StepArgs), C.c_int]
    lib.zso_shard_step.restype = C.c_uint32
    lib.zso_scaler_update.argtypes = [C.POINTER(ScalerState), C.c_uint32]
    lib.zso_model_state_bytes.argtypes = [C.c_double, C.c_double, C.c_int, C.c_double]
    lib.zso_model_state_bytes.restype = C.c_double
    lib.zso_ring_allreduce_time.argtypes = [C.c_double] * 4
    lib.zso_ring_allreduce_time.restype = C.c_double
    if not lib.zso_fp_env_ok():
        raise RuntimeError("oracle: floating-point environment flushes subnormals "
                           "or does not round to nearest-even")
    _lib = lib
    return lib


class AdamWConsts(C.Structure):
    _fields_ = [("alpha", C.c_float), ("b2", C.c_float), ("delta", C.c_float),
                ("c1", C.c_float), ("c2", C.c_float), ("beta1", C.c_float),
                ("beta2", C.c_float), ("eps", C.c_float)]


class _StepArgs(C.Structure):
    _fields_ = [("world", C.c_uint32), ("rank", C.c_uint32), ("n", C.c_uint64),
                ("grad_dtype", C.c_int), ("param_dtype", C.c_int),
                ("part", C.POINTER(C.POINTER(C.c_uint16))),
                ("acc_in", C.POINTER(C.c_float)),
                ("master_in", C.POINTER(C.c_float)), ("m_in", C.POINTER(C.c_float)),
                ("v_in", C.POINTER(C.c_float)),
                ("master_out", C.POINTER(C.c_float)), ("m_out", C.POINTER(C.c_float)),
                ("v_out", C.POINTER(C.c_float)),
                ("param_out", C.POINTER(C.c_uint16)),
                ("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float),
                ("eps", C.c_float), ("weight_decay", C.c_float), ("loss_scale", C.c_float),
                ("step_t", C.c_uint32), ("wire", C.c_int)]


class ScalerState(C.Structure):
    _fields_ = [("scale", C.c_float), ("clean", C.c_uint32), ("interval", C.c_uint32),
                ("t", C.c_uint64), ("skipped", C.c_uint64)]


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(C.POINTER(C.c_float))


def _u16(a):
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return a, a.ctypes.data_as(C.POINTER(C.c_uint16))


def _parts(parts):
    keep = [np.ascontiguousarray(p, dtype=np.uint16) for p in parts]
    arr = (C.POINTER(C.c_uint16) * len(keep))(*[p.ctypes.data_as(C.POINTER(C.c_uint16)) for p in keep])
    return keep, arr


def dtype_code(dtype):
    return _DTYPES[dtype]


# ---- a1: partition --------------------------------------------------------

def partition(phi, world, rank):
    """(chunk P, offset, count) of rank `rank` in a flat buffer of phi elements."""
    lib = _load()
    p, o, c = C.c_uint64(), C.c_uint64(), C.c_uint64()
    if lib.zso_partition(phi, world, rank, C.byref(p), C.byref(o), C.byref(c)) != 0:
        raise ValueError("bad partition arguments")
    return p.value, o.value, c.value


# ---- 16-bit formats -------------------------------------------------------

def half_to_float(bits, dtype):
    lib = _load()
    bits, bp = _u16(bits)
    out = np.empty(bits.shape, np.float32)
    lib.zso_halves_to_floats(bp, out.ctypes.data_as(C.POINTER(C.c_float)), bits.size, dtype_code(dtype))
    return out


def float_to_half(x, dtype):
    lib = _load()
    x, xp = _f32(x)
    out = np.empty(x.shape, np.uint16)
    lib.zso_floats_to_halves(xp, out.ctypes.data_as(C.POINTER(C.c_uint16)), x.size, dtype_code(dtype))
    return out


# ---- a2: the ring ---------------------------------------------------------

def ring_reduce_scatter(bufs, sigma, steps):
    """In place on a (W, W*L) float32 array; see zs_oracle.h."""
    lib = _load()
    assert bufs.dtype == np.float32 and bufs.flags.c_contiguous and bufs.ndim == 2
    w = bufs.shape[0]
    assert bufs.shape[1] % w == 0
    rc = lib.zso_ring_reduce_scatter(w, bufs.shape[1] // w, sigma, steps,
                                     bufs.ctypes.data_as(C.POINTER(C.c_float)))
    if rc != 0:
        raise ValueError("bad ring arguments")
    return bufs


def ring_all_gather(bufs, sigma, steps):
    lib = _load()
    assert bufs.dtype == np.float32 and bufs.flags.c_contiguous and bufs.ndim == 2
    w = bufs.shape[0]
    rc = lib.zso_ring_all_gather(w, bufs.shape[1] // w, sigma, steps,
                                 bufs.ctypes.data_as(C.POINTER(C.c_float)))
    if rc != 0:
        raise ValueError("bad ring arguments")
    return bufs


def ring_held_chunk(world, rank, sigma):
    return _load().zso_ring_held_chunk(world, rank, sigma)


def ring_chunk_sum(parts, rank, dtype, wire=None):
    """Ring-order sum of rank `rank`'s partition (parts in worker order), the
    partials carried in fp32 (default) or rounded to `wire` at every hop."""
    lib = _load()
    keep, arr = _parts(parts)
    n = keep[0].size
    out = np.empty(n, np.float32)
    if _WIRES[wire] == WIRE_FP32:
        lib.zso_ring_chunk_sum(len(keep), rank, arr, dtype_code(dtype), n,
                               out.ctypes.data_as(C.POINTER(C.c_float)))
    else:
        lib.zso_ring_chunk_sum_wire(len(keep), rank, arr, dtype_code(dtype), _WIRES[wire], n,
                                    out.ctypes.data_as(C.POINTER(C.c_float)))
    return out


# ---- a3-a5 ----------------------------------------------------------------

def reduce_avg(parts, rank, dtype, out, accumulate, loss_scale, wire=None):
    """out = ring_sum/W (or out += ring_sum/W); returns the overflow flag."""
    lib = _load()
    keep, arr = _parts(parts)
    assert out.dtype == np.float32 and out.flags.c_contiguous and out.size == keep[0].size
    return int(lib.zso_reduce_avg_wire(len(keep), rank, arr, dtype_code(dtype), _WIRES[wire],
                                       out.size, out.ctypes.data_as(C.POINTER(C.c_float)),
                                       1 if accumulate else 0, loss_scale))


def check_overflow(a, loss_scale):
    lib = _load()
    a, ap = _f32(a)
    return int(lib.zso_check_overflow(ap, a.size, loss_scale))


# ---- a7 -------------------------------------------------------------------

def adamw_consts(lr, beta1, beta2, eps, weight_decay, t):
    k = AdamWConsts()
    _load().zso_adamw_consts_make(lr, beta1, beta2, eps, weight_decay, t, C.byref(k))
    return {f: getattr(k, f) for f, _ in AdamWConsts._fields_}


def adamw(master, m, v, a, loss_scale, lr, beta1, beta2, eps, weight_decay, t):
    """In-place AdamW on float32 arrays; g = a / loss_scale."""
    lib = _load()
    for x in (master, m, v):
        assert x.dtype == np.float32 and x.flags.c_contiguous
    a, ap = _f32(a)
    k = AdamWConsts()
    lib.zso_adamw_consts_make(lr, beta1, beta2, eps, weight_decay, t, C.byref(k))
    lib.zso_adamw(master.ctypes.data_as(C.POINTER(C.c_float)),
                  m.ctypes.data_as(C.POINTER(C.c_float)),
                  v.ctypes.data_as(C.POINTER(C.c_float)), ap, master.size, loss_scale, C.byref(k))


# ---- the whole step -------------------------------------------------------

def shard_step(parts, rank, grad_dtype, param_dtype, master, m, v, *, lr, beta1, beta2,
               eps, weight_decay, loss_scale, step_t, acc_in=None, threads=1, wire=None):
    """One shard step; returns (flag, master_out, m_out, v_out, param_out_bits)."""
    lib = _load()
    keep, arr = _parts(parts)
    n = keep[0].size
    master, mp = _f32(master)
    m, m_p = _f32(m)
    v, vp = _f32(v)
    assert master.size == m.size == v.size == n
    outs = [np.empty(n, np.float32) for _ in range(3)]
    pout = np.empty(n, np.uint16)
    a = _StepArgs()
    a.world, a.rank, a.n = len(keep), rank, n
    a.grad_dtype, a.param_dtype = dtype_code(grad_dtype), dtype_code(param_dtype)
    a.part = arr
    if acc_in is not None:
        acc_in, accp = _f32(acc_in)
        assert acc_in.size == n
        a.acc_in = accp
    a.master_in, a.m_in, a.v_in = mp, m_p, vp
    a.master_out, a.m_out, a.v_out = [o.ctypes.data_as(C.POINTER(C.c_float)) for o in outs]
    a.param_out = pout.ctypes.data_as(C.POINTER(C.c_uint16))
    a.lr, a.beta1, a.beta2, a.eps = lr, beta1, beta2, eps
    a.weight_decay, a.loss_scale, a.step_t = weight_decay, loss_scale, step_t
    a.wire = _WIRES[wire]
    flag = lib.zso_shard_step(C.byref(a), threads)
    if flag == 0xFFFFFFFF:
        raise MemoryError("oracle: thread allocation failed")
    return int(flag), outs[0], outs[1], outs[2], pout


# ---- a6: scaler; accounting ------------------------------------------------

class Scaler:
    """Dynamic loss scaler (halve on overflow, double after `interval` clean steps)."""

    def __init__(self, scale, interval, t=0):
        self.s = ScalerState(scale=scale, clean=0, interval=interval, t=t, skipped=0)

    def update(self, overflow):
        _load().zso_scaler_update(C.byref(self.s), 1 if overflow else 0)

    scale = property(lambda self: self.s.scale)
    t = property(lambda self: self.s.t)
    clean = property(lambda self: self.s.clean)
    skipped = property(lambda self: self.s.skipped)


def model_state_bytes(psi, n_gpus, stage, k=12.0):
    return _load().zso_model_state_bytes(psi, n_gpus, stage, k)


def ring_allreduce_time(msg_bytes, world, alpha, beta):
    return _load().zso_ring_allreduce_time(msg_bytes, world, alpha, beta)
