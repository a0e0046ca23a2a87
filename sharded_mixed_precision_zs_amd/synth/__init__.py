"""Seeded synthetic inputs for the shard step (host and device twins).

This module generates inputs only; it holds none of the step's arithmetic.
Values are a pure function of (seed, stream, worker, step, micro-batch, flat
index) -- see ``synth_core.h`` for the definition -- so the device can fill
multi-GB buffers in HBM while the host regenerates any window of them for the
oracle. A worker's gradient at flat index ``i`` does not depend on how the flat
buffer is partitioned.

Workloads
---------
The five workloads below are the shard-step configurations this library is
tested and benchmarked on. Distributions ``N(0, s)`` take ``s`` as the standard
deviation; 16-bit gradients are the fp32 sample truncated toward zero.
"""
import ctypes as C
import math
import os
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libzssynth_host.so")
DEV_LIB = os.path.join(HERE, "libzssynth_dev.so")

BF16, FP16 = 0, 1
STREAM_GRAD, STREAM_MASTER, STREAM_M, STREAM_V, STREAM_INJECT = 1, 2, 3, 4, 5
_IH_STD = math.sqrt((2.0 ** 32 - 1.0) / 3.0)  # std of a sum of four 16-bit uniforms


@dataclass(frozen=True)
class Workload:
    name: str
    phi: int                      # flat parameter count of the model
    world: int                    # W data-parallel workers
    rank: int                     # the rank whose shard is stepped
    grad_dtype: int
    param_dtype: int
    grad_sigma: float             # std of the unscaled gradient
    master_sigma: float
    m_sigma: float                # 0: m starts at zero
    v_hi: float                   # 0: v starts at zero; else U(0, v_hi)
    lr: float
    beta1: float
    beta2: float
    eps: float
    weight_decay: float
    loss_scale: float             # initial (dynamic) or fixed (static) scale
    dynamic_scale: bool
    scale_interval: int           # clean steps before the scale doubles
    steps: int
    accum: int                    # micro-batches per optimizer step
    inject_steps: Tuple[int, ...] = ()
    inject_rate: float = 0.0
    seed: int = 0
    bucket: int = 0               # bucket size in elements (0: one bucket)
    tensors: Tuple[int, ...] = field(default=())
    description: str = ""

    @property
    def chunk(self):
        return -(-self.phi // self.world)

    @property
    def offset(self):
        return self.rank * self.chunk

    @property
    def n(self):
        return max(0, min(self.chunk, self.phi - self.offset))

    def bytes_per_param(self):
        """Algorithmic HBM bytes per parameter of one optimizer step
        (read, write) for the single-pass step with micro-batch accumulation."""
        w, a = self.world, self.accum
        read = 2 * w * a + 4 * (a - 1) + 12
        write = 4 * (a - 1) + 14
        return read, write


WORKLOADS = {
    "mlp9-w3": Workload(
        name="mlp9-w3", phi=2 ** 20, world=3, rank=0, grad_dtype=BF16, param_dtype=BF16,
        grad_sigma=1e-3, master_sigma=0.02, m_sigma=0.0, v_hi=0.0,
        lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01,
        loss_scale=1024.0, dynamic_scale=False, scale_interval=0, steps=1, accum=1, seed=0,
        tensors=(116508,) * 8 + (116512,),
        description="9-tensor MLP, flat phi=2^20, W=3, bf16 grads x1024, static scale 1024"),
    "gpt2s-w8": Workload(
        name="gpt2s-w8", phi=124_439_808, world=8, rank=0, grad_dtype=BF16, param_dtype=BF16,
        grad_sigma=1e-3, master_sigma=0.02, m_sigma=1e-4, v_hi=1e-6,
        lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01,
        loss_scale=65536.0, dynamic_scale=False, scale_interval=0, steps=5, accum=1, seed=1,
        bucket=25_000_000,
        description="GPT-2-small-shaped flat phi=124,439,808, W=8, bf16 grads x65536, warm m/v"),
    "7p5b-shard-w64": Workload(
        name="7p5b-shard-w64", phi=7_500_000_000, world=64, rank=0, grad_dtype=BF16,
        param_dtype=BF16, grad_sigma=1e-3, master_sigma=0.02, m_sigma=0.0, v_hi=0.0,
        lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01,
        loss_scale=1.0, dynamic_scale=False, scale_interval=0, steps=3, accum=1, seed=2,
        description="7.5B model, rank-0 shard at N=64 (117,187,500 params), 64 bf16 workers"),
    "7b-full-w1": Workload(
        name="7b-full-w1", phi=7_000_000_000, world=1, rank=0, grad_dtype=BF16,
        param_dtype=BF16, grad_sigma=1e-3, master_sigma=0.02, m_sigma=0.0, v_hi=0.0,
        lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1,
        loss_scale=1.0, dynamic_scale=False, scale_interval=0, steps=2, accum=1, seed=3,
        description="7B model, full state on one rank (W=1), bf16 grads"),
    "1p3b-w4-acc4-fp16": Workload(
        name="1p3b-w4-acc4-fp16", phi=1_300_000_000, world=4, rank=0, grad_dtype=FP16,
        param_dtype=FP16, grad_sigma=1e-3, master_sigma=0.02, m_sigma=0.0, v_hi=0.0,
        lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01,
        loss_scale=65536.0, dynamic_scale=True, scale_interval=4, steps=10, accum=4,
        inject_steps=(3, 7), inject_rate=1e-3, seed=4,
        description="1.3B, W=4, 4 micro-batches, fp16 grads x dynamic scale, inf/NaN at steps 3, 7"),
}


def ks_normal(sigma, scale=1.0):
    """fp32 multiplier turning the centred Irwin-Hall integer into N(0, sigma)*scale."""
    k = np.float32(sigma / _IH_STD)
    s = np.float32(scale)
    if scale != 1.0 and (math.frexp(scale)[0] != 0.5):
        raise ValueError("gradient scale must be a power of two (exact multiply)")
    return np.float32(k * s)


def ku_uniform(hi):
    return np.float32(hi / 2.0 ** 24)


def inject_threshold(rate):
    return int(math.floor(rate * 2.0 ** 32))


# ---- host library ---------------------------------------------------------

_host = None


def _host_lib():
    global _host
    if _host is not None:
        return _host
    if not os.path.exists(HOST_LIB):
        from .. import build as _b
        _b.build_synth_host()
    lib = C.CDLL(HOST_LIB)
    lib.zsg_key_host.argtypes = [C.c_uint64, C.c_uint32, C.c_uint32, C.c_uint32, C.c_uint32]
    lib.zsg_key_host.restype = C.c_uint64
    lib.zsg_fill_normal_f32.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64, C.c_float, C.c_void_p]
    lib.zsg_fill_uniform_f32.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64, C.c_float, C.c_void_p]
    lib.zsg_fill_grad16.argtypes = [C.c_uint64, C.c_uint64, C.c_uint32, C.c_uint64, C.c_uint64,
                                    C.c_float, C.c_int, C.c_void_p]
    _host = lib
    return lib


def key(seed, stream, worker=0, step=0, micro=0):
    return int(_host_lib().zsg_key_host(seed, stream, worker, step, micro))


def normal_f32(k, first, n, ks):
    out = np.empty(n, np.float32)
    _host_lib().zsg_fill_normal_f32(k, first, n, float(ks), out.ctypes.data)
    return out


def uniform_f32(k, first, n, ku):
    out = np.empty(n, np.float32)
    _host_lib().zsg_fill_uniform_f32(k, first, n, float(ku), out.ctypes.data)
    return out


def grad16(k, kinj, threshold, first, n, ks, dtype):
    out = np.empty(n, np.uint16)
    _host_lib().zsg_fill_grad16(k, kinj, threshold, first, n, float(ks), dtype, out.ctypes.data)
    return out


# ---- workload-level host generation (flat indices) --------------------------

def grad_scale_at(wl: Workload, scale: Optional[float]):
    return wl.loss_scale if scale is None else scale


def host_grad(wl: Workload, worker, step, micro, first, n, scale=None):
    """Worker `worker`'s 16-bit gradient bits at flat indices [first, first+n)
    for optimizer step `step` (1-based) and micro-batch `micro`."""
    ks = ks_normal(wl.grad_sigma, grad_scale_at(wl, scale))
    kg = key(wl.seed, STREAM_GRAD, worker, step, micro)
    thr = inject_threshold(wl.inject_rate) if step in wl.inject_steps else 0
    kinj = key(wl.seed, STREAM_INJECT, worker, step, micro)
    return grad16(kg, kinj, thr, first, n, ks, wl.grad_dtype)


def host_state(wl: Workload, first, n):
    """Initial (master, m, v) at flat indices [first, first+n)."""
    master = normal_f32(key(wl.seed, STREAM_MASTER), first, n, ks_normal(wl.master_sigma))
    m = (normal_f32(key(wl.seed, STREAM_M), first, n, ks_normal(wl.m_sigma))
         if wl.m_sigma else np.zeros(n, np.float32))
    v = (uniform_f32(key(wl.seed, STREAM_V), first, n, ku_uniform(wl.v_hi))
         if wl.v_hi else np.zeros(n, np.float32))
    return master, m, v


# ---- device library -------------------------------------------------------

_dev = None


def _dev_lib():
    global _dev
    if _dev is not None:
        return _dev
    if not os.path.exists(DEV_LIB):
        raise RuntimeError(f"device generator not built: {DEV_LIB} (run __graft_entry__.build())")
    lib = C.CDLL(DEV_LIB)
    lib.zsg_dev_fill_normal_f32.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64, C.c_float,
                                            C.c_void_p, C.c_void_p]
    lib.zsg_dev_fill_uniform_f32.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64, C.c_float,
                                             C.c_void_p, C.c_void_p]
    lib.zsg_dev_fill_grad16.argtypes = [C.c_uint64, C.c_uint64, C.c_uint32, C.c_uint64,
                                        C.c_uint64, C.c_float, C.c_int, C.c_void_p, C.c_void_p]
    for f in (lib.zsg_dev_fill_normal_f32, lib.zsg_dev_fill_uniform_f32, lib.zsg_dev_fill_grad16):
        f.restype = C.c_int
    _dev = lib
    return lib


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"device generator: {what} failed")


def _stream_ptr(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def dev_grad(wl: Workload, worker, step, micro, first, out, scale=None, stream=None):
    """Fill `out` (torch uint16/int16/bf16/fp16 CUDA tensor, contiguous) with the
    same bits as host_grad(wl, worker, step, micro, first, out.numel())."""
    ks = ks_normal(wl.grad_sigma, grad_scale_at(wl, scale))
    kg = key(wl.seed, STREAM_GRAD, worker, step, micro)
    thr = inject_threshold(wl.inject_rate) if step in wl.inject_steps else 0
    kinj = key(wl.seed, STREAM_INJECT, worker, step, micro)
    assert out.is_cuda and out.is_contiguous() and out.element_size() == 2
    _check(_dev_lib().zsg_dev_fill_grad16(kg, kinj, thr, first, out.numel(), float(ks),
                                          wl.grad_dtype, out.data_ptr(), _stream_ptr(stream)),
           "grad16")


def dev_state(wl: Workload, first, master, m, v, stream=None):
    """Fill fp32 CUDA tensors (master, m, v) with host_state(wl, first, n)."""
    lib = _dev_lib()
    sp = _stream_ptr(stream)
    n = master.numel()
    for t in (master, m, v):
        assert t.is_cuda and t.is_contiguous() and t.numel() == n and t.element_size() == 4
    _check(lib.zsg_dev_fill_normal_f32(key(wl.seed, STREAM_MASTER), first, n,
                                       float(ks_normal(wl.master_sigma)), master.data_ptr(), sp),
           "master")
    if wl.m_sigma:
        _check(lib.zsg_dev_fill_normal_f32(key(wl.seed, STREAM_M), first, n,
                                           float(ks_normal(wl.m_sigma)), m.data_ptr(), sp), "m")
    else:
        m.zero_()
    if wl.v_hi:
        _check(lib.zsg_dev_fill_uniform_f32(key(wl.seed, STREAM_V), first, n,
                                            float(ku_uniform(wl.v_hi)), v.data_ptr(), sp), "v")
    else:
        v.zero_()
