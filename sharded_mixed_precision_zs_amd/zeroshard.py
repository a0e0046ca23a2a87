"""Python binding of libzeroshard (ctypes): argument marshalling only.

Each function has the name of the C entry point it calls (include/zeroshard.h
documents the semantics and cites the pages). Device buffers are torch CUDA
tensors (or raw integer device addresses); torch supplies memory and the
stream, every step of the computation runs in the library's HIP kernels.
The binding checks that each tensor is a contiguous CUDA tensor of the right
element size holding at least the elements the kernel will touch, then passes
plain pointers. There is no fallback: if the library is missing, importing
this module raises.
"""
import ctypes as C
import os
from typing import Optional, Sequence

from . import build as _build

ZS_ABI_VERSION = 7
ZS_MAX_WORLD = 64
ZS_BF16, ZS_FP16 = 0, 1
ZS_WIRE_FP32, ZS_WIRE_BF16, ZS_WIRE_FP16 = 0, 1, 2
ZS_STATE_SPLIT, ZS_STATE_GROUPED = 0, 1
ZS_STATE_GROUP = 1024
ZS_OK, ZS_ERR_INVALID_ARG, ZS_ERR_UNSUPPORTED, ZS_ERR_ALIAS, ZS_ERR_HIP = range(5)

LIB_PATH = _build.LIB


class ZsError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__(f"{fn}: {zs_status_string(status)}: {detail}")
        self.status = status


class zs_adamw_hparams(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float),
                ("eps", C.c_float), ("weight_decay", C.c_float),
                ("loss_scale", C.c_float), ("step_t", C.c_uint32)]


class zs_step_args(C.Structure):
    _fields_ = [("world", C.c_uint32), ("rank", C.c_uint32), ("n", C.c_uint64),
                ("grad_dtype", C.c_int32), ("param_dtype", C.c_int32),
                ("worker_grads", C.POINTER(C.c_void_p)),
                ("acc_in", C.c_void_p),
                ("master_in", C.c_void_p), ("m_in", C.c_void_p), ("v_in", C.c_void_p),
                ("master_out", C.c_void_p), ("m_out", C.c_void_p), ("v_out", C.c_void_p),
                ("gather_buf", C.c_void_p), ("gather_offset", C.c_uint64),
                ("overflow_flag", C.c_void_p),
                ("hp", zs_adamw_hparams), ("wire_dtype", C.c_int32),
                ("state_layout", C.c_int32)]


def grouped_len(n):
    """Floats in a grouped state buffer for n elements (whole groups)."""
    return -(-n // ZS_STATE_GROUP) * 3 * ZS_STATE_GROUP


class zs_loss_scaler(C.Structure):
    _fields_ = [("scale", C.c_float), ("clean_steps", C.c_uint32),
                ("growth_interval", C.c_uint32), ("dynamic", C.c_uint32),
                ("step_t", C.c_uint64), ("skipped", C.c_uint64)]


class zs_device_scaler(C.Structure):
    _fields_ = [("scale", C.c_float), ("clean_steps", C.c_uint32),
                ("growth_interval", C.c_uint32), ("dynamic", C.c_uint32),
                ("step_t", C.c_uint64), ("skipped", C.c_uint64),
                ("beta1_t", C.c_double), ("beta2_t", C.c_double),
                ("epoch", C.c_uint64), ("flag_epoch", C.c_uint64), ("checked_epoch", C.c_uint64),
                ("last_flag", C.c_uint32), ("bad_scale", C.c_uint32),
                ("last_alpha", C.c_float), ("last_bc2", C.c_float)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libzeroshard is not built ({LIB_PATH}); "
                          "run __graft_entry__.build() -- there is no fallback path")
    # the library maps torch's HIP runtime whatever the import order (see
    # build.py), so it shares torch's streams and allocations
    lib = C.CDLL(LIB_PATH)
    vp, u32, u64, f32, i32 = C.c_void_p, C.c_uint32, C.c_uint64, C.c_float, C.c_int
    sig = {
        "zs_abi_version": ([], i32),
        "zs_status_string": ([i32], C.c_char_p),
        "zs_last_error": ([], C.c_char_p),
        "zs_partition": ([u64, u32, u32, C.POINTER(u64), C.POINTER(u64), C.POINTER(u64)], i32),
        "zs_reduce_scatter_avg": ([C.POINTER(vp), i32, i32, u32, u32, u64, vp, i32, vp, f32, vp],
                                  i32),
        "zs_check_overflow": ([vp, u64, f32, vp, vp], i32),
        "zs_adamw_step": ([vp, vp, vp, vp, u64, C.POINTER(zs_adamw_hparams), vp, vp], i32),
        "zs_cast_gather": ([vp, vp, i32, u64, u64, vp, vp], i32),
        "zs_step_fused": ([C.POINTER(zs_step_args), vp], i32),
        "zs_scaler_update": ([C.POINTER(zs_loss_scaler), u32], i32),
        "zs_step_commit": ([C.POINTER(zs_step_args), C.POINTER(zs_loss_scaler), vp, vp, vp, vp,
                            C.POINTER(C.c_int)], i32),
        "zs_step_commit_noalloc": ([C.POINTER(zs_step_args), C.POINTER(zs_loss_scaler), vp, vp,
                                    vp, vp, C.POINTER(C.c_int)], i32),
        "zs_all_gather_step": ([C.POINTER(vp), u32, u64, u32, u32, vp], i32),
        "zs_cpu_step": ([vp, vp, vp, vp, u64, C.POINTER(zs_adamw_hparams), vp, i32, i32,
                         C.POINTER(u32)], i32),
        "zs_cpu_update": ([vp, vp, vp, vp, u64, C.POINTER(zs_adamw_hparams), vp, i32, i32], i32),
        "zs_device_scaler_make": ([C.POINTER(zs_loss_scaler), f32, f32,
                                   C.POINTER(zs_device_scaler)], i32),
        "zs_step_device": ([C.POINTER(zs_step_args), vp, vp, vp, vp], i32),
        "zs_offload_step": ([vp, vp, vp, vp, vp, vp, vp, u64, C.POINTER(zs_adamw_hparams), i32,
                             vp, vp, i32, i32, vp, C.POINTER(C.c_int)], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes, f.restype = args, res
    if lib.zs_abi_version() != ZS_ABI_VERSION:
        raise ImportError("libzeroshard ABI version mismatch")
    return lib


_lib = _load()


# ---- marshalling helpers ----------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t, explicit):
    if explicit is not None:
        return int(explicit)
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ZS_BF16
    if t.dtype == torch.float16:
        return ZS_FP16
    raise TypeError(f"16-bit float tensor expected, got {t.dtype}; pass the dtype explicitly")


def _ptr(x, n, elem, what, offset=0):
    """Device address of x after checking it holds offset+n elements of `elem` bytes."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError(f"{what}: CUDA tensor expected")
    if not x.is_contiguous():
        raise ValueError(f"{what}: contiguous tensor expected")
    if x.element_size() != elem:
        raise ValueError(f"{what}: {elem}-byte elements expected, got {x.element_size()}")
    if x.numel() < offset + n:
        raise ValueError(f"{what}: needs {offset + n} elements, has {x.numel()}")
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return C.c_void_p(_torch().cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def _check(fn, status, detail=None):
    if status != ZS_OK:
        raise ZsError(fn, status, detail if detail is not None else zs_last_error())


# The host update (offload_cpu.cpp) reports status codes only.
_CPU_DETAIL = {
    ZS_ERR_INVALID_ARG: "a null pointer, a bad param dtype, a loss scale that is not finite "
                        "and > 0, step_t == 0, or a hyper-parameter out of range",
    ZS_ERR_UNSUPPORTED: "n exceeds 2^48 elements",
}


def hparams(lr, beta1, beta2, eps, weight_decay, loss_scale, step_t):
    return zs_adamw_hparams(lr, beta1, beta2, eps, weight_decay, loss_scale, step_t)


# ---- entry points -----------------------------------------------------------

def zs_abi_version():
    return _lib.zs_abi_version()


def zs_status_string(status):
    return _lib.zs_status_string(status).decode()


def zs_last_error():
    return _lib.zs_last_error().decode()


def zs_partition(phi, world, rank):
    """Returns (chunk, offset, count)."""
    p, o, c = C.c_uint64(), C.c_uint64(), C.c_uint64()
    _check("zs_partition", _lib.zs_partition(phi, world, rank, C.byref(p), C.byref(o), C.byref(c)))
    return p.value, o.value, c.value


def _grad_array(worker_grads, n):
    ptrs = [_ptr(g, n, 2, f"worker_grads[{k}]") for k, g in enumerate(worker_grads)]
    return (C.c_void_p * len(ptrs))(*ptrs)


def zs_reduce_scatter_avg(worker_grads: Sequence, grad_dtype: Optional[int], world: int,
                          rank: int, n: int, grad_part, accumulate=False,
                          overflow_flag=None, loss_scale=1.0, stream=None,
                          wire_dtype=ZS_WIRE_FP32):
    if len(worker_grads) != world:
        raise ValueError("len(worker_grads) must equal world")
    arr = _grad_array(worker_grads, n)
    dt = _dtype_code(worker_grads[0], grad_dtype) if world else 0
    _check("zs_reduce_scatter_avg", _lib.zs_reduce_scatter_avg(
        arr, dt, wire_dtype, world, rank, n, _ptr(grad_part, n, 4, "grad_part"),
        1 if accumulate else 0, _ptr(overflow_flag, 1, 4, "overflow_flag"), loss_scale,
        _stream(stream)))


def zs_check_overflow(grad_part, n, loss_scale, overflow_flag, stream=None):
    _check("zs_check_overflow", _lib.zs_check_overflow(
        _ptr(grad_part, n, 4, "grad_part"), n, loss_scale,
        _ptr(overflow_flag, 1, 4, "overflow_flag"), _stream(stream)))


def zs_adamw_step(master, m, v, grad_part, n, hp: zs_adamw_hparams, overflow_flag=None,
                  stream=None):
    _check("zs_adamw_step", _lib.zs_adamw_step(
        _ptr(master, n, 4, "master"), _ptr(m, n, 4, "m"), _ptr(v, n, 4, "v"),
        _ptr(grad_part, n, 4, "grad_part"), n, C.byref(hp),
        _ptr(overflow_flag, 1, 4, "overflow_flag"), _stream(stream)))


def zs_cast_gather(master, gather_buf, param_dtype: Optional[int], offset, n,
                   overflow_flag=None, stream=None):
    dt = _dtype_code(gather_buf, param_dtype)
    _check("zs_cast_gather", _lib.zs_cast_gather(
        _ptr(master, n, 4, "master"), _ptr(gather_buf, n, 2, "gather_buf", offset), dt,
        offset, n, _ptr(overflow_flag, 1, 4, "overflow_flag"), _stream(stream)))


class StepArgs:
    """A prepared zs_step_args: built once, re-pointed cheaply between steps
    (swap() exchanges the input and output sets after a committed step)."""

    def __init__(self, worker_grads, rank, n, master_in, m_in, v_in, master_out, m_out, v_out,
                 gather_buf, gather_offset, overflow_flag, hp: zs_adamw_hparams,
                 acc_in=None, grad_dtype=None, param_dtype=None, gather_in=None,
                 wire_dtype=ZS_WIRE_FP32, state_layout=ZS_STATE_SPLIT):
        """state_layout ZS_STATE_GROUPED: master_in / master_out are grouped
        state buffers (grouped_len(n) floats); m_in, v_in, m_out, v_out None."""
        world = len(worker_grads)
        self._grads = _grad_array(worker_grads, n)
        a = zs_step_args()
        a.world, a.rank, a.n = world, rank, n
        a.grad_dtype = _dtype_code(worker_grads[0], grad_dtype)
        a.param_dtype = _dtype_code(gather_buf, param_dtype)
        a.worker_grads = C.cast(self._grads, C.POINTER(C.c_void_p))
        a.acc_in = _ptr(acc_in, n, 4, "acc_in")
        ns = grouped_len(n) if state_layout == ZS_STATE_GROUPED else n
        a.master_in, a.m_in, a.v_in = (_ptr(master_in, ns, 4, "master_in"), _ptr(m_in, n, 4, "m_in"),
                                       _ptr(v_in, n, 4, "v_in"))
        a.master_out, a.m_out, a.v_out = (_ptr(master_out, ns, 4, "master_out"),
                                          _ptr(m_out, n, 4, "m_out"), _ptr(v_out, n, 4, "v_out"))
        a.state_layout = state_layout
        a.gather_buf = _ptr(gather_buf, n, 2, "gather_buf", gather_offset)
        # Optional second gather buffer: with one per set, a skipped step also
        # leaves the current set's 16-bit parameters untouched.
        self._gather_in = _ptr(gather_in, n, 2, "gather_in", gather_offset)
        a.gather_offset = gather_offset
        a.overflow_flag = _ptr(overflow_flag, 1, 4, "overflow_flag")
        a.hp = hp
        a.wire_dtype = wire_dtype
        self.args = a

    def set_grads(self, worker_grads):
        n = self.args.n
        for k, g in enumerate(worker_grads):
            self._grads[k] = _ptr(g, n, 2, f"worker_grads[{k}]")

    def swap(self):
        a = self.args
        a.master_in, a.master_out = a.master_out, a.master_in
        a.m_in, a.m_out = a.m_out, a.m_in
        a.v_in, a.v_out = a.v_out, a.v_in
        if self._gather_in is not None:
            a.gather_buf, self._gather_in = self._gather_in, a.gather_buf


def zs_step_fused(args, stream=None):
    """args: a StepArgs (or a raw zs_step_args)."""
    raw = args.args if isinstance(args, StepArgs) else args
    _check("zs_step_fused", _lib.zs_step_fused(C.byref(raw), _stream(stream)))


def zs_scaler_update(state: zs_loss_scaler, overflow):
    _check("zs_scaler_update", _lib.zs_scaler_update(C.byref(state), 1 if overflow else 0))


def zs_step_commit(args, scaler: zs_loss_scaler, host_flag, stream=None, ev_start=None,
                   ev_stop=None):
    """Fused step + flag readback + scaler update (blocks). host_flag: a
    (pinned) host tensor or address of at least 4 bytes. Returns committed."""
    raw = args.args if isinstance(args, StepArgs) else args
    hf = host_flag if isinstance(host_flag, int) else host_flag.data_ptr()
    committed = C.c_int(0)
    _check("zs_step_commit", _lib.zs_step_commit(C.byref(raw), C.byref(scaler), hf,
                                                 _stream(stream), ev_start, ev_stop,
                                                 C.byref(committed)))
    return bool(committed.value)


def zs_step_commit_noalloc(args, scaler: zs_loss_scaler, host_flag, stream=None, ev_start=None,
                           ev_stop=None):
    """zs_step_commit with the overflow word in the library's own device
    memory (args' overflow_flag is not used). Returns committed."""
    raw = args.args if isinstance(args, StepArgs) else args
    hf = host_flag if isinstance(host_flag, int) else host_flag.data_ptr()
    committed = C.c_int(0)
    _check("zs_step_commit_noalloc",
           _lib.zs_step_commit_noalloc(C.byref(raw), C.byref(scaler), hf, _stream(stream),
                                       ev_start, ev_stop, C.byref(committed)))
    return bool(committed.value)


DEVICE_SCALER_BYTES = C.sizeof(zs_device_scaler)


def zs_device_scaler_make(scaler: zs_loss_scaler, beta1: float, beta2: float) -> zs_device_scaler:
    """Host image of a device-resident scaler continuing from `scaler`."""
    out = zs_device_scaler()
    _check("zs_device_scaler_make", _lib.zs_device_scaler_make(C.byref(scaler), beta1, beta2,
                                                               C.byref(out)))
    return out


def device_scaler_upload(image: zs_device_scaler, device="cuda"):
    """A device buffer (uint8 CUDA tensor) holding `image`."""
    torch = _torch()
    raw = bytes(memoryview(image).cast("B"))
    host = torch.frombuffer(bytearray(raw), dtype=torch.uint8)
    return host.to(device)


def device_scaler_read(dev_buf) -> zs_device_scaler:
    """Host copy of a device scaler buffer. Waits for all work on the
    buffer's device first: steps may be queued on any stream."""
    torch = _torch()
    torch.cuda.synchronize(dev_buf.device)
    raw = dev_buf[:DEVICE_SCALER_BYTES].cpu().numpy().tobytes()
    return zs_device_scaler.from_buffer_copy(raw)


def device_scaler_write(dev_buf, image: zs_device_scaler):
    """Overwrite a device scaler buffer with `image`. Waits for all work on
    the device before and after the copy, so no queued step on any stream
    sees a partly written scaler."""
    torch = _torch()
    raw = bytes(memoryview(image).cast("B"))
    torch.cuda.synchronize(dev_buf.device)
    dev_buf[:DEVICE_SCALER_BYTES].copy_(torch.frombuffer(bytearray(raw), dtype=torch.uint8))
    torch.cuda.synchronize(dev_buf.device)


def _dev_scaler_ptr(dev):
    return _ptr(dev, DEVICE_SCALER_BYTES, 1, "device scaler")


def zs_step_device(args, dev, stream=None, ev_start=None, ev_stop=None):
    """Fused step + on-device commit or skip (never waits). dev: the device
    scaler buffer (device_scaler_upload) or its address."""
    raw = args.args if isinstance(args, StepArgs) else args
    _check("zs_step_device", _lib.zs_step_device(C.byref(raw), _dev_scaler_ptr(dev),
                                                 _stream(stream), ev_start, ev_stop))


def zs_all_gather_step(replicas: Sequence, phi: int, step: int, sigma: int = 0, stream=None):
    """One ring all-gather step over len(replicas) flat 16-bit buffers."""
    ptrs = [_ptr(r, phi, 2, f"replicas[{k}]") for k, r in enumerate(replicas)]
    arr = (C.c_void_p * len(ptrs))(*ptrs)
    _check("zs_all_gather_step", _lib.zs_all_gather_step(arr, len(ptrs), phi, sigma, step,
                                                         _stream(stream)))


def _host_args(fn, master, m, v, grad_part, params16, param_dtype):
    """Pointers and size of host tensors/arrays (torch CPU tensors or numpy
    arrays, contiguous) for the host update entry points."""
    def hptr(x, elem, what):
        if hasattr(x, "data_ptr"):
            if x.is_cuda or not x.is_contiguous() or x.element_size() != elem:
                raise ValueError(f"{what}: contiguous host tensor of {elem}-byte elements expected")
            return x.data_ptr(), x.numel()
        if not x.flags.c_contiguous or x.itemsize != elem:
            raise ValueError(f"{what}: contiguous array of {elem}-byte elements expected")
        return x.ctypes.data, x.size
    (pm, n), (p1, n1), (p2, n2), (pg, n3) = (hptr(master, 4, "master"), hptr(m, 4, "m"),
                                              hptr(v, 4, "v"), hptr(grad_part, 4, "grad_part"))
    pp, n4 = hptr(params16, 2, "params16")
    if not (n == n1 == n2 == n3 <= n4):
        raise ValueError(f"{fn}: size mismatch")
    if param_dtype is None:
        param_dtype = _dtype_code(params16, None) if hasattr(params16, "dtype") and \
            str(params16.dtype).startswith("torch") else ZS_BF16
    return pm, p1, p2, pg, n, pp, param_dtype


def zs_cpu_step(master, m, v, grad_part, hp: zs_adamw_hparams, params16, param_dtype=None,
                threads=0):
    """ZeRO-Offload update on host memory. Returns the overflow flag (1: skipped)."""
    pm, p1, p2, pg, n, pp, dt = _host_args("zs_cpu_step", master, m, v, grad_part, params16,
                                           param_dtype)
    flag = C.c_uint32(0)
    rc = _lib.zs_cpu_step(pm, p1, p2, pg, n, C.byref(hp), pp, dt, threads, C.byref(flag))
    _check("zs_cpu_step", rc, _CPU_DETAIL.get(rc, ""))
    return int(flag.value)


def zs_cpu_update(master, m, v, grad_part, hp: zs_adamw_hparams, params16, param_dtype=None,
                  threads=0):
    """zs_cpu_step without its check (the caller has checked the gradient)."""
    pm, p1, p2, pg, n, pp, dt = _host_args("zs_cpu_update", master, m, v, grad_part, params16,
                                           param_dtype)
    rc = _lib.zs_cpu_update(pm, p1, p2, pg, n, C.byref(hp), pp, dt, threads)
    _check("zs_cpu_update", rc, _CPU_DETAIL.get(rc, ""))


def _host_ptr(x, n, elem, what):
    """Address of a contiguous host (CPU) tensor or array of >= n elements of
    `elem` bytes."""
    if hasattr(x, "data_ptr"):
        if x.is_cuda or not x.is_contiguous() or x.element_size() != elem or x.numel() < n:
            raise ValueError(f"{what}: contiguous host tensor of >= {n} {elem}-byte elements "
                             "expected")
        return x.data_ptr()
    if not x.flags.c_contiguous or x.itemsize != elem or x.size < n:
        raise ValueError(f"{what}: contiguous array of >= {n} {elem}-byte elements expected")
    return x.ctypes.data


def zs_offload_step(grad_dev, grad_host, master, m, v, params_host, params_dev,
                    hp: zs_adamw_hparams, flag_dev, flag_host, param_dtype=None, threads=0,
                    pieces=16, stream=None):
    """Pipelined ZeRO-Offload step (blocks until the host update is done).
    grad_dev, params_dev, flag_dev: CUDA tensors; grad_host, master, m, v,
    params_host, flag_host: host tensors (the staging ones pinned). n is
    master's length. Returns True when committed, False when skipped."""
    n = master.numel() if hasattr(master, "numel") else master.size
    if param_dtype is None:
        param_dtype = _dtype_code(params_dev, None)
    committed = C.c_int(0)
    rc = _lib.zs_offload_step(
        _ptr(grad_dev, n, 4, "grad_dev"), _host_ptr(grad_host, n, 4, "grad_host"),
        _host_ptr(master, n, 4, "master"), _host_ptr(m, n, 4, "m"), _host_ptr(v, n, 4, "v"),
        _host_ptr(params_host, n, 2, "params_host"), _ptr(params_dev, n, 2, "params_dev"), n,
        C.byref(hp), param_dtype, _ptr(flag_dev, 1, 4, "flag_dev"),
        _host_ptr(flag_host, 1, 4, "flag_host"), threads, pieces, _stream(stream),
        C.byref(committed))
    _check("zs_offload_step", rc)
    return bool(committed.value)
