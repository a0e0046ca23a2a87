"""Host-side driver of one rank's ZeRO-2 shard step (built on the C ABI only).

`ShardState` owns this rank's optimizer shard in HBM -- two sets of fp32
(master, m, v) and two 16-bit gather buffers (ping-pong), the overflow flag
and the loss scaler -- and runs one optimizer step in one of two ways.
step() decides on the host:

    zs_step_fused(in-set -> out-set)    one pass over HBM
    flag -> host (4 bytes)              the only synchronization
    flag == 0: swap sets, t += 1        commit
    flag == 1: keep the in-set          skip (scale halves when dynamic)

step_device() (device_commit=True) decides on the GPU with no host round
trip: the fused pass reads the scale from a device-resident scaler, a
commit kernel restores the out-set on a skip and updates the scaler, and
the sets swap every step. Both follow the owner's update sequence of the DeepSpeed ZeRO notes (section
三): gradients averaged and unscaled in fp32, moments and master updated, the
16-bit copy refreshed for the all-gather. Micro-batches before the last are
reduced into an fp32 accumulator with zs_reduce_scatter_avg (lecture 7,
"Gradient Accumulation"). All arithmetic runs in libzeroshard's kernels;
torch only allocates memory and provides the stream.
"""
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

from . import zeroshard as zs


@dataclass
class AdamW:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01


class ShardState:
    """One rank's shard: n parameters at flat offset `offset` of a model with
    `world` data-parallel ranks; gather buffers hold `gather_len` elements.
    state_layout: "split" (master, m and v as three arrays) or "grouped"
    (one buffer per set in libzeroshard's grouped layout, ZS_STATE_GROUPED)."""

    FLAG_RING = 256  # flags zeroed in bulk, one slot per step
    FILL_CHUNK = 1 << 26  # elements per piece when filling a grouped set

    def __init__(self, n, world, rank, offset, gather_len, param_dtype, grad_dtype,
                 opt: AdamW, loss_scale, dynamic=False, growth_interval=0,
                 device="cuda", accumulate=False, wire_dtype=zs.ZS_WIRE_FP32,
                 device_commit=False, state_layout="split"):
        self.n, self.world, self.rank, self.offset = n, world, rank, offset
        self.wire_dtype = wire_dtype  # precision of the ring's partial sums
        self.param_dtype, self.grad_dtype = param_dtype, grad_dtype
        self.opt = opt
        layouts = {"split": zs.ZS_STATE_SPLIT, "grouped": zs.ZS_STATE_GROUPED}
        if state_layout not in layouts:
            raise ValueError(f"state_layout must be one of {sorted(layouts)}")
        self.state_layout = layouts[state_layout]
        f32 = dict(dtype=torch.float32, device=device)
        if self.state_layout == zs.ZS_STATE_GROUPED:
            self.sets = [[torch.empty(zs.grouped_len(n), **f32)] for _ in range(2)]
        else:
            self.sets = [[torch.empty(n, **f32) for _ in range(3)] for _ in range(2)]
        pdt = torch.bfloat16 if param_dtype == zs.ZS_BF16 else torch.float16
        self.gather = [torch.zeros(gather_len, dtype=pdt, device=device) for _ in range(2)]
        self.cur = 0
        self.acc = torch.empty(n, **f32) if accumulate else None
        self.flags = torch.zeros(self.FLAG_RING, dtype=torch.int32, device=device)
        self.flag_host = torch.zeros(1, dtype=torch.int32, pin_memory=True)
        self.slot = 0
        self.scaler = zs.zs_loss_scaler(scale=loss_scale, clean_steps=0,
                                        growth_interval=growth_interval,
                                        dynamic=1 if dynamic else 0, step_t=0, skipped=0)
        self.last_flag = 0
        self._prepared = {}
        self._flag_base = self.flags.data_ptr()
        self._bound = None
        # device-resident commit-or-skip: the scaler lives in HBM and steps
        # are queued without waiting (step_device); self.scaler is refreshed
        # by sync_scaler()
        self.device_commit = device_commit
        self._dev_betas = None
        self.dev = self._upload_scaler() if device_commit else None
        self.device = device

    # -- state access -------------------------------------------------------
    def _array(self, k):
        """Array k (0 master, 1 m, 2 v) of the current set: the tensor itself
        (split), or a (groups, 1024) strided view of the grouped buffer."""
        x = self.sets[self.cur]
        if self.state_layout == zs.ZS_STATE_GROUPED:
            return x[0].view(-1, 3, zs.ZS_STATE_GROUP)[:, k, :]
        return x[k]

    @property
    def master(self):
        return self._array(0)

    @property
    def m(self):
        return self._array(1)

    @property
    def v(self):
        return self._array(2)

    def state(self, k, first=0, count=None):
        """Elements [first, first + count) of array k (0 master, 1 m, 2 v) of
        the current set as a contiguous device tensor: a view with the split
        layout, a copy of the groups it spans with the grouped one."""
        count = self.n - first if count is None else count
        if self.state_layout != zs.ZS_STATE_GROUPED:
            return self.sets[self.cur][k][first:first + count]
        G = zs.ZS_STATE_GROUP
        g0, g1 = first // G, -(-(first + count) // G)
        flat = self._array(k)[g0:g1].reshape(-1)
        return flat[first - g0 * G:first - g0 * G + count]

    def write_state(self, k, first, src):
        """Copy the device tensor src into elements [first, first + len(src))
        of array k of the current set."""
        count = src.numel()
        if self.state_layout != zs.ZS_STATE_GROUPED:
            self.sets[self.cur][k][first:first + count].copy_(src)
            return
        G = zs.ZS_STATE_GROUP
        g0, g1 = first // G, -(-(first + count) // G)
        blk = self._array(k)[g0:g1]
        flat = blk.reshape(-1).clone()
        flat[first - g0 * G:first - g0 * G + count] = src
        blk.copy_(flat.view(g1 - g0, G))

    def fill_state(self, fill):
        """fill(first, count, master, m, v) writes elements [first, first +
        count) of the three arrays into the contiguous fp32 device tensors it
        is given; this calls it once (split) or in pieces of FILL_CHUNK
        elements (grouped) and stores the result in the current set."""
        if self.state_layout != zs.ZS_STATE_GROUPED:
            fill(0, self.n, *self.sets[self.cur])
            return
        dev = self.sets[self.cur][0].device
        for first in range(0, self.n, self.FILL_CHUNK):
            count = min(self.FILL_CHUNK, self.n - first)
            tmp = [torch.empty(count, dtype=torch.float32, device=dev) for _ in range(3)]
            fill(first, count, *tmp)
            for k in range(3):
                self.write_state(k, first, tmp[k])

    @property
    def params(self):
        """This rank's slice of the current 16-bit gather buffer."""
        return self.gather[self.cur][self.offset:self.offset + self.n]

    @property
    def t(self):
        return int(self.scaler.step_t)

    @property
    def loss_scale(self):
        return float(self.scaler.scale)

    # -- checkpoint / resume ---------------------------------------------------
    def state_dict(self):
        """Host copy of everything the next step depends on: the current fp32
        set, this rank's 16-bit parameters and the scaler (waits for every
        queued step, on any stream)."""
        torch.cuda.synchronize(self.sets[0][0].device)
        if self.device_commit:
            self.sync_scaler()
        sc = self.scaler
        return {"master": self.state(0).cpu(), "m": self.state(1).cpu(), "v": self.state(2).cpu(),
                "params": self.params.cpu(),
                "scaler": {"scale": float(sc.scale), "clean_steps": int(sc.clean_steps),
                           "growth_interval": int(sc.growth_interval), "dynamic": int(sc.dynamic),
                           "step_t": int(sc.step_t), "skipped": int(sc.skipped)}}

    def load_state_dict(self, sd):
        """Restore a state_dict() into the current set (shapes must match;
        waits for every queued step first, on any stream)."""
        torch.cuda.synchronize(self.sets[0][0].device)
        for key in ("master", "m", "v"):
            if tuple(sd[key].shape) != (self.n,) or sd[key].dtype != torch.float32:
                raise ValueError(f"state_dict[{key!r}] has the wrong shape or dtype")
        if sd["params"].shape != self.params.shape or sd["params"].dtype != self.params.dtype:
            raise ValueError("state_dict['params'] has the wrong shape or dtype")
        for k, key in enumerate(("master", "m", "v")):
            self.write_state(k, 0, sd[key].to(self.sets[0][0].device))
        self.params.copy_(sd["params"])
        for k, v in sd["scaler"].items():
            setattr(self.scaler, k, v)
        if self.device_commit:
            zs.device_scaler_write(self.dev, self._scaler_image())

    # -- device-resident scaler ---------------------------------------------
    def _scaler_image(self):
        """Device-scaler image continuing self.scaler with the current betas."""
        self._dev_betas = (self.opt.beta1, self.opt.beta2)
        return zs.zs_device_scaler_make(self.scaler, self.opt.beta1, self.opt.beta2)

    def _upload_scaler(self):
        return zs.device_scaler_upload(self._scaler_image(), self.sets[0][0].device)

    def sync_scaler(self):
        """Wait for the queued steps and copy the device scaler into
        self.scaler; returns the device image."""
        d = zs.device_scaler_read(self.dev)
        for k in ("scale", "clean_steps", "growth_interval", "dynamic", "step_t", "skipped"):
            setattr(self.scaler, k, getattr(d, k))
        self.last_flag = int(d.last_flag)
        return d

    def hparams(self):
        o = self.opt
        return zs.hparams(o.lr, o.beta1, o.beta2, o.eps, o.weight_decay, self.loss_scale,
                          self.t + 1)

    def _refresh_hparams(self, args):
        """Write the step's settings into prepared arguments: self.opt may
        change between steps (a learning-rate schedule), the scale and t
        change with every commit or skip."""
        args.args.hp = self.hparams()

    # -- flag ring ----------------------------------------------------------
    def _next_flag_addr(self, stream=None):
        """Device address of a fresh zeroed uint32 flag slot. The ring is
        re-zeroed on the stream of the step that will use it (the earlier
        slots' steps ran on that stream or were waited for)."""
        if self.slot == self.FLAG_RING:
            if stream is None:
                stream = torch.cuda.current_stream()
            elif isinstance(stream, int):
                stream = torch.cuda.ExternalStream(stream)
            with torch.cuda.stream(stream):
                self.flags.zero_()
            self.slot = 0
        addr = self._flag_base + 4 * self.slot
        self.slot += 1
        return addr

    def _next_flag(self, stream=None):
        addr = self._next_flag_addr(stream)
        i = (addr - self._flag_base) // 4
        return self.flags[i:i + 1]

    # -- micro-batches before the last one ------------------------------------
    def reduce_micro(self, worker_grads: Sequence[torch.Tensor], first: bool, stream=None):
        """acc = mean of this micro-batch's worker gradients (first) or
        acc += that mean (later micro-batches). No overflow check here: a
        non-finite partial stays non-finite through the accumulation, and the
        step's fused pass checks (acc + last average) / scale."""
        zs.zs_reduce_scatter_avg(worker_grads, self.grad_dtype, self.world, self.rank, self.n,
                                 self.acc, accumulate=not first, overflow_flag=None,
                                 loss_scale=1.0, stream=stream, wire_dtype=self.wire_dtype)

    # -- one optimizer step -------------------------------------------------
    def _args(self, worker_grads, acc_in):
        """Prepared zs_step_args for the current direction (cached by pointers)."""
        key = (self.cur, tuple(g.data_ptr() for g in worker_grads),
               acc_in.data_ptr() if acc_in is not None else 0)
        args = self._prepared.get(key)
        if args is None:
            src, dst = self.sets[self.cur], self.sets[1 - self.cur]
            if self.state_layout == zs.ZS_STATE_GROUPED:
                src, dst = [src[0], None, None], [dst[0], None, None]
            args = zs.StepArgs(worker_grads, self.rank, self.n, src[0], src[1], src[2],
                               dst[0], dst[1], dst[2], self.gather[1 - self.cur], self.offset,
                               self.flags[0:1], self.hparams(), acc_in=acc_in,
                               grad_dtype=self.grad_dtype, param_dtype=self.param_dtype,
                               wire_dtype=self.wire_dtype, state_layout=self.state_layout)
            if len(self._prepared) > 16:
                self._prepared.clear()
            self._prepared[key] = args
        return args

    def launch(self, worker_grads: Sequence[torch.Tensor], acc_in: Optional[torch.Tensor] = None,
               stream=None):
        """Enqueue the fused step without waiting; returns the device flag
        slot it ORs into (finish() reads it back)."""
        flag = self._next_flag(stream)
        args = self._args(worker_grads, acc_in)
        self._refresh_hparams(args)
        args.args.overflow_flag = flag.data_ptr()
        zs.zs_step_fused(args, stream)
        return flag

    def finish(self, flag, stream=None):
        """Read the flag back (the step's only synchronization), then commit or
        skip. `stream` must be the one launch() used: the copy is ordered
        after the step on it."""
        if stream is None:
            s = torch.cuda.current_stream()
        elif isinstance(stream, int):
            s = torch.cuda.ExternalStream(stream)
        else:
            s = stream
        with torch.cuda.stream(s):
            self.flag_host.copy_(flag, non_blocking=True)
        s.synchronize()
        self.last_flag = int(self.flag_host[0])
        zs.zs_scaler_update(self.scaler, self.last_flag)
        if self.last_flag == 0:
            self.cur = 1 - self.cur
        return self.last_flag == 0

    def _step_args(self, worker_grads, acc_in):
        if worker_grads is not None:
            args = self._args(worker_grads, acc_in)
        elif self._bound is None:
            raise RuntimeError("no gradients given and none bound: call bind() first")
        else:
            args = self._bound[self.cur]
        self._refresh_hparams(args)
        return args

    def bind(self, worker_grads: Sequence[torch.Tensor], acc_in: Optional[torch.Tensor] = None):
        """Prepare both directions' arguments once for gradients that stay at
        the same addresses every step; step() with no gradients uses them."""
        saved = self.cur
        pair = []
        for c in (0, 1):
            self.cur = c
            pair.append(self._args(worker_grads, acc_in))
        self.cur = saved
        self._bound = pair

    def step(self, worker_grads=None, acc_in=None, stream=None, ev_start=None, ev_stop=None):
        """One optimizer step through zs_step_commit (launch, flag readback,
        scaler update in one native call); returns True when committed.
        ev_start / ev_stop: optional raw hipEvent_t handles around the kernel."""
        args = self._step_args(worker_grads, acc_in)
        args.args.overflow_flag = self._next_flag_addr(stream)
        ok = zs.zs_step_commit(args, self.scaler, self.flag_host, stream, ev_start, ev_stop)
        self.last_flag = 0 if ok else 1
        if ok:
            self.cur = 1 - self.cur
        return ok

    def step_device(self, worker_grads=None, acc_in=None, stream=None, ev_start=None,
                    ev_stop=None):
        """One optimizer step through zs_step_device: queued, never waits. The
        commit or skip happens on the device, which leaves the state after
        the step in the output set either way, so the sets swap every call;
        sync_scaler() reads the outcome. lr, eps and weight decay are read
        from self.opt at every call; the beta powers live on the device, so
        a change of betas waits for the queued steps once and re-forms
        beta^(t+1) from the new values (what the host flow computes)."""
        if not self.device_commit:
            raise RuntimeError("ShardState was built without device_commit=True")
        if (self.opt.beta1, self.opt.beta2) != self._dev_betas:
            self.sync_scaler()
            zs.device_scaler_write(self.dev, self._scaler_image())
        args = self._step_args(worker_grads, acc_in)
        zs.zs_step_device(args, self.dev, stream, ev_start, ev_stop)
        self.cur = 1 - self.cur

    def capture(self, worker_grads=None, acc_in=None):
        """Capture two device-commit steps, one per direction of the ping-pong
        sets, into a HIP graph and return a function that replays them (two
        steps per call; the sets end where they started). For shards small
        enough that launching from Python costs more than the kernels.
        The graph holds this moment's hyper-parameters and gradient
        addresses: refill the same gradient buffers between replays, and
        capture again after changing the settings."""
        if not self.device_commit:
            raise RuntimeError("ShardState was built without device_commit=True")
        if worker_grads is not None:
            self.bind(worker_grads, acc_in)
        if self._bound is None:
            raise RuntimeError("no gradients given and none bound: call bind() first")
        if (self.opt.beta1, self.opt.beta2) != self._dev_betas:   # waits: not inside a capture
            self.sync_scaler()
            zs.device_scaler_write(self.dev, self._scaler_image())
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                self.step_device()
                self.step_device()
        torch.cuda.current_stream().wait_stream(side)
        return graph.replay


class OffloadShard:
    """ZeRO-Offload variant of one rank's shard (the DeepSpeed introduction,
    item (16)): fp32 master, m and v live in host memory and the update runs
    on the host; the GPU keeps the W-way ring-order reduction
    (zs_reduce_scatter_avg) and the 16-bit parameters. Per step, 4 bytes per
    parameter cross PCIe to the host (the averaged fp32 gradient) and 2 back
    (the parameters), against the fused GPU step's 12 B/param of optimizer
    state kept in HBM. The arithmetic is the fused step's, element for
    element, so both variants produce the same bits.

    A step is one native call (zs_offload_step): the overflow check runs on
    the GPU and its flag reaches the host first, so a skipped step does no
    host work; the gradient then comes back in `pieces` pieces while the host
    pool updates the pieces already there, and each finished piece's
    parameters go back at once."""

    def __init__(self, n, world, rank, offset, gather_len, param_dtype, grad_dtype,
                 opt: AdamW, loss_scale, dynamic=False, growth_interval=0, device="cuda",
                 threads=0, wire_dtype=zs.ZS_WIRE_FP32, pieces=16):
        self.n, self.world, self.rank, self.offset = n, world, rank, offset
        self.param_dtype, self.grad_dtype, self.opt = param_dtype, grad_dtype, opt
        self.threads, self.wire_dtype, self.pieces = threads, wire_dtype, pieces
        pdt = torch.bfloat16 if param_dtype == zs.ZS_BF16 else torch.float16
        self.master = torch.empty(n, dtype=torch.float32)
        self.m = torch.zeros(n, dtype=torch.float32)
        self.v = torch.zeros(n, dtype=torch.float32)
        self.grad = torch.empty(n, dtype=torch.float32, device=device)   # reduced, on the GPU
        self.grad_host = torch.empty(n, dtype=torch.float32, pin_memory=True)
        self.params_host = torch.empty(n, dtype=pdt, pin_memory=True)
        self.gather = torch.zeros(gather_len, dtype=pdt, device=device)
        self.scaler = zs.zs_loss_scaler(scale=loss_scale, clean_steps=0,
                                        growth_interval=growth_interval,
                                        dynamic=1 if dynamic else 0, step_t=0, skipped=0)
        self.last_flag = 0
        self.flag_dev = torch.zeros(1, dtype=torch.int32, device=device)
        self.flag_host = torch.zeros(1, dtype=torch.int32, pin_memory=True)

    @property
    def params(self):
        return self.gather[self.offset:self.offset + self.n]

    @property
    def t(self):
        return int(self.scaler.step_t)

    @property
    def loss_scale(self):
        return float(self.scaler.scale)

    def reduce_micro(self, worker_grads, first: bool, stream=None):
        """Reduce one micro-batch's gradients into the device partition."""
        zs.zs_reduce_scatter_avg(worker_grads, self.grad_dtype, self.world, self.rank, self.n,
                                 self.grad, accumulate=not first, overflow_flag=None,
                                 loss_scale=self.loss_scale, stream=stream,
                                 wire_dtype=self.wire_dtype)

    def step(self, worker_grads=None, first=True, stream=None):
        """Reduce the last micro-batch (unless worker_grads is None, when it
        was reduced already), then the pipelined check, transfer and host
        update of zs_offload_step. Returns True when committed."""
        if worker_grads is not None:
            self.reduce_micro(worker_grads, first, stream)
        o = self.opt
        hp = zs.hparams(o.lr, o.beta1, o.beta2, o.eps, o.weight_decay, self.loss_scale,
                        self.t + 1)
        ok = zs.zs_offload_step(self.grad, self.grad_host, self.master, self.m, self.v,
                                self.params_host, self.params, hp, self.flag_dev, self.flag_host,
                                self.param_dtype, self.threads, self.pieces, stream)
        flag = 0 if ok else 1
        zs.zs_scaler_update(self.scaler, flag)
        self.last_flag = flag
        return ok
