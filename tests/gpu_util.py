"""Helpers for the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np

F32 = np.float32


def announce(msg):
    """Name the case on stderr before GPU work (survives pytest capture)."""
    sys.__stderr__.write(f"[gpu] {msg}\n")
    sys.__stderr__.flush()


def torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype in (0, "bf16") else torch.float16


def up16(bits, dtype):
    """uint16 numpy bits -> torch CUDA tensor of the 16-bit float dtype."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).cuda()
    return t.view(torch_dtype(dtype))


def up32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, F32).copy()).cuda()


def down16(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def down32(t):
    return t.cpu().numpy()


def bits32(x):
    return np.ascontiguousarray(x, F32).view(np.uint32)


def assert_bits_equal(got, want, what):
    """Bit-exact fp32 equality; NaNs compared by class."""
    got, want = np.asarray(got, F32), np.asarray(want, F32)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    bad = bits32(got)[~gn] != bits32(want)[~wn]
    if bad.any():
        i = np.flatnonzero(~gn)[np.flatnonzero(bad)[0]]
        raise AssertionError(f"{what}: {bad.sum()} of {got.size} differ; first at {i}: "
                             f"got {got[i]!r} want {want[i]!r}")


def assert_rel(got, want, rtol, what):
    """|got - want| <= rtol * |want| elementwise (0 must be exact); NaN by class.
    Returns the number of elements that are not bit-identical."""
    got, want = np.asarray(got, F32), np.asarray(want, F32)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    g, w = got[~gn].astype(np.float64), want[~wn].astype(np.float64)
    inf = np.isinf(w)
    assert np.array_equal(g[inf], w[inf]), f"{what}: inf mismatch"
    g, w = g[~inf], w[~inf]
    err = np.abs(g - w)
    bad = err > rtol * np.abs(w)
    if bad.any():
        i = np.flatnonzero(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {w.size} beyond rtol {rtol}; "
                             f"e.g. got {g[i]!r} want {w[i]!r}")
    return int((bits32(got)[~gn] != bits32(want)[~wn]).sum())


def _ordered16(bits, dtype):
    """Map 16-bit float bits to integers ordered like the values."""
    b = np.asarray(bits, np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def assert_ulp16(got, want, dtype, max_ulp, what):
    got, want = np.asarray(got, np.uint16), np.asarray(want, np.uint16)
    nanmask = 0x7F80 if dtype in (0, "bf16") else 0x7C00
    fracmask = 0x007F if dtype in (0, "bf16") else 0x03FF

    def isnan(b):
        b = b.astype(np.int32)
        return ((b & nanmask) == nanmask) & ((b & fracmask) != 0)

    gn, wn = isnan(got), isnan(want)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    d = np.abs(_ordered16(got[~gn], dtype) - _ordered16(want[~wn], dtype))
    if (d > max_ulp).any():
        i = np.flatnonzero(d > max_ulp)[0]
        raise AssertionError(f"{what}: {int((d > max_ulp).sum())} beyond {max_ulp} ulp; "
                             f"e.g. {got[~gn][i]:#06x} vs {want[~wn][i]:#06x}")
    return int((d != 0).sum())


def oracle_offload_update(master, m, v, grad, loss_scale, lr, beta1, beta2, eps, weight_decay,
                          t, param_dtype):
    """What the oracle computes for one ZeRO-Offload update of an averaged,
    still loss-scaled fp32 gradient partition: the overflow flag of the
    unscaled gradient; on a clean step the AdamW update of copies of
    (master, m, v) and the 16-bit cast of the new master; on a skipped step
    the inputs unchanged and no parameters (None)."""
    import oracle
    flag = oracle.check_overflow(grad, loss_scale)
    state = [np.array(x, F32, copy=True) for x in (master, m, v)]
    if flag:
        return flag, state, None
    oracle.adamw(*state, grad, loss_scale, lr, beta1, beta2, eps, weight_decay, t)
    return flag, state, oracle.float_to_half(state[0], param_dtype)


def assert_offload_matches_oracle(host_state, params_bits, want, param_dtype, what):
    """host_state (master, m, v as numpy) and the device parameters against
    oracle_offload_update's result, at the parity bar (fp32 within 1e-6
    relative, 16-bit within 1 ulp); returns the elements not bit-identical."""
    flag, state, params = want
    nonbit = 0
    for got, ref, name in zip(host_state, state, ("master", "m", "v")):
        nonbit += assert_rel(got, ref, 1e-6, f"{what} {name} vs oracle")
    if params is not None:
        nonbit += assert_ulp16(params_bits, params, param_dtype, 1, f"{what} params vs oracle")
    return nonbit
